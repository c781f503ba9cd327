"""CPU oracle of the layer around the write/read op (test infrastructure only: the tests, ``smoke()`` and the bench's
``cpu_baseline`` leg may use it; the product path never does).

What it computes (sparse-delta-memory README.md, usage example ``SparseDeltaMemoryArgs(dim, num_heads,
slots_per_head, num_writes, num_reads, chunk_size)`` and "Behavior changes": a layer call runs the projections, the
top-k and the bank copy, then the op; README "ideas": the gated delta-rule update of Gated DeltaNet, whose A/dt
parameterisation of the gates the layer matches). The pages name the parts but not their shapes; the reading taken
here (the plainest one) is:

* one input map ``x w_in^T`` whose output rows are, in order, the write keys (H F dk, head-major), the read queries
  (H F dk), the values (H d), the forget-gate inputs a (H) and the input-gate inputs b (H);
* forget gate ``alpha = exp(-exp(A_log[h]) * softplus(a + dt_bias[h]))`` and input gate ``beta = sigmoid(b)``;
* the write/read op (``sdm_oracle.write_read``) on those tensors and the bank;
* the output map ``o w_out^T`` from the H d op outputs back to the model width.

Every tensor between the steps is a bfloat16 tensor (the layer runs in bfloat16, README usage example), so the
oracle rounds each to bfloat16 (nearest, ties to even) after computing it in fp64.

Pins (``tests/test_layer_oracle_pins.py``): the dense map against a brute-force sum with the weight's row/column
roles fixed by a non-square example; softplus against ``numpy.logaddexp``; the gates' closed forms (alpha = 1 when
A = 0 or when a + dt_bias runs to minus infinity, alpha = e^-1 when A = 1 and softplus = 1, beta = 1/2 at b = 0);
bfloat16 rounding on halfway cases; the whole layer with 0/1 weights that copy slices of x into the keys,
queries and values, against the op oracle called on those slices directly (fixes the split order and layout).
"""
from __future__ import annotations

import numpy as np

from . import sdm_oracle


def round_bf16_array(x) -> np.ndarray:
    """Nearest bfloat16 (8 significant bits, ties to even) of every fp64 element, as float64. Normal range only
    (zeros pass through); no subnormal or overflow handling, which the layer's magnitudes never reach."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def dense(x, w) -> np.ndarray:
    """y[..., n] = sum_k x[..., k] w[n, k] in fp64 (the weight in out-features x in-features order)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x @ w.T


def softplus(x) -> np.ndarray:
    """log(1 + e^x) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 30.0, x, np.log1p(np.exp(np.minimum(x, 30.0))))


def gates(a, b, a_log, dt_bias):
    """Forget and input gates of Gated DeltaNet with the A/dt parameterisation (per head h on the last axis):
    alpha = exp(-exp(A_log[h]) * softplus(a + dt_bias[h])), beta = 1 / (1 + exp(-b)). fp64."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    A = np.exp(np.asarray(a_log, dtype=np.float64))
    alpha = np.exp(-A * softplus(a + np.asarray(dt_bias, dtype=np.float64)))
    beta = 1.0 / (1.0 + np.exp(-b))
    return alpha, beta


def split_projection(p, heads, widths, subkey_dim, head_dim):
    """The input map's output [B, T, N] cut into keys, queries [B, T, H, F dk], values [B, T, H, d], a, b [B, T, H]."""
    B, T, _ = p.shape
    H, P, d = int(heads), len(widths) * int(subkey_dim), int(head_dim)
    o = 0
    keys = p[..., o:o + H * P].reshape(B, T, H, P); o += H * P
    queries = p[..., o:o + H * P].reshape(B, T, H, P); o += H * P
    values = p[..., o:o + H * d].reshape(B, T, H, d); o += H * d
    a = p[..., o:o + H]; o += H
    b = p[..., o:o + H]; o += H
    assert o == p.shape[-1]
    return keys, queries, values, a, b


def initial_bank_copy(initial_bank, batch) -> np.ndarray:
    """The per-sequence copy of a learned initial bank [H, rows, d] into every batch row: [B, H, rows, d]
    (README model wiring: the bank is learned when backprop_on_memory=true; the layer copies it before the op)."""
    init = np.asarray(initial_bank, dtype=np.float32)
    return np.ascontiguousarray(np.broadcast_to(init[None], (int(batch),) + init.shape))


def layer_forward(x, w_in, a_log, dt_bias, w_out, subkeys, bank, *, heads, widths, num_writes, num_reads,
                  bank_bf16=False, nthreads=None, initial_bank=None):
    """The layer's forward on bfloat16 tensors (given as float arrays of bfloat16 values). Returns a dict with every
    intermediate (keys, queries, values, a, b, alpha, beta: bfloat16 values as float64; the op's result dict `op`;
    y [B, T, Dm] bfloat16 values as float64). The bank is not modified (the op oracle advances a copy). With
    initial_bank [H, rows, d] the op starts from its copy in every batch row instead of `bank`."""
    if initial_bank is not None:
        bank = initial_bank_copy(initial_bank, np.asarray(x).shape[0])
    dk = np.asarray(subkeys).shape[-1]
    d = np.asarray(bank).shape[-1]
    p = round_bf16_array(dense(x, w_in))
    keys, queries, values, a, b = split_projection(p, heads, widths, dk, d)
    alpha, beta = gates(a, b, a_log, dt_bias)
    alpha, beta = round_bf16_array(alpha), round_bf16_array(beta)
    op = sdm_oracle.write_read(keys, queries, values, alpha, beta, subkeys, bank, widths, num_writes, num_reads,
                               bank_bf16=bank_bf16, act_bf16=True, nthreads=nthreads)
    B, T = p.shape[:2]
    o = np.asarray(op["out"], dtype=np.float64).reshape(B, T, -1)
    y = round_bf16_array(dense(o, w_out))
    return {"keys": keys, "queries": queries, "values": values, "a": a, "b": b, "alpha": alpha, "beta": beta,
            "op": op, "y": y}
