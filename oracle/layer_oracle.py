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

The backward (``layer_backward``) is the chain rule through those steps, last first; the gradients passed between
steps are bfloat16 like the tensors they belong to. Pins of the backward (``tests/test_layer_oracle_backward_pins.py``):
central finite differences of the unrounded layer along random directions in every input and parameter, the gates'
derivatives against finite differences and closed forms, and the dense maps' transposes by hand-summed loops.

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
                  bank_bf16=False, nthreads=None, initial_bank=None, rounded=True):
    """The layer's forward on bfloat16 tensors (given as float arrays of bfloat16 values). Returns a dict with every
    intermediate (keys, queries, values, a, b, alpha, beta: bfloat16 values as float64; the op's result dict `op`;
    o [B, T, H d] the op's output; y [B, T, Dm] bfloat16 values as float64). The bank is not modified (the op oracle
    advances a copy). With initial_bank [H, rows, d] the op starts from its copy in every batch row instead of
    `bank`. rounded=False: the same steps with no bfloat16 rounding anywhere and the op's bank states in fp64 (its
    inputs still pass as float32), the smooth function that the backward differentiates (finite-difference pins)."""
    if initial_bank is not None:
        bank = initial_bank_copy(initial_bank, np.asarray(x).shape[0])
    rnd = round_bf16_array if rounded else (lambda v: np.asarray(v, dtype=np.float64))
    dk = np.asarray(subkeys).shape[-1]
    d = np.asarray(bank).shape[-1]
    p = rnd(dense(x, w_in))
    keys, queries, values, a, b = split_projection(p, heads, widths, dk, d)
    alpha, beta = gates(a, b, a_log, dt_bias)
    alpha, beta = rnd(alpha), rnd(beta)
    if rounded:
        op = sdm_oracle.write_read(keys, queries, values, alpha, beta, subkeys, bank, widths, num_writes, num_reads,
                                   bank_bf16=bank_bf16, act_bf16=True, nthreads=nthreads)
    else:  # the fp64-state forward of the op (its backward run with zero upstream gradients)
        B0, T0 = p.shape[:2]
        op = sdm_oracle.write_read_backward(keys, queries, values, alpha, beta, subkeys, bank,
                                            np.zeros((B0, T0, heads, d)), None, widths, num_writes, num_reads,
                                            exact=True, want_forward=True, nthreads=nthreads)
    B, T = p.shape[:2]
    o = np.asarray(op["out"], dtype=np.float64).reshape(B, T, -1)
    y = rnd(dense(o, w_out))
    return {"keys": keys, "queries": queries, "values": values, "a": a, "b": b, "alpha": alpha, "beta": beta,
            "op": op, "o": o, "y": y, "bank_in": np.asarray(bank)}


def sigmoid(x) -> np.ndarray:
    """1 / (1 + e^-x) in fp64, without overflow for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gates_backward(a, b, a_log, dt_bias, d_alpha, d_beta):
    """The chain rule through gates() (fp64; alpha and beta recomputed from a and b, unrounded). With z = a + dt_bias[h]
    and A = exp(a_log[h]): alpha = exp(-A softplus(z)), so d alpha / d a = d alpha / d dt_bias = -alpha A sigmoid(z)
    (the derivative of softplus is the sigmoid) and d alpha / d a_log = -alpha A softplus(z); beta = sigmoid(b), so
    d beta / d b = beta (1 - beta). Returns d_a, d_b (the shape of a) and d_a_log, d_dt_bias [H], summed over every
    leading index."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    A = np.exp(np.asarray(a_log, dtype=np.float64))
    z = a + np.asarray(dt_bias, dtype=np.float64)
    sp = softplus(z)
    alpha = np.exp(-A * sp)
    beta = sigmoid(b)
    da_ = np.asarray(d_alpha, dtype=np.float64)
    d_a = da_ * alpha * (-A) * sigmoid(z)
    d_b = np.asarray(d_beta, dtype=np.float64) * beta * (1.0 - beta)
    lead = tuple(range(d_a.ndim - 1))
    d_a_log = np.sum(da_ * alpha * (-A * sp), axis=lead)
    d_dt_bias = np.sum(d_a, axis=lead)
    return d_a, d_b, d_a_log, d_dt_bias


def layer_backward(x, w_in, a_log, dt_bias, w_out, subkeys, bank, grad_y, grad_bank=None, *, heads, widths,
                   num_writes, num_reads, bank_bf16=False, nthreads=None, initial_bank=None, rounded=True, fwd=None):
    """Gradients of the layer (the chain rule through layer_forward's steps, last step first). grad_y [B, T, Dm] is
    the gradient of the loss with respect to y and grad_bank (the bank's shape, or None for zero) the one with
    respect to the bank after the call. Every tensor between the steps is bfloat16 (rounded=True, as in the
    forward), so the gradients passed between them are rounded to bfloat16 too: d o (into the op's backward) and
    d p (the input map's output, assembled from the op's key, query and value gradients and the gate inputs'
    gradients). Parameter and input gradients are fp64:
      d o = grad_y w_out,  d w_out = sum over (b, t) of grad_y^T o
      the op's backward (sdm_oracle.write_read_backward) on d o and grad_bank
      d a, d b, d a_log, d dt_bias: gates_backward on the op's d alpha, d beta
      d x = d p w_in,  d w_in = sum over (b, t) of d p^T x
    Returns d_o, d_p (as bfloat16 values when rounded), d_x, d_w_in, d_a_log, d_dt_bias, d_w_out, d_subkeys, d_bank
    (with respect to the bank the op started from), the op's result `op`, d_a, d_b, the forward `fwd`, and with
    initial_bank d_initial_bank (d_bank summed over the batch)."""
    kw = dict(heads=heads, widths=widths, num_writes=num_writes, num_reads=num_reads, bank_bf16=bank_bf16,
              nthreads=nthreads, initial_bank=initial_bank, rounded=rounded)
    f = fwd if fwd is not None else layer_forward(x, w_in, a_log, dt_bias, w_out, subkeys, bank, **kw)
    rnd = round_bf16_array if rounded else (lambda v: np.asarray(v, dtype=np.float64))
    x = np.asarray(x, dtype=np.float64)
    w_in = np.asarray(w_in, dtype=np.float64)
    w_out = np.asarray(w_out, dtype=np.float64)
    gy = np.asarray(grad_y, dtype=np.float64)
    B, T, _ = x.shape
    H = int(heads)
    d = np.asarray(f["bank_in"]).shape[-1]
    o = f["o"]
    d_o = rnd(gy @ w_out)                                  # [B, T, H d]
    d_w_out = np.einsum("btn,btk->nk", gy, o)             # [Dm, H d]
    ob = sdm_oracle.write_read_backward(f["keys"], f["queries"], f["values"], f["alpha"], f["beta"], subkeys,
                                        f["bank_in"], d_o.reshape(B, T, H, d), grad_bank, widths, num_writes,
                                        num_reads, bank_bf16=bank_bf16, exact=not rounded, nthreads=nthreads)
    d_a, d_b, d_a_log, d_dt_bias = gates_backward(f["a"], f["b"], a_log, dt_bias, ob["d_alpha"], ob["d_beta"])
    d_p = rnd(np.concatenate([ob["d_wkeys"].reshape(B, T, -1), ob["d_rq"].reshape(B, T, -1),
                              ob["d_values"].reshape(B, T, -1), d_a, d_b], axis=-1))
    res = {"d_o": d_o, "d_p": d_p, "d_x": d_p @ w_in, "d_w_in": np.einsum("btn,btk->nk", d_p, x),
           "d_a_log": d_a_log, "d_dt_bias": d_dt_bias, "d_w_out": d_w_out, "d_subkeys": ob["d_subkeys"],
           "d_bank": ob["d_bank"], "op": ob, "d_a": d_a, "d_b": d_b, "fwd": f}
    if initial_bank is not None:
        res["d_initial_bank"] = ob["d_bank"].sum(axis=0)
    return res
