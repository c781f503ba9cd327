"""Parity of the layer's forward (sdm_layer_forward, through the C ABI) with the layer oracle, step by step.

The projections decide the top-k, so the steps are compared on the same inputs the way the method takes its
integer decisions: (1) the input map against the oracle's fp64 product of the same bf16 x and w_in, within the
bound of a float32-accumulated, bfloat16-rounded dot product; (2) the gates against the oracle's formula applied to
the GPU's own gate inputs; (3) the op against the op oracle run on the GPU's own keys, queries, values and gates
(slot ids bit-exact, out and bank within the op's tolerances); (4) the output map against the oracle's product of
the GPU's op output and w_out. Then repeatability, and the layer_65k shapes at model width 2048 on sampled rows.

Dense-map bound, per element: |y - y*| <= g S + 2^-8 (|y*| + g S), with y* the exact product, S = sum_k |x_k w_k|,
g = K 2^-24 (a float32 sum of K products in any order, first order), and 2^-8 the unit roundoff of bfloat16.
Gate bound: 2^-8 |ref| (the bfloat16 rounding) + 1e-6 (float32 exp / log1p on values of order one).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import layer_oracle as lo
from gated_delta_rule_product_amd import binding, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
RTOL = {"f32": 1e-5, "bf16": 2e-2}


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)


def to_np(t):
    return t.float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def rowwise_rel(got, ref):
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    err = np.abs(got - ref).max(axis=1)
    scale = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((err / scale).max())


def dense_ok(got, x, w):
    """got (bf16 values) against x w^T with the dense-map bound; returns the largest error / bound ratio."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    ref = lo.dense(x, w)
    S = np.abs(x) @ np.abs(w).T
    g = x.shape[-1] * 2.0 ** -24
    bound = g * S + 2.0 ** -8 * (np.abs(ref) + g * S) + 1e-30
    return float((np.abs(np.asarray(got, np.float64) - ref) / bound).max())


def run_layer(s, Dm, seed=0, bank_dt=torch.float32):
    x = synth.make_layer_inputs(s, Dm, seed)
    bank = to_dev(x["bank"], bank_dt)
    bank0 = to_np(bank)
    y, widx, ridx, ws = binding.sdm_layer_forward(
        to_dev(x["x"], torch.bfloat16), to_dev(x["w_in"], torch.bfloat16), to_dev(x["a_log"], torch.float32),
        to_dev(x["dt_bias"], torch.float32), to_dev(x["w_out"], torch.bfloat16), to_dev(x["subkeys"], torch.bfloat16),
        bank, heads=s.heads, widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
        chunk_size=s.chunk_size, want_index=True, return_workspace=True)
    torch.cuda.synchronize()
    v = binding.layer_workspace_views(x["x"].shape, s.heads, s.widths, s.subkey_dim, s.head_dim, ws)
    got = {k: to_np(t) for k, t in v.items()}
    got.update(y=to_np(y), widx=to_np(widx), ridx=to_np(ridx), bank=to_np(bank))
    return x, bank0, got


CASES = {
    # ragged last chunk (70 = 64 + 6), two heads, two factors
    "small": (synth.Shape(2, 70, 2, (16, 16), 32, 64, 8, 8, 64, "bf16", "f32"), 256),
    # bf16 bank, three factors, odd model width multiple of 32, N not a multiple of the GEMM tile
    "bf16_bank_3f": (synth.Shape(1, 40, 3, (8, 8, 4), 16, 96, 5, 7, 16, "bf16", "bf16"), 160),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_steps_against_oracle(name):
    s, Dm = CASES[name]
    bank_dt = torch.bfloat16 if s.bank == "bf16" else torch.float32
    x, bank0, got = run_layer(s, Dm, seed=3, bank_dt=bank_dt)
    H, P, d = s.heads, len(s.widths) * s.subkey_dim, s.head_dim
    # (1) input map, piece by piece (the split order is the header's)
    w = x["w_in"]
    o = 0
    for key, n in (("keys", H * P), ("queries", H * P), ("values", H * d), ("gin", 2 * H)):
        r = dense_ok(got[key].reshape(s.batch, s.tokens, n), x["x"], w[o:o + n])
        assert r <= 1.0, f"{key}: error {r} x the bound"
        o += n
    # (2) gates from the GPU's own gate inputs
    a, b = got["gin"][..., :H], got["gin"][..., H:]
    ra, rb = lo.gates(a, b, x["a_log"], x["dt_bias"])
    for key, ref in (("alpha", ra), ("beta", rb)):
        err = np.abs(got[key] - ref) - (2.0 ** -8 * np.abs(ref) + 1e-6)
        assert err.max() <= 0.0, f"{key} beyond its bound by {err.max()}"
    # (3) the op on the GPU's own inputs
    ref = oracle.write_read(got["keys"], got["queries"], got["values"], got["alpha"], got["beta"], x["subkeys"],
                            bank0, s.widths, s.num_writes, s.num_reads, bank_bf16=s.bank == "bf16", act_bf16=True)
    assert np.array_equal(got["widx"], ref["widx"]), "write slot ids differ"
    assert np.array_equal(got["ridx"], ref["ridx"]), "read slot ids differ"
    assert rowwise_rel(got["o"], ref["out"]) <= max(RTOL["bf16"], RTOL[s.bank])
    assert rowwise_rel(got["bank"], ref["bank"]) <= RTOL[s.bank]
    # (4) output map from the GPU's own op output
    r = dense_ok(got["y"], got["o"].reshape(s.batch, s.tokens, H * d), x["w_out"])
    assert r <= 1.0, f"y: error {r} x the bound"


def test_layer_repeatable():
    s, Dm = CASES["small"]
    _, _, g1 = run_layer(s, Dm, seed=4)
    _, _, g2 = run_layer(s, Dm, seed=4)
    for k in ("y", "bank", "widx", "ridx", "keys", "alpha"):
        assert np.array_equal(g1[k], g2[k]), k


def test_layer_65k_width_2048_sampled():
    """The layer at the layer_65k op shapes (B 2, T 4096, H 2, d 1024, 65536 slots, W = R = 64, chunk 64, float32
    bank) and model width 2048: the dense maps and the top-k on 48 sampled token rows, the gates everywhere."""
    s = synth.WORKLOADS["layer_65k"]
    Dm = 2048
    print("layer 65k: GPU", flush=True)
    x, _, got = run_layer(s, Dm, seed=0)
    H, P, d = s.heads, len(s.widths) * s.subkey_dim, s.head_dim
    rng = np.random.default_rng(1)
    rows = rng.choice(s.batch * s.tokens, 48, replace=False)
    xf = x["x"].reshape(-1, Dm)[rows]
    o = 0
    for key, n in (("keys", H * P), ("queries", H * P), ("values", H * d), ("gin", 2 * H)):
        r = dense_ok(got[key].reshape(-1, n)[rows], xf, x["w_in"][o:o + n])
        assert r <= 1.0, f"{key}: error {r} x the bound"
        o += n
    a, b = got["gin"][..., :H], got["gin"][..., H:]
    ra, rb = lo.gates(a, b, x["a_log"], x["dt_bias"])
    assert (np.abs(got["alpha"] - ra) <= 2.0 ** -8 * np.abs(ra) + 1e-6).all()
    assert (np.abs(got["beta"] - rb) <= 2.0 ** -8 * np.abs(rb) + 1e-6).all()
    print("layer 65k: oracle top-k on sampled rows", flush=True)
    for key, ids, k in (("keys", "widx", s.num_writes), ("queries", "ridx", s.num_reads)):
        q = got[key].reshape(-1, 1, H, P)[rows]  # [48, 1, H, P]
        rid, _ = oracle.topk(q, x["subkeys"], s.widths, k)
        assert np.array_equal(got[ids].reshape(-1, 1, H, k)[rows], rid), f"{ids} differ on sampled rows"
    r = dense_ok(got["y"].reshape(-1, Dm)[rows], got["o"].reshape(-1, H * d)[rows], x["w_out"])
    assert r <= 1.0, f"y: error {r} x the bound"


def test_layer_padded_bank_pitch():
    """A bank whose rows are padded (the pitch the bench uses for 4 KiB rows): the same bits as a dense bank, and
    the padding never written."""
    s, Dm = CASES["small"]
    x = synth.make_layer_inputs(s, Dm, seed=6)
    args = [to_dev(x["x"], torch.bfloat16), to_dev(x["w_in"], torch.bfloat16), to_dev(x["a_log"], torch.float32),
            to_dev(x["dt_bias"], torch.float32), to_dev(x["w_out"], torch.bfloat16),
            to_dev(x["subkeys"], torch.bfloat16)]
    kw = dict(heads=s.heads, widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
              chunk_size=s.chunk_size)
    dense = to_dev(x["bank"], torch.float32)
    pitch = s.head_dim + 32
    buf = torch.full((s.batch, s.heads, s.rows, pitch), 1234.5, dtype=torch.float32, device=DEV)
    padded = buf[..., :s.head_dim]
    padded.copy_(dense)
    y1, _, _ = binding.sdm_layer_forward(*args, dense, **kw)
    y2, _, _ = binding.sdm_layer_forward(*args, padded, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(dense, padded)
    assert bool((buf[..., s.head_dim:] == 1234.5).all())
