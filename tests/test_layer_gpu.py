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


def test_layer_learned_initial_bank():
    """A learned initial bank (README model wiring; the layer's bank copy runs before the op): every batch row of the
    bank starts from the copy, bit for bit the layer on a bank filled with the copy beforehand; the op then matches
    the oracle started from the copy; rows past N and the row padding are never written."""
    s = synth.Shape(3, 70, 2, (16, 16), 32, 64, 8, 8, 64, "bf16", "f32", bank_rows=300)
    Dm = 256
    x = synth.make_layer_inputs(s, Dm, 5)
    rng = np.random.default_rng(6)
    init_np = (0.02 * rng.standard_normal((s.heads, s.rows, s.head_dim))).astype(np.float32)
    pitch, SENT = 80, 777.0
    t = {k: to_dev(x[k], torch.bfloat16) for k in ("x", "w_in", "w_out", "subkeys")}
    g = {k: to_dev(x[k], torch.float32) for k in ("a_log", "dt_bias")}
    kw = dict(heads=s.heads, widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
              chunk_size=s.chunk_size, want_index=True, return_workspace=True)
    ibuf = torch.full((s.heads, s.rows, pitch), SENT, device=DEV)
    init = ibuf[..., :s.head_dim]
    init.copy_(to_dev(init_np, torch.float32))
    bbuf = torch.full((s.batch, s.heads, s.rows, pitch), SENT, device=DEV)
    bank = bbuf[..., :s.head_dim]
    print("layer with a learned initial bank", flush=True)
    y, widx, ridx, ws = binding.sdm_layer_forward(t["x"], t["w_in"], g["a_log"], g["dt_bias"], t["w_out"],
                                                  t["subkeys"], bank, initial_bank=init, **kw)
    # the same layer on a bank filled with the copy beforehand
    bbuf2 = torch.full_like(bbuf, SENT)
    bank2 = bbuf2[..., :s.head_dim]
    bank2[:, :, :s.slots].copy_(init[:, :s.slots].unsqueeze(0).expand(s.batch, -1, -1, -1))
    y2, widx2, _, _ = binding.sdm_layer_forward(t["x"], t["w_in"], g["a_log"], g["dt_bias"], t["w_out"],
                                                t["subkeys"], bank2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(widx, widx2) and torch.equal(bbuf, bbuf2)
    assert bool((bbuf[..., s.head_dim:] == SENT).all()) and bool((bbuf[:, :, s.slots:] == SENT).all())
    v = binding.layer_workspace_views(x["x"].shape, s.heads, s.widths, s.subkey_dim, s.head_dim, ws)
    got = {k: to_np(u) for k, u in v.items()}
    start = lo.initial_bank_copy(init_np[:, :s.slots], s.batch)
    ref = oracle.write_read(got["keys"], got["queries"], got["values"], got["alpha"], got["beta"], x["subkeys"],
                            start, s.widths, s.num_writes, s.num_reads, act_bf16=True)
    assert np.array_equal(to_np(widx), ref["widx"]) and np.array_equal(to_np(ridx), ref["ridx"])
    assert rowwise_rel(got["o"], ref["out"]) <= RTOL["bf16"]
    assert rowwise_rel(to_np(bank[:, :, :s.slots]), ref["bank"]) <= RTOL["f32"]


def test_bank_grad_sum():
    """The learned bank's gradient: the op's per-stream bank gradients summed over the batch in order, each element
    within the a-priori bound of a float32 sum of B terms ((B - 1) 2^-24 times the sum of their magnitudes) of the
    fp64 sum, bitwise repeatable; rows past N and the padding are not written."""
    B, H, rows, d, pitch, N = 5, 3, 70, 48, 52, 64
    rng = np.random.default_rng(7)
    gb_np = rng.standard_normal((B, H, rows, d)).astype(np.float32) * np.exp(rng.standard_normal((B, H, rows, 1)))
    gbuf = torch.zeros((B, H, rows, pitch), device=DEV)
    gb = gbuf[..., :d]
    gb.copy_(to_dev(gb_np, torch.float32))
    obuf = torch.full((H, rows, pitch), 5.0, device=DEV)
    out = obuf[..., :d]
    print("bank gradient sum", flush=True)
    binding.sdm_bank_grad_sum(gb, heads=H, widths=(8, 8), head_dim=d, out=out)
    out2 = torch.full_like(obuf, 5.0)[..., :d]
    binding.sdm_bank_grad_sum(gb, heads=H, widths=(8, 8), head_dim=d, out=out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    got = to_np(out)[:, :N]
    ref = gb_np[:, :, :N].astype(np.float64).sum(axis=0)
    bound = (B - 1) * 2.0 ** -24 * np.abs(gb_np[:, :, :N].astype(np.float64)).sum(axis=0) * 1.01
    assert np.all(np.abs(got - ref) <= bound)
    assert bool((obuf[:, N:] == 5.0).all()) and bool((obuf[..., d:] == 5.0).all())


# ---------------------------------------------------------------------------------------------------------- backward
# The layer's backward (sdm_layer_forward_save + sdm_layer_backward), step by step on the GPU's own intermediates,
# each against the oracle's definition of that step (oracle/layer_oracle.py: layer_backward):
#   d o       bfloat16(grad_y w_out): the dense-map bound above (K = Dm)
#   d w_out   grad_y^T o (float32 result): |err| <= K 2^-24 S, K = B T, S = sum |terms| (float32 sums in any order)
#   the op    sdm_oracle's backward with its a-priori bounds (write_read_backward_bounds) on the GPU's keys, queries,
#             values, gates and d o, after the bound's hypothesis (the GPU's forward rows within the op's tolerance)
#   d p       its key, query and value columns the GPU's own float32 gradients rounded to nearest even (bit for
#             bit); its gate columns against gates_backward on the GPU's d alpha, d beta and gate inputs: one
#             bfloat16 rounding plus a float32 evaluation of exp, log1p and a few products (EVAL u (1 + |A softplus|)
#             relative, EVAL = 16)
#   d a_log, d dt_bias   the same terms summed in float32 over B T rows: (B T 2^-24 + EVAL u (1 + max |A softplus|))
#             times the sum of the terms' magnitudes
#   d x, d w_in   d p w_in and d p^T x in float32: K 2^-24 S (K = the padded input width, or B T)
# and the bank stepped back to its state before the forward bit for bit.
EVAL = 16
U32 = 2.0 ** -24
EPS_ROW = {"f32": 1e-5, "bf16": 2e-2}


def f32_ok(got, ref, S, K):
    bound = 1.01 * K * U32 * S + 1e-30
    return float((np.abs(np.asarray(got, np.float64) - ref) / bound).max())


BWD_CASES = {
    # float32 bank, model width 64 (every dense map on the LDS-tiled kernel)
    "small": (synth.Shape(2, 40, 2, (16, 16), 8, 32, 8, 8, 16, "bf16", "f32"), 64, False),
    # bfloat16 bank, model width 96 (d o's map, K = 96, on the register-only kernel), ragged chunk
    "bf16_bank_w96": (synth.Shape(1, 36, 2, (8, 8), 8, 32, 6, 5, 8, "bf16", "bf16"), 96, False),
    # a learned initial bank copied into every batch row; its gradient the batch sum of the bank gradient
    "learned_bank": (synth.Shape(3, 24, 2, (16, 16), 8, 32, 8, 8, 8, "bf16", "f32"), 64, True),
    # the 65,536-slot op shapes at model width 2048 (256 tokens a stream)
    "w2048_65k": (synth.WORKLOADS["layer_65k"].with_(tokens=256), 2048, False),
}


@pytest.mark.parametrize("name", list(BWD_CASES))
def test_layer_backward_steps_against_oracle(name):
    s, Dm, learned = BWD_CASES[name]
    bank_dt = torch.float32 if s.bank == "f32" else torch.bfloat16
    x = synth.make_layer_inputs(s, Dm, 3)
    rng = np.random.default_rng(31)
    gy_np = synth.round_bf16_rne(rng.standard_normal((s.batch, s.tokens, Dm)).astype(np.float32))
    gb_np = rng.standard_normal((s.batch, s.heads, s.rows, s.head_dim)).astype(np.float32)
    t = {k: to_dev(x[k], torch.bfloat16) for k in ("x", "w_in", "w_out", "subkeys")}
    t.update({k: to_dev(x[k], torch.float32) for k in ("a_log", "dt_bias")})
    bank = to_dev(x["bank"], bank_dt)
    init = None
    if learned:  # the op starts from this bank's copy in every batch row; the caller's bank is overwritten
        init_np = (0.02 * rng.standard_normal((s.heads, s.rows, s.head_dim))).astype(np.float32)
        init = to_dev(init_np, bank_dt)
        x["bank"] = np.ascontiguousarray(np.broadcast_to(init_np[None], x["bank"].shape))
    kw = dict(heads=s.heads, widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, chunk_size=s.chunk_size)
    print(f"layer backward {name}: {s} Dm {Dm}", flush=True)
    y, snap, ws, widx, ridx = binding.sdm_layer_forward_save(t["x"], t["w_in"], t["a_log"], t["dt_bias"], t["w_out"],
                                                             t["subkeys"], bank, want_index=True, initial_bank=init,
                                                             **kw)
    torch.cuda.synchronize()
    fv = {k: to_np(v) for k, v in binding.layer_workspace_views(x["x"].shape, s.heads, s.widths, s.subkey_dim,
                                                                s.head_dim, ws).items()}
    fwd_bank = to_np(bank)
    fwd_snap = to_np(snap)
    bank0 = to_dev(x["bank"], bank_dt)  # the bank the op started from
    gbank = to_dev(gb_np, torch.float32)
    g = binding.sdm_layer_backward(t["x"], t["w_in"], t["a_log"], t["dt_bias"], t["w_out"], t["subkeys"], bank, snap,
                                   to_dev(gy_np, torch.bfloat16), ws, gbank, **kw)
    torch.cuda.synchronize()
    assert torch.equal(bank, bank0), "the backward did not restore the bank bit for bit"
    lc = binding._layer_config(t["x"], bank, s.heads, s.widths, s.subkey_dim, s.num_writes, s.num_reads,
                               s.chunk_size)
    bv = {k: to_np(v) for k, v in binding.layer_backward_workspace_views(x["x"].shape, s.heads, s.widths,
                                                                         s.subkey_dim, s.head_dim, lc, ws).items()}
    got = {k: to_np(v) for k, v in g.items()}
    B, T, H, d, P = s.batch, s.tokens, s.heads, s.head_dim, len(s.widths) * s.subkey_dim
    M = B * T
    gy = gy_np.astype(np.float64)
    w_out = x["w_out"].astype(np.float64)
    o = fv["o"].reshape(B, T, H * d).astype(np.float64)
    # the output map
    r = dense_ok(bv["d_o"].reshape(B, T, H * d), gy, w_out.T)
    assert r <= 1.0, f"d o beyond its bound ({r:.3g})"
    ref = np.einsum("btn,btk->nk", gy, o)
    S = np.einsum("btn,btk->nk", np.abs(gy), np.abs(o))
    r = f32_ok(got["w_out"], ref, S, M)
    assert r <= 1.0, f"d w_out beyond its bound ({r:.3g})"
    # the op's backward on the GPU's own inputs
    ob = oracle.write_read_backward_bounds(fv["keys"], fv["queries"], fv["values"], fv["alpha"], fv["beta"],
                                           x["subkeys"], x["bank"], bv["d_o"], gb_np, s.widths, s.num_writes,
                                           s.num_reads, eps_row=EPS_ROW[s.bank], bank_bf16=s.bank == "bf16",
                                           want_snapshot=True)
    assert np.array_equal(to_np(widx), ob_ids(fv, x, s)[0]) and np.array_equal(to_np(ridx), ob_ids(fv, x, s)[1])
    for gpu_rows, ref_rows, what in ((fwd_snap, ob["snapshot"], "snapshot"), (fwd_bank, ob["bank"], "bank")):
        gr = np.asarray(gpu_rows, np.float64).reshape(-1, d)
        rr = np.asarray(ref_rows, np.float64).reshape(-1, d)
        allow = EPS_ROW[s.bank] * np.abs(rr).max(axis=1, keepdims=True)
        assert np.all(np.abs(gr - rr) <= allow), f"the forward's {what} rows beyond the op's tolerance"
    pairs = (("d_keys", "wkeys"), ("d_queries", "rq"), ("d_values", "values"), ("d_alpha", "alpha"),
             ("d_beta", "beta"))
    for gk, ok in pairs:
        err = np.abs(bv[gk].astype(np.float64) - ob["d_" + ok])
        assert np.all(err <= 1.01 * ob["e_" + ok] + 1e-30), f"op gradient {gk} beyond its bound"
    for gk, ok in (("subkeys", "subkeys"), ("bank", "bank")):
        err = np.abs(got[gk].astype(np.float64) - ob["d_" + ok])
        assert np.all(err <= 1.01 * ob["e_" + ok] + 1e-30), f"gradient {gk} beyond its bound"
    # d p: the op's gradients rounded, then the gate inputs' gradients
    dp = bv["d_p"].reshape(M, -1).astype(np.float64)
    HP, Hd = H * P, H * d
    np.testing.assert_array_equal(dp[:, :HP], synth.round_bf16_rne(bv["d_keys"].reshape(M, HP)))
    np.testing.assert_array_equal(dp[:, HP:2 * HP], synth.round_bf16_rne(bv["d_queries"].reshape(M, HP)))
    np.testing.assert_array_equal(dp[:, 2 * HP:2 * HP + Hd], synth.round_bf16_rne(bv["d_values"].reshape(M, Hd)))
    nin = 2 * HP + Hd + 2 * H
    assert np.all(dp[:, nin:] == 0.0)
    gin = fv["gin"].reshape(M, 2 * H).astype(np.float64)
    a_, b_ = gin[:, :H], gin[:, H:]
    da_alpha = bv["d_alpha"].reshape(M, H).astype(np.float64)
    da_beta = bv["d_beta"].reshape(M, H).astype(np.float64)
    d_a, d_b, d_alog, d_dtb = lo.gates_backward(a_, b_, x["a_log"], x["dt_bias"], da_alpha, da_beta)
    A = np.exp(x["a_log"].astype(np.float64))
    Asp = A * lo.softplus(a_ + x["dt_bias"].astype(np.float64))
    ev = EVAL * U32 * (1.0 + Asp)
    for cols, ref in ((slice(2 * HP + Hd, 2 * HP + Hd + H), d_a), (slice(2 * HP + Hd + H, nin), d_b)):
        err = np.abs(dp[:, cols] - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + ev * np.abs(ref) * 1.01 + 1e-30), "gate gradients"
    t_alog = np.abs(da_alpha * np.exp(-Asp) * Asp)
    t_dtb = np.abs(d_a)
    for gv_, ref, tm in ((got["a_log"], d_alog, t_alog), (got["dt_bias"], d_dtb, t_dtb)):
        bound = (M * U32 + EVAL * U32 * (1.0 + Asp.max(axis=0))) * tm.sum(axis=0) * 1.01 + 1e-30
        assert np.all(np.abs(gv_.astype(np.float64) - ref) <= bound), "gate parameter gradients"
    # the input map
    xx = x["x"].reshape(M, Dm).astype(np.float64)
    w_in = x["w_in"].astype(np.float64)
    Np = dp.shape[1]
    ref = dp[:, :nin] @ w_in
    r = f32_ok(got["x"].reshape(M, Dm), ref, np.abs(dp[:, :nin]) @ np.abs(w_in), Np)
    assert r <= 1.0, f"d x beyond its bound ({r:.3g})"
    ref = dp[:, :nin].T @ xx
    r = f32_ok(got["w_in"], ref, np.abs(dp[:, :nin]).T @ np.abs(xx), M)
    assert r <= 1.0, f"d w_in beyond its bound ({r:.3g})"
    if learned:  # the learned bank's gradient: the batch sum, in order, of the bank gradient (within its bounds)
        gi = binding.sdm_bank_grad_sum(g["bank"], heads=H, widths=s.widths, head_dim=d)
        torch.cuda.synchronize()
        ref = ob["d_bank"].sum(axis=0)
        bound = 1.01 * (ob["e_bank"].sum(axis=0) + (B - 1) * U32 * np.abs(ob["d_bank"]).sum(axis=0)) + 1e-30
        N = int(np.prod(s.widths))
        assert np.all(np.abs(to_np(gi)[:, :N] - ref[:, :N]) <= bound[:, :N]), "the learned bank's gradient"


def ob_ids(fv, x, s):
    """The op oracle's selected slots on the GPU's keys and queries (its top-k: the backward recomputes them)."""
    ids_w, _ = oracle.topk(fv["keys"], x["subkeys"], s.widths, s.num_writes)
    ids_r, _ = oracle.topk(fv["queries"], x["subkeys"], s.widths, s.num_reads)
    return ids_w, ids_r
