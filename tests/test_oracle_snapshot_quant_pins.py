"""Pins of the oracle's quantized backward snapshots (no GPU).

The reading (sdm_oracle.c, "Quantized backward snapshots"): a float32 snapshot row is stored in groups of 16 columns,
each with the smallest power-of-two scale s that brings the group's largest magnitude to at most the format's largest
value (448 for OCP FP8 E4M3, 7 for int4), every element as the format's nearest value to x / s (ties to even), read
back as that value times s. Pinned here: the E4M3 rounding against torch's float8_e4m3fn conversion (a library
routine) and by hand on ties and subnormals; the scale rule's closed forms; the quantized rows' error bounds, group
independence and exact rows; and the backward with such a snapshot like the bfloat16 one: value and bank gradients
untouched, rows already in the format change nothing, the one-token gate gradients by hand with the quantized row.
"""
import numpy as np
import pytest
import torch

import oracle


def test_e4m3_rounding_matches_torch_float8():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-2.0 ** -5, 2.0 ** -5, 20000),
                        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000)) * rng.choice([-1, 1], 20000)])
    v = v.astype(np.float32).astype(np.float64)
    ours = np.array([oracle.e4m3_round(x) for x in v])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_values_ties_and_subnormals():
    # every finite E4M3 value is its own rounding (exponent field 0..15, 3 mantissa bits, bias 7; S.1111.111 is NaN)
    vals = []
    for E in range(16):
        for M in range(8):
            if E == 15 and M == 7:
                continue
            vals.append(M * 2.0 ** -9 if E == 0 else (1 + M / 8) * 2.0 ** (E - 7))
    for x in vals:
        assert oracle.e4m3_round(x) == x and oracle.e4m3_round(-x) == -x
    assert max(vals) == 448.0
    assert oracle.e4m3_round(1 + 1 / 16) == 1.0          # tie between 1 (mantissa 0) and 1.125: even
    assert oracle.e4m3_round(1 + 3 / 16) == 1.25         # tie between 1.125 and 1.25: even
    assert oracle.e4m3_round(2.0 ** -10) == 0.0          # half the subnormal spacing: to zero (even)
    assert oracle.e4m3_round(3 * 2.0 ** -10) == 2.0 ** -8
    assert oracle.e4m3_round(440.0) == 448.0 and oracle.e4m3_round(431.0) == 416.0


def test_scale_exponent_closed_forms():
    for k in (-20, -3, 0, 5):
        assert oracle.snap_scale_exp(448.0 * 2.0 ** k, 448.0) == k        # exactly the largest value
        assert oracle.snap_scale_exp(448.0 * 2.0 ** k * 1.0001, 448.0) == k + 1
        assert oracle.snap_scale_exp(7.0 * 2.0 ** k, 7.0) == k
        assert oracle.snap_scale_exp(7.0 * 2.0 ** k * 1.0001, 7.0) == k + 1
        assert oracle.snap_scale_exp(256.0 * 2.0 ** k, 448.0) == k       # (256 / 2^-1 = 512 > 448)


@pytest.mark.parametrize("mode", ["fp8", "int4"])
def test_quantized_rows(mode):
    rng = np.random.default_rng(2)
    x = (0.02 * rng.standard_normal((200, 64))).astype(np.float32).astype(np.float64)
    x[3, 16:32] = 0.0
    q = oracle.snap_rows(x, mode)
    g = np.abs(x).reshape(200, 4, 16).max(axis=2)  # group maxima
    qmax = 448.0 if mode == "fp8" else 7.0
    s = np.array([[2.0 ** oracle.snap_scale_exp(a, qmax) if a > 0 else 0.0 for a in row] for row in g])
    s_el = np.repeat(s, 16, axis=1)
    err = np.abs(q - x)
    if mode == "fp8":
        assert np.all(err <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * s_el)
    else:
        assert np.all(err <= s_el / 2) and np.all(np.abs(q / np.where(s_el > 0, s_el, 1)) <= 7)
    assert np.all(q[3, 16:32] == 0.0)
    # groups are independent: changing one group's values leaves the other groups' quantization alone
    y = x.copy()
    y[:, :16] *= 3.0
    qy = oracle.snap_rows(y, mode)
    assert np.array_equal(qy[:, 16:], q[:, 16:])
    # rows already in the format (a power-of-two scale times format values) come back unchanged
    assert np.array_equal(oracle.snap_rows(q, mode), q)


def _case(seed, B, T, H, widths, dk, d):
    rng = np.random.default_rng(seed)
    F = len(widths)
    x = {"wkeys": rng.standard_normal((B, T, H, F * dk)).astype(np.float32),
         "rq": rng.standard_normal((B, T, H, F * dk)).astype(np.float32),
         "values": rng.standard_normal((B, T, H, d)).astype(np.float32),
         "alpha": (1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32),
         "beta": (1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32),
         "subkeys": rng.standard_normal((H, sum(widths), dk)).astype(np.float32),
         "bank": (0.3 * rng.standard_normal((B, H, int(np.prod(widths)), d))).astype(np.float32)}
    dout = rng.standard_normal((B, T, H, d)).astype(np.float32)
    dbank = rng.standard_normal(x["bank"].shape).astype(np.float32)
    return x, dout, dbank


def _bwd(x, dout, dbank, widths, W, R, **kw):
    return oracle.write_read_backward(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"],
                                      x["bank"], dout, dbank, widths, W, R, nthreads=1, **kw)


@pytest.mark.parametrize("mode", ["fp8", "int4"])
def test_quantized_snapshot_leaves_value_and_bank_gradients_alone(mode):
    x, dout, dbank = _case(3, 1, 12, 2, (4, 4), 3, 16)
    a = _bwd(x, dout, dbank, (4, 4), 3, 2)
    b = _bwd(x, dout, dbank, (4, 4), 3, 2, snap_quant=mode)
    assert np.array_equal(a["d_values"], b["d_values"]) and np.array_equal(a["d_bank"], b["d_bank"])
    assert not np.array_equal(a["d_alpha"], b["d_alpha"])  # the row-reading gradients do change


@pytest.mark.parametrize("mode", ["fp8", "int4"])
def test_quantized_snapshot_of_rows_in_the_format_changes_nothing(mode):
    """With alpha = 1 and beta = 0 the rows never change; if they are already in the format, every gradient equals
    the float32 snapshot's."""
    x, dout, _ = _case(4, 1, 10, 2, (4, 4), 3, 32)
    x["alpha"][:] = 1.0
    x["beta"][:] = 0.0
    x["bank"] = oracle.snap_rows(x["bank"], mode).astype(np.float32)
    a = _bwd(x, dout, None, (4, 4), 3, 3)
    b = _bwd(x, dout, None, (4, 4), 3, 3, snap_quant=mode)
    for k in ("d_wkeys", "d_rq", "d_values", "d_alpha", "d_beta", "d_subkeys", "d_bank"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("mode", ["fp8", "int4"])
def test_quantized_snapshot_one_token_gate_gradients_by_hand(mode):
    """One token writing and reading one slot: d alpha = (1 - beta) <dout, P~>, d beta = <dout, v - alpha P~> with
    P~ the quantized row."""
    rng = np.random.default_rng(12)
    widths, dk, d = (4,), 2, 32
    q = rng.standard_normal((1, 1, 1, dk)).astype(np.float32)
    x = {"wkeys": q, "rq": q.copy(), "values": rng.standard_normal((1, 1, 1, d)).astype(np.float32),
         "alpha": np.array([[[0.7]]], np.float32), "beta": np.array([[[0.3]]], np.float32),
         "subkeys": rng.standard_normal((1, 4, dk)).astype(np.float32),
         "bank": (rng.standard_normal((1, 1, 4, d)) / 3).astype(np.float32)}
    dout = rng.standard_normal((1, 1, 1, d)).astype(np.float32)
    ids, _ = oracle.topk(q, x["subkeys"], widths, 1)
    P = x["bank"][0, 0, ids[0, 0, 0, 0]].astype(np.float64)
    Pq = oracle.snap_rows(P[None], mode)[0]
    assert not np.array_equal(P, Pq)
    a, be = np.float64(x["alpha"][0, 0, 0]), np.float64(x["beta"][0, 0, 0])
    g = dout[0, 0, 0].astype(np.float64)
    v = x["values"][0, 0, 0].astype(np.float64)
    r = _bwd(x, dout, None, widths, 1, 1, snap_quant=mode)
    assert abs(r["d_alpha"][0, 0, 0] - (1 - be) * (g @ Pq)) <= 1e-12
    assert abs(r["d_beta"][0, 0, 0] - g @ (v - a * Pq)) <= 1e-12


def _rbf16(x):
    return np.array([oracle.round_bf16(float(v)) for v in np.ravel(x)]).reshape(np.shape(x))


def test_bank_gradient_accumulated_in_bfloat16_by_hand():
    """The pages' default bank-gradient accumulation on a bfloat16 bank (CHANGELOG 2.0.0, "Deterministic": float32
    accumulation is the opt-in): every update of the adjoint bank is rounded to bfloat16. One token writing and reading
    one slot (W = R = 1, weights 1): G[j] = rnd(dbank[j] + dout), then G[j] = rnd(alpha (1 - beta) G[j]); every other
    row keeps dbank; every entry is a bfloat16 value."""
    rng = np.random.default_rng(13)
    widths, dk, d = (4,), 2, 8
    q = rng.standard_normal((1, 1, 1, dk)).astype(np.float32)
    x = {"wkeys": q, "rq": q.copy(), "values": rng.standard_normal((1, 1, 1, d)).astype(np.float32),
         "alpha": np.array([[[0.7]]], np.float32), "beta": np.array([[[0.3]]], np.float32),
         "subkeys": rng.standard_normal((1, 4, dk)).astype(np.float32),
         "bank": _rbf16(rng.standard_normal((1, 1, 4, d)) / 3).astype(np.float32)}
    dout = _rbf16(rng.standard_normal((1, 1, 1, d))).astype(np.float32)
    dbank = _rbf16(rng.standard_normal((1, 1, 4, d))).astype(np.float32)
    j = int(oracle.topk(q, x["subkeys"], widths, 1)[0][0, 0, 0, 0])
    r = oracle.write_read_backward(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                                   dout, dbank, widths, 1, 1, bank_bf16=True, grad_bank_bf16=True, nthreads=1)
    a, b = float(x["alpha"][0, 0, 0]), float(x["beta"][0, 0, 0])
    g = _rbf16(dbank[0, 0, j].astype(np.float64) + dout[0, 0, 0].astype(np.float64))
    expect = _rbf16(a * g - a * b * 1.0 * g)
    assert np.array_equal(r["d_bank"][0, 0, j], expect)
    others = [i for i in range(4) if i != j]
    assert np.array_equal(r["d_bank"][0, 0, others], dbank[0, 0, others].astype(np.float64))
    f = oracle.write_read_backward(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                                   dout, dbank, widths, 1, 1, bank_bf16=True, nthreads=1)
    assert not np.array_equal(f["d_bank"], r["d_bank"])  # float32 (fp64 here) accumulation keeps the low bits


def test_bank_gradient_in_bfloat16_holds_bfloat16_values():
    x, dout, dbank = _case(5, 1, 16, 2, (4, 4), 3, 16)
    x["bank"] = _rbf16(x["bank"]).astype(np.float32)
    dbank = _rbf16(dbank).astype(np.float32)
    r = _bwd(x, dout, dbank, (4, 4), 3, 2, bank_bf16=True, grad_bank_bf16=True)
    assert np.array_equal(r["d_bank"], _rbf16(r["d_bank"]))
