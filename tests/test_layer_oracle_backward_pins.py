"""Pins of the layer oracle's backward (oracle/layer_oracle.py, no GPU): its gradients are the derivatives of the
layer's forward.

The backward with rounded=False differentiates the smooth function the forward computes without bfloat16 rounding
(bank states in fp64; the op's inputs still pass as float32). Central finite differences of the loss
L = <U_y, y> + <U_bank, bank after the call> along a random direction in one input or parameter at a time must equal
<gradient, direction>, with every selected slot set unchanged by the perturbation (checked with the oracle's top-k
on the perturbed keys and queries). The gates' derivatives are also pinned on their own (finite differences in
fp64 and closed forms), and with rounding on, the gradients passed between the steps are bfloat16 values.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import layer_oracle as lo


def test_gates_backward_finite_differences():
    rng = np.random.default_rng(11)
    H = 3
    a, b = rng.standard_normal((4, 5, H)) * 2, rng.standard_normal((4, 5, H)) * 2
    a_log, dt_bias = rng.standard_normal(H) * 0.5, rng.standard_normal(H)
    ga, gb = rng.standard_normal(a.shape), rng.standard_normal(b.shape)

    def loss(a_, b_, al_, dt_):
        alpha, beta = lo.gates(a_, b_, al_, dt_)
        return float(np.sum(ga * alpha) + np.sum(gb * beta))

    d_a, d_b, d_alog, d_dtb = lo.gates_backward(a, b, a_log, dt_bias, ga, gb)
    eps = 1e-6
    for name, arr, g in (("a", a, d_a), ("b", b, d_b), ("a_log", a_log, d_alog), ("dt_bias", dt_bias, d_dtb)):
        v = rng.standard_normal(arr.shape)
        args = {"a": a, "b": b, "a_log": a_log, "dt_bias": dt_bias}
        plus, minus = dict(args), dict(args)
        plus[name], minus[name] = arr + eps * v, arr - eps * v
        fd = (loss(plus["a"], plus["b"], plus["a_log"], plus["dt_bias"]) -
              loss(minus["a"], minus["b"], minus["a_log"], minus["dt_bias"])) / (2 * eps)
        an = float(np.sum(g * v))
        assert abs(fd - an) <= 1e-7 * (abs(an) + float(np.sum(np.abs(g * v)))), (name, fd, an)


def test_gates_backward_closed_forms():
    # A = 1, z = a + dt_bias = 0: softplus = ln 2, alpha = 1/2, sigmoid(0) = 1/2
    d_a, d_b, d_alog, d_dtb = lo.gates_backward(np.zeros((1, 1)), np.zeros((1, 1)), np.zeros(1), np.zeros(1),
                                                np.ones((1, 1)), np.ones((1, 1)))
    assert abs(d_a[0, 0] + 0.25) < 1e-15             # -alpha A sigmoid(z)
    assert abs(d_alog[0] + 0.5 * math.log(2.0)) < 1e-15  # -alpha A softplus(z)
    assert d_dtb[0] == d_a[0, 0]                     # dt_bias enters like a
    assert d_b[0, 0] == 0.25                         # beta (1 - beta) at b = 0
    # A = 0: alpha = 1 whatever a, so no gradient reaches a, dt_bias or a_log
    d_a, _, d_alog, _ = lo.gates_backward(np.array([[3.0]]), np.zeros((1, 1)), np.array([-np.inf]), np.zeros(1),
                                          np.ones((1, 1)), np.zeros((1, 1)))
    assert d_a[0, 0] == 0.0 and d_alog[0] == 0.0
    # saturated input gate: no gradient through beta
    _, d_b, _, _ = lo.gates_backward(np.zeros((1, 1)), np.array([[800.0]]), np.zeros(1), np.zeros(1),
                                     np.zeros((1, 1)), np.ones((1, 1)))
    assert d_b[0, 0] == 0.0
    # head-wise sums: the parameter gradients add every (b, t) row of their head only
    d_a, _, _, d_dtb = lo.gates_backward(np.zeros((2, 3, 2)), np.zeros((2, 3, 2)), np.zeros(2), np.zeros(2),
                                         np.stack([np.ones((2, 3)), np.zeros((2, 3))], axis=-1), np.zeros((2, 3, 2)))
    assert d_dtb[0] == 6 * -0.25 and d_dtb[1] == 0.0


B, T, H, WIDTHS, DK, D, W, R, DM = 1, 5, 2, (4, 4), 2, 4, 3, 2, 12
P = len(WIDTHS) * DK
NIN = 2 * H * P + H * D + 2 * H
KW = dict(heads=H, widths=WIDTHS, num_writes=W, num_reads=R, nthreads=1)


def _selection(f):
    """Sorted selected slot sets of the op's keys and queries (as float32, the op's input)."""
    return (np.sort(oracle.topk(np.asarray(f["keys"], np.float32), SUB32, WIDTHS, W)[0], axis=-1),
            np.sort(oracle.topk(np.asarray(f["queries"], np.float32), SUB32, WIDTHS, R)[0], axis=-1))


def _case(seed):
    rng = np.random.default_rng(seed)
    for _ in range(200):  # draw until every selection has a clear margin (finite differences keep it)
        p = {"x": rng.standard_normal((B, T, DM)), "w_in": 0.3 * rng.standard_normal((NIN, DM)),
             "a_log": 0.3 * rng.standard_normal(H), "dt_bias": rng.standard_normal(H),
             "w_out": 0.3 * rng.standard_normal((DM, H * D)), "subkeys": rng.standard_normal((H, sum(WIDTHS), DK)),
             "bank": 0.3 * rng.standard_normal((B, H, 16, D))}
        p["subkeys"] = p["subkeys"].astype(np.float32).astype(np.float64)
        f = lo.layer_forward(p["x"], p["w_in"], p["a_log"], p["dt_bias"], p["w_out"], p["subkeys"],
                             p["bank"].astype(np.float32), rounded=False, **KW)
        ok = True
        for name, k in (("keys", W), ("queries", R)):
            _, sc = oracle.topk(np.asarray(f[name], np.float32), p["subkeys"].astype(np.float32), WIDTHS, k + 1)
            ok &= bool(((sc[..., k - 1] - sc[..., k]) > 0.01).all())
        if ok:
            return p, rng.standard_normal((B, T, DM)), rng.standard_normal((B, H, 16, D))
    raise AssertionError("no case with separated selections")


SUB32 = None


def _loss(p, u_y, u_bank, initial_bank=None):
    f = lo.layer_forward(p["x"], p["w_in"], p["a_log"], p["dt_bias"], p["w_out"], p["subkeys"],
                         p["bank"].astype(np.float32), rounded=False, initial_bank=initial_bank, **KW)
    return float(np.sum(f["y"] * u_y) + np.sum(np.asarray(f["op"]["bank"], np.float64) * u_bank)), f


GRADS = {"x": "d_x", "w_in": "d_w_in", "a_log": "d_a_log", "dt_bias": "d_dt_bias", "w_out": "d_w_out",
         "subkeys": "d_subkeys", "bank": "d_bank"}


@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("name", list(GRADS) + ["initial_bank"])
def test_layer_gradient_equals_finite_difference(seed, name):
    global SUB32
    p, u_y, u_bank = _case(seed)
    SUB32 = p["subkeys"].astype(np.float32)
    init = None
    if name == "initial_bank":
        init = (0.3 * np.random.default_rng(seed + 50).standard_normal((H, 16, D))).astype(np.float32)
    L0, f0 = _loss(p, u_y, u_bank, init)
    g = lo.layer_backward(p["x"], p["w_in"], p["a_log"], p["dt_bias"], p["w_out"], p["subkeys"],
                          p["bank"].astype(np.float32), u_y, u_bank, rounded=False, initial_bank=init, fwd=f0, **KW)
    rng = np.random.default_rng(1000 + seed)
    base = p[name] if name != "initial_bank" else init.astype(np.float64)
    v = rng.standard_normal(base.shape)
    eps = 1e-4
    if name in ("bank", "initial_bank", "subkeys"):
        # float32 inputs of the op: the direction actually taken is the rounded difference
        hi = (base + eps * v).astype(np.float32).astype(np.float64)
        lo_ = (base - eps * v).astype(np.float32).astype(np.float64)
        v = (hi - lo_) / (2 * eps)
    else:
        hi, lo_ = base + eps * v, base - eps * v
    sel0 = _selection(f0)
    Ls = []
    for val in (hi, lo_):
        q = dict(p)
        ib = init
        if name == "initial_bank":
            ib = val.astype(np.float32)
        else:
            q[name] = val
        if name == "subkeys":
            SUB32 = q["subkeys"].astype(np.float32)
        L, f = _loss(q, u_y, u_bank, ib)
        sel = _selection(f)
        assert all(np.array_equal(s0, s1) for s0, s1 in zip(sel0, sel)), "a selection changed"
        Ls.append(L)
    SUB32 = p["subkeys"].astype(np.float32)
    fd = (Ls[0] - Ls[1]) / (2 * eps)
    key = "d_initial_bank" if name == "initial_bank" else GRADS[name]
    an = float(np.sum(g[key] * v))
    scale = float(np.sum(np.abs(g[key] * v)))
    assert abs(fd - an) <= 2e-3 * scale + 1e-9, (name, fd, an, scale)


def test_rounded_backward_passes_bfloat16_gradients():
    """With rounding on (the library's arithmetic), the gradients passed between steps are bfloat16 values and the
    op's backward receives exactly d_o."""
    rng = np.random.default_rng(4)
    r = lambda *shape: lo.round_bf16_array(rng.standard_normal(shape))
    x, w_in, w_out = r(B, T, DM), r(NIN, DM) * 0.25, r(DM, H * D) * 0.25
    sub = r(H, sum(WIDTHS), DK)
    bank = (0.1 * rng.standard_normal((B, H, 16, D))).astype(np.float32)
    gy = r(B, T, DM)
    g = lo.layer_backward(x, w_in, np.zeros(H), np.zeros(H), w_out, sub, bank, gy, None, **KW)
    for k in ("d_o", "d_p"):
        np.testing.assert_array_equal(lo.round_bf16_array(g[k]), g[k])
    np.testing.assert_array_equal(g["d_o"], lo.round_bf16_array(gy @ w_out))
    np.testing.assert_allclose(g["d_x"], g["d_p"] @ w_in, rtol=1e-13, atol=1e-13)
