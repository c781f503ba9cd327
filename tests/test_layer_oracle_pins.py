"""Pins of the layer oracle (oracle/layer_oracle.py) against values fixed by the mathematics, not by the oracle:
the dense map's roles of rows and columns, softplus, the gates' closed forms, bfloat16 rounding, and the split of
the input map (a whole layer whose 0/1 weights copy slices of x, against the op oracle on those slices)."""
import math

import numpy as np
import pytest

from oracle import layer_oracle as lo
from oracle import sdm_oracle


def test_dense_is_x_times_w_transposed():
    """Non-square shapes make a transposed operand fail: y[m, n] = sum_k x[m, k] w[n, k], summed by hand."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 3, 5))
    w = rng.standard_normal((7, 5))
    y = lo.dense(x, w)
    assert y.shape == (2, 3, 7)
    for i in range(2):
        for t in range(3):
            for n in range(7):
                s = 0.0
                for k in range(5):
                    s += x[i, t, k] * w[n, k]
                assert abs(y[i, t, n] - s) <= 1e-12 * (1 + abs(s))


def test_softplus_against_logaddexp():
    x = np.linspace(-40.0, 40.0, 801)
    np.testing.assert_allclose(lo.softplus(x), np.logaddexp(0.0, x), rtol=1e-14, atol=1e-300)


def test_gates_closed_forms():
    # A = exp(A_log) = 1 and softplus(a + dt_bias) = 1 (a + dt_bias = log(e - 1)): alpha = e^-1
    al, be = lo.gates(np.array([[math.log(math.e - 1.0)]]), np.array([[0.0]]), np.array([0.0]), np.array([0.0]))
    assert abs(al[0, 0] - math.exp(-1.0)) < 1e-15
    assert be[0, 0] == 0.5
    # A = 0 (A_log = -inf): no decay whatever the input
    al, _ = lo.gates(np.array([[5.0]]), np.array([[1.0]]), np.array([-np.inf]), np.array([0.0]))
    assert al[0, 0] == 1.0
    # a + dt_bias -> -inf: softplus -> 0, alpha -> 1; large positive input: alpha -> 0
    al, _ = lo.gates(np.array([[-800.0, 800.0]]), np.array([[0.0, 0.0]]), np.array([0.0, 0.0]), np.array([0.0, 0.0]))
    assert al[0, 0] == 1.0 and al[0, 1] == 0.0
    # sigmoid symmetry and saturation
    _, be = lo.gates(np.zeros((1, 3)), np.array([[2.0, -2.0, 50.0]]), np.zeros(3), np.zeros(3))
    assert abs(be[0, 0] + be[0, 1] - 1.0) < 1e-15 and abs(be[0, 2] - 1.0) < 1e-15
    # per-head parameters are taken along the last axis: head 1 decays, head 0 does not
    al, _ = lo.gates(np.zeros((2, 2)), np.zeros((2, 2)), np.array([-np.inf, 0.0]), np.array([0.0, 0.0]))
    assert (al[:, 0] == 1.0).all() and np.allclose(al[:, 1], math.exp(-math.log(2.0)))


def test_round_bf16_halfway_and_exact():
    r = lo.round_bf16_array
    assert r(1.0 + 2.0 ** -8) == 1.0                      # halfway between 1 and 1 + 2^-7: to even (1.0)
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6     # halfway between 1 + 2^-7 and 1 + 2^-6: to even
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7  # just above halfway
    assert r(-3.0) == -3.0 and r(0.0) == 0.0
    assert r(255.5) == 256.0                             # 8 significant bits
    x = np.random.default_rng(0).standard_normal(1000)
    y = r(x)
    np.testing.assert_array_equal(r(y), y)               # idempotent
    _, e = np.frexp(x)                                   # |x| in [2^(e-1), 2^e): bf16 spacing 2^(e-8)
    assert np.all(np.abs(y - x) <= np.ldexp(1.0, e - 9))  # within half a spacing
    for v in (0.1, -7.3, 1e-3):                          # the same as the op oracle's scalar rounding
        assert r(v) == sdm_oracle.round_bf16(v)


def test_layer_split_order_with_copy_weights():
    """w_in copies slices of x into keys, queries and values (0/1 weights; bf16-exact), w_out copies o back: the
    layer must equal the op oracle run on those slices directly, with the gates from their own formula."""
    rng = np.random.default_rng(5)
    B, T, H, widths, dk, d, W, R = 1, 6, 2, (4, 4), 2, 4, 3, 2
    P = len(widths) * dk
    n_in = 2 * H * P + H * d + 2 * H
    Dm = n_in
    x = lo.round_bf16_array(rng.standard_normal((B, T, Dm)))
    # row n of w_in copies column perm[n] of x (a permutation, so each piece takes different columns)
    perm = rng.permutation(Dm)
    w_in = np.zeros((n_in, Dm))
    w_in[np.arange(n_in), perm] = 1.0
    a_log = np.array([0.3, -0.5])
    dt_bias = np.array([-1.0, 0.5])
    w_out = np.eye(Dm, H * d)  # y[:, :, j] = o[:, :, j] for j < H d, else 0
    sub = lo.round_bf16_array(rng.standard_normal((H, sum(widths), dk)))
    bank = rng.standard_normal((B, H, 16, d)).astype(np.float32) * 0.1
    res = lo.layer_forward(x, w_in, a_log, dt_bias, w_out, sub, bank, heads=H, widths=widths, num_writes=W,
                           num_reads=R, nthreads=1)
    xs = x[..., perm]
    o = 0
    keys = xs[..., o:o + H * P].reshape(B, T, H, P); o += H * P
    queries = xs[..., o:o + H * P].reshape(B, T, H, P); o += H * P
    values = xs[..., o:o + H * d].reshape(B, T, H, d); o += H * d
    a = xs[..., o:o + H]; o += H
    b = xs[..., o:o + H]
    alpha = lo.round_bf16_array(np.exp(-np.exp(a_log) * np.logaddexp(0.0, a + dt_bias)))
    beta = lo.round_bf16_array(1.0 / (1.0 + np.exp(-b)))
    ref = sdm_oracle.write_read(keys, queries, values, alpha, beta, sub, bank, widths, W, R, act_bf16=True,
                                nthreads=1)
    np.testing.assert_array_equal(res["op"]["widx"], ref["widx"])
    np.testing.assert_array_equal(res["op"]["ridx"], ref["ridx"])
    np.testing.assert_array_equal(res["alpha"], alpha)
    np.testing.assert_array_equal(res["beta"], beta)
    y_ref = np.zeros((B, T, Dm))
    y_ref[..., :H * d] = np.asarray(ref["out"], dtype=np.float64).reshape(B, T, H * d)
    np.testing.assert_array_equal(res["y"], y_ref)


@pytest.mark.parametrize("seed", [0, 1])
def test_layer_oracle_mistakes_are_caught(seed):
    """The copy-weight pin above fails for a plausible layout mistake: swapping keys and queries changes the ids."""
    rng = np.random.default_rng(seed)
    H, widths, dk = 1, (8, 8), 2
    P = len(widths) * dk
    k = lo.round_bf16_array(rng.standard_normal((1, 4, H, P)))
    q = lo.round_bf16_array(rng.standard_normal((1, 4, H, P)))
    sub = lo.round_bf16_array(rng.standard_normal((H, 16, dk)))
    v = np.ones((1, 4, H, 4))
    g = np.full((1, 4, H), 0.5)
    bank = np.zeros((1, H, 64, 4), dtype=np.float32)
    r1 = sdm_oracle.write_read(k, q, v, g, g, sub, bank, widths, 3, 3, nthreads=1)
    r2 = sdm_oracle.write_read(q, k, v, g, g, sub, bank, widths, 3, 3, nthreads=1)
    assert not np.array_equal(r1["widx"], r2["widx"])


def test_initial_bank_copy_is_the_op_on_every_batch_row():
    """A learned initial bank: the layer starts every batch row from its copy, so each batch row's op equals the op
    oracle run on that row alone from the initial bank (the rows are independent streams)."""
    rng = np.random.default_rng(9)
    B, T, H, widths, dk, d, Dm = 3, 5, 2, (4, 4), 4, 8, 32
    P = len(widths) * dk
    nin = 2 * H * P + H * d + 2 * H
    r = lambda *shape: lo.round_bf16_array(rng.standard_normal(shape))
    x, w_in, w_out = r(B, T, Dm), r(nin, Dm) * 0.2, r(Dm, H * d) * 0.2
    sub = r(H, sum(widths), dk)
    init = (0.1 * rng.standard_normal((H, 16, d))).astype(np.float32)
    a_log, dt_bias = np.zeros(H), np.zeros(H)
    kw = dict(heads=H, widths=widths, num_writes=3, num_reads=2)
    full = lo.layer_forward(x, w_in, a_log, dt_bias, w_out, sub, np.zeros((B, H, 16, d), np.float32),
                            initial_bank=init, **kw)
    cp = lo.initial_bank_copy(init, B)
    assert cp.shape == (B, H, 16, d) and all(np.array_equal(cp[b], init) for b in range(B))
    for b in range(B):
        one = lo.layer_forward(x[b:b + 1], w_in, a_log, dt_bias, w_out, sub, init[None], **kw)
        assert np.array_equal(one["y"][0], full["y"][b])
        assert np.array_equal(one["op"]["bank"][0], full["op"]["bank"][b])
