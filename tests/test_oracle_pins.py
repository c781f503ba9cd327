"""Pins of the CPU oracle against facts fixed by the pages and by mathematics (no GPU).

Each test checks the oracle against something other than itself: exact rational arithmetic, an independent Python
enumeration of every slot, closed forms of the tie order (tests/golden/tie_zero_query.txt), the textbook top-k for
one factor, closed forms of the gated delta rule (no-op gates, a single write, alpha = beta = 1), the dense Gated
DeltaNet recurrence (all slots selected), linearity, and read-after-write order.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gated_delta_rule_product_amd.synth import round_bf16_rne

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------------------------------------ exact arithmetic
def fl32_of_fraction(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even (no intermediate rounding)."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    lsb = max(e - 23, -149)
    r = round(a / Fraction(2) ** lsb)  # Fraction rounding: nearest integer, ties to even
    val = Fraction(r) * Fraction(2) ** lsb
    if val >= Fraction(2) ** 128:
        return np.float32(sign * math.inf)
    return np.float32(sign * float(val))


def exact_dot(q, c) -> Fraction:
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q, c)), Fraction(0))


def fma_chain_emulated(q, c) -> np.float32:
    """fp64 FMA chain emulated with exact rationals: each step is the correctly rounded fp64 of a*b+acc."""
    acc = 0.0
    for a, b in zip(q, c):
        acc = float(Fraction(float(a)) * Fraction(float(b)) + Fraction(acc))
    return np.float32(acc)


def bf16_normal(rng, shape):
    return round_bf16_rne(rng.standard_normal(shape).astype(np.float32))


# ------------------------------------------------------------------------------------------------ rounding
def test_round_bf16_ties_and_no_double_rounding(oracle_lib):
    r = oracle_lib.round_bf16
    assert r(1.0) == 1.0
    assert r(1.0 + 2**-8) == 1.0                      # tie -> even mantissa (0)
    assert r(1.0 + 3 * 2**-8) == 1.0 + 2**-6          # tie -> even mantissa (2)
    assert r(1.0 + 2**-8 + 2**-40) == 1.0 + 2**-7     # just above the tie: up (through float32 it would tie down)
    assert r(-(1.0 + 2**-8 + 2**-40)) == -(1.0 + 2**-7)
    assert r(2.0**-133) == 2.0**-133                  # smallest bfloat16 subnormal
    assert r(3.39e38) == (2 - 2**-7) * 2.0**127               # rounds to the largest finite bfloat16
    assert math.isinf(r(3.4e38))                              # past the last rounding boundary
    # agrees with the input module's independent float32 -> bfloat16 bit rounding on random float32 values
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(2000) * np.exp(rng.uniform(-20, 20, 2000))).astype(np.float32)
    ours = np.array([r(float(v)) for v in x], dtype=np.float32)
    assert np.array_equal(ours, round_bf16_rne(x))


# ------------------------------------------------------------------------------------------------ factor scores
@pytest.mark.parametrize("dk", [16, 64])
def test_factor_score_bf16_equals_rounded_exact_dot(oracle_lib, dk):
    rng = np.random.default_rng(dk)
    q = bf16_normal(rng, dk)
    C = bf16_normal(rng, (24, dk))
    s = oracle_lib.factor_scores(q, C)
    want = np.array([fl32_of_fraction(exact_dot(q, C[i])) for i in range(C.shape[0])], dtype=np.float32)
    assert np.array_equal(s, want)


def test_factor_score_fp32_is_the_ordered_fma_chain(oracle_lib):
    rng = np.random.default_rng(7)
    dk = 32
    q = rng.standard_normal(dk).astype(np.float32)
    C = rng.standard_normal((16, dk)).astype(np.float32)
    s = oracle_lib.factor_scores(q, C)
    chain = np.array([fma_chain_emulated(q, C[i]) for i in range(16)], dtype=np.float32)
    assert np.array_equal(s, chain)
    exact = np.array([fl32_of_fraction(exact_dot(q, C[i])) for i in range(16)], dtype=np.float32)
    ulp = np.spacing(np.abs(exact))
    assert np.all(np.abs(s.astype(np.float64) - exact) <= ulp)


def test_factor_score_unit_query_selects_coordinate(oracle_lib):
    rng = np.random.default_rng(3)
    C = rng.standard_normal((10, 8)).astype(np.float32)
    for c in range(8):
        q = np.zeros(8, np.float32)
        q[c] = 1.0
        assert np.array_equal(oracle_lib.factor_scores(q, C), C[:, c])


# ------------------------------------------------------------------------------------------------ softmax
def test_softmax_closed_forms(oracle_lib):
    assert np.array_equal(oracle_lib.softmax(np.zeros(4, np.float32)), np.full(4, 0.25))
    w = oracle_lib.softmax(np.array([1000.0, 1000.0], np.float32))  # max-subtracted: no overflow
    assert np.array_equal(w, np.array([0.5, 0.5]))
    s = np.array([0.0, math.log(3.0)], np.float32)
    w = oracle_lib.softmax(s)
    assert abs(w[1] / w[0] - math.exp(float(s[1]))) < 1e-12 and abs(w.sum() - 1.0) < 1e-15


# ------------------------------------------------------------------------------------------------ top-k
def python_brute_topk(q, sub, widths, k):
    """Independent enumeration of every slot: exact-rational factor scores, float32 slot sums, full sort."""
    F = len(widths)
    dk = sub.shape[1]
    offs = np.concatenate([[0], np.cumsum(widths)])
    fs, pos = [], []
    for f in range(F):
        s = [fl32_of_fraction(exact_dot(q[f * dk:(f + 1) * dk], sub[offs[f] + i])) for i in range(widths[f])]
        order = sorted(range(widths[f]), key=lambda i: (-float(s[i]), i))
        p = [0] * widths[f]
        for rank, i in enumerate(order):
            p[i] = rank
        fs.append(s)
        pos.append(p)
    slots = []
    for digits in itertools.product(*[range(n) for n in widths]):  # factor 0 most significant
        S = fs[0][digits[0]]
        for f in range(1, F):
            S = np.float32(S + fs[f][digits[f]])
        ps = [pos[f][digits[f]] for f in range(F)]
        sid = 0
        for f in range(F):
            sid = sid * widths[f] + digits[f]
        slots.append((-float(S), sum(ps), tuple(ps), sid, np.float32(S)))
    slots.sort(key=lambda t: (t[0], t[1], t[2]))
    top = slots[:k]
    return np.array([t[3] for t in top], np.int32), np.array([t[4] for t in top], np.float32)


def _tie_data(rng, widths, dk, kind):
    F = len(widths)
    if kind == "ternary":  # small integers: exact scores, many equal
        q = rng.integers(-1, 2, F * dk).astype(np.float32)
        sub = rng.integers(-1, 2, (sum(widths), dk)).astype(np.float32)
    elif kind == "duplicate_rows":
        q = bf16_normal(rng, F * dk)
        sub = bf16_normal(rng, (sum(widths), dk))
        for _ in range(sum(widths) // 2):
            i, j = rng.integers(0, sum(widths), 2)
            sub[j] = sub[i]
    else:
        q = bf16_normal(rng, F * dk)
        sub = bf16_normal(rng, (sum(widths), dk))
    return q, sub


@pytest.mark.parametrize("widths,dk,k", [((8, 8), 4, 5), ((8, 8), 4, 64), ((4, 3, 5), 3, 7), ((6, 5), 5, 12),
                                         ((3, 2, 2, 3), 2, 9), ((16,), 4, 6)])
@pytest.mark.parametrize("kind", ["random", "ternary", "duplicate_rows"])
def test_topk_equals_independent_brute_force(oracle_lib, widths, dk, k, kind):
    rng = np.random.default_rng(hash((widths, dk, k, kind)) & 0xFFFF)
    for _ in range(3):
        q, sub = _tie_data(rng, widths, dk, kind)
        ids, sc = oracle_lib.topk_one(q, sub, widths, k)
        want_ids, want_sc = python_brute_topk(q, sub, widths, k)
        assert np.array_equal(ids, want_ids)
        assert np.array_equal(sc, want_sc)


def test_topk_zero_query_golden(oracle_lib):
    with open(os.path.join(GOLDEN, "tie_zero_query.txt")) as f:
        rows = [ln for ln in f.read().splitlines() if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 3
    rng = np.random.default_rng(0)
    for ln in rows:
        w, k, ids = [x.strip() for x in ln.split(";")]
        widths = [int(x) for x in w.split(",")]
        k = int(k)
        want = np.array([int(x) for x in ids.split(",")], np.int32)
        dk = 8
        q = np.zeros(len(widths) * dk, np.float32)
        sub = rng.standard_normal((sum(widths), dk)).astype(np.float32)
        got, sc = oracle_lib.topk_one(q, sub, widths, k)
        assert np.array_equal(got, want), (widths, k, got, want)
        assert np.all(sc == 0.0)


def test_topk_one_factor_is_textbook_topk(oracle_lib):
    rng = np.random.default_rng(11)
    for n, k in [(50, 7), (33, 33), (64, 1)]:
        q = rng.standard_normal(6).astype(np.float32)
        sub = rng.standard_normal((n, 6)).astype(np.float32)
        sub[5] = sub[9]  # a tie: the smaller index must come first
        s = oracle_lib.factor_scores(q, sub)
        want = np.argsort(-s.astype(np.float64), kind="stable")[:k].astype(np.int32)
        got, sc = oracle_lib.topk_one(q, sub, [n], k)
        assert np.array_equal(got, want)
        assert np.array_equal(sc, s[want])


def test_topk_batched_matches_single(oracle_lib):
    rng = np.random.default_rng(5)
    B, T, H, widths, dk, k = 2, 3, 2, (8, 4), 4, 6
    q = rng.standard_normal((B, T, H, 2 * dk)).astype(np.float32)
    sub = rng.standard_normal((H, 12, dk)).astype(np.float32)
    ids, sc = oracle_lib.topk(q, sub, widths, k, nthreads=3)
    for b, t, h in itertools.product(range(B), range(T), range(H)):
        i1, s1 = oracle_lib.topk_one(q[b, t, h], sub[h], widths, k)
        assert np.array_equal(ids[b, t, h], i1) and np.array_equal(sc[b, t, h], s1)


# ------------------------------------------------------------------------------------------------ write / read
def _wr_inputs(rng, B, T, H, widths, dk, d, N):
    F = len(widths)
    return dict(
        wkeys=rng.standard_normal((B, T, H, F * dk)).astype(np.float32),
        rq=rng.standard_normal((B, T, H, F * dk)).astype(np.float32),
        values=rng.standard_normal((B, T, H, d)).astype(np.float32),
        alpha=(1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32),
        beta=(1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32),
        subkeys=rng.standard_normal((H, sum(widths), dk)).astype(np.float32),
        bank=(0.02 * rng.standard_normal((B, H, N, d))).astype(np.float32),
    )


def _softmax_np(s):
    s = np.asarray(s, np.float64)
    e = np.exp(s - s.max())
    return e / e.sum()


def test_noop_gates_leave_bank_and_read_is_weighted_gather(oracle_lib):
    rng = np.random.default_rng(21)
    B, T, H, widths, dk, d, W, R = 1, 12, 2, (8, 8), 4, 8, 4, 5
    x = _wr_inputs(rng, B, T, H, widths, dk, d, 64)
    x["alpha"][:] = 1.0
    x["beta"][:] = 0.0
    res = oracle_lib.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                                widths, W, R)
    assert np.array_equal(res["bank"], x["bank"])
    for b, t, h in itertools.product(range(B), range(T), range(H)):
        rho = _softmax_np(res["rscore"][b, t, h])
        want = (rho[:, None] * x["bank"][b, h][res["ridx"][b, t, h]].astype(np.float64)).sum(0)
        np.testing.assert_allclose(res["out"][b, t, h], want, rtol=1e-6, atol=1e-9)


def test_single_write_closed_form(oracle_lib):
    """W = 1: the weight is exactly 1, so M[j] <- alpha (1 - beta) M[j] + beta v."""
    rng = np.random.default_rng(22)
    B, T, H, widths, dk, d = 1, 30, 1, (4, 4), 3, 5
    x = _wr_inputs(rng, B, T, H, widths, dk, d, 16)
    res = oracle_lib.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                                widths, 1, 1)
    M = x["bank"][0, 0].astype(np.float64).copy()
    for t in range(T):
        j = res["widx"][0, t, 0, 0]
        a, be = float(x["alpha"][0, t, 0]), float(x["beta"][0, t, 0])
        M[j] = (a * (1 - be) * M[j] + be * x["values"][0, t, 0]).astype(np.float32)
    np.testing.assert_allclose(res["bank"][0, 0], M, rtol=2e-6, atol=1e-9)


def test_full_gates_store_value_exactly_and_read_after_write(oracle_lib):
    """alpha = beta = 1, W = R = 1 with the read query equal to the write key: the written row becomes v exactly
    and the same token's read returns it (a read before the write would return the old row)."""
    rng = np.random.default_rng(23)
    B, T, H, widths, dk, d = 1, 10, 1, (4, 4), 3, 6
    x = _wr_inputs(rng, B, T, H, widths, dk, d, 16)
    x["alpha"][:] = 1.0
    x["beta"][:] = 1.0
    res = oracle_lib.write_read(x["wkeys"], x["wkeys"], x["values"], x["alpha"], x["beta"], x["subkeys"],
                                x["bank"], widths, 1, 1)
    assert np.array_equal(res["out"], x["values"])
    last = {}
    for t in range(T):
        last[int(res["widx"][0, t, 0, 0])] = t
    for j, t in last.items():
        assert np.array_equal(res["bank"][0, 0, j], x["values"][0, t, 0])


def test_unselected_rows_are_untouched(oracle_lib):
    rng = np.random.default_rng(24)
    B, T, H, widths, dk, d, W, R = 2, 20, 1, (16, 16), 4, 4, 3, 3
    x = _wr_inputs(rng, B, T, H, widths, dk, d, 256)
    res = oracle_lib.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                                widths, W, R)
    for b in range(B):
        written = set(res["widx"][b, :, 0].ravel().tolist())
        untouched = np.array(sorted(set(range(256)) - written))
        assert len(untouched) > 150
        assert np.array_equal(res["bank"][b, 0, untouched], x["bank"][b, 0, untouched])
        assert not np.array_equal(res["bank"][b, 0, sorted(written)], x["bank"][b, 0, sorted(written)])


def test_dense_limit_is_gated_deltanet(oracle_lib):
    """W = R = N: every slot is selected, and the recurrence is Gated DeltaNet in slot space with key w:
    M_t = alpha (I - beta w w^T) M_{t-1} + beta w v^T,   o_t = M_t^T rho."""
    rng = np.random.default_rng(25)
    B, T, H, widths, dk, d = 1, 12, 2, (4, 4), 3, 6
    N = 16
    x = _wr_inputs(rng, B, T, H, widths, dk, d, N)
    x["bank"] *= 50.0
    res = oracle_lib.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                                widths, N, N)
    for h in range(H):
        M = x["bank"][0, h].astype(np.float64).copy()
        for t in range(T):
            w = np.zeros(N)
            w[res["widx"][0, t, h]] = _softmax_np(res["wscore"][0, t, h])
            rho = np.zeros(N)
            rho[res["ridx"][0, t, h]] = _softmax_np(res["rscore"][0, t, h])
            a, be = float(x["alpha"][0, t, h]), float(x["beta"][0, t, h])
            v = x["values"][0, t, h].astype(np.float64)
            M = a * (np.eye(N) - be * np.outer(w, w)) @ M + be * np.outer(w, v)
            np.testing.assert_allclose(res["out"][0, t, h], M.T @ rho, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(res["bank"][0, h], M, rtol=1e-5, atol=1e-6)


def test_linear_in_bank_and_values(oracle_lib):
    rng = np.random.default_rng(26)
    B, T, H, widths, dk, d, W, R = 1, 25, 1, (8, 8), 4, 8, 4, 4
    x = _wr_inputs(rng, B, T, H, widths, dk, d, 64)
    y = _wr_inputs(rng, B, T, H, widths, dk, d, 64)

    def run(bank, values):
        return oracle_lib.write_read(x["wkeys"], x["rq"], values, x["alpha"], x["beta"], x["subkeys"], bank,
                                     widths, W, R)

    ra = run(x["bank"], x["values"])
    rb = run(y["bank"], y["values"])
    rc = run((x["bank"] + 2 * y["bank"]).astype(np.float32), (x["values"] + 2 * y["values"]).astype(np.float32))
    np.testing.assert_allclose(rc["out"], ra["out"] + 2 * rb["out"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(rc["bank"], ra["bank"] + 2 * rb["bank"], rtol=1e-5, atol=1e-5)


def test_bf16_bank_rows_stay_bf16(oracle_lib):
    rng = np.random.default_rng(27)
    B, T, H, widths, dk, d, W, R = 1, 15, 1, (8, 8), 4, 8, 4, 4
    x = _wr_inputs(rng, B, T, H, widths, dk, d, 64)
    bank = round_bf16_rne(x["bank"])
    res = oracle_lib.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], bank,
                                widths, W, R, bank_bf16=True, act_bf16=True)
    assert np.array_equal(res["bank"], round_bf16_rne(res["bank"]))
    assert np.array_equal(res["out"], round_bf16_rne(res["out"]))


def test_streams_are_independent_and_threads_do_not_matter(oracle_lib):
    rng = np.random.default_rng(28)
    B, T, H, widths, dk, d, W, R = 2, 9, 3, (8, 4), 4, 4, 3, 2
    x = _wr_inputs(rng, B, T, H, widths, dk, d, 32)
    args = (x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"], widths, W, R)
    r1 = oracle_lib.write_read(*args, nthreads=1)
    r4 = oracle_lib.write_read(*args, nthreads=4)
    for k in ("out", "bank", "widx", "ridx"):
        assert np.array_equal(r1[k], r4[k])
    # stream (1, 2) alone gives the same result as inside the batch
    sl = lambda a: a[1:2, :, 2:3]
    r = oracle_lib.write_read(sl(x["wkeys"]), sl(x["rq"]), sl(x["values"]), sl(x["alpha"]), sl(x["beta"]),
                              x["subkeys"][2:3], x["bank"][1:2, 2:3], widths, W, R)
    assert np.array_equal(r["out"][0, :, 0], r1["out"][1, :, 2])
    assert np.array_equal(r["bank"][0, 0], r1["bank"][1, 2])
