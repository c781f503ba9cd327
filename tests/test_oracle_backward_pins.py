"""Pins of the oracle's backward (no GPU): its gradients are the derivatives of the forward.

Central finite differences of the loss L = <U_out, out> + <U_bank, bank after the call>, taken on the oracle's
fp64-state forward (exact=True) along a random direction in one input at a time, must equal <gradient, direction>.
Perturbed inputs are float32 arrays, so the direction used is the exact difference of the rounded perturbed inputs;
key perturbations must leave every selected slot unchanged (checked with the oracle's top-k). Small banks make slots
collide across tokens, so every term of the reverse recurrence carries weight. The fp64-state forward itself is
pinned to oracle.write_read, and the rounded-state forward that the backward replays equals it bit for bit.
"""
import numpy as np
import pytest

import oracle


def _case(seed, B, T, H, widths, dk, d, W, R):
    rng = np.random.default_rng(seed)
    F = len(widths)
    x = {
        "wkeys": rng.standard_normal((B, T, H, F * dk)).astype(np.float32),
        "rq": rng.standard_normal((B, T, H, F * dk)).astype(np.float32),
        "values": rng.standard_normal((B, T, H, d)).astype(np.float32),
        "alpha": (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32),
        "beta": (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32),
        "subkeys": rng.standard_normal((H, sum(widths), dk)).astype(np.float32),
        "bank": (0.5 * rng.standard_normal((B, H, int(np.prod(widths)), d))).astype(np.float32),
    }
    # resample queries whose k-th and (k+1)-th slot scores are closer than 0.05, so that a finite-difference step
    # of the keys (score changes below 0.01) never changes a selected set
    N = int(np.prod(widths))
    for name, k in (("wkeys", W), ("rq", R)):
        if k >= N:
            continue
        for _ in range(50):
            _, sc = oracle.topk(x[name], x["subkeys"], widths, k + 1)
            close = (sc[..., k - 1] - sc[..., k]) < 0.05
            if not close.any():
                break
            x[name][close] = rng.standard_normal((int(close.sum()), F * dk)).astype(np.float32)
        else:
            raise AssertionError("could not separate the selected sets")
    u_out = rng.standard_normal((B, T, H, d)).astype(np.float32)
    u_bank = rng.standard_normal(x["bank"].shape).astype(np.float32)
    return x, u_out, u_bank, (widths, W, R)


def _loss(x, u_out, u_bank, cfg):
    widths, W, R = cfg
    r = oracle.write_read_backward(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                                   u_out, u_bank, widths, W, R, exact=True, want_forward=True, nthreads=1)
    L = float(np.sum(r["out"] * u_out.astype(np.float64)) + np.sum(r["bank"] * u_bank.astype(np.float64)))
    return L, r


def _ids(x, cfg):
    """The selected slot sets (sorted ids: the order inside a top-k only changes the rounding of the sums)."""
    widths, W, R = cfg
    return (np.sort(oracle.topk(x["wkeys"], x["subkeys"], widths, W)[0], axis=-1),
            np.sort(oracle.topk(x["rq"], x["subkeys"], widths, R)[0], axis=-1))


GRAD = {"wkeys": "d_wkeys", "rq": "d_rq", "values": "d_values", "alpha": "d_alpha", "beta": "d_beta",
        "subkeys": "d_subkeys", "bank": "d_bank"}
CASES = [
    # seed, B, T, H, widths, dk, d, W, R
    (1, 2, 10, 2, (4, 4), 3, 5, 4, 3),      # 16 slots, 4 writes a token: slots collide across tokens
    (2, 1, 12, 1, (12,), 4, 6, 3, 5),       # one factor
    (3, 1, 8, 2, (3, 2, 3), 2, 4, 5, 4),    # three factors
    (4, 1, 6, 1, (2, 2), 3, 3, 4, 4),       # every slot written and read by every token (dense limit)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
@pytest.mark.parametrize("name", list(GRAD))
def test_gradient_equals_finite_difference(case, name):
    seed, B, T, H, widths, dk, d, W, R = case
    x, u_out, u_bank, cfg = _case(seed, B, T, H, widths, dk, d, W, R)
    _, r = _loss(x, u_out, u_bank, cfg)
    g = r[GRAD[name]]
    rng = np.random.default_rng(100 + seed)
    direction = rng.standard_normal(x[name].shape)
    smooth = name in ("values", "bank", "alpha", "beta")
    h = 1e-4 if smooth else 1e-3
    if name in ("alpha", "beta"):
        h = 1e-4 * 0.25  # stays inside (0, 1)
    xp, xm = dict(x), dict(x)
    xp[name] = (x[name] + h * direction).astype(np.float32)
    xm[name] = (x[name] - h * direction).astype(np.float32)
    if not smooth:
        ids0 = _ids(x, cfg)
        for y in (xp, xm):
            for a, b in zip(ids0, _ids(y, cfg)):
                assert np.array_equal(a, b), "the perturbation changed a selected slot"
    Lp, _ = _loss(xp, u_out, u_bank, cfg)
    Lm, _ = _loss(xm, u_out, u_bank, cfg)
    step = xp[name].astype(np.float64) - xm[name].astype(np.float64)  # the exact float32 perturbation
    fd = Lp - Lm
    an = float(np.sum(g * step))
    scale = float(np.sum(np.abs(g * step)))
    # smooth inputs: the loss is polynomial in them, the error is fp64 rounding and O(h^2);
    # keys: the float32 rounding of the perturbed scores adds about 1e-7 / 1e-3 relative
    tol = 1e-6 if smooth else 3e-3
    assert abs(fd - an) <= tol * scale, f"{name}: finite difference {fd} vs gradient {an} (scale {scale})"


def test_exact_forward_matches_the_oracle_forward():
    x, u_out, u_bank, cfg = _case(5, 2, 16, 2, (4, 8), 4, 8, 6, 5)
    widths, W, R = cfg
    _, r = _loss(x, u_out, u_bank, cfg)
    ref = oracle.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"], widths,
                            W, R)
    assert np.max(np.abs(r["out"] - ref["out"])) <= 1e-5 * max(1.0, np.max(np.abs(ref["out"])))
    assert np.max(np.abs(r["bank"] - ref["bank"])) <= 1e-5 * max(1.0, np.max(np.abs(ref["bank"])))


@pytest.mark.parametrize("bank_bf16", [False, True])
def test_rounded_replay_equals_the_oracle_forward_bitwise(bank_bf16):
    x, u_out, u_bank, cfg = _case(6, 1, 20, 2, (4, 8), 4, 8, 6, 5)
    widths, W, R = cfg
    if bank_bf16:
        x["bank"] = np.array([[[[oracle.round_bf16(float(v)) for v in row] for row in m] for m in s] for s in
                              x["bank"]], dtype=np.float32)
    r = oracle.write_read_backward(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                                   u_out, None, widths, W, R, bank_bf16=bank_bf16, want_forward=True)
    ref = oracle.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"], widths,
                            W, R, bank_bf16=bank_bf16)
    assert np.array_equal(r["out"].astype(np.float32), ref["out"])
    assert np.array_equal(r["bank"].astype(np.float32), ref["bank"])


def test_zero_upstream_gradient_gives_zero_and_bank_gradient_passes_untouched_rows():
    x, u_out, u_bank, cfg = _case(7, 1, 5, 1, (8, 8), 3, 4, 2, 2)
    widths, W, R = cfg
    z = np.zeros_like(u_out)
    r = oracle.write_read_backward(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                                   z, None, widths, W, R)
    for k in GRAD.values():
        assert not np.any(r[k])
    r = oracle.write_read_backward(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                                   z, u_bank, widths, W, R)
    wid, rid = _ids(x, cfg)
    touched = set(wid[0, :, 0].ravel()) | set(rid[0, :, 0].ravel())
    untouched = [s for s in range(64) if s not in touched]
    assert untouched
    assert np.array_equal(r["d_bank"][0, 0, untouched], u_bank[0, 0, untouched].astype(np.float64))


# ------------------------------------------------------------------ bfloat16 snapshot (CHANGELOG 2.0.0, "New")
def _bwd(x, dout, dbank, widths, W, R, **kw):
    return oracle.write_read_backward(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"],
                                      x["bank"], dout, dbank, widths, W, R, nthreads=1, **kw)


def _rbf16(a):
    return np.vectorize(oracle.round_bf16)(np.asarray(a, dtype=np.float64))


def test_bf16_snapshot_leaves_value_and_bank_gradients_alone():
    """The rounded rows feed only the key, gate and query gradients: d_values and d_bank use no row."""
    x = _case(7, 1, 12, 2, (4, 4), 3, 5, 3, 2)[0]
    rng = np.random.default_rng(8)
    dout = rng.standard_normal(x["values"].shape).astype(np.float32)
    dbank = rng.standard_normal(x["bank"].shape).astype(np.float32)
    a = _bwd(x, dout, dbank, (4, 4), 3, 2)
    b = _bwd(x, dout, dbank, (4, 4), 3, 2, snap_bf16=True)
    np.testing.assert_array_equal(a["d_values"], b["d_values"])
    np.testing.assert_array_equal(a["d_bank"], b["d_bank"])
    assert not np.array_equal(a["d_alpha"], b["d_alpha"])  # the rows are not bf16-exact here


def test_bf16_snapshot_of_exact_rows_changes_nothing():
    """Rows that are bfloat16 values already (a bf16 bank that never changes: alpha = 1, beta = 0) round to
    themselves: every gradient equals the float32 snapshot's."""
    x = _case(9, 1, 10, 1, (4, 4), 3, 6, 3, 3)[0]
    x["bank"] = _rbf16(x["bank"]).astype(np.float32)
    x["alpha"][:] = 1.0
    x["beta"][:] = 0.0
    rng = np.random.default_rng(10)
    dout = rng.standard_normal(x["values"].shape).astype(np.float32)
    a = _bwd(x, dout, None, (4, 4), 3, 3)
    b = _bwd(x, dout, None, (4, 4), 3, 3, snap_bf16=True)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_bf16_snapshot_one_token_gate_gradients_by_hand():
    """One token, one slot written and read (the same key and query): g = dout, D = dout, r = P, so
    d alpha = (1 - beta) <dout, P~> and d beta = <dout, v - alpha P~> with P~ the row rounded to bfloat16."""
    rng = np.random.default_rng(11)
    widths, dk, d = (4,), 2, 6
    q = rng.standard_normal((1, 1, 1, dk)).astype(np.float32)
    x = {"wkeys": q, "rq": q.copy(), "values": rng.standard_normal((1, 1, 1, d)).astype(np.float32),
         "alpha": np.array([[[0.7]]], np.float32), "beta": np.array([[[0.3]]], np.float32),
         "subkeys": rng.standard_normal((1, 4, dk)).astype(np.float32),
         "bank": (rng.standard_normal((1, 1, 4, d)) / 3).astype(np.float32)}
    dout = rng.standard_normal((1, 1, 1, d)).astype(np.float32)
    ids, _ = oracle.topk(q, x["subkeys"], widths, 1)
    P = x["bank"][0, 0, ids[0, 0, 0, 0]].astype(np.float64)
    Pq = _rbf16(P)
    assert not np.array_equal(P, Pq)
    a, be = np.float64(x["alpha"][0, 0, 0]), np.float64(x["beta"][0, 0, 0])
    g = dout[0, 0, 0].astype(np.float64)
    v = x["values"][0, 0, 0].astype(np.float64)
    for Prow, kw in ((P, {}), (Pq, {"snap_bf16": True})):
        r = _bwd(x, dout, None, widths, 1, 1, **kw)
        assert abs(r["d_alpha"][0, 0, 0] - (1 - be) * (g @ Prow)) <= 1e-12
        assert abs(r["d_beta"][0, 0, 0] - g @ (v - a * Prow)) <= 1e-12


def test_bf16_snapshot_rounds_a_read_row_only_if_a_later_token_writes_its_slot():
    """Token 0 reads slot s; token 1 writes s (and token 0 does not). Rounding the row read at token 0 is what
    the in-place restore from a bfloat16 snapshot gives; with one token (nothing later) the read gradient matches
    the float32 snapshot's exactly."""
    rng = np.random.default_rng(12)
    widths, dk, d = (4,), 2, 5
    sub = np.zeros((1, 4, dk), np.float32)
    sub[0, :, 0] = [3.0, 2.0, 1.0, 0.0]  # query (1, 0) ranks slots 0, 1, 2, 3; query (-1, 0) ranks 3, 2, 1, 0
    q_best0 = np.array([1.0, 0.0], np.float32)
    q_best3 = np.array([-1.0, 0.0], np.float32)
    x = {"wkeys": np.stack([q_best3, q_best0])[None, :, None, :],    # writes: token 0 slot 3, token 1 slot 0
         "rq": np.stack([q_best0, q_best3])[None, :, None, :],       # reads (R = 2): token 0 slots 0, 1
         "values": rng.standard_normal((1, 2, 1, d)).astype(np.float32),
         "alpha": np.array([[[0.9], [0.8]]], np.float32), "beta": np.array([[[0.4], [0.6]]], np.float32),
         "subkeys": sub, "bank": (rng.standard_normal((1, 1, 4, d)) / 3).astype(np.float32)}
    dout = rng.standard_normal((1, 2, 1, d)).astype(np.float32)
    a = _bwd(x, dout, None, widths, 1, 2)
    b = _bwd(x, dout, None, widths, 1, 2, snap_bf16=True)
    assert not np.array_equal(a["d_rq"][0, 0], b["d_rq"][0, 0])  # token 0 read slot 0, which token 1 rewrites
    one = {k: v[:, :1] for k, v in x.items() if k not in ("subkeys", "bank")}
    one.update(subkeys=x["subkeys"], bank=x["bank"])
    a1 = _bwd(one, dout[:, :1], None, widths, 1, 2)
    b1 = _bwd(one, dout[:, :1], None, widths, 1, 2, snap_bf16=True)
    np.testing.assert_array_equal(a1["d_rq"], b1["d_rq"])
