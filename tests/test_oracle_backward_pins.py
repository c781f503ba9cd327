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
