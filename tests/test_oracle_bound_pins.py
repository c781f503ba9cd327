"""Pins of the oracle's backward error bounds (no GPU).

oracle.write_read_backward_bounds returns, with each gradient element, a bound on how far another evaluation of the
same backward may be from the fp64 one: an evaluation that reads rows within eps_row of the oracle's (relative to
each row's largest magnitude), has softmax weights within eps_w, and rounds every other operation with unit
roundoff u in any order (first-order running error analysis; sdm_oracle.c, the comment above bound_par_t).

Pinned here against an independent evaluation: the same chain rule written out below in plain float32 numpy, token
by token (its own forward in float32 too, so its rows carry float32 rounding). With eps_row set to the deviation its
rows actually have (measured row by row in the test, the hypothesis of the bound) and u = 2^-24, every element of
every gradient must be inside the bound; and a float32 evaluation with one term of the chain rule dropped or with a
wrong sign must fall outside it somewhere, so the bound is tight enough to see such mistakes. With u = eps_row =
eps_w = 0 the bounds are exactly zero.
"""
import numpy as np
import pytest

import oracle

f32 = np.float32


def _inputs(seed, B, T, H, widths, dk, d, bank_scale=0.5):
    rng = np.random.default_rng(seed)
    F = len(widths)
    return {
        "wkeys": rng.standard_normal((B, T, H, F * dk)).astype(f32),
        "rq": rng.standard_normal((B, T, H, F * dk)).astype(f32),
        "values": rng.standard_normal((B, T, H, d)).astype(f32),
        "alpha": (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(f32),
        "beta": (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(f32),
        "subkeys": rng.standard_normal((H, sum(widths), dk)).astype(f32),
        "bank": (bank_scale * rng.standard_normal((B, H, int(np.prod(widths)), d))).astype(f32),
    }, rng.standard_normal((B, T, H, d)).astype(f32), rng.standard_normal((B, H, int(np.prod(widths)), d)).astype(f32)


def _softmax32(s):
    s = s.astype(f32)
    e = np.exp(s - s.max()).astype(f32)
    return (e / e.sum(dtype=f32)).astype(f32)


def _float32_backward(x, dout, dbank, widths, W, R, mutate=None):
    """The write/read's chain rule evaluated in float32 (forward replay included). mutate names one planted mistake."""
    B, T, H, Fdk = x["wkeys"].shape
    F = len(widths)
    dk = Fdk // F
    d = x["values"].shape[-1]
    wid, wsc = oracle.topk(x["wkeys"], x["subkeys"], widths, W)
    rid, rsc = oracle.topk(x["rq"], x["subkeys"], widths, R)
    g = {k: np.zeros(x[k].shape, f32) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    g["bank"] = np.zeros(x["bank"].shape, f32)
    rows_P = np.zeros((B, H, T, W, d), f32)
    offs = np.concatenate([[0], np.cumsum(widths)[:-1]])

    def digits(sid):
        out = []
        for f in range(F - 1, -1, -1):
            out.append(sid % widths[f])
            sid //= widths[f]
        return out[::-1]

    def score_bwd(sid, ds, q, dq, dsub):
        for f, i in enumerate(digits(int(sid))):
            c = x["subkeys"][h, offs[f] + i]
            dq[f * dk:(f + 1) * dk] += f32(ds) * c
            dsub[offs[f] + i] += f32(ds) * q[f * dk:(f + 1) * dk]

    for b in range(B):
        for h in range(H):
            M = x["bank"][b, h].copy()
            trace = []
            for t in range(T):
                S, Rr = wid[b, t, h], rid[b, t, h]
                w, rho = _softmax32(wsc[b, t, h]), _softmax32(rsc[b, t, h])
                a, be, v = x["alpha"][b, t, h], x["beta"][b, t, h], x["values"][b, t, h]
                P = M[S].copy()
                r = (w[:, None] * P).sum(axis=0, dtype=f32)
                dl = (be * (v - a * r)).astype(f32)
                M[S] = (a * P + w[:, None] * dl[None, :]).astype(f32)
                V = M[Rr].copy()
                rows_P[b, h, t] = P
                trace.append((S, Rr, w, rho, a, be, v, P, r, dl, V))
            G = (dbank[b, h] if dbank is not None else np.zeros_like(M)).astype(f32).copy()
            for t in range(T - 1, -1, -1):
                S, Rr, w, rho, a, be, v, P, r, dl, V = trace[t]
                do = dout[b, t, h]
                drho = (V * do[None, :]).sum(axis=1, dtype=f32)
                G[Rr] += (rho[:, None] * do[None, :]).astype(f32)
                ssum = (rho * drho).sum(dtype=f32)
                for j in range(R):
                    score_bwd(Rr[j], rho[j] * (drho[j] - ssum), x["rq"][b, t, h], g["rq"][b, t, h], g["subkeys"][h])
                gi = G[S].copy()
                D = (w[:, None] * gi).sum(axis=0, dtype=f32)
                g["values"][b, t, h] = be * D
                g["beta"][b, t, h] = (D * (v - a * r)).sum(dtype=f32)
                dal = (gi * P).sum(dtype=f32) - be * (D * r).sum(dtype=f32)
                if mutate == "alpha_sign":
                    dal = (gi * P).sum(dtype=f32) + be * (D * r).sum(dtype=f32)
                g["alpha"][b, t, h] = dal
                dw = (gi * dl[None, :]).sum(axis=1, dtype=f32) - a * be * (D[None, :] * P).sum(axis=1, dtype=f32)
                if mutate == "dw_no_P":
                    dw = (gi * dl[None, :]).sum(axis=1, dtype=f32)
                upd = (a * gi - a * be * w[:, None] * D[None, :]).astype(f32)
                if mutate == "adjoint_no_D":
                    upd = (a * gi).astype(f32)
                G[S] = upd
                ssum = (w * dw).sum(dtype=f32)
                for i in range(W):
                    ds = w[i] * (dw[i] - ssum)
                    if mutate == "uncentred":
                        ds = w[i] * dw[i]
                    score_bwd(S[i], ds, x["wkeys"][b, t, h], g["wkeys"][b, t, h], g["subkeys"][h])
            g["bank"][b, h] = G
    return g, rows_P


def _row_dev(got, ref):
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    return float((np.abs(got - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-300)).max())


GRADS = {"wkeys": "d_wkeys", "rq": "d_rq", "values": "d_values", "alpha": "d_alpha", "beta": "d_beta",
         "subkeys": "d_subkeys", "bank": "d_bank"}

CASES = [  # seed, B, T, H, widths, dk, d, W, R: small banks, so slots collide across tokens
    (1, 1, 24, 2, (4, 4), 4, 16, 4, 3),
    (2, 2, 16, 1, (8, 4), 3, 8, 8, 5),
    (3, 1, 20, 1, (4, 2, 2), 4, 12, 6, 6),
]


def _bounds(x, dout, dbank, widths, W, R, eps_row, **kw):
    return oracle.write_read_backward_bounds(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"],
                                             x["subkeys"], x["bank"], dout, dbank, widths, W, R, eps_row=eps_row,
                                             want_snapshot=True, nthreads=1, **kw)


@pytest.mark.parametrize("case", CASES)
def test_float32_evaluation_within_bounds(case):
    seed, B, T, H, widths, dk, d, W, R = case
    x, dout, dbank = _inputs(seed, B, T, H, widths, dk, d)
    g32, P32 = _float32_backward(x, dout, dbank, widths, W, R)
    # the hypothesis: rows within eps_row; measured on this evaluation's pre-write rows (read rows are later
    # pre-write rows or final rows, which come from the same float32 recurrence)
    probe = _bounds(x, dout, dbank, widths, W, R, eps_row=0.0)
    eps_row = max(_row_dev(P32, probe["snapshot"]), 2.0 ** -24)
    res = _bounds(x, dout, dbank, widths, W, R, eps_row=2 * eps_row)
    for k, r in GRADS.items():
        err = np.abs(g32[k].astype(np.float64) - res[r])
        bound = res["e_" + k] * 1.01
        assert np.all(err <= bound), (k, float((err - bound).max()))
        assert np.all(res["e_" + k] >= 0)


@pytest.mark.parametrize("mutate,grad", [("alpha_sign", "alpha"), ("dw_no_P", "wkeys"), ("adjoint_no_D", "bank"),
                                         ("uncentred", "wkeys")])
def test_bounds_see_planted_mistakes(mutate, grad):
    seed, B, T, H, widths, dk, d, W, R = CASES[0]
    x, dout, dbank = _inputs(seed, B, T, H, widths, dk, d)
    g32, P32 = _float32_backward(x, dout, dbank, widths, W, R, mutate=mutate)
    probe = _bounds(x, dout, dbank, widths, W, R, eps_row=0.0)
    eps_row = max(_row_dev(P32, probe["snapshot"]), 2.0 ** -24)
    res = _bounds(x, dout, dbank, widths, W, R, eps_row=2 * eps_row)
    err = np.abs(g32[grad].astype(np.float64) - res[GRADS[grad]])
    assert np.any(err > res["e_" + grad] * 1.01), f"{mutate} not seen in d {grad}"


def test_bounds_zero_without_rounding_and_gradients_unchanged():
    seed, B, T, H, widths, dk, d, W, R = CASES[1]
    x, dout, dbank = _inputs(seed, B, T, H, widths, dk, d)
    res = _bounds(x, dout, dbank, widths, W, R, eps_row=0.0, u=0.0, eps_w=0.0)
    for k in GRADS:
        assert not np.any(res["e_" + k]), k
    ref = oracle.write_read_backward(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"],
                                     x["bank"], dout, dbank, widths, W, R, want_forward=True, nthreads=1)
    for k in list(GRADS.values()) + ["out", "bank"]:
        assert np.array_equal(res[k], ref[k]), k
