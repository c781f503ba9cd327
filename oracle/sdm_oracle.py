"""ctypes wrapper around the C oracle (``sdm_oracle.c``). Test infrastructure only.

All tensors cross the boundary as contiguous float32 numpy arrays whose values are already rounded to their dtype
(bfloat16 values are exact in float32); the oracle rounds written bank rows and outputs to the requested dtypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sdm_oracle.c")
_LIB = os.path.join(_HERE, "libsdm_oracle.so")
_lock = threading.Lock()
_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE arithmetic: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-pthread",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=False)
            lib = ctypes.CDLL(_LIB)
            lib.oracle_round_bf16.restype = ctypes.c_double
            lib.oracle_round_bf16.argtypes = [ctypes.c_double]
            lib.oracle_factor_scores.restype = None
            lib.oracle_factor_scores.argtypes = [ctypes.c_int, ctypes.c_int, _f32p, _f32p, _f32p]
            lib.oracle_softmax.restype = None
            lib.oracle_softmax.argtypes = [ctypes.c_int, _f32p, _f64p]
            lib.oracle_topk_one.restype = ctypes.c_int
            lib.oracle_topk_one.argtypes = [ctypes.c_int, _i32p, ctypes.c_int, _f32p, _f32p, ctypes.c_int, _i32p,
                                            _f32p]
            lib.oracle_topk.restype = ctypes.c_int
            lib.oracle_topk.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, ctypes.c_int,
                                        _f32p, _f32p, ctypes.c_int, _i32p, _f32p, ctypes.c_int]
            vp = ctypes.c_void_p
            lib.oracle_write_read.restype = ctypes.c_int
            lib.oracle_write_read.argtypes = [
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, ctypes.c_int, ctypes.c_int,
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int64, _f32p,
                vp, vp, vp, vp, ctypes.c_int]
            lib.oracle_write_read_backward.restype = ctypes.c_int
            lib.oracle_write_read_backward.argtypes = [
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, ctypes.c_int, ctypes.c_int,
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int64, _f32p, vp,
                _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, vp, vp, ctypes.c_int]
            lib.oracle_e4m3_round.restype = ctypes.c_double
            lib.oracle_e4m3_round.argtypes = [ctypes.c_double]
            lib.oracle_snap_scale_exp.restype = ctypes.c_int
            lib.oracle_snap_scale_exp.argtypes = [ctypes.c_double, ctypes.c_double]
            lib.oracle_snap_rows.restype = None
            lib.oracle_snap_rows.argtypes = [_f64p, _f64p, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
            lib.oracle_write_read_backward_bounds.restype = ctypes.c_int
            lib.oracle_write_read_backward_bounds.argtypes = [
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, ctypes.c_int, ctypes.c_int,
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int64, _f32p, vp,
                _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, vp, vp, vp, _f64p,
                _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int]
            _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def round_bf16(x: float) -> float:
    """Nearest bfloat16 (ties to even) of an fp64 value."""
    return float(_load().oracle_round_bf16(float(x)))


def factor_scores(q, C) -> np.ndarray:
    """float32 rounding of the fp64 FMA chain <q, C[i]> for every row i of C. q: [dk], C: [n, dk]."""
    q = _f32(q)
    C = _f32(C)
    n, dk = C.shape
    assert q.shape == (dk,)
    s = np.empty(n, dtype=np.float32)
    _load().oracle_factor_scores(n, dk, q, C, s)
    return s


def softmax(scores) -> np.ndarray:
    s = _f32(scores)
    w = np.empty(s.shape[0], dtype=np.float64)
    _load().oracle_softmax(s.shape[0], s, w)
    return w


def topk_one(q, subkeys, widths, k):
    """Exact product-key top-k of one query q [F*dk] against one head's stacked sub-key tables [sum n_f, dk]."""
    widths = np.ascontiguousarray(np.asarray(widths, dtype=np.int32))
    q = _f32(q)
    sub = _f32(subkeys)
    dk = sub.shape[1]
    ids = np.empty(k, dtype=np.int32)
    sc = np.empty(k, dtype=np.float32)
    rc = _load().oracle_topk_one(len(widths), widths, dk, q, sub, k, ids, sc)
    if rc != 0:
        raise ValueError("oracle_topk_one rejected its arguments")
    return ids, sc


def topk(queries, subkeys, widths, k, nthreads: int | None = None):
    """queries [B, T, H, F*dk], subkeys [H, sum n_f, dk] -> ids int32 [B, T, H, k], scores float32 [B, T, H, k]."""
    q = _f32(queries)
    sub = _f32(subkeys)
    B, T, H, _ = q.shape
    widths = np.ascontiguousarray(np.asarray(widths, dtype=np.int32))
    dk = sub.shape[2]
    ids = np.empty((B, T, H, k), dtype=np.int32)
    sc = np.empty((B, T, H, k), dtype=np.float32)
    nt = nthreads or min(os.cpu_count() or 1, 16)
    rc = _load().oracle_topk(B, T, H, len(widths), widths, dk, q, sub, k, ids, sc, nt)
    if rc != 0:
        raise ValueError("oracle_topk rejected its arguments")
    return ids, sc


def write_read(wkeys, rq, values, alpha, beta, subkeys, bank, widths, num_writes, num_reads, *, bank_bf16=False,
               act_bf16=False, nthreads: int | None = None, want_index=True):
    """Sequential per-token SDM write/read over every stream (b, h).

    Arguments (float32 arrays, values already in their dtype): wkeys/rq [B, T, H, F*dk], values [B, T, H, d],
    alpha/beta [B, T, H], subkeys [H, sum n_f, dk], bank [B, H, bank_rows, d] (not modified: a copy advances).
    Returns dict(out [B,T,H,d] float32, bank [B,H,bank_rows,d] float32, widx, ridx, wscore, rscore).
    """
    wk = _f32(wkeys)
    rqa = _f32(rq)
    v = _f32(values)
    al = _f32(alpha)
    be = _f32(beta)
    sub = _f32(subkeys)
    M = np.array(bank, dtype=np.float32, copy=True, order="C")
    B, T, H, Fdk = wk.shape
    d = v.shape[-1]
    widths = np.ascontiguousarray(np.asarray(widths, dtype=np.int32))
    dk = sub.shape[2]
    W, R = int(num_writes), int(num_reads)
    out = np.empty((B, T, H, d), dtype=np.float32)
    res = {"out": out, "bank": M}
    ptrs = []
    for name, k in (("widx", W), ("ridx", R)):
        arr = np.empty((B, T, H, k), dtype=np.int32) if want_index else None
        res[name] = arr
        ptrs.append(arr.ctypes.data if arr is not None else None)
    for name, k in (("wscore", W), ("rscore", R)):
        arr = np.empty((B, T, H, k), dtype=np.float32) if want_index else None
        res[name] = arr
        ptrs.append(arr.ctypes.data if arr is not None else None)
    nt = nthreads or min(os.cpu_count() or 1, 16)
    rc = _load().oracle_write_read(B, T, H, len(widths), widths, dk, d, W, R, int(bool(bank_bf16)),
                                   int(bool(act_bf16)), wk, rqa, v, al, be, sub, M, M.shape[2], out,
                                   ptrs[0], ptrs[1], ptrs[2], ptrs[3], nt)
    if rc != 0:
        raise ValueError("oracle_write_read rejected its arguments")
    return res


SNAP_MODES = {"none": 0, "bf16": 1, "fp8": 2, "int4": 3}


def _snap_mode(snap_bf16, snap_quant):
    if snap_quant is not None:
        return SNAP_MODES[snap_quant]
    return 1 if snap_bf16 else 0


def e4m3_round(v: float) -> float:
    """Nearest OCP FP8 E4M3 value to v (|v| <= 448), ties to even (sdm_oracle.c)."""
    return float(_load().oracle_e4m3_round(float(v)))


def snap_scale_exp(amax: float, qmax: float) -> int:
    """The smallest e with amax / 2^e <= qmax: a quantized snapshot group's scale exponent."""
    return int(_load().oracle_snap_scale_exp(float(amax), float(qmax)))


def snap_rows(rows, snap_quant: str) -> np.ndarray:
    """Rows [..., d] (float32 values) as a snapshot of the mode stores them: "bf16" rounded, "fp8" / "int4" quantized
    in groups of 16 columns with a power-of-two scale and read back (d % 16 == 0). fp64 result."""
    x = np.ascontiguousarray(np.asarray(rows, dtype=np.float64))
    out = np.empty_like(x)
    d = x.shape[-1]
    _load().oracle_snap_rows(x, out, x.size // d if d else 0, d, SNAP_MODES[snap_quant])
    return out


def write_read_backward(wkeys, rq, values, alpha, beta, subkeys, bank, dout, dbank, widths, num_writes, num_reads,
                        *, bank_bf16=False, exact=False, snap_bf16=False, want_forward=False,
                        nthreads: int | None = None, snap_quant=None, grad_bank_bf16=False):
    """Gradients of the write/read (the chain rule through the per-token recurrence, in reverse; sdm_oracle.c).

    bank is the bank before the call [B, H, bank_rows, d]; dout [B, T, H, d] and dbank (same shape as bank, or None
    for zero) are the gradients of the loss with respect to out and to the bank after the call. exact=True keeps
    the bank states in fp64 (no rounding to the bank dtype). Returns fp64 arrays d_wkeys, d_rq, d_values, d_alpha,
    d_beta, d_subkeys, d_bank (with respect to the bank before the call), and with want_forward=True also out and
    bank (the forward in fp64, rounded to the bank dtype after every token unless exact). snap_bf16=True: the
    backward of a bfloat16 snapshot (CHANGELOG 2.0.0, "New"): every pre-write row it reads rounded to bfloat16 (r and
    delta rebuilt from them), and a row read at token t whose slot a later token writes rounded too (the bank is
    restored in place from the snapshot as the sweep goes back).
    """
    wk, rqa, v, al, be, sub = (_f32(x) for x in (wkeys, rq, values, alpha, beta, subkeys))
    M = _f32(bank)
    g_out = _f32(dout)
    g_bank = None if dbank is None else _f32(dbank)
    B, T, H, Fdk = wk.shape
    d = v.shape[-1]
    widths = np.ascontiguousarray(np.asarray(widths, dtype=np.int32))
    dk = sub.shape[2]
    W, R = int(num_writes), int(num_reads)
    res = {"d_wkeys": np.zeros(wk.shape), "d_rq": np.zeros(rqa.shape), "d_values": np.zeros(v.shape),
           "d_alpha": np.zeros(al.shape), "d_beta": np.zeros(be.shape), "d_subkeys": np.zeros(sub.shape),
           "d_bank": np.zeros(M.shape)}
    fwd = [None, None]
    if want_forward:
        res["out"] = np.zeros((B, T, H, d))
        res["bank"] = np.zeros(M.shape)
        fwd = [res["out"].ctypes.data, res["bank"].ctypes.data]
    nt = nthreads or min(os.cpu_count() or 1, 16)
    rc = _load().oracle_write_read_backward(
        B, T, H, len(widths), widths, dk, d, W, R, int(bool(bank_bf16)), int(bool(exact)),
        _snap_mode(snap_bf16, snap_quant), int(bool(grad_bank_bf16)),
        wk, rqa, v, al, be, sub,
        M, M.shape[2], g_out, None if g_bank is None else g_bank.ctypes.data, res["d_wkeys"], res["d_rq"],
        res["d_values"], res["d_alpha"], res["d_beta"], res["d_subkeys"], res["d_bank"], fwd[0], fwd[1], nt)
    if rc != 0:
        raise ValueError("oracle_write_read_backward rejected its arguments")
    return res


U_F32 = 2.0 ** -24  # unit roundoff of float32 (round to nearest)


def write_read_backward_bounds(wkeys, rq, values, alpha, beta, subkeys, bank, dout, dbank, widths, num_writes,
                               num_reads, *, eps_row, eps_w=2 * U_F32, u=U_F32, q_rel=0.0, q_grp=0.0,
                               bank_bf16=False, snap_bf16=False, want_snapshot=False, nthreads: int | None = None,
                               snap_quant=None, grad_bank_bf16=False, g_rel=2.0 ** -7):
    """write_read_backward (rounded bank states, as the forward stores them) plus, for every gradient element, a
    bound on how far another evaluation of the same backward may be from it (sdm_oracle.c, the comment above
    bound_par_t): one that reads pre-write and read rows within eps_row of each row's largest magnitude (plus q_rel
    of an element and q_grp of its 16-column group's largest magnitude for rows read from a rounded or quantized
    snapshot, snap_quant "bf16", "fp8" or "int4"), has softmax weights within eps_w relative, and does every other
    operation with unit roundoff u in any order. Returns the gradients as write_read_backward does, the
    bounds as e_wkeys, e_rq, e_values, e_alpha, e_beta, e_subkeys, e_bank, the forward's out and bank (fp64; the
    bank rounded to its dtype after every token), and with want_snapshot the pre-write rows of every write event
    as the backward reads them, float32 [B, H, T, W, d]."""
    wk, rqa, v, al, be, sub = (_f32(x) for x in (wkeys, rq, values, alpha, beta, subkeys))
    M = _f32(bank)
    g_out = _f32(dout)
    g_bank = None if dbank is None else _f32(dbank)
    B, T, H, Fdk = wk.shape
    d = v.shape[-1]
    widths = np.ascontiguousarray(np.asarray(widths, dtype=np.int32))
    dk = sub.shape[2]
    W, R = int(num_writes), int(num_reads)
    z = np.zeros
    res = {"d_wkeys": z(wk.shape), "d_rq": z(rqa.shape), "d_values": z(v.shape), "d_alpha": z(al.shape),
           "d_beta": z(be.shape), "d_subkeys": z(sub.shape), "d_bank": z(M.shape), "out": z((B, T, H, d)),
           "bank": z(M.shape)}
    for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys", "bank"):
        res["e_" + k] = z(res["d_" + k].shape)
    snap = np.empty((B, H, T, W, d), np.float32) if want_snapshot else None
    par = np.array([u, eps_row, eps_w, q_rel, q_grp, g_rel], np.float64)
    nt = nthreads or min(os.cpu_count() or 1, 16)
    rc = _load().oracle_write_read_backward_bounds(
        B, T, H, len(widths), widths, dk, d, W, R, int(bool(bank_bf16)), _snap_mode(snap_bf16, snap_quant),
        int(bool(grad_bank_bf16)), wk, rqa, v,
        al, be,
        sub, M, M.shape[2], g_out, None if g_bank is None else g_bank.ctypes.data, res["d_wkeys"], res["d_rq"],
        res["d_values"], res["d_alpha"], res["d_beta"], res["d_subkeys"], res["d_bank"], res["out"].ctypes.data,
        res["bank"].ctypes.data, None if snap is None else snap.ctypes.data, par, res["e_wkeys"], res["e_rq"],
        res["e_values"], res["e_alpha"], res["e_beta"], res["e_subkeys"], res["e_bank"], nt)
    if rc != 0:
        raise ValueError("oracle_write_read_backward_bounds rejected its arguments")
    if want_snapshot:
        res["snapshot"] = snap
    return res
