"""Thin ctypes binding of libsdm.so (include/sdm.h): argument marshalling only.

Every step of the write/read, the top-k and the decode step runs in the library's HIP kernels. Torch supplies
device memory (outputs and the workspace) and the current stream. If the library is missing the binding raises; it
never falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdm.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "sdm.h")

SDM_OK, SDM_ERR_DTYPE, SDM_ERR_RANGE, SDM_ERR_BANK_TOO_SMALL, SDM_ERR_ALIAS = 0, 1, 2, 3, 4
SDM_ERR_LAYOUT, SDM_ERR_WORKSPACE, SDM_ERR_DEVICE, SDM_ERR_HIP, SDM_ERR_NULL = 5, 6, 7, 8, 9
STATUS_NAMES = {0: "SDM_OK", 1: "SDM_ERR_DTYPE", 2: "SDM_ERR_RANGE", 3: "SDM_ERR_BANK_TOO_SMALL", 4: "SDM_ERR_ALIAS",
                5: "SDM_ERR_LAYOUT", 6: "SDM_ERR_WORKSPACE", 7: "SDM_ERR_DEVICE", 8: "SDM_ERR_HIP", 9: "SDM_ERR_NULL"}
SDM_F32, SDM_BF16, SDM_F16, SDM_FP8, SDM_INT4 = 0, 1, 2, 3, 4
SDM_OP_TOPK, SDM_OP_WRITE_READ, SDM_OP_DECODE, SDM_OP_BACKWARD, SDM_OP_DECODE_STEPS = 0, 1, 2, 3, 4
SCORING = {"auto": 0, "direct": 1, "filtered": 2}


class UnsupportedConfigurationError(ValueError):
    """Raised when the library refuses a call before doing any work."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class SdmConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("tokens", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("num_factors", ctypes.c_int32), ("factor_widths", ctypes.c_int32 * 4), ("subkey_dim", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("num_writes", ctypes.c_int32), ("num_reads", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("bank_dtype", ctypes.c_int32),
        ("bank_rows", ctypes.c_int64), ("bank_row_stride", ctypes.c_int64),
        ("shared_bank", ctypes.c_int32), ("snapshot_dtype", ctypes.c_int32), ("topk_scoring", ctypes.c_int32),
        ("grad_bank_dtype", ctypes.c_int32),
    ]


class SdmLayerConfig(ctypes.Structure):
    _fields_ = [("op", SdmConfig), ("model_dim", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def make_config(batch, tokens, heads, widths, subkey_dim, head_dim=1, num_writes=1, num_reads=1, chunk_size=1,
                act_dtype=SDM_F32, bank_dtype=SDM_F32, bank_rows=None, bank_row_stride=0,
                shared_bank=False, snapshot_dtype=0, topk_scoring=0, grad_bank_dtype=0) -> SdmConfig:
    c = SdmConfig()
    c.batch, c.tokens, c.heads = int(batch), int(tokens), int(heads)
    c.num_factors = len(widths)
    for i in range(4):
        c.factor_widths[i] = int(widths[i]) if i < len(widths) else 0
    c.subkey_dim, c.head_dim = int(subkey_dim), int(head_dim)
    c.num_writes, c.num_reads, c.chunk_size = int(num_writes), int(num_reads), int(chunk_size)
    c.act_dtype, c.bank_dtype = int(act_dtype), int(bank_dtype)
    n = 1
    for w in widths:
        n *= int(w)
    c.bank_rows = int(bank_rows) if bank_rows is not None else n
    c.bank_row_stride = int(bank_row_stride)
    c.shared_bank = 1 if shared_bank else 0
    c.snapshot_dtype = int(snapshot_dtype)
    c.topk_scoring = SCORING[topk_scoring] if isinstance(topk_scoring, str) else int(topk_scoring)
    c.grad_bank_dtype = int(grad_bank_dtype)
    return c


_SNAP = {"none": 0, "bf16": SDM_BF16, "fp8": SDM_FP8, "int4": SDM_INT4}


def _snapshot_dtype(snapshot_quant: str, bank: torch.Tensor):
    """(config code, torch dtype) of the backward snapshot: "none" = the bank dtype, "bf16" = bfloat16."""
    if snapshot_quant not in _SNAP:
        raise ValueError(f"snapshot_quant must be one of {sorted(_SNAP)}, not {snapshot_quant!r}")
    if snapshot_quant in ("fp8", "int4"):
        return _SNAP[snapshot_quant], torch.uint8  # bytes: elements, then scales (include/sdm.h)
    return _SNAP[snapshot_quant], (torch.bfloat16 if snapshot_quant == "bf16" else bank.dtype)


def _snapshot_shape(cfg, scode, B, H, T, W, d):
    """Shape of the snapshot tensor: [B, H, T, W, d] rows, or the byte count of a quantized snapshot."""
    if scode in (SDM_FP8, SDM_INT4):
        n = ctypes.c_size_t(0)
        _check(load().sdm_snapshot_bytes(ctypes.byref(cfg), ctypes.byref(n)))
        return (n.value,)
    return (B, H, T, W, d)


def bank_pitch(head_dim: int, dtype: torch.dtype) -> int:
    """Row pitch (elements) for a bank on MI355X: rows whose byte size is a multiple of 512 get 128 bytes of padding,
    so that gathering rows in column slices spreads over the HBM channels instead of hitting one channel group."""
    es = torch.empty(0, dtype=dtype).element_size()
    return head_dim + (128 // es if (head_dim * es) % 512 == 0 else 0)


def alloc_bank(batch, heads, rows, head_dim, dtype, device, pitch=None) -> torch.Tensor:
    """Uninitialised bank [batch, heads, rows, head_dim] whose rows are `pitch` elements apart (a view)."""
    ld = bank_pitch(head_dim, dtype) if pitch is None else int(pitch)
    buf = torch.empty((batch, heads, rows, ld), dtype=dtype, device=device)
    return buf[..., :head_dim]


def _bank_ld(bank: torch.Tensor, name: str) -> int:
    """Row stride of a bank tensor [B, H, rows, d] whose rows may be padded (unit column stride)."""
    if not bank.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    B, H, rows, d = bank.shape
    ld = bank.stride(2) if rows > 1 else max(d, bank.stride(2))
    if bank.stride(3) != 1 or ld < d or (H > 1 and bank.stride(1) != rows * ld) or \
            (B > 1 and bank.stride(0) != H * rows * ld):
        raise ValueError(f"{name} must be [B, H, rows, d] with unit column stride and a uniform row pitch "
                         f"(strides {tuple(bank.stride())})")
    return ld


_lib = None
_lock = threading.Lock()
_vp = ctypes.c_void_p


def load():
    """Load libsdm.so (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() (no fallback exists)")
            lib = ctypes.CDLL(LIB_PATH)
            cfgp = ctypes.POINTER(SdmConfig)
            lib.sdm_last_error.restype = ctypes.c_char_p
            lib.sdm_last_error.argtypes = []
            lib.sdm_workspace_size.restype = ctypes.c_int
            lib.sdm_workspace_size.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
            lib.topk_product_keys.restype = ctypes.c_int
            lib.topk_product_keys.argtypes = [cfgp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, ctypes.c_size_t, _vp]
            lib.sdm_write_read.restype = ctypes.c_int
            lib.sdm_write_read.argtypes = [cfgp] + [_vp] * 11 + [ctypes.c_size_t, _vp]
            lib.sdm_write_read_save.restype = ctypes.c_int
            lib.sdm_write_read_save.argtypes = [cfgp] + [_vp] * 12 + [ctypes.c_size_t, _vp]
            lib.sdm_write_read_backward.restype = ctypes.c_int
            lib.sdm_write_read_backward.argtypes = [cfgp] + [_vp] * 17 + [ctypes.c_size_t, _vp]
            lib.sdm_decode_step.restype = ctypes.c_int
            lib.sdm_decode_step.argtypes = [cfgp] + [_vp] * 12 + [ctypes.c_size_t, _vp]
            lib.sdm_decode_steps.restype = ctypes.c_int
            lib.sdm_decode_steps.argtypes = [cfgp] + [_vp] * 12 + [ctypes.c_size_t, _vp]
            lib.sdm_decode_step_noalloc.restype = ctypes.c_int
            lib.sdm_decode_step_noalloc.argtypes = [cfgp] + [_vp] * 12
            lib.sdm_shared_bank_check.restype = ctypes.c_int
            lib.sdm_shared_bank_check.argtypes = [cfgp, _vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32), _vp]
            lib.sdm_profile_enable.restype = ctypes.c_int
            lcfgp = ctypes.POINTER(SdmLayerConfig)
            lib.sdm_layer_workspace_size.argtypes = [lcfgp, ctypes.POINTER(ctypes.c_size_t)]
            lib.sdm_layer_workspace_size.restype = ctypes.c_int
            lib.sdm_layer_forward.argtypes = [lcfgp] + [_vp] * 12 + [ctypes.c_size_t, _vp]
            lib.sdm_snapshot_bytes.restype = ctypes.c_int
            lib.sdm_snapshot_bytes.argtypes = [cfgp, ctypes.POINTER(ctypes.c_size_t)]
            lib.sdm_bank_grad_sum.restype = ctypes.c_int
            lib.sdm_bank_grad_sum.argtypes = [cfgp, _vp, _vp, _vp]
            lib.sdm_layer_forward.restype = ctypes.c_int
            lib.sdm_layer_forward_save.argtypes = [lcfgp] + [_vp] * 13 + [ctypes.c_size_t, _vp]
            lib.sdm_layer_forward_save.restype = ctypes.c_int
            lib.sdm_layer_backward_workspace_size.argtypes = [lcfgp, ctypes.POINTER(ctypes.c_size_t)]
            lib.sdm_layer_backward_workspace_size.restype = ctypes.c_int
            lib.sdm_layer_backward.argtypes = [lcfgp] + [_vp] * 17 + [ctypes.c_size_t, _vp]
            lib.sdm_layer_backward.restype = ctypes.c_int
            lib.sdm_profile_enable.argtypes = [ctypes.c_int32]
            lib.sdm_profile_read.restype = ctypes.c_int
            lib.sdm_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
            _lib = lib
    return _lib


def declared_functions() -> list:
    """Names of the functions include/sdm.h declares."""
    src = open(HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", src, flags=re.M)


def last_error() -> str:
    return load().sdm_last_error().decode()


def _check(status: int):
    if status != SDM_OK:
        msg = last_error()
        raise UnsupportedConfigurationError(status, msg)


def workspace_size(cfg: SdmConfig, op: int, k: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(load().sdm_workspace_size(ctypes.byref(cfg), op, k, ctypes.byref(n)))
    return n.value


KERNELS = ("cand", "topk", "plan", "loop", "decode", "copy", "bwd", "dense")


def profile_enable(on: bool = True):
    """Start (and reset) or stop HIP-event timing of the library's kernel launches."""
    _check(load().sdm_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{kernel: (total ms, launches)} since timing was enabled (waits for the recorded events)."""
    ms = (ctypes.c_double * len(KERNELS))()
    n = (ctypes.c_int64 * len(KERNELS))()
    _check(load().sdm_profile_read(ms, n))
    return {k: (ms[i], n[i]) for i, k in enumerate(KERNELS)}


_DT = {torch.float32: SDM_F32, torch.bfloat16: SDM_BF16, torch.float16: SDM_F16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise UnsupportedConfigurationError(SDM_ERR_DTYPE, f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, shape=None, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _workspace(nbytes: int, device, workspace=None):
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: {nbytes} bytes needed")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def topk_product_keys(queries: torch.Tensor, subkeys: torch.Tensor, widths, k: int, want_scores=True,
                      workspace=None, scoring="auto"):
    """queries [B, T, H, F*dk], subkeys [H, sum n_f, dk] (same dtype) -> (ids int32 [B,T,H,k], scores f32 or None).
    scoring: "auto", "direct" or "filtered" (the factor-scoring kernel; the results are the same)."""
    B, T, H, Fdk = queries.shape
    F = len(widths)
    dk = Fdk // F
    _need(queries, "queries")
    _need(subkeys, "subkeys", (H, sum(widths), dk), queries.dtype)
    cfg = make_config(B, T, H, widths, dk, act_dtype=_dt(queries), topk_scoring=scoring)
    ws = _workspace(workspace_size(cfg, SDM_OP_TOPK, k), queries.device, workspace)
    ids = torch.empty((B, T, H, k), dtype=torch.int32, device=queries.device)
    scores = torch.empty((B, T, H, k), dtype=torch.float32, device=queries.device) if want_scores else None
    _check(load().topk_product_keys(ctypes.byref(cfg), _ptr(queries), _ptr(subkeys), k, _ptr(ids), _ptr(scores),
                                    _ptr(ws), 0 if ws is None else ws.numel(), _stream(queries.device)))
    return ids, scores


class SlotConflictError(ValueError):
    """A shared-bank write/read whose streams address a common slot (the call wrote neither the bank nor out)."""


def sdm_write_read(write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank, *, widths, num_writes,
                   num_reads, chunk_size, want_index=False, out=None, workspace=None, shared_bank=False):
    """Chunked SDM write/read. bank [B, H, bank_rows, d] advances in place. Returns (out, write_idx, read_idx).

    shared_bank=True: bank is [H, bank_rows, d], shared by the B streams of each head, whose slots must be disjoint;
    the library checks this on the device and this function waits for the check (it synchronises the stream) and
    raises SlotConflictError if it failed."""
    B, T, H, Fdk = write_keys.shape
    F = len(widths)
    dk = Fdk // F
    d = values.shape[-1]
    act = write_keys.dtype
    for name, t, shp in (("write_keys", write_keys, (B, T, H, Fdk)), ("read_queries", read_queries, (B, T, H, Fdk)),
                         ("values", values, (B, T, H, d)), ("forget_gate", forget_gate, (B, T, H)),
                         ("input_gate", input_gate, (B, T, H)), ("subkeys", subkeys, (H, sum(widths), dk))):
        _need(t, name, shp, act)
    if shared_bank:
        if bank.dim() != 3 or bank.shape[0] != H or bank.shape[2] != d:
            raise ValueError(f"shared bank has shape {tuple(bank.shape)}, expected ({H}, bank_rows, {d})")
        ld = _bank_ld(bank.unsqueeze(0), "bank")
        rows = bank.shape[1]
    else:
        if bank.dim() != 4 or bank.shape[0] != B or bank.shape[1] != H or bank.shape[3] != d:
            raise ValueError(f"bank has shape {tuple(bank.shape)}, expected ({B}, {H}, bank_rows, {d})")
        ld = _bank_ld(bank, "bank")
        rows = bank.shape[2]
    cfg = make_config(B, T, H, widths, dk, d, num_writes, num_reads, chunk_size, _dt(write_keys), _dt(bank),
                      rows, ld, shared_bank)
    ws = _workspace(workspace_size(cfg, SDM_OP_WRITE_READ), bank.device, workspace)
    if out is None:
        out = torch.empty((B, T, H, d), dtype=act, device=bank.device)
    else:
        _need(out, "out", (B, T, H, d), act)
    widx = torch.empty((B, T, H, num_writes), dtype=torch.int32, device=bank.device) if want_index else None
    ridx = torch.empty((B, T, H, num_reads), dtype=torch.int32, device=bank.device) if want_index else None
    _check(load().sdm_write_read(ctypes.byref(cfg), _ptr(write_keys), _ptr(read_queries), _ptr(values),
                                 _ptr(forget_gate), _ptr(input_gate), _ptr(subkeys), _ptr(bank), _ptr(out),
                                 _ptr(widx), _ptr(ridx), _ptr(ws), 0 if ws is None else ws.numel(),
                                 _stream(bank.device)))
    if shared_bank:
        conflict = ctypes.c_int32(0)
        _check(load().sdm_shared_bank_check(ctypes.byref(cfg), _ptr(ws), 0 if ws is None else ws.numel(),
                                            ctypes.byref(conflict), _stream(bank.device)))
        if conflict.value:
            raise SlotConflictError("shared_bank=True but the streams of a head address a common slot "
                                    "(the bank and out were not written)")
    return out, widx, ridx


def layer_in_features(heads, widths, subkey_dim, head_dim) -> int:
    """Rows of the layer's input map: write keys and read queries (H F dk each), values (H d), two gate inputs (2 H)."""
    return 2 * heads * len(widths) * subkey_dim + heads * head_dim + 2 * heads


def sdm_layer_forward(x, w_in, a_log, dt_bias, w_out, subkeys, bank, *, heads, widths, num_writes, num_reads,
                      chunk_size, want_index=False, y=None, workspace=None, return_workspace=False,
                      initial_bank=None):
    """The layer's forward: projections of x [B, T, Dm] (bf16) by w_in, gates, the write/read op on bank
    [B, H, bank_rows, d] (advances in place), output projection by w_out [Dm, H d]. Returns (y, write_idx,
    read_idx), plus the workspace (uint8) with return_workspace (its first regions: layer_workspace_views)."""
    B, T, Dm = x.shape
    H = int(heads)
    dk = subkeys.shape[-1]
    d = bank.shape[-1]
    _need(x, "x", None, torch.bfloat16)
    _need(w_in, "w_in", (layer_in_features(H, widths, dk, d), Dm), torch.bfloat16)
    _need(a_log, "a_log", (H,), torch.float32)
    _need(dt_bias, "dt_bias", (H,), torch.float32)
    _need(w_out, "w_out", (Dm, H * d), torch.bfloat16)
    _need(subkeys, "subkeys", (H, sum(widths), dk), torch.bfloat16)
    if bank.dim() != 4 or bank.shape[0] != B or bank.shape[1] != H:
        raise ValueError(f"bank has shape {tuple(bank.shape)}, expected ({B}, {H}, bank_rows, d)")
    ld = _bank_ld(bank, "bank")
    if initial_bank is not None:
        if tuple(initial_bank.shape) != (H,) + tuple(bank.shape[2:]) or initial_bank.dtype != bank.dtype or \
                _bank_ld(initial_bank.unsqueeze(0), "initial_bank") != ld:
            raise ValueError("initial_bank must be [heads, bank_rows, d] with the bank's dtype and row stride")
    lc = SdmLayerConfig()
    lc.op = make_config(B, T, H, widths, dk, d, num_writes, num_reads, chunk_size, SDM_BF16, _dt(bank),
                        bank.shape[2], ld)
    lc.model_dim = int(Dm)
    n = ctypes.c_size_t(0)
    _check(load().sdm_layer_workspace_size(ctypes.byref(lc), ctypes.byref(n)))
    ws = _workspace(n.value, x.device, workspace)
    if y is None:
        y = torch.empty((B, T, Dm), dtype=torch.bfloat16, device=x.device)
    else:
        _need(y, "y", (B, T, Dm), torch.bfloat16)
    widx = torch.empty((B, T, H, num_writes), dtype=torch.int32, device=x.device) if want_index else None
    ridx = torch.empty((B, T, H, num_reads), dtype=torch.int32, device=x.device) if want_index else None
    _check(load().sdm_layer_forward(ctypes.byref(lc), _ptr(x), _ptr(w_in), _ptr(a_log), _ptr(dt_bias), _ptr(w_out),
                                    _ptr(subkeys), _ptr(initial_bank), _ptr(bank), _ptr(y), _ptr(widx), _ptr(ridx), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(x.device)))
    return (y, widx, ridx, ws) if return_workspace else (y, widx, ridx)


def _layer_config(x, bank, heads, widths, dk, num_writes, num_reads, chunk_size, snapshot_dtype=0,
                  grad_bank_dtype=0):
    B, T, Dm = x.shape
    ld = _bank_ld(bank, "bank")
    lc = SdmLayerConfig()
    lc.op = make_config(B, T, int(heads), widths, dk, bank.shape[-1], num_writes, num_reads, chunk_size, SDM_BF16,
                        _dt(bank), bank.shape[2], ld, snapshot_dtype=snapshot_dtype, grad_bank_dtype=grad_bank_dtype)
    lc.model_dim = int(Dm)
    return lc


def _check_layer_args(x, w_in, a_log, dt_bias, w_out, subkeys, bank, heads, widths):
    B, T, Dm = x.shape
    H = int(heads)
    dk = subkeys.shape[-1]
    d = bank.shape[-1]
    _need(x, "x", None, torch.bfloat16)
    _need(w_in, "w_in", (layer_in_features(H, widths, dk, d), Dm), torch.bfloat16)
    _need(a_log, "a_log", (H,), torch.float32)
    _need(dt_bias, "dt_bias", (H,), torch.float32)
    _need(w_out, "w_out", (Dm, H * d), torch.bfloat16)
    _need(subkeys, "subkeys", (H, sum(widths), dk), torch.bfloat16)
    if bank.dim() != 4 or bank.shape[0] != B or bank.shape[1] != H:
        raise ValueError(f"bank has shape {tuple(bank.shape)}, expected ({B}, {H}, bank_rows, d)")
    return B, T, Dm, H, dk, d


def layer_backward_workspace_size(lc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().sdm_layer_backward_workspace_size(ctypes.byref(lc), ctypes.byref(n)))
    return n.value


def sdm_layer_forward_save(x, w_in, a_log, dt_bias, w_out, subkeys, bank, *, heads, widths, num_writes, num_reads,
                           chunk_size, initial_bank=None, snapshot_quant="none", want_index=False, y=None,
                           snapshot=None, workspace=None):
    """The layer's training forward: sdm_layer_forward with the op saving its backward snapshot. Returns (y, snapshot,
    workspace, write_idx, read_idx); pass the snapshot and the workspace (uint8, layer_backward_workspace_size
    bytes; do not reuse it in between) to sdm_layer_backward."""
    B, T, Dm, H, dk, d = _check_layer_args(x, w_in, a_log, dt_bias, w_out, subkeys, bank, heads, widths)
    scode, sdt = _snapshot_dtype(snapshot_quant, bank)
    lc = _layer_config(x, bank, H, widths, dk, num_writes, num_reads, chunk_size, snapshot_dtype=scode)
    if initial_bank is not None:
        if tuple(initial_bank.shape) != (H,) + tuple(bank.shape[2:]) or initial_bank.dtype != bank.dtype or \
                _bank_ld(initial_bank.unsqueeze(0), "initial_bank") != lc.op.bank_row_stride:
            raise ValueError("initial_bank must be [heads, bank_rows, d] with the bank's dtype and row stride")
    ws = _workspace(layer_backward_workspace_size(lc), x.device, workspace)
    shp = _snapshot_shape(lc.op, scode, B, H, T, num_writes, d)
    if snapshot is None:
        snapshot = torch.empty(shp, dtype=sdt, device=x.device)
    _need(snapshot, "snapshot", shp, sdt)
    if y is None:
        y = torch.empty((B, T, Dm), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", (B, T, Dm), torch.bfloat16)
    widx = torch.empty((B, T, H, num_writes), dtype=torch.int32, device=x.device) if want_index else None
    ridx = torch.empty((B, T, H, num_reads), dtype=torch.int32, device=x.device) if want_index else None
    _check(load().sdm_layer_forward_save(ctypes.byref(lc), _ptr(x), _ptr(w_in), _ptr(a_log), _ptr(dt_bias),
                                         _ptr(w_out), _ptr(subkeys), _ptr(initial_bank), _ptr(bank), _ptr(y),
                                         _ptr(snapshot), _ptr(widx), _ptr(ridx), _ptr(ws), ws.numel(),
                                         _stream(x.device)))
    return y, snapshot, ws, widx, ridx


def sdm_layer_backward(x, w_in, a_log, dt_bias, w_out, subkeys, bank, snapshot, grad_y, workspace, grad_bank=None, *,
                       heads, widths, num_writes, num_reads, chunk_size, snapshot_quant="none",
                       grad_bank_dtype=torch.float32):
    """Backward of the layer (after sdm_layer_forward_save with the same arguments; bank as it left it, stepped back
    here). grad_y [B, T, Dm] bfloat16; grad_bank (the bank's shape and strides, float32 or bfloat16 on a bfloat16
    bank) the gradient w.r.t. the bank after the forward (None: zeros), replaced by the one w.r.t. the bank the op
    started from. Returns float32 gradients x, w_in, a_log, dt_bias, w_out, subkeys, and bank (grad_bank)."""
    B, T, Dm, H, dk, d = _check_layer_args(x, w_in, a_log, dt_bias, w_out, subkeys, bank, heads, widths)
    _need(grad_y, "grad_y", (B, T, Dm), torch.bfloat16)
    scode, sdt = _snapshot_dtype(snapshot_quant, bank)
    dev = x.device
    ld = _bank_ld(bank, "bank")
    if grad_bank is None:
        grad_bank = torch.zeros((B, H, bank.shape[2], ld), dtype=grad_bank_dtype, device=dev)[..., :d]
    if grad_bank.dtype not in (torch.float32, torch.bfloat16) or tuple(grad_bank.shape) != tuple(bank.shape) or \
            grad_bank.stride() != bank.stride():
        raise ValueError("grad_bank must be float32 or bfloat16 with the bank's shape and strides")
    lc = _layer_config(x, bank, H, widths, dk, num_writes, num_reads, chunk_size, snapshot_dtype=scode,
                       grad_bank_dtype=_dt(grad_bank))
    _need(snapshot, "snapshot", _snapshot_shape(lc.op, scode, B, H, T, num_writes, d), sdt)
    f32 = torch.float32
    g = {"x": torch.empty((B, T, Dm), dtype=f32, device=dev), "w_in": torch.empty(tuple(w_in.shape), dtype=f32,
                                                                                 device=dev),
         "a_log": torch.empty((H,), dtype=f32, device=dev), "dt_bias": torch.empty((H,), dtype=f32, device=dev),
         "w_out": torch.empty((Dm, H * d), dtype=f32, device=dev),
         "subkeys": torch.empty(tuple(subkeys.shape), dtype=f32, device=dev), "bank": grad_bank}
    _check(load().sdm_layer_backward(ctypes.byref(lc), _ptr(x), _ptr(w_in), _ptr(a_log), _ptr(dt_bias), _ptr(w_out),
                                     _ptr(subkeys), _ptr(bank), _ptr(snapshot), _ptr(grad_y), _ptr(grad_bank),
                                     _ptr(g["x"]), _ptr(g["w_in"]), _ptr(g["a_log"]), _ptr(g["dt_bias"]),
                                     _ptr(g["w_out"]), _ptr(g["subkeys"]), _ptr(workspace), workspace.numel(),
                                     _stream(dev)))
    return g


def layer_backward_workspace_views(x_shape, heads, widths, subkey_dim, head_dim, lc, ws):
    """Views of what sdm_layer_backward leaves in its workspace after the forward's regions (include/sdm.h): d o
    [B, T, H, d] bf16, the op's float32 gradients d keys, d queries [B, T, H, F dk], d values [B, T, H, d], d alpha,
    d beta [B, T, H], and d p [B, T, Np] bf16 (Np: the input map's width rounded up to 64)."""
    B, T, _ = x_shape
    H, P, d = int(heads), len(widths) * int(subkey_dim), int(head_dim)
    al = lambda n: (n + 255) // 256 * 256
    off = 0
    for n in (B * T * H * P * 2, B * T * H * P * 2, B * T * H * d * 2, B * T * 2 * H * 2, B * T * H * 2,
              B * T * H * 2, B * T * H * d * 2):
        off = al(off + n)
    opsize = max(workspace_size(lc.op, SDM_OP_WRITE_READ), workspace_size(lc.op, SDM_OP_BACKWARD))
    off = al(off + opsize)
    nin = 2 * H * P + H * d + 2 * H
    Np = (nin + 63) // 64 * 64
    out = {}
    for name, shp, dt, es in (("d_o", (B, T, H, d), torch.bfloat16, 2), ("d_keys", (B, T, H, P), torch.float32, 4),
                              ("d_queries", (B, T, H, P), torch.float32, 4), ("d_values", (B, T, H, d), torch.float32, 4),
                              ("d_alpha", (B, T, H), torch.float32, 4), ("d_beta", (B, T, H), torch.float32, 4),
                              ("d_p", (B, T, Np), torch.bfloat16, 2)):
        n = 1
        for v in shp:
            n *= v
        out[name] = ws[off:off + es * n].view(dt).view(shp)
        off = al(off + es * n)
    return out


def layer_workspace_views(x_shape, heads, widths, subkey_dim, head_dim, ws):
    """Views of the projections and gates the last sdm_layer_forward left in its workspace `ws` (bf16 tensors):
    write keys, read queries [B, T, H, F dk], values [B, T, H, d], gate inputs [B, T, 2 H], alpha, beta [B, T, H],
    o [B, T, H, d] (the layout of the layer's workspace, in order, each region 256-byte aligned)."""
    B, T, _ = x_shape
    H, P, d = int(heads), len(widths) * int(subkey_dim), int(head_dim)
    shapes = [("keys", (B, T, H, P)), ("queries", (B, T, H, P)), ("values", (B, T, H, d)), ("gin", (B, T, 2 * H)),
              ("alpha", (B, T, H)), ("beta", (B, T, H)), ("o", (B, T, H, d))]
    out, off = {}, 0
    for name, shp in shapes:
        n = 1
        for v in shp:
            n *= v
        out[name] = ws[off:off + 2 * n].view(torch.bfloat16).view(shp)
        off = (off + 2 * n + 255) // 256 * 256
    return out


def sdm_write_read_save(write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank, *, widths,
                        num_writes, num_reads, chunk_size, want_index=False, out=None, snapshot=None, workspace=None,
                        snapshot_quant="none"):
    """sdm_write_read that also saves the backward's snapshot [B, H, T, W, d] (bank dtype, or bfloat16 with
    snapshot_quant="bf16"): the row of every write event before it. Returns (out, write_idx, read_idx, snapshot)."""
    B, T, H, Fdk = write_keys.shape
    F = len(widths)
    dk = Fdk // F
    d = values.shape[-1]
    act = write_keys.dtype
    for name, t, shp in (("write_keys", write_keys, (B, T, H, Fdk)), ("read_queries", read_queries, (B, T, H, Fdk)),
                         ("values", values, (B, T, H, d)), ("forget_gate", forget_gate, (B, T, H)),
                         ("input_gate", input_gate, (B, T, H)), ("subkeys", subkeys, (H, sum(widths), dk))):
        _need(t, name, shp, act)
    if bank.dim() != 4 or bank.shape[0] != B or bank.shape[1] != H or bank.shape[3] != d:
        raise ValueError(f"bank has shape {tuple(bank.shape)}, expected ({B}, {H}, bank_rows, {d})")
    ld = _bank_ld(bank, "bank")
    scode, sdt = _snapshot_dtype(snapshot_quant, bank)
    cfg = make_config(B, T, H, widths, dk, d, num_writes, num_reads, chunk_size, _dt(write_keys), _dt(bank),
                      bank.shape[2], ld, snapshot_dtype=scode)
    ws = _workspace(workspace_size(cfg, SDM_OP_WRITE_READ), bank.device, workspace)
    if out is None:
        out = torch.empty((B, T, H, d), dtype=act, device=bank.device)
    else:
        _need(out, "out", (B, T, H, d), act)
    sshape = _snapshot_shape(cfg, scode, B, H, T, num_writes, d)
    if snapshot is None:
        snapshot = torch.empty(sshape, dtype=sdt, device=bank.device)
    else:
        _need(snapshot, "snapshot", sshape, sdt)
    widx = torch.empty((B, T, H, num_writes), dtype=torch.int32, device=bank.device) if want_index else None
    ridx = torch.empty((B, T, H, num_reads), dtype=torch.int32, device=bank.device) if want_index else None
    _check(load().sdm_write_read_save(ctypes.byref(cfg), _ptr(write_keys), _ptr(read_queries), _ptr(values),
                                      _ptr(forget_gate), _ptr(input_gate), _ptr(subkeys), _ptr(bank), _ptr(out),
                                      _ptr(snapshot), _ptr(widx), _ptr(ridx), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(bank.device)))
    return out, widx, ridx, snapshot


def sdm_write_read_backward(write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank, snapshot,
                            grad_out, grad_bank=None, *, widths, num_writes, num_reads, chunk_size, workspace=None,
                            snapshot_quant="none", grad_bank_dtype=torch.float32):
    """Backward of sdm_write_read_save (the same snapshot_quant). bank (as the forward left it) steps back to its
    state before the forward (with a bfloat16 snapshot of a float32 bank, written rows come back rounded).
    grad_bank: float32, or bfloat16 on a bfloat16 bank (every update rounded), with the bank's shape and row stride,
    the gradient w.r.t. the bank after the forward (None: zeros of grad_bank_dtype), replaced in place by the
    gradient w.r.t. the bank before it. Returns a dict of gradients: write_keys, read_queries, values, forget_gate,
    input_gate, subkeys (float32) and bank (grad_bank)."""
    B, T, H, Fdk = write_keys.shape
    F = len(widths)
    dk = Fdk // F
    d = values.shape[-1]
    act = write_keys.dtype
    for name, t, shp in (("write_keys", write_keys, (B, T, H, Fdk)), ("read_queries", read_queries, (B, T, H, Fdk)),
                         ("values", values, (B, T, H, d)), ("forget_gate", forget_gate, (B, T, H)),
                         ("input_gate", input_gate, (B, T, H)), ("subkeys", subkeys, (H, sum(widths), dk)),
                         ("grad_out", grad_out, (B, T, H, d))):
        _need(t, name, shp, act)
    if bank.dim() != 4 or bank.shape[0] != B or bank.shape[1] != H or bank.shape[3] != d:
        raise ValueError(f"bank has shape {tuple(bank.shape)}, expected ({B}, {H}, bank_rows, {d})")
    ld = _bank_ld(bank, "bank")
    scode, sdt = _snapshot_dtype(snapshot_quant, bank)
    dev = bank.device
    if grad_bank is None:
        grad_bank = torch.zeros((B, H, bank.shape[2], ld), dtype=grad_bank_dtype, device=dev)[..., :d]
    if grad_bank.dtype not in (torch.float32, torch.bfloat16) or tuple(grad_bank.shape) != tuple(bank.shape) or \
            grad_bank.stride() != bank.stride():
        raise ValueError("grad_bank must be float32 or bfloat16 with the bank's shape and strides")
    cfg = make_config(B, T, H, widths, dk, d, num_writes, num_reads, chunk_size, _dt(write_keys), _dt(bank),
                      bank.shape[2], ld, snapshot_dtype=scode, grad_bank_dtype=_dt(grad_bank))
    _need(snapshot, "snapshot", _snapshot_shape(cfg, scode, B, H, T, num_writes, d), sdt)
    ws = _workspace(workspace_size(cfg, SDM_OP_BACKWARD), dev, workspace)
    f32 = torch.float32
    g = {"write_keys": torch.empty((B, T, H, Fdk), dtype=f32, device=dev),
         "read_queries": torch.empty((B, T, H, Fdk), dtype=f32, device=dev),
         "values": torch.empty((B, T, H, d), dtype=f32, device=dev),
         "forget_gate": torch.empty((B, T, H), dtype=f32, device=dev),
         "input_gate": torch.empty((B, T, H), dtype=f32, device=dev),
         "subkeys": torch.empty((H, sum(widths), dk), dtype=f32, device=dev),
         "bank": grad_bank}
    _check(load().sdm_write_read_backward(
        ctypes.byref(cfg), _ptr(write_keys), _ptr(read_queries), _ptr(values), _ptr(forget_gate), _ptr(input_gate),
        _ptr(subkeys), _ptr(bank), _ptr(snapshot), _ptr(grad_out), _ptr(grad_bank), _ptr(g["write_keys"]),
        _ptr(g["read_queries"]), _ptr(g["values"]), _ptr(g["forget_gate"]), _ptr(g["input_gate"]),
        _ptr(g["subkeys"]), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)))
    return g


def sdm_decode_step(write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank_in, bank_out=None, *,
                    widths, num_writes, num_reads, want_index=False, out=None, workspace=None):
    """One decode step. bank_out None or bank_in: donated (in place); else a disjoint successor buffer.
    Inputs [B, 1, H, ...]. Returns (out, write_idx, read_idx, bank_out)."""
    if bank_out is None:
        bank_out = bank_in
    B, T, H, Fdk = write_keys.shape
    F = len(widths)
    dk = Fdk // F
    d = values.shape[-1]
    act = write_keys.dtype
    for name, t, shp in (("write_keys", write_keys, (B, T, H, Fdk)), ("read_queries", read_queries, (B, T, H, Fdk)),
                         ("values", values, (B, T, H, d)), ("forget_gate", forget_gate, (B, T, H)),
                         ("input_gate", input_gate, (B, T, H)), ("subkeys", subkeys, (H, sum(widths), dk))):
        _need(t, name, shp, act)
    if bank_in.dim() != 4 or bank_in.shape[0] != B or bank_in.shape[1] != H or bank_in.shape[3] != d:
        raise ValueError(f"bank_in has shape {tuple(bank_in.shape)}, expected ({B}, {H}, bank_rows, {d})")
    ld = _bank_ld(bank_in, "bank_in")
    if tuple(bank_out.shape) != tuple(bank_in.shape) or bank_out.dtype != bank_in.dtype or \
            bank_out.stride() != bank_in.stride():
        raise ValueError("bank_out must have bank_in's shape, dtype and strides")
    cfg = make_config(B, T, H, widths, dk, d, num_writes, num_reads, 1, _dt(write_keys), _dt(bank_in),
                      bank_in.shape[2], ld)
    ws = _workspace(workspace_size(cfg, SDM_OP_DECODE), bank_in.device, workspace)
    if out is None:
        out = torch.empty((B, T, H, d), dtype=act, device=bank_in.device)
    widx = torch.empty((B, T, H, num_writes), dtype=torch.int32, device=bank_in.device) if want_index else None
    ridx = torch.empty((B, T, H, num_reads), dtype=torch.int32, device=bank_in.device) if want_index else None
    _check(load().sdm_decode_step(ctypes.byref(cfg), _ptr(write_keys), _ptr(read_queries), _ptr(values),
                                  _ptr(forget_gate), _ptr(input_gate), _ptr(subkeys), _ptr(bank_in), _ptr(bank_out),
                                  _ptr(out), _ptr(widx), _ptr(ridx), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(bank_in.device)))
    return out, widx, ridx, bank_out


def sdm_decode_steps(write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank_in, bank_out=None, *,
                     widths, num_writes, num_reads, want_index=False, out=None, workspace=None):
    """K consecutive decode steps in one call: inputs [B, K, H, ...], token k of each stream is step k's input;
    bank_out None or bank_in: in place (donated), else a disjoint successor buffer that receives bank_in's copy.
    Bitwise equal to K sdm_decode_step calls. Returns (out [B, K, H, d], write_idx, read_idx, bank_out)."""
    if bank_out is None:
        bank_out = bank_in
    B, K, H, Fdk = write_keys.shape
    F = len(widths)
    dk = Fdk // F
    d = values.shape[-1]
    act = write_keys.dtype
    for name, t, shp in (("write_keys", write_keys, (B, K, H, Fdk)), ("read_queries", read_queries, (B, K, H, Fdk)),
                         ("values", values, (B, K, H, d)), ("forget_gate", forget_gate, (B, K, H)),
                         ("input_gate", input_gate, (B, K, H)), ("subkeys", subkeys, (H, sum(widths), dk))):
        _need(t, name, shp, act)
    if bank_in.dim() != 4 or bank_in.shape[0] != B or bank_in.shape[1] != H or bank_in.shape[3] != d:
        raise ValueError(f"bank_in has shape {tuple(bank_in.shape)}, expected ({B}, {H}, bank_rows, {d})")
    ld = _bank_ld(bank_in, "bank_in")
    if tuple(bank_out.shape) != tuple(bank_in.shape) or bank_out.dtype != bank_in.dtype or \
            bank_out.stride() != bank_in.stride():
        raise ValueError("bank_out must have bank_in's shape, dtype and strides")
    cfg = make_config(B, K, H, widths, dk, d, num_writes, num_reads, 1, _dt(write_keys), _dt(bank_in),
                      bank_in.shape[2], ld)
    ws = _workspace(workspace_size(cfg, SDM_OP_DECODE_STEPS), bank_in.device, workspace)
    if out is None:
        out = torch.empty((B, K, H, d), dtype=act, device=bank_in.device)
    else:
        _need(out, "out", (B, K, H, d), act)
    widx = torch.empty((B, K, H, num_writes), dtype=torch.int32, device=bank_in.device) if want_index else None
    ridx = torch.empty((B, K, H, num_reads), dtype=torch.int32, device=bank_in.device) if want_index else None
    _check(load().sdm_decode_steps(ctypes.byref(cfg), _ptr(write_keys), _ptr(read_queries), _ptr(values),
                                   _ptr(forget_gate), _ptr(input_gate), _ptr(subkeys), _ptr(bank_in), _ptr(bank_out),
                                   _ptr(out), _ptr(widx), _ptr(ridx), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(bank_in.device)))
    return out, widx, ridx, bank_out


def sdm_bank_grad_sum(grad_bank, *, heads, widths, head_dim, out=None):
    """Gradient of a learned initial bank copied into every batch row: grad_bank [B, H, bank_rows, d] float32 or
    bfloat16 (rows possibly padded) summed over the batch in order, in float32, into [H, bank_rows, d] float32 (the
    same row stride in elements; rows >= N and the padding are left as `out` had them, zeros when out is None)."""
    B, H, rows, d = grad_bank.shape
    ld = _bank_ld(grad_bank, "grad_bank")
    if grad_bank.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("grad_bank must be float32 or bfloat16")
    if out is None:
        out = torch.zeros((H, rows, ld), dtype=torch.float32, device=grad_bank.device)[..., :d]
    if tuple(out.shape) != (H, rows, d) or _bank_ld(out.unsqueeze(0), "out") != ld:
        raise ValueError("out must be [heads, bank_rows, d] float32 with grad_bank's row stride")
    gdt = _dt(grad_bank)
    cfg = make_config(B, 1, H, widths, 1, d, 1, 1, 1, SDM_F32, gdt, rows, ld, grad_bank_dtype=gdt)
    _check(load().sdm_bank_grad_sum(ctypes.byref(cfg), _ptr(grad_bank), _ptr(out), _stream(grad_bank.device)))
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20  # SDM_NOALLOC_SCRATCH_BYTES in include/sdm.h


def sdm_decode_step_noalloc(write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank_in,
                            bank_out=None, *, widths, num_writes, num_reads, out, write_idx=None, read_idx=None):
    """sdm_decode_step without a workspace (the library's per-GPU scratch array instead): for callers that cannot
    allocate device memory. Every output tensor is the caller's (out [B, 1, H, d]; write_idx / read_idx optional);
    nothing is allocated here. Returns out."""
    if bank_out is None:
        bank_out = bank_in
    B, T, H, Fdk = write_keys.shape
    F = len(widths)
    dk = Fdk // F
    d = values.shape[-1]
    act = write_keys.dtype
    for name, t, shp in (("write_keys", write_keys, (B, T, H, Fdk)), ("read_queries", read_queries, (B, T, H, Fdk)),
                         ("values", values, (B, T, H, d)), ("forget_gate", forget_gate, (B, T, H)),
                         ("input_gate", input_gate, (B, T, H)), ("subkeys", subkeys, (H, sum(widths), dk)),
                         ("out", out, (B, T, H, d))):
        _need(t, name, shp, act)
    for name, t, k in (("write_idx", write_idx, num_writes), ("read_idx", read_idx, num_reads)):
        if t is not None:
            _need(t, name, (B, T, H, k), torch.int32)
    if bank_in.dim() != 4 or bank_in.shape[0] != B or bank_in.shape[1] != H or bank_in.shape[3] != d:
        raise ValueError(f"bank_in has shape {tuple(bank_in.shape)}, expected ({B}, {H}, bank_rows, {d})")
    ld = _bank_ld(bank_in, "bank_in")
    if tuple(bank_out.shape) != tuple(bank_in.shape) or bank_out.dtype != bank_in.dtype or \
            bank_out.stride() != bank_in.stride():
        raise ValueError("bank_out must have bank_in's shape, dtype and strides")
    cfg = make_config(B, T, H, widths, dk, d, num_writes, num_reads, 1, _dt(write_keys), _dt(bank_in),
                      bank_in.shape[2], ld)
    _check(load().sdm_decode_step_noalloc(ctypes.byref(cfg), _ptr(write_keys), _ptr(read_queries), _ptr(values),
                                          _ptr(forget_gate), _ptr(input_gate), _ptr(subkeys), _ptr(bank_in),
                                          _ptr(bank_out), _ptr(out), _ptr(write_idx), _ptr(read_idx),
                                          _stream(bank_in.device)))
    return out


class DecodeStep:
    """A prepared single-token decode step for fixed shapes (serving loops): the config and the workspace are made
    once, and a call only hands the tensors' pointers to sdm_decode_step (which still validates the config, the
    ranges and the aliasing on every call). Tensors must have the shapes, dtypes and bank layout given here
    (contiguous inputs [batch, 1, heads, ...]; bank [batch, heads, bank_rows, head_dim] with row stride
    bank_row_stride). Returns out [batch, 1, heads, head_dim]."""

    def __init__(self, batch, heads, widths, subkey_dim, head_dim, num_writes, num_reads, act_dtype, bank_dtype,
                 bank_rows, device, bank_row_stride=0, workspace=None):
        self._cfg = make_config(batch, 1, heads, widths, subkey_dim, head_dim, num_writes, num_reads, 1,
                                _DT[act_dtype], _DT[bank_dtype], bank_rows, bank_row_stride)
        self._cfgp = ctypes.byref(self._cfg)
        self._ws = _workspace(workspace_size(self._cfg, SDM_OP_DECODE), device, workspace)
        self._wsp = _ptr(self._ws)
        self._wsn = 0 if self._ws is None else self._ws.numel()
        self._fn = load().sdm_decode_step
        self._device = device
        self._out_shape = (batch, 1, heads, head_dim)
        self._act = act_dtype

    def __call__(self, write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank_in, bank_out=None,
                 out=None, write_idx=None, read_idx=None):
        if out is None:
            out = torch.empty(self._out_shape, dtype=self._act, device=self._device)
        _check(self._fn(self._cfgp, write_keys.data_ptr(), read_queries.data_ptr(), values.data_ptr(),
                        forget_gate.data_ptr(), input_gate.data_ptr(), subkeys.data_ptr(), bank_in.data_ptr(),
                        (bank_out if bank_out is not None else bank_in).data_ptr(), out.data_ptr(),
                        _ptr(write_idx), _ptr(read_idx), self._wsp, self._wsn,
                        torch.cuda.current_stream(self._device).cuda_stream))
        return out
