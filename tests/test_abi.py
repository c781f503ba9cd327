"""The C ABI on the host (no GPU): the library loads, exports every function include/sdm.h declares, sizes its
workspace, and refuses bad calls before any device work with the documented status codes."""
import ctypes
import os

import pytest

from gated_delta_rule_product_amd import binding as B


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from gated_delta_rule_product_amd import build

        build.build()
    return B.load()


def test_exports_every_declared_function(lib):
    names = B.declared_functions()
    assert set(names) >= {"sdm_last_error", "sdm_workspace_size", "topk_product_keys", "sdm_write_read",
                          "sdm_decode_step"}
    for n in names:
        assert hasattr(lib, n), n


def test_exports_no_other_c_function():
    """Every unmangled function the library exports is one the header declares (helpers keep internal linkage)."""
    import shutil
    import subprocess
    if not os.path.exists(B.LIB_PATH) or shutil.which("nm") is None:
        pytest.skip("needs the built library and nm")
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True)
    exported = {f[2] for f in (ln.split() for ln in out.stdout.splitlines())
                if len(f) == 3 and f[1] == "T" and not f[2].startswith("_Z")}
    assert exported <= set(B.declared_functions()), sorted(exported - set(B.declared_functions()))


def test_binding_refuses_to_run_without_the_library(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libsdm.so")
    with pytest.raises(RuntimeError):
        B.load()


def _cfg(**kw):
    base = dict(batch=2, tokens=256, heads=2, widths=(32, 32), subkey_dim=16, head_dim=64, num_writes=4,
                num_reads=4, chunk_size=64, act_dtype=B.SDM_F32, bank_dtype=B.SDM_F32)
    base.update(kw)
    return B.make_config(**base)


def _status(cfg, op=B.SDM_OP_WRITE_READ, k=0):
    n = ctypes.c_size_t(0)
    return B.load().sdm_workspace_size(ctypes.byref(cfg), op, k, ctypes.byref(n)), n.value


def test_workspace_sizes(lib):
    s, n = _status(_cfg())
    assert s == B.SDM_OK and n > 0
    s2, n2 = _status(_cfg(tokens=512))
    assert s2 == B.SDM_OK and n2 > n
    s, n = _status(_cfg(), B.SDM_OP_DECODE)
    assert s == B.SDM_ERR_RANGE  # decode needs tokens == 1
    s, n = _status(_cfg(tokens=1), B.SDM_OP_DECODE)
    assert s == B.SDM_OK and n > 0
    s, n = _status(_cfg(), B.SDM_OP_TOPK, 64)
    assert s == B.SDM_OK and n > 0


@pytest.mark.parametrize("kw,status", [
    (dict(act_dtype=B.SDM_F16), B.SDM_ERR_DTYPE),
    (dict(bank_dtype=B.SDM_F16), B.SDM_ERR_DTYPE),
    (dict(act_dtype=7), B.SDM_ERR_DTYPE),
    (dict(widths=(2, 2, 2, 2, 2)[:4], subkey_dim=400), B.SDM_ERR_RANGE),   # F * dk > 1024
    (dict(widths=(0, 32)), B.SDM_ERR_RANGE),
    (dict(widths=(4096, 4096)), B.SDM_ERR_RANGE),                          # N >= 2^31 ... 2^24 fine, see below
    (dict(num_writes=2000), B.SDM_ERR_RANGE),
    (dict(num_writes=0), B.SDM_ERR_RANGE),
    (dict(widths=(2, 2), num_writes=5), B.SDM_ERR_RANGE),                  # more writes than slots
    (dict(num_reads=1025), B.SDM_ERR_RANGE),
    (dict(head_dim=(1 << 20) + 4), B.SDM_ERR_RANGE),
    (dict(head_dim=66), B.SDM_ERR_LAYOUT),
    (dict(head_dim=68, bank_dtype=B.SDM_BF16), B.SDM_ERR_LAYOUT),
    (dict(chunk_size=65537), B.SDM_ERR_RANGE),
    (dict(chunk_size=0), B.SDM_ERR_RANGE),
    (dict(bank_rows=1023), B.SDM_ERR_BANK_TOO_SMALL),
    (dict(bank_row_stride=60), B.SDM_ERR_LAYOUT),                          # pitch below head_dim
    (dict(bank_row_stride=66), B.SDM_ERR_LAYOUT),                          # pitch not a 16-byte multiple
    (dict(tokens=-1), B.SDM_ERR_RANGE),
    (dict(topk_scoring=3), B.SDM_ERR_RANGE),
    (dict(topk_scoring=-1), B.SDM_ERR_RANGE),
])
def test_refusals(lib, kw, status):
    if kw.get("widths") == (4096, 4096):
        # 2^24 slots is fine; a product past 2^31 is not
        assert _status(_cfg(**kw))[0] == B.SDM_OK
        kw = dict(widths=(4096, 4096, 256))
    s, _ = _status(_cfg(**kw))
    assert s == status, (kw, B.STATUS_NAMES.get(s), B.last_error())
    assert B.last_error() != ""


def test_shared_bank_settings(lib):
    s0, n0 = _status(_cfg())
    s1, n1 = _status(_cfg(shared_bank=True))
    assert s0 == B.SDM_OK and s1 == B.SDM_OK
    assert n1 >= n0 + 2 * 1024 * 4  # the owner table: one int32 per (head, slot)
    cfg = _cfg(tokens=1, shared_bank=True)
    assert _status(cfg, B.SDM_OP_DECODE)[0] == B.SDM_ERR_RANGE  # a decode step's streams own their banks
    assert "shared_bank" in B.last_error()
    cfg = _cfg()
    cfg.shared_bank = 2
    assert _status(cfg)[0] == B.SDM_ERR_RANGE
    # the check entry point refuses a config without a shared bank and a NULL result pointer
    c = ctypes.c_int32(0)
    assert lib.sdm_shared_bank_check(ctypes.byref(_cfg()), None, 0, ctypes.byref(c), None) == B.SDM_ERR_RANGE
    assert lib.sdm_shared_bank_check(ctypes.byref(_cfg(shared_bank=True)), None, 0, None, None) == B.SDM_ERR_NULL


def test_padded_pitch_accepted_and_sized(lib):
    s0, n0 = _status(_cfg(bank_row_stride=0))
    s1, n1 = _status(_cfg(bank_row_stride=96))
    assert s0 == B.SDM_OK and s1 == B.SDM_OK and n0 == n1  # the workspace does not depend on the pitch


def test_candidate_limit(lib):
    # four factors with k = 512 give more than 4096 candidate tuples
    s, _ = _status(_cfg(widths=(16, 16, 16, 16), num_writes=512, num_reads=4, chunk_size=16))
    assert s == B.SDM_ERR_RANGE and "candidate" in B.last_error()


def _gpu_visible():
    """True when a GPU device node or a HIP device is visible to this process. Calls with fake device addresses
    are meant to stop at a host check; on a machine with a GPU a mistake in such a test would launch kernels on
    unmapped memory, so those tests run only where no GPU is visible."""
    if os.path.exists("/dev/kfd"):
        return True
    try:
        import torch

        return torch.cuda.device_count() > 0  # counts devices without initialising HIP
    except Exception:
        return False


fake_pointers = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses are only passed where no GPU is "
                                   "visible")


def _fake(addr):
    return ctypes.c_void_p(addr)


@fake_pointers
def test_write_read_refuses_before_device_work(lib):
    cfg = _cfg()
    n = ctypes.c_size_t(0)
    assert lib.sdm_workspace_size(ctypes.byref(cfg), B.SDM_OP_WRITE_READ, 0, ctypes.byref(n)) == B.SDM_OK
    base = 1 << 40  # fake, never dereferenced: every check below fails before any HIP call
    step = 1 << 32
    ptrs = [_fake(base + i * step) for i in range(10)]
    args = lambda p, ws, wsn: (ctypes.byref(cfg), *p, ws, wsn, None)
    # NULL input
    p = list(ptrs)
    p[0] = None
    assert lib.sdm_write_read(*args(p, ptrs[9], n.value)) == B.SDM_ERR_NULL
    # workspace too small / misaligned
    assert lib.sdm_write_read(*args(ptrs[:9] + [None], _fake(base + 20 * step), n.value - 1)) == B.SDM_ERR_WORKSPACE
    assert lib.sdm_write_read(*args(ptrs[:9] + [None], _fake(base + 20 * step + 8), n.value)) == B.SDM_ERR_WORKSPACE
    # misaligned bank
    p = list(ptrs[:9]) + [None]
    p[6] = _fake(base + 6 * step + 4)
    assert lib.sdm_write_read(*args(p, _fake(base + 20 * step), n.value)) == B.SDM_ERR_LAYOUT
    # out overlapping the bank
    p = list(ptrs[:9]) + [None]
    p[7] = _fake(base + 6 * step + 4096)
    assert lib.sdm_write_read(*args(p, _fake(base + 20 * step), n.value)) == B.SDM_ERR_ALIAS
    # out overlapping an input (values)
    p = list(ptrs[:9]) + [None]
    p[7] = p[2]
    assert lib.sdm_write_read(*args(p, _fake(base + 20 * step), n.value)) == B.SDM_ERR_ALIAS
    assert "overlaps" in B.last_error()


@fake_pointers
def test_decode_partial_overlap_refused(lib):
    cfg = _cfg(tokens=1)
    n = ctypes.c_size_t(0)
    assert lib.sdm_workspace_size(ctypes.byref(cfg), B.SDM_OP_DECODE, 0, ctypes.byref(n)) == B.SDM_OK
    base, step = 1 << 40, 1 << 32
    p = [_fake(base + i * step) for i in range(11)]
    p[7] = _fake(base + 6 * step + 256)  # bank_out starts inside bank_in
    st = lib.sdm_decode_step(ctypes.byref(cfg), *p, _fake(base + 20 * step), n.value, None)
    assert st == B.SDM_ERR_ALIAS and "bank_out" in B.last_error()


def test_backward_settings_and_refusals(lib):
    s0, n0 = _status(_cfg(), B.SDM_OP_BACKWARD)
    assert s0 == B.SDM_OK and n0 > 0
    assert _status(_cfg(tokens=512), B.SDM_OP_BACKWARD)[1] > n0  # partial sums grow with the tokens
    assert _status(_cfg(shared_bank=True), B.SDM_OP_BACKWARD)[0] == B.SDM_ERR_RANGE
    # a snapshot of 2^31 rows (batch * heads * tokens * num_writes) is refused before any work
    big = _cfg(batch=64, heads=64, tokens=4096, num_writes=128)
    assert _status(big, B.SDM_OP_BACKWARD)[0] == B.SDM_ERR_RANGE and "snapshot" in B.last_error()
    assert _status(_cfg(batch=64, heads=64, tokens=4096, num_writes=64), B.SDM_OP_BACKWARD)[0] == B.SDM_OK
    assert _status(_cfg(), 5)[0] == B.SDM_ERR_RANGE  # no op 5


@fake_pointers
def test_save_and_backward_refuse_before_device_work(lib):
    cfg = _cfg()
    n = ctypes.c_size_t(0)
    assert lib.sdm_workspace_size(ctypes.byref(cfg), B.SDM_OP_WRITE_READ, 0, ctypes.byref(n)) == B.SDM_OK
    base, step = 1 << 40, 1 << 36  # fake, never dereferenced: every check below fails before any HIP call
    # keys, queries, values, gates (2), sub-keys, bank, out, snapshot, write ids, read ids
    p = [_fake(base + i * step) for i in range(11)]
    ws = _fake(base + 40 * step)
    # the saving forward: NULL snapshot, shared bank, snapshot overlapping the bank
    q = list(p)
    q[8] = None
    assert lib.sdm_write_read_save(ctypes.byref(cfg), *q, ws, n.value, None) == B.SDM_ERR_NULL
    assert "snapshot" in B.last_error()
    shared = _cfg(shared_bank=True)
    assert lib.sdm_write_read_save(ctypes.byref(shared), *p, ws, n.value, None) == B.SDM_ERR_RANGE
    q = list(p)
    q[8] = _fake(base + 6 * step + 4096)  # inside the bank
    assert lib.sdm_write_read_save(ctypes.byref(cfg), *q, ws, n.value, None) == B.SDM_ERR_ALIAS
    # the backward: NULL gradient, misaligned grad_bank, a gradient overlapping an input
    nb = ctypes.c_size_t(0)
    assert lib.sdm_workspace_size(ctypes.byref(cfg), B.SDM_OP_BACKWARD, 0, ctypes.byref(nb)) == B.SDM_OK
    # inputs (6), bank, snapshot, grad_out, grad_bank, then the six gradients
    g = [_fake(base + i * step) for i in range(16)]
    q = list(g)
    q[11] = None  # grad_read_queries
    assert lib.sdm_write_read_backward(ctypes.byref(cfg), *q, ws, nb.value, None) == B.SDM_ERR_NULL
    q = list(g)
    q[9] = _fake(base + 9 * step + 4)  # grad_bank
    assert lib.sdm_write_read_backward(ctypes.byref(cfg), *q, ws, nb.value, None) == B.SDM_ERR_LAYOUT
    q = list(g)
    q[12] = q[2]  # grad_values = values
    assert lib.sdm_write_read_backward(ctypes.byref(cfg), *q, ws, nb.value, None) == B.SDM_ERR_ALIAS
    assert lib.sdm_write_read_backward(ctypes.byref(cfg), *g, ws, nb.value - 1, None) == B.SDM_ERR_WORKSPACE


def _layer_cfg(model_dim=256, **kw):
    base = dict(act_dtype=B.SDM_BF16)
    base.update(kw)
    lc = B.SdmLayerConfig()
    lc.op = _cfg(**base)
    lc.model_dim = model_dim
    return lc


def _layer_ws(lc):
    n = ctypes.c_size_t(0)
    return B.load().sdm_layer_workspace_size(ctypes.byref(lc), ctypes.byref(n)), n.value


def test_layer_settings_and_refusals(lib):
    s, n = _layer_ws(_layer_cfg())
    assert s == B.SDM_OK
    op_s, op_n = _status(_layer_cfg().op)
    assert op_s == B.SDM_OK and n > op_n  # the projections, gates and o come before the op's workspace
    assert _layer_ws(_layer_cfg(act_dtype=B.SDM_F32))[0] == B.SDM_ERR_DTYPE
    assert _layer_ws(_layer_cfg(model_dim=48))[0] == B.SDM_ERR_RANGE
    assert _layer_ws(_layer_cfg(model_dim=0))[0] == B.SDM_ERR_RANGE
    assert _layer_ws(_layer_cfg(shared_bank=True))[0] == B.SDM_ERR_RANGE
    assert _layer_ws(_layer_cfg(head_dim=72, heads=1))[0] == B.SDM_ERR_RANGE  # H d = 72: not a multiple of 32
    lc = _layer_cfg()
    lc.reserved = 1
    assert _layer_ws(lc)[0] == B.SDM_ERR_RANGE
    assert _layer_ws(_layer_cfg(widths=(32, 32), bank_rows=100))[0] == B.SDM_ERR_BANK_TOO_SMALL


@fake_pointers
def test_layer_refuses_before_device_work(lib):
    lc = _layer_cfg()
    s, n = _layer_ws(lc)
    assert s == B.SDM_OK
    base = 1 << 40  # fake, never dereferenced: every check below fails before any HIP call
    step = 1 << 32
    # x w_in a_log dt_bias w_out subkeys initial_bank bank y widx ridx ws (initial_bank NULL)
    p = [_fake(base + i * step) for i in range(11)]
    call = lambda q, wsn=n: lib.sdm_layer_forward(ctypes.byref(lc), *q[:6], None, *q[6:10], q[10], wsn, None)
    q = list(p)
    q[6] = None  # bank
    assert call(q) == B.SDM_ERR_NULL
    q = list(p)
    q[7] = _fake(base + 6 * step + 64)  # y inside the bank
    assert call(q) == B.SDM_ERR_ALIAS
    q = list(p)
    q[8] = p[0]  # write ids over x
    assert call(q) == B.SDM_ERR_ALIAS
    q = list(p)
    q[5] = _fake(base + 5 * step + 8)  # misaligned sub-keys
    assert call(q) == B.SDM_ERR_LAYOUT
    assert call(list(p), n - 1) == B.SDM_ERR_WORKSPACE


def test_layer_backward_workspace(lib):
    """The training calls' workspace: the forward's as a prefix plus the op's backward and the layer backward's
    regions (larger than the forward's); the op's own backward refusals surface through it."""
    lc = _layer_cfg()
    _, nf = _layer_ws(lc)
    n = ctypes.c_size_t(0)
    assert lib.sdm_layer_backward_workspace_size(ctypes.byref(lc), ctypes.byref(n)) == B.SDM_OK
    assert n.value > nf
    # settings the op's backward refuses (a bfloat16 snapshot of a float32 bank outside the held-row loop)
    bad = _layer_cfg(snapshot_dtype=B.SDM_BF16, chunk_size=7)
    assert _layer_ws(bad)[0] == B.SDM_OK  # the plain forward does not need the backward
    assert lib.sdm_layer_backward_workspace_size(ctypes.byref(bad), ctypes.byref(n)) == B.SDM_ERR_RANGE


@fake_pointers
def test_layer_training_calls_refuse_before_device_work(lib):
    lc = _layer_cfg()
    n = ctypes.c_size_t(0)
    assert lib.sdm_layer_backward_workspace_size(ctypes.byref(lc), ctypes.byref(n)) == B.SDM_OK
    nb = n.value
    _, nf = _layer_ws(lc)
    base, step = 1 << 40, 1 << 34
    # x w_in a_log dt_bias w_out subkeys initial_bank bank y snapshot widx ridx ws
    p = [_fake(base + i * step) for i in range(13)]
    p[6] = None
    fwd = lambda q, wsn: lib.sdm_layer_forward_save(ctypes.byref(lc), *q, wsn, None)
    assert fwd(p, nf) == B.SDM_ERR_WORKSPACE  # the forward's size is not enough: the backward reads this one
    q = list(p)
    q[9] = None
    assert fwd(q, nb) == B.SDM_ERR_NULL  # no snapshot
    q = list(p)
    q[9] = _fake(base + 7 * step + 256)  # the snapshot inside the bank
    assert fwd(q, nb) == B.SDM_ERR_ALIAS
    # x w_in a_log dt_bias w_out subkeys bank snapshot grad_y grad_bank grad_x grad_w_in grad_a_log grad_dt_bias
    # grad_w_out grad_subkeys ws
    g = [_fake(base + i * step) for i in range(17)]
    bwd = lambda q, wsn=nb: lib.sdm_layer_backward(ctypes.byref(lc), *q, wsn, None)
    assert bwd(g, nb - 1) == B.SDM_ERR_WORKSPACE
    q = list(g)
    q[8] = None
    assert bwd(q) == B.SDM_ERR_NULL  # no grad_y
    q = list(g)
    q[10] = g[0]  # grad_x over x
    assert bwd(q) == B.SDM_ERR_ALIAS
    q = list(g)
    q[11] = _fake(base + 11 * step + 4)  # misaligned grad_w_in
    assert bwd(q) == B.SDM_ERR_LAYOUT


@fake_pointers
def test_snapshot_dtype_settings_and_refusals(lib):
    """snapshot_dtype: 0 (the bank dtype) or SDM_BF16; a bfloat16 snapshot of a float32 bank needs the held-row
    loop and the fast reverse sweep, else SDM_ERR_RANGE, before any device work; on a bfloat16 bank it is the same
    as 0."""
    n = ctypes.c_size_t(0)
    base, step = 1 << 40, 1 << 36
    p = [_fake(base + i * step) for i in range(11)]
    ws = _fake(base + 40 * step)
    g = [_fake(base + i * step) for i in range(16)]

    def save(cfg, short=0):
        assert lib.sdm_workspace_size(ctypes.byref(cfg), B.SDM_OP_WRITE_READ, 0, ctypes.byref(n)) == B.SDM_OK
        return lib.sdm_write_read_save(ctypes.byref(cfg), *p, ws, n.value - short, None)

    def bwd(cfg):
        assert lib.sdm_workspace_size(ctypes.byref(cfg), B.SDM_OP_BACKWARD, 0, ctypes.byref(n)) == B.SDM_OK
        return lib.sdm_write_read_backward(ctypes.byref(cfg), *g, ws, n.value, None)

    assert save(_cfg(snapshot_dtype=7)) == B.SDM_ERR_DTYPE
    assert bwd(_cfg(snapshot_dtype=7)) == B.SDM_ERR_DTYPE
    ragged = _cfg(snapshot_dtype=B.SDM_BF16, chunk_size=7)  # no held-row loop for chunk 7
    assert save(ragged) == B.SDM_ERR_RANGE and "no native route" in B.last_error()
    assert bwd(ragged) == B.SDM_ERR_RANGE
    wide = _cfg(snapshot_dtype=B.SDM_BF16, num_writes=160, num_reads=16, chunk_size=8, widths=(32, 32))
    assert save(wide) == B.SDM_ERR_RANGE  # W > 128: no fast reverse sweep
    # a bfloat16 bank ignores it: the checks after it run as for 0. The workspace is one byte short, so the call
    # stops at the workspace check (which follows the route check) on every machine, never at the route refusal
    bf = _cfg(snapshot_dtype=B.SDM_BF16, chunk_size=7, act_dtype=B.SDM_BF16, bank_dtype=B.SDM_BF16)
    assert save(bf, short=1) == B.SDM_ERR_WORKSPACE


@fake_pointers
def test_grad_bank_dtype_settings_and_refusals(lib):
    """grad_bank_dtype: 0 (float32) or SDM_BF16, the latter only on a bfloat16 bank and, in the backward, within the
    fast reverse sweep (num_writes, num_reads <= 128); refusals come before any device work. A bfloat16 gradient is
    half the bytes: an output that overlaps it only past that size is not an alias."""
    n = ctypes.c_size_t(0)
    base, step = 1 << 40, 1 << 36
    g = [_fake(base + i * step) for i in range(16)]
    ws = _fake(base + 40 * step)

    def bwd(cfg, ptrs=g):
        assert lib.sdm_workspace_size(ctypes.byref(cfg), B.SDM_OP_BACKWARD, 0, ctypes.byref(n)) == B.SDM_OK
        return lib.sdm_write_read_backward(ctypes.byref(cfg), *ptrs, ws, n.value, None)

    bf = dict(act_dtype=B.SDM_BF16, bank_dtype=B.SDM_BF16)
    assert bwd(_cfg(grad_bank_dtype=5, **bf)) == B.SDM_ERR_DTYPE
    assert bwd(_cfg(grad_bank_dtype=B.SDM_BF16)) == B.SDM_ERR_RANGE  # float32 bank
    assert "float32 bank" in B.last_error()
    wide = _cfg(grad_bank_dtype=B.SDM_BF16, num_writes=160, num_reads=16, chunk_size=8, **bf)
    assert bwd(wide) == B.SDM_ERR_RANGE and "no native route" in B.last_error()
    # aliasing is sized by the gradient's element: grad_write_keys placed right after a bfloat16 grad_bank
    cfg = _cfg(grad_bank_dtype=B.SDM_BF16, **bf)
    nbank = cfg.batch * cfg.heads * cfg.bank_rows * cfg.head_dim
    q = list(g)
    q[10] = _fake(base + 9 * step + 2 * nbank)  # starts where the bfloat16 gradient ends
    st = bwd(cfg, q)
    assert st != B.SDM_ERR_ALIAS and st in (B.SDM_ERR_DEVICE, B.SDM_ERR_HIP), B.last_error()
    q[10] = _fake(base + 9 * step + 2 * nbank - 16)  # one lane inside it
    assert bwd(cfg, q) == B.SDM_ERR_ALIAS
    f32 = _cfg(**bf)
    q[10] = _fake(base + 9 * step + 2 * nbank)  # inside a float32 gradient of the same shape
    assert bwd(f32, q) == B.SDM_ERR_ALIAS
    # the batch sum reads the same field
    gs = _cfg(grad_bank_dtype=B.SDM_BF16)
    assert lib.sdm_bank_grad_sum(ctypes.byref(gs), g[0], g[1], None) == B.SDM_ERR_RANGE
    gs = _cfg(grad_bank_dtype=7, **bf)
    assert lib.sdm_bank_grad_sum(ctypes.byref(gs), g[0], g[1], None) == B.SDM_ERR_DTYPE


@fake_pointers
def test_decode_noalloc_refuses_before_device_work(lib):
    """sdm_decode_step_noalloc: the decode step's host checks, and a step whose workspace exceeds the per-GPU
    scratch (SDM_NOALLOC_SCRATCH_BYTES) refused with SDM_ERR_RANGE, all before any device work."""
    base, step = 1 << 40, 1 << 36
    p = [_fake(base + i * step) for i in range(11)]  # keys queries values gates(2) sub-keys bank_in bank_out out ids
    cfg = _cfg(tokens=1)
    q = list(p)
    q[8] = None  # out
    assert lib.sdm_decode_step_noalloc(ctypes.byref(cfg), *q, None) == B.SDM_ERR_NULL
    q = list(p)
    q[7] = _fake(base + 6 * step + 256)  # bank_out starts inside bank_in
    assert lib.sdm_decode_step_noalloc(ctypes.byref(cfg), *q, None) == B.SDM_ERR_ALIAS
    big = _cfg(tokens=1, batch=2048, num_writes=512, num_reads=512, widths=(32, 32))
    assert B.workspace_size(big, B.SDM_OP_DECODE) > B.NOALLOC_SCRATCH_BYTES
    assert lib.sdm_decode_step_noalloc(ctypes.byref(big), *p, None) == B.SDM_ERR_RANGE
    assert "scratch" in B.last_error()


def test_decode_steps_settings(lib):
    """sdm_decode_steps: its workspace grows with the steps (ids and scores of every token), a shared bank is
    refused, and shapes outside the one-launch step (W > 64, wide factors) are refused before any device work."""
    s1, n1 = _status(_cfg(tokens=1), B.SDM_OP_DECODE_STEPS)
    s8, n8 = _status(_cfg(tokens=8), B.SDM_OP_DECODE_STEPS)
    assert s1 == B.SDM_OK and s8 == B.SDM_OK and n8 > n1
    assert _status(_cfg(tokens=8, shared_bank=True), B.SDM_OP_DECODE_STEPS)[0] == B.SDM_ERR_RANGE


@fake_pointers
def test_decode_steps_refuses_before_device_work(lib):
    base, step = 1 << 40, 1 << 36
    p = [_fake(base + i * step) for i in range(11)]
    ws = _fake(base + 40 * step)
    for cfg in (_cfg(tokens=4, num_writes=96, widths=(32, 32)), _cfg(tokens=4, widths=(512, 2))):
        n = B.workspace_size(cfg, B.SDM_OP_DECODE_STEPS)
        assert lib.sdm_decode_steps(ctypes.byref(cfg), *p, ws, n, None) == B.SDM_ERR_RANGE
        assert "sdm_decode_step per token" in B.last_error()
    cfg = _cfg(tokens=4)
    n = B.workspace_size(cfg, B.SDM_OP_DECODE_STEPS)
    q = list(p)
    q[7] = _fake(base + 6 * step + 256)  # bank_out starts inside bank_in
    assert lib.sdm_decode_steps(ctypes.byref(cfg), *q, ws, n, None) == B.SDM_ERR_ALIAS
    assert lib.sdm_decode_steps(ctypes.byref(cfg), *p, ws, n - 1, None) == B.SDM_ERR_WORKSPACE


def test_large_chunks_run_as_sub_chunks(lib):
    """chunk_size above the kernels' 128 tokens / 8192 events runs as equal sub-chunks (its largest divisor within
    them): the workspace (chunk plans) is that of the sub-chunk."""
    base = dict(widths=(256, 256), num_writes=64, num_reads=64, tokens=1024)
    n128 = _status(_cfg(chunk_size=128, **base))[1]
    s256, n256 = _status(_cfg(chunk_size=256, **base))
    assert s256 == B.SDM_OK and n256 == n128
    s, n = _status(_cfg(chunk_size=128, widths=(256, 256), num_writes=128, num_reads=64, tokens=1024))
    assert s == B.SDM_OK and n == _status(_cfg(chunk_size=64, widths=(256, 256), num_writes=128, num_reads=64,
                                               tokens=1024))[1]
    assert _status(_cfg(chunk_size=131))[0] == B.SDM_OK  # a prime above 128: chunks of one token


def test_quantized_snapshot_routes_and_sizes(lib):
    """fp8 / int4 snapshots: the pages' refusals (head_dim above 16384, not a multiple of 4, not splitting into
    ceil(head_dim / 128) equal slices of 16-byte rows; int4 with slices 4 mod 8 wide), this library's (a bfloat16
    bank, head_dim not a multiple of 16, no held-row route), all before any work; sizes per include/sdm.h."""
    def snap(**kw):
        base = dict(widths=(32, 32), num_writes=8, num_reads=8, chunk_size=16, tokens=64)
        base.update(kw)
        cfg = _cfg(**base)
        n = ctypes.c_size_t(0)
        st = lib.sdm_snapshot_bytes(ctypes.byref(cfg), ctypes.byref(n))
        return st, n.value
    rows = 2 * 2 * 64 * 8
    for d in (64, 400, 1024):
        assert snap(head_dim=d, snapshot_dtype=B.SDM_FP8) == (B.SDM_OK, rows * (d + d // 16))
    assert snap(head_dim=64, snapshot_dtype=B.SDM_INT4) == (B.SDM_OK, rows * (64 // 2 + 64 // 16))
    assert snap(head_dim=64) == (B.SDM_OK, rows * 64 * 4)
    assert snap(head_dim=64, snapshot_dtype=B.SDM_BF16) == (B.SDM_OK, rows * 64 * 2)
    refused = [dict(head_dim=400, snapshot_dtype=B.SDM_INT4),           # 4 slices of 100 columns: 4 mod 8
               dict(head_dim=12, snapshot_dtype=B.SDM_INT4),            # 1 slice of 12: 4 mod 8
               dict(head_dim=16400, snapshot_dtype=B.SDM_FP8),          # above 16384
               dict(head_dim=136, snapshot_dtype=B.SDM_FP8),            # groups of 16 columns
               dict(head_dim=64, snapshot_dtype=B.SDM_FP8, bank_dtype=B.SDM_BF16, act_dtype=B.SDM_BF16),
               dict(head_dim=64, snapshot_dtype=B.SDM_FP8, chunk_size=7)]  # no held-row route
    for kw in refused:
        st, _ = snap(**kw)
        assert st == B.SDM_ERR_RANGE, (kw, B.last_error())
    assert "4 mod 8" in (snap(head_dim=400, snapshot_dtype=B.SDM_INT4), B.last_error())[1]
    assert snap(head_dim=64, snapshot_dtype=9)[0] == B.SDM_ERR_DTYPE
