"""GPU parity of the backward (sdm_write_read_save + sdm_write_read_backward, through the C ABI) against the oracle's
backward (fp64, bank states rounded like the forward after every token).

Checked: every gradient (write keys, read queries, values, both gates, sub-keys, the bank before the call) element
by element within an a-priori bound; the bank stepped back to its state before the forward bit for bit; the
snapshot's rows of each stream's first token equal the initial bank rows bit for bit; repeated backward calls give
the same bits.

The bound (oracle.write_read_backward_bounds; sdm_oracle.c, the comment above bound_par_t) is a first-order running
error analysis of the backward evaluated alongside the oracle's: the GPU computes the same chain rule in float32
(unit roundoff u = 2^-24, sums in its own fixed orders, which the any-order bound gamma(n) = n u / (1 - n u) times
the sum of the terms' magnitudes covers), its softmax weights are the float32 rounding of an fp64 softmax of the
bit-exact slot scores (within 2u), and the rows it reads (the snapshot's pre-write rows, the rows read after a
write) come from its own forward. That last condition is checked first, against the oracle's forward: every
snapshot row and every final bank row within eps_row of the oracle's (row-wise, relative to the row's largest
magnitude), with eps_row the forward's tolerance for the bank dtype (1e-5 float32, 2e-2 bfloat16); with a bfloat16
snapshot each element may also round the other way, one bfloat16 spacing (q_rel = 2^-7 of the element). The bound
propagates exactly these deviations; the only slack is a factor 1.01 for the second-order terms the analysis leaves
out. Nothing in it is taken from a measurement of the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_product_amd import binding, synth

DEV = torch.device("cuda:0")
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
pytestmark = pytest.mark.gpu


def rowwise_rel(got, ref):
    """max over rows of |got - ref|_inf / |ref row|_inf."""
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    err = np.abs(got - ref).max(axis=1)
    scale = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((err / scale).max())


def rows_within(got, ref, eps, q_rel=0.0):
    """Every element within eps of its row's largest magnitude (plus q_rel of the element and of that allowance)."""
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    allow = eps * np.abs(ref).max(axis=1, keepdims=True)
    allow = allow + q_rel * (np.abs(ref) + allow)
    return bool(np.all(np.abs(got - ref) <= allow)), rowwise_rel(got, ref)


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)


EPS_ROW = {"f32": 1e-5, "bf16": 2e-2}  # the forward's row tolerance per bank dtype
Q_BF16 = 2.0 ** -7                    # one bfloat16 spacing, relative to the element
SLACK = 1.01                          # second-order terms of the running error analysis


def _upstream(s, seed, with_bank_grad):
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal((s.batch, s.tokens, s.heads, s.head_dim)).astype(np.float32)
    if s.act == "bf16":
        dout = synth.round_bf16_rne(dout)
    dbank = rng.standard_normal((s.batch, s.heads, s.rows, s.head_dim)).astype(np.float32) if with_bank_grad else None
    return dout, dbank


def run_gpu(s, x, dout, dbank, pitch=None, gdt=torch.float32):
    at, bt = TORCH_DT[s.act], TORCH_DT[s.bank]
    t = {k: to_dev(x[k], at) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    if pitch is None:
        bank = to_dev(x["bank"], bt)
    else:
        buf = torch.zeros((s.batch, s.heads, s.rows, pitch), dtype=bt, device=DEV)
        bank = buf[..., :s.head_dim]
        bank.copy_(to_dev(x["bank"], bt))
    bank0 = bank.clone()
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, chunk_size=s.chunk_size)
    out, widx, _, snap = binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"],
                                                     t["subkeys"], bank, want_index=True, **kw)
    torch.cuda.synchronize()
    fwd = {"snapshot": snap.float().cpu().numpy(), "bank": bank.float().cpu().numpy()}
    gbank = None
    if dbank is not None:
        ld = bank.stride(2)
        gbank = torch.zeros((s.batch, s.heads, s.rows, ld), dtype=gdt, device=DEV)[..., :s.head_dim]
        gbank.copy_(to_dev(dbank, torch.float32))
    g = binding.sdm_write_read_backward(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                        snap, to_dev(dout, at), gbank, grad_bank_dtype=gdt, **kw)
    assert g["bank"].dtype == gdt
    torch.cuda.synchronize()
    assert torch.equal(bank, bank0), "the backward did not restore the bank bit for bit"
    # the first token's snapshot rows are initial bank rows
    w0 = widx[:, 0].long()  # [B, H, W]
    first = torch.stack([torch.stack([bank0[b, h, w0[b, h]] for h in range(s.heads)]) for b in range(s.batch)])
    assert torch.equal(snap[:, :, 0], first)
    fwd["out"] = out.float().cpu().numpy()
    return {k: v.float().cpu().numpy() for k, v in g.items()}, fwd


def run_oracle(s, x, dout, dbank, snap_bf16=False, grad_bank_bf16=False):
    """The oracle's backward with its error bounds for a float32 evaluation reading rows within the forward's
    tolerance (EPS_ROW of the bank dtype; plus one bfloat16 spacing per element with a bfloat16 snapshot)."""
    return oracle.write_read_backward_bounds(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"],
                                             x["bank"], dout, dbank, s.widths, s.num_writes, s.num_reads,
                                             eps_row=EPS_ROW[s.bank], q_rel=Q_BF16 if snap_bf16 else 0.0,
                                             bank_bf16=s.bank == "bf16", snap_bf16=snap_bf16, want_snapshot=True,
                                             grad_bank_bf16=grad_bank_bf16, g_rel=Q_BF16)



BOUNDS = {"write_keys": "wkeys", "read_queries": "rq", "values": "values", "subkeys": "subkeys", "bank": "bank",
          "forget_gate": "alpha", "input_gate": "beta"}


def check(s, got, ref, fwd=None, snap_bf16=False):
    """The bound's hypothesis (the GPU's forward rows within EPS_ROW of the oracle's), then every gradient element
    within its bound. fwd: the GPU's snapshot and bank after its forward (None: rows not available)."""
    eps = EPS_ROW[s.bank]
    if fwd is not None:
        ok, e = rows_within(fwd["snapshot"], ref["snapshot"], eps, Q_BF16 if snap_bf16 else 0.0)
        assert ok, f"snapshot rows beyond {eps} of the oracle's (row-wise {e:.3g})"
        ok, e = rows_within(fwd["bank"], ref["bank"], eps)
        assert ok, f"bank after the forward beyond {eps} of the oracle's (row-wise {e:.3g})"
    ratios = {}
    for k, r in BOUNDS.items():
        err = np.abs(np.asarray(got[k], np.float64) - ref["d_" + r])
        bound = SLACK * ref["e_" + r]
        ratios[k] = float((err / np.maximum(bound, 1e-300)).max())
    print("gradient error / bound (max)", {k: f"{v:.3g}" for k, v in ratios.items()}, flush=True)
    bad = {k: v for k, v in ratios.items() if not v <= 1.0}
    assert not bad, f"gradients beyond their a-priori bounds: {bad}"


CASES = [
    # name, shape, with a bank gradient
    ("tiny", synth.WORKLOADS["tiny_1k"].with_(tokens=96, batch=2, heads=2, chunk_size=32), True),
    ("ragged_c7", synth.WORKLOADS["tiny_1k"].with_(tokens=50, batch=1, heads=2, chunk_size=7), False),
    ("collide", synth.Shape(1, 64, 2, (8, 8), 4, 32, 16, 16, 16, name="collide"), True),
    ("three_factors", synth.Shape(1, 40, 2, (8, 4, 4), 8, 32, 16, 12, 16, name="f3"), True),
    ("bf16_act", synth.Shape(2, 48, 2, (16, 16), 8, 64, 8, 8, 16, "bf16", "f32", name="bf16a"), True),
    ("bf16_bank", synth.Shape(1, 48, 2, (16, 16), 8, 64, 8, 8, 16, "bf16", "bf16", name="bf16b"), True),
    ("wide_w", synth.Shape(1, 24, 1, (16, 16), 8, 48, 160, 136, 8, name="wide"), True),
    # held-row loop with more slots written several times per chunk than its LDS keeps (~300 of 512 slots): the
    # events of those slots are applied, and their snapshot rows stored, from the plan region
    ("held_many_multi", synth.Shape(1, 96, 1, (16, 32), 8, 32, 32, 32, 32, name="multi"), True),
    # enough streams x 16-column slices (32 x 16 = 512) that the sweep keeps 16-column slices; the shapes above take
    # 8-column slices (two token chains per CU)
    ("slices16", synth.Shape(8, 24, 4, (16, 16), 8, 256, 16, 12, 8, name="s16"), True),
    # steps of up to four consecutive tokens with disjoint slots (W, R <= 32 on 16-column slices), 4,096 slots so
    # that runs of every length occur, and a token count that is not a multiple of four
    ("token_runs", synth.Shape(2, 61, 2, (64, 64), 8, 64, 12, 20, 16, name="runs"), True),
    # more than 8192 terms in a row block of the sub-key sums (16 rows x 560 terms): the one-wave kernel instead of
    # the sorting one
    ("subkey_one_wave", synth.Shape(1, 20, 1, (32, 32), 8, 16, 300, 260, 4, name="sk1w"), True),
    # sub-keys of 96 coordinates: the sub-key sums in two column blocks, the second one partly past dk
    ("dk96", synth.Shape(1, 24, 2, (16, 16), 96, 32, 8, 8, 8, name="dk96"), True),
]


@pytest.mark.parametrize("name,s,bank_grad", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(name, s, bank_grad):
    x = synth.make_inputs(s, seed=41)
    dout, dbank = _upstream(s, 42, bank_grad)
    print(f"backward {name}: {s}", flush=True)
    got, fwd = run_gpu(s, x, dout, dbank)
    check(s, got, run_oracle(s, x, dout, dbank), fwd)


GB16_CASES = [
    # name, shape (bfloat16 banks), with a bank gradient
    ("bf16_bank", synth.Shape(1, 48, 2, (16, 16), 8, 64, 8, 8, 16, "bf16", "bf16", name="bf16b"), True),
    # 64 slots, 16 reads and 16 writes a token: most tokens read rows they also write
    ("collide", synth.Shape(1, 64, 2, (8, 8), 4, 32, 16, 16, 16, "bf16", "bf16", name="collide16"), True),
    ("f32_act", synth.Shape(1, 40, 2, (8, 4, 4), 8, 32, 16, 12, 16, "f32", "bf16", name="f3b"), False),
    ("slices16", synth.Shape(8, 24, 4, (16, 16), 8, 256, 16, 12, 8, "bf16", "bf16", name="s16b"), True),
]


@pytest.mark.parametrize("name,s,bank_grad", GB16_CASES, ids=[c[0] for c in GB16_CASES])
def test_bf16_bank_gradient(name, s, bank_grad):
    """The bank gradient in the bank dtype of a bfloat16 bank (CHANGELOG 2.0.0 "Deterministic": float32 accumulation
    is the opt-in): every gradient within the oracle's bounds for an adjoint bank rounded to bfloat16 at every
    update (one bfloat16 spacing per update that may round the other way); the gradient is bfloat16-valued, the
    bank is restored bit for bit, and two calls give the same bits."""
    x = synth.make_inputs(s, seed=51)
    dout, dbank = _upstream(s, 52, bank_grad)
    if dbank is not None:
        dbank = synth.round_bf16_rne(dbank)
    print(f"bf16 bank gradient {name}: {s}", flush=True)
    got, fwd = run_gpu(s, x, dout, dbank, gdt=torch.bfloat16)
    again, _ = run_gpu(s, x, dout, dbank, gdt=torch.bfloat16)
    for k in got:
        assert np.array_equal(got[k], again[k]), f"{k} differs between calls"
    assert np.array_equal(synth.round_bf16_rne(got["bank"].astype(np.float32)), got["bank"])
    ref = run_oracle(s, x, dout, dbank, grad_bank_bf16=True)
    check(s, got, ref, fwd)


def test_bf16_bank_gradient_batch_sum():
    """sdm_bank_grad_sum over a bfloat16 bank gradient: the float32 sum over the batch in order, bit for bit (each
    term widened exactly), rows past N and the padding not written."""
    B, H, rows, d, pitch, N = 4, 2, 70, 48, 56, 64
    rng = np.random.default_rng(9)
    gb_np = synth.round_bf16_rne(rng.standard_normal((B, H, rows, d)).astype(np.float32))
    gbuf = torch.zeros((B, H, rows, pitch), dtype=torch.bfloat16, device=DEV)
    gb = gbuf[..., :d]
    gb.copy_(to_dev(gb_np, torch.float32))
    obuf = torch.full((H, rows, pitch), 5.0, device=DEV)
    out = obuf[..., :d]
    print("bf16 bank gradient sum", flush=True)
    binding.sdm_bank_grad_sum(gb, heads=H, widths=(8, 8), head_dim=d, out=out)
    torch.cuda.synchronize()
    acc = gb_np[0, :, :N].copy()
    for b in range(1, B):
        acc = (acc + gb_np[b, :, :N]).astype(np.float32)
    assert np.array_equal(out.cpu().numpy()[:, :N], acc)
    assert bool((obuf[:, N:] == 5.0).all()) and bool((obuf[..., d:] == 5.0).all())


def test_backward_padded_pitch_and_repeatable():
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=64, batch=1, heads=2, chunk_size=16)
    x = synth.make_inputs(s, seed=43)
    dout, dbank = _upstream(s, 44, True)
    print("backward pitch 80 / repeat", flush=True)
    a, fwd_a = run_gpu(s, x, dout, dbank, pitch=80)
    b, fwd_b = run_gpu(s, x, dout, dbank)
    assert np.array_equal(fwd_a["out"], fwd_b["out"])
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{k} differs between calls"
    check(s, a, run_oracle(s, x, dout, dbank), fwd_a)


def test_save_forward_matches_plain_forward_within_rounding():
    """The saving forward runs the segmented loop; its outputs equal the plain forward's up to rounding."""
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=80, batch=2, heads=2, chunk_size=16)
    x = synth.make_inputs(s, seed=45)
    t = {k: to_dev(x[k], torch.float32) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, chunk_size=s.chunk_size)
    b1, b2 = to_dev(x["bank"], torch.float32), to_dev(x["bank"], torch.float32)
    o1, _, _ = binding.sdm_write_read(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], b1, **kw)
    o2, _, _, _ = binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"],
                                              b2, **kw)
    torch.cuda.synchronize()
    assert rowwise_rel(o2.cpu().numpy(), o1.cpu().numpy()) <= 1e-5
    assert rowwise_rel(b2.cpu().numpy(), b1.cpu().numpy()) <= 1e-5


def test_backward_layer_65k_full_size():
    """The 65,536-slot layer workload at full size (B 2, T 4096, H 2, d 1024, W = R = 64, chunk 64, bf16 activations
    on a float32 bank, padded row pitch): every gradient against the oracle's backward, bank restored bit for bit."""
    s = synth.WORKLOADS["layer_65k"]
    print("full-size backward: inputs", flush=True)
    x = synth.make_inputs(s)
    dout, dbank = _upstream(s, 46, True)
    print("full-size backward: GPU", flush=True)
    got, fwd = run_gpu(s, x, dout, dbank, pitch=binding.bank_pitch(s.head_dim, torch.float32))
    print("full-size backward: oracle", flush=True)
    ref = run_oracle(s, x, dout, dbank)
    check(s, got, ref, fwd)


def test_training_step_graph_replay_equals_eager():
    """The saving forward and the backward captured into one HIP graph (the gradient bank reset by a fill kernel
    inside it) and replayed several times, with eager work and synchronisations between the replays: every replay
    gives the eager outputs and gradients bit for bit, and leaves the bank as it found it."""
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=96, batch=2, heads=2, chunk_size=32)
    x = synth.make_inputs(s, seed=47)
    dout, _ = _upstream(s, 48, False)
    t = {k: to_dev(x[k], torch.float32) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    g_out = to_dev(dout, torch.float32)
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, chunk_size=s.chunk_size)
    cfg = binding.make_config(s.batch, s.tokens, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes,
                              s.num_reads, s.chunk_size, binding.SDM_F32, binding.SDM_F32, s.rows)
    wsf = torch.empty(binding.workspace_size(cfg, binding.SDM_OP_WRITE_READ), dtype=torch.uint8, device=DEV)
    wsb = torch.empty(binding.workspace_size(cfg, binding.SDM_OP_BACKWARD), dtype=torch.uint8, device=DEV)
    bank = to_dev(x["bank"], torch.float32)
    bank0 = bank.clone()
    out = torch.empty((s.batch, s.tokens, s.heads, s.head_dim), device=DEV)
    snap = torch.empty((s.batch, s.heads, s.tokens, s.num_writes, s.head_dim), device=DEV)
    gbank = torch.zeros_like(bank)
    grads = {}

    def step():
        gbank.zero_()
        binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                    out=out, snapshot=snap, workspace=wsf, **kw)
        grads.update(binding.sdm_write_read_backward(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"],
                                                     t["subkeys"], bank, snap, g_out, gbank, workspace=wsb, **kw))

    print("training step graph replay", flush=True)
    step()
    torch.cuda.synchronize()
    ref_out = out.clone()
    ref = {k: v.clone() for k, v in grads.items()}
    assert torch.equal(bank, bank0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    captured = dict(grads)  # the gradient tensors the graph writes
    for r in range(3):
        out.fill_(float("nan"))
        for v in captured.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: out differs"
        for k, v in captured.items():
            assert torch.equal(v, ref[k]), f"replay {r}: gradient {k} differs"
        assert torch.equal(bank, bank0), f"replay {r}: bank not restored"
        step()  # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------------------ bfloat16 snapshot of a float32 bank
SNAP_CASES = [
    ("tiny", synth.WORKLOADS["tiny_1k"].with_(tokens=96, batch=2, heads=2, chunk_size=32), True),
    ("collide", synth.Shape(1, 64, 2, (8, 8), 4, 32, 16, 16, 16, name="collide"), True),
    ("bf16_act", synth.Shape(2, 48, 2, (16, 16), 8, 64, 8, 8, 16, "bf16", "f32", name="bf16a"), False),
]


def _padded(arr, pitch):
    """A float32 bank view [B, H, rows, d] on rows `pitch` elements apart (pitch None: dense)."""
    if pitch is None:
        return to_dev(arr, torch.float32)
    B, H, rows, d = arr.shape
    v = torch.zeros((B, H, rows, pitch), dtype=torch.float32, device=DEV)[..., :d]
    v.copy_(to_dev(arr, torch.float32))
    return v


def _bf16_snapshot_case(s, bank_grad, pitch=None):
    x = synth.make_inputs(s, seed=51)
    dout, dbank = _upstream(s, 52, bank_grad)
    at = TORCH_DT[s.act]
    t = {k: to_dev(x[k], at) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, chunk_size=s.chunk_size)
    bank0 = _padded(x["bank"], pitch)
    b_none, b_q = _padded(x["bank"], pitch), _padded(x["bank"], pitch)
    o1, w1, _, snap_none = binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"],
                                                       t["subkeys"], b_none, want_index=True, **kw)
    o2, w2, _, snap_q = binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"],
                                                    t["subkeys"], b_q, want_index=True, snapshot_quant="bf16", **kw)
    torch.cuda.synchronize()
    assert snap_q.dtype == torch.bfloat16
    assert torch.equal(o1, o2) and torch.equal(b_none, b_q) and torch.equal(w1, w2)
    assert torch.equal(snap_q, snap_none.to(torch.bfloat16))
    del snap_none
    fwd = {"snapshot": snap_q.float().cpu().numpy(), "bank": b_q.float().cpu().numpy()}
    gbank = None
    if dbank is not None:
        gbank = torch.zeros((s.batch, s.heads, s.rows, b_q.stride(2)), dtype=torch.float32, device=DEV)[..., :s.head_dim]
        gbank.copy_(to_dev(dbank, torch.float32))
    g = binding.sdm_write_read_backward(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], b_q,
                                        snap_q, to_dev(dout, at), gbank, snapshot_quant="bf16", **kw)
    torch.cuda.synchronize()
    written = torch.zeros((s.batch, s.heads, s.rows), dtype=torch.bool, device=DEV)
    for b in range(s.batch):
        for h in range(s.heads):
            written[b, h, w1[b, :, h].reshape(-1).long()] = True
    expect = torch.where(written[..., None], bank0.to(torch.bfloat16).float(), bank0)
    assert torch.equal(b_q, expect), "the bank is not the rounded restore"
    ref = run_oracle(s, x, dout, dbank, snap_bf16=True)
    check(s, {k: v.cpu().numpy() for k, v in g.items()}, ref, fwd, snap_bf16=True)


@pytest.mark.parametrize("name,s,bank_grad", SNAP_CASES, ids=[c[0] for c in SNAP_CASES])
def test_bf16_snapshot(name, s, bank_grad):
    """CHANGELOG 2.0.0, "New" (bf16 snapshots on a float32 bank): the saving forward with a bfloat16 snapshot
    equals the float32 snapshot's forward bit for bit, its snapshot is that snapshot rounded to nearest even, the
    backward matches the oracle's bfloat16-snapshot backward, and the bank comes back with exactly the rows the
    forward wrote rounded to bfloat16 (it is restored from the rounded rows)."""
    _bf16_snapshot_case(s, bank_grad)


def test_bf16_snapshot_layer_65k_full_size():
    """The same at the full layer_65k workload (2 GiB bfloat16 snapshot, padded row pitch, 8-column sweep)."""
    s = synth.WORKLOADS["layer_65k"]
    print("full-size bf16 snapshot", flush=True)
    _bf16_snapshot_case(s, True, pitch=binding.bank_pitch(s.head_dim, torch.float32))


def test_bf16_snapshot_refused_without_a_native_route():
    """A bfloat16 snapshot of a float32 bank needs the held-row loop (chunk 7 is not a power of two): refused
    before any work, like the pages' training calls that have no native route."""
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=50, batch=1, heads=2, chunk_size=7)
    x = synth.make_inputs(s, seed=1)
    t = {k: to_dev(x[k], torch.float32) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    bank = to_dev(x["bank"], torch.float32)
    bank0 = bank.clone()
    with pytest.raises(binding.UnsupportedConfigurationError, match="no native route"):
        binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                    widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
                                    chunk_size=s.chunk_size, snapshot_quant="bf16")
    torch.cuda.synchronize()
    assert torch.equal(bank, bank0)


# ------------------------------------------------------------------ fp8 / int4 snapshots of a float32 bank
QUANT = {  # mode: (q_rel, q_grp) of the bound: one rounding that falls the other way on each side
    "fp8": (2.0 ** -2, 2.0 ** -14),   # an E4M3 spacing is at most 2^-3 of the element (subnormals: 2^-9 scale units)
    "int4": (0.0, 1.0 / 3.0),         # an int4 step is at most 2/7 of the group's largest magnitude (6/7 of it stored)
}


def _quantize_ref(rows, mode):
    """The snapshot bytes of float32 rows [n, d] by this library's format, computed here with torch (E4M3 by
    torch's float8_e4m3fn conversion, int4 by torch.round): elements then scale bytes."""
    x = rows.reshape(-1, rows.shape[-1] // 16, 16).to(torch.float64)
    amax = x.abs().amax(dim=2)
    m, ex = torch.frexp(amax)  # amax = m 2^ex, m in [0.5, 1): amax = (2m) 2^(ex - 1)
    k = 8 if mode == "fp8" else 2
    e = ex - 1 - k + (2 * m > 1.75).to(ex.dtype)
    e = torch.where(amax > 0, e, torch.full_like(e, -127))
    y = x * torch.pow(2.0, -e.to(torch.float64)).unsqueeze(2)
    if mode == "fp8":
        el = y.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).reshape(rows.shape[0], -1)
    else:
        q = (torch.round(y).to(torch.int32) & 0xF).reshape(rows.shape[0], -1)
        el = (q[:, 0::2] | (q[:, 1::2] << 4)).to(torch.uint8)
    sc = (e + 127).clamp(0, 255).to(torch.uint8)
    return torch.cat([el.reshape(-1), sc.reshape(-1)])


def _quant_case(s, mode, bank_grad, exact_rows=False):
    x = synth.make_inputs(s, seed=53)
    if exact_rows:  # rows never change (alpha 1, beta 0) and are already in the format: no rounding anywhere
        x["alpha"][:] = 1.0
        x["beta"][:] = 0.0
        x["bank"] = oracle.snap_rows(x["bank"], mode).astype(np.float32)
    dout, dbank = _upstream(s, 54, bank_grad)
    at = TORCH_DT[s.act]
    t = {k: to_dev(x[k], at) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, chunk_size=s.chunk_size)
    b_none, b_q = to_dev(x["bank"], torch.float32), to_dev(x["bank"], torch.float32)
    o1, w1, _, snap_none = binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"],
                                                       t["subkeys"], b_none, want_index=True, **kw)
    o2, w2, _, snap_q = binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"],
                                                    t["subkeys"], b_q, want_index=True, snapshot_quant=mode, **kw)
    torch.cuda.synchronize()
    assert snap_q.dtype == torch.uint8
    assert torch.equal(o1, o2) and torch.equal(b_none, b_q) and torch.equal(w1, w2)
    # the quantized snapshot is this format's quantization of the float32 snapshot, byte for byte
    assert torch.equal(snap_q, _quantize_ref(snap_none.reshape(-1, s.head_dim), mode))
    del snap_none
    fwd = {"bank": b_q.float().cpu().numpy()}
    g = binding.sdm_write_read_backward(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], b_q,
                                        snap_q, to_dev(dout, at),
                                        None if dbank is None else to_dev(dbank, torch.float32),
                                        snapshot_quant=mode, **kw)
    torch.cuda.synchronize()
    # the bank comes back with exactly the written rows as the snapshot stores them
    written = np.zeros((s.batch, s.heads, s.rows), bool)
    wi = w1.cpu().numpy()
    for b in range(s.batch):
        for h in range(s.heads):
            written[b, h, wi[b, :, h].reshape(-1)] = True
    expect = np.where(written[..., None], oracle.snap_rows(x["bank"], mode), x["bank"])
    assert np.array_equal(b_q.cpu().numpy(), expect.astype(np.float32)), "the bank is not the quantized restore"
    q_rel, q_grp = (0.0, 0.0) if exact_rows else QUANT[mode]
    eps = 0.0 if exact_rows else EPS_ROW[s.bank]
    ref = oracle.write_read_backward_bounds(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"],
                                            x["bank"], dout, dbank, s.widths, s.num_writes, s.num_reads,
                                            eps_row=eps, q_rel=q_rel, q_grp=q_grp, snap_quant=mode,
                                            want_snapshot=True)
    ok, e = rows_within(fwd["bank"], ref["bank"], EPS_ROW[s.bank])
    assert ok, f"bank after the forward beyond the tolerance ({e:.3g})"
    check(s, {k: v.cpu().numpy() for k, v in g.items()}, ref)


@pytest.mark.parametrize("mode", ["fp8", "int4"])
@pytest.mark.parametrize("name,s,bank_grad", SNAP_CASES, ids=[c[0] for c in SNAP_CASES])
def test_quantized_snapshot(name, s, bank_grad, mode):
    """CHANGELOG 2.0.0, "New" / "Behavior changes" (fp8 and int4 snapshots): the saving forward's out, bank and ids
    equal the float32 snapshot's bit for bit, the snapshot is that snapshot quantized byte for byte (groups of 16
    columns, power-of-two scales, E4M3 by torch's float8 conversion, int4 by torch.round), the bank comes back with
    exactly the written rows quantized, and the gradients match the oracle's quantized-snapshot backward within its
    a-priori bound (rows within the forward tolerance, plus one quantization step where a rounding may fall the
    other way)."""
    print(f"quantized snapshot {mode} {name}", flush=True)
    _quant_case(s, mode, bank_grad)


@pytest.mark.parametrize("mode", ["fp8", "int4"])
def test_quantized_snapshot_exact_rows(mode):
    """Rows that never change (forget gate 1, input gate 0) and are already in the format: the GPU's snapshot rows
    equal the oracle's exactly, so the bound is the float32 arithmetic's alone (no row allowance)."""
    s = synth.Shape(2, 64, 2, (16, 16), 8, 64, 8, 8, 16, name="qexact")
    print(f"quantized snapshot {mode}, exact rows", flush=True)
    _quant_case(s, mode, True, exact_rows=True)


def test_quantized_snapshot_refused_before_any_work():
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=50, batch=1, heads=2, chunk_size=16, head_dim=40)
    x = synth.make_inputs(s, seed=2)
    t = {k: to_dev(x[k], torch.float32) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    bank = to_dev(x["bank"], torch.float32)
    bank0 = bank.clone()
    with pytest.raises(binding.UnsupportedConfigurationError, match="groups of 16"):
        binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                    widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
                                    chunk_size=s.chunk_size, snapshot_quant="fp8")
    torch.cuda.synchronize()
    assert torch.equal(bank, bank0)


@pytest.mark.slow
def test_fp8_snapshot_layer_65k_full_size():
    """fp8 snapshot at the full layer_65k workload (8-column sweep slices sharing each group's scale)."""
    s = synth.WORKLOADS["layer_65k"]
    print("full-size fp8 snapshot", flush=True)
    _quant_case(s, "fp8", True)
