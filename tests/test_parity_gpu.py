"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded synthetic inputs.

Bar: slot ids and float32 slot scores bit-exact; outputs and bank rows within 1e-5 (float32) / 2e-2 (bfloat16) of the
oracle, measured row-wise as max|gpu - ref| <= rtol * max|ref| per output row and per bank row; GPU results bitwise
repeatable; a donated decode step equal to a copied one bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_product_amd import binding, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
RTOL = {"f32": 1e-5, "bf16": 2e-2}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def rowwise_rel(got, ref):
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    err = np.abs(got - ref).max(axis=1)
    scale = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((err / scale).max())


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)


def to_np(t):
    return t.float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


SENTINEL = 1234.5


def padded_bank(arr, dtype, pitch):
    """Device bank view [B, H, rows, d] with rows `pitch` elements apart; padding filled with a sentinel."""
    B, H, rows, d = arr.shape
    buf = torch.full((B, H, rows, pitch), SENTINEL, dtype=dtype, device=DEV)
    g = buf[..., :d]
    g.copy_(torch.from_numpy(np.ascontiguousarray(arr)).to(DEV).to(dtype))
    return g


def run_gpu(s, x, chunk_size=None, bank=None, pitch=None):
    at, bt = TORCH_DT[s.act], TORCH_DT[s.bank]
    t = {k: to_dev(x[k], at) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    src = x["bank"] if bank is None else bank
    g_bank = to_dev(src, bt) if pitch is None else padded_bank(src, bt, pitch)
    out, widx, ridx = binding.sdm_write_read(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"],
                                             g_bank, widths=s.widths, num_writes=s.num_writes,
                                             num_reads=s.num_reads, chunk_size=chunk_size or s.chunk_size,
                                             want_index=True)
    torch.cuda.synchronize()
    if pitch is not None and pitch > s.head_dim:
        pad = g_bank._base[..., s.head_dim:]
        assert bool((pad == SENTINEL).all()), "padding columns of the bank were written"
    return to_np(out), to_np(g_bank), to_np(widx), to_np(ridx)


def run_oracle(s, x):
    return oracle.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                             s.widths, s.num_writes, s.num_reads, bank_bf16=s.bank == "bf16",
                             act_bf16=s.act == "bf16")


def check_parity(s, gpu, ref):
    out, bank, widx, ridx = gpu
    assert np.array_equal(widx, ref["widx"]), "write slot ids differ"
    assert np.array_equal(ridx, ref["ridx"]), "read slot ids differ"
    e_out = rowwise_rel(out, ref["out"])
    e_bank = rowwise_rel(bank, ref["bank"])
    # out is read from bank rows: its tolerance is that of the coarser of its own dtype and the bank dtype
    assert e_out <= max(RTOL[s.act], RTOL[s.bank]), f"out rel err {e_out}"
    assert e_bank <= RTOL[s.bank], f"bank rel err {e_bank}"
    return e_out, e_bank


# ------------------------------------------------------------------------------------------------ top-k
def _topk_case(widths, dk, k, act, kind, B=1, T=24, H=2, seed=0, scoring="auto"):
    rng = np.random.default_rng(seed)
    F = len(widths)
    if kind == "ternary":
        q = rng.integers(-1, 2, (B, T, H, F * dk)).astype(np.float32)
        sub = rng.integers(-1, 2, (H, sum(widths), dk)).astype(np.float32)
    else:
        q = rng.standard_normal((B, T, H, F * dk)).astype(np.float32)
        sub = rng.standard_normal((H, sum(widths), dk)).astype(np.float32)
        if kind == "dup":
            for _ in range(sum(widths) // 3):
                i, j = rng.integers(0, sum(widths), 2)
                sub[:, j] = sub[:, i]
    if act == "bf16":
        q, sub = synth.round_bf16_rne(q), synth.round_bf16_rne(sub)
    ids, sc = binding.topk_product_keys(to_dev(q, TORCH_DT[act]), to_dev(sub, TORCH_DT[act]), widths, k,
                                        scoring=scoring)
    torch.cuda.synchronize()
    rid, rsc = oracle.topk(q, sub, widths, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.array_equal(sc.cpu().numpy(), rsc)


@pytest.mark.parametrize("widths,dk,k", [((32, 32), 16, 4), ((32, 32), 16, 64), ((8, 8), 4, 5), ((4, 3, 5), 3, 7),
                                         ((16,), 4, 6), ((3, 2, 2, 3), 2, 9), ((7, 9), 5, 63), ((64, 32, 32), 8, 64),
                                         ((32, 32), 16, 512)])  # the largest k
@pytest.mark.parametrize("kind", ["random", "ternary", "dup"])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_topk_exact(widths, dk, k, kind, act):
    print(f"topk widths={widths} dk={dk} k={k} kind={kind} act={act}", flush=True)
    _topk_case(widths, dk, k, act, kind)


@pytest.mark.parametrize("widths,dk,k", [((32, 32), 32, 64), ((64, 32, 16), 64, 64), ((16,), 32, 9),
                                         ((256, 256), 64, 64), ((48, 16), 96, 33), ((32, 32), 128, 17),
                                         ((512, 16), 32, 64), ((1024, 32), 64, 40),
                                         # selection buffers too large for the score rows (the per-wave layout)
                                         ((512, 64), 64, 200), ((1024, 32), 32, 254)])
@pytest.mark.parametrize("kind", ["random", "ternary", "dup"])
@pytest.mark.parametrize("scoring", ["filtered", "direct"])
def test_topk_exact_filtered(widths, dk, k, kind, scoring):
    """bf16 shapes the MFMA-filtered scoring can serve (widths multiples of 16, dk a multiple of 32 up to 128), with
    each scoring forced: ids and scores bit-exact, including the many exact ties of ternary inputs and duplicated
    sub-keys."""
    print(f"topk {scoring} widths={widths} dk={dk} k={k} kind={kind}", flush=True)
    _topk_case(widths, dk, k, "bf16", kind, T=40, scoring=scoring)


@pytest.mark.parametrize("kind", ["ternary_onehot", "binary_onehot"])
@pytest.mark.parametrize("scoring", ["filtered", "direct"])
def test_topk_massive_ties(kind, scoring):
    """Queries with one nonzero coordinate (+-1) per factor over ternary or 0/1 sub-keys (1024 of them, k 64): 300 to
    650 sub-keys of a factor tie at its k_p-th score, so the filtered scoring's first stage keeps that many (its
    widest listed selection, and past 512 the keys taken from registers) and the tie rule (smaller index first)
    decides the ids; both scorings against the oracle, bit for bit."""
    widths, dk, k, T, H = (1024, 32), 64, 64, 40, 2
    rng = np.random.default_rng(11)
    q = np.zeros((1, T, H, 2 * dk), np.float32)
    for f in range(2):
        j = rng.integers(0, dk, (1, T, H))
        sign = rng.choice([-1.0, 1.0], (1, T, H, 1)).astype(np.float32)
        np.put_along_axis(q[..., f * dk:(f + 1) * dk], j[..., None], sign, -1)
    if kind == "ternary_onehot":
        sub = rng.integers(-1, 2, (H, sum(widths), dk)).astype(np.float32)
    else:
        sub = (rng.random((H, sum(widths), dk)) < 0.6).astype(np.float32)
    print(f"topk massive ties {kind} {scoring}", flush=True)
    ids, sc = binding.topk_product_keys(to_dev(q, torch.bfloat16), to_dev(sub, torch.bfloat16), widths, k,
                                        scoring=scoring)
    torch.cuda.synchronize()
    rid, rsc = oracle.topk(q, sub, widths, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.array_equal(sc.cpu().numpy(), rsc)


@pytest.mark.parametrize("name", ["layer_65k", "large_1m"])
def test_topk_filtered_equals_direct(name):
    """The filtered (MFMA) scoring and the direct fp64 scoring return identical ids and scores at full size."""
    s = synth.WORKLOADS[name]
    x = synth.make_step_inputs(s.with_(tokens=256))
    q = to_dev(x["wkeys"], torch.bfloat16)
    sub = to_dev(synth.make_subkeys(s), torch.bfloat16)
    print(f"topk filtered vs direct, {name} T=256", flush=True)
    ids_f, sc_f = binding.topk_product_keys(q, sub, s.widths, s.num_writes, scoring="filtered")
    torch.cuda.synchronize()
    ids_d, sc_d = binding.topk_product_keys(q, sub, s.widths, s.num_writes, scoring="direct")
    torch.cuda.synchronize()
    assert torch.equal(ids_f, ids_d)
    assert torch.equal(sc_f, sc_d)


def test_topk_filtered_nonfinite_equals_direct():
    """Inputs the MFMA filter cannot bound: a NaN and an infinite sub-key row, NaN and infinite query values, and a
    query whose norm times the largest sub-key norm passes 2^127 (finite scores). The filtered scoring keeps every
    sub-key of such a factor and returns the direct scoring's ids and score bits."""
    widths, dk, k = (1024, 32), 64, 40
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 48, 3, 2 * dk)).astype(np.float32)
    sub = rng.standard_normal((3, sum(widths), dk)).astype(np.float32)
    sub[0, 17, 3] = np.nan            # head 0, factor 0
    sub[1, 1024 + 5, 0] = np.inf      # head 1, factor 1
    q[0, 3, 0, 7] = np.nan            # head 0, factor 0
    q[0, 4, 1, dk + 2] = -np.inf      # head 1, factor 1
    q[0, 5, 2, :dk] = 5e36            # head 2 (finite sub-keys), factor 0: |x| |c| > 2^127
    qd, sd = to_dev(q, torch.bfloat16), to_dev(sub, torch.bfloat16)
    print("topk filtered vs direct, non-finite inputs", flush=True)
    ids_f, sc_f = binding.topk_product_keys(qd, sd, widths, k, scoring="filtered")
    torch.cuda.synchronize()
    ids_d, sc_d = binding.topk_product_keys(qd, sd, widths, k, scoring="direct")
    torch.cuda.synchronize()
    assert torch.equal(ids_f, ids_d)
    assert torch.equal(sc_f.view(torch.int32), sc_d.view(torch.int32))
    assert bool(torch.isfinite(sc_d[0, 5, 2]).all())  # the large query's scores stay finite


def test_topk_zero_query_tie_order():
    q = np.zeros((1, 1, 1, 2 * 8), np.float32)
    sub = np.random.default_rng(0).standard_normal((1, 64, 8)).astype(np.float32)
    ids, sc = binding.topk_product_keys(to_dev(q, torch.float32), to_dev(sub, torch.float32), (32, 32), 4)
    assert ids.cpu().numpy().ravel().tolist() == [0, 1, 32, 2]


@pytest.mark.parametrize("name", ["layer_65k", "three_factor_65k", "large_1m"])
def test_topk_full_size_factors_sampled(name):
    """The full-size factor tables (65,536 and 1,048,576 slots) on sampled token rows."""
    s = synth.WORKLOADS[name]
    x = synth.make_step_inputs(s.with_(tokens=8))
    sub = synth.make_subkeys(s)
    print(f"topk full-size {name}", flush=True)
    for key in ("wkeys", "rq"):
        ids, sc = binding.topk_product_keys(to_dev(x[key], TORCH_DT[s.act]), to_dev(sub, TORCH_DT[s.act]), s.widths,
                                            s.num_writes)
        torch.cuda.synchronize()
        rid, rsc = oracle.topk(x[key], sub, s.widths, s.num_writes)
        assert np.array_equal(ids.cpu().numpy(), rid)
        assert np.array_equal(sc.cpu().numpy(), rsc)


# ------------------------------------------------------------------------------------------------ write / read
def test_write_read_tiny():
    s = synth.WORKLOADS["tiny_1k"]
    x = synth.make_inputs(s)
    print("write/read tiny_1k", flush=True)
    e = check_parity(s, run_gpu(s, x), run_oracle(s, x))
    print("errors", e)


@pytest.mark.parametrize("chunk", [1, 7, 16, 64, 128])
def test_write_read_chunk_sizes_ragged(chunk):
    """chunk_size changes results only through rounding; T = 200 leaves a ragged last chunk."""
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=200, batch=2, heads=2, chunk_size=chunk)
    x = synth.make_inputs(s, seed=3)
    print(f"write/read chunk={chunk}", flush=True)
    check_parity(s, run_gpu(s, x), run_oracle(s, x))


@pytest.mark.parametrize("act,bank", [("bf16", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
def test_write_read_dtypes(act, bank):
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=130, batch=2, act=act, bank=bank, head_dim=64, chunk_size=32)
    x = synth.make_inputs(s, seed=4)
    print(f"write/read act={act} bank={bank}", flush=True)
    check_parity(s, run_gpu(s, x), run_oracle(s, x))


def test_write_read_collisions_heavy():
    """A tiny bank (64 slots, W = R = 16) makes most writes collide inside a chunk."""
    s = synth.Shape(1, 96, 2, (8, 8), 4, 32, 16, 16, 32, name="collide")
    x = synth.make_inputs(s, seed=5)
    print("write/read collisions", flush=True)
    check_parity(s, run_gpu(s, x), run_oracle(s, x))


def test_write_read_dense_limit():
    """W = R = N: every slot is written and read by every token (Gated DeltaNet in slot space)."""
    s = synth.Shape(1, 40, 1, (4, 4), 3, 16, 16, 16, 8, name="dense")
    x = synth.make_inputs(s, seed=6)
    print("write/read dense limit", flush=True)
    check_parity(s, run_gpu(s, x), run_oracle(s, x))


@pytest.mark.parametrize("act,bank", [("f32", "f32"), ("bf16", "bf16")])
def test_write_read_largest_k(act, bank):
    """W = R = 512, the largest top-k, on 1024 slots: chunk 16 (16 x 512 = 8192 write events, the loop's largest
    chunk), 40 tokens (a ragged last chunk); half the slots written and read by every token."""
    s = synth.Shape(1, 40, 2, (32, 32), 16, 64, 512, 512, 16, act, bank, name="k512")
    x = synth.make_inputs(s, seed=30)
    print(f"write/read W = R = 512 act={act} bank={bank}", flush=True)
    check_parity(s, run_gpu(s, x), run_oracle(s, x))


def test_write_read_three_factors_small():
    s = synth.Shape(1, 80, 2, (8, 4, 4), 8, 32, 16, 12, 16, "bf16", "bf16", name="f3")
    x = synth.make_inputs(s, seed=7)
    print("write/read three factors", flush=True)
    check_parity(s, run_gpu(s, x), run_oracle(s, x))


# Shapes served by the 16-byte-slice chunk loop: gpt = 512 / C lanes per token share its W write and R read terms
# (at most 16 of each per lane); bf16 banks, and float32 banks whose chunk gives a 64-byte slice too many terms.
NARROW = [
    # act, bank, chunk, W, R, widths, tokens
    ("bf16", "bf16", 128, 64, 64, (16, 8, 8), 300),   # the three-factor workload's chunk split (16 terms per lane)
    ("bf16", "f32", 128, 64, 64, (32, 32), 200),      # float32 bank, 16 terms per lane
    ("f32", "bf16", 64, 32, 24, (32, 32), 150),       # 4 and 3 terms per lane
    ("bf16", "bf16", 32, 16, 32, (16, 16), 100),      # 1 and 2 terms per lane
    ("f32", "bf16", 8, 64, 128, (16, 16), 37),        # one wave per token
]


@pytest.mark.parametrize("act,bank,chunk,W,R,widths,T", NARROW)
def test_write_read_narrow_slices(act, bank, chunk, W, R, widths, T):
    s = synth.Shape(2, T, 2, widths, 8, 64, W, R, chunk, act, bank, name="narrow")
    x = synth.make_inputs(s, seed=21)
    print(f"write/read narrow act={act} bank={bank} C={chunk} W={W} R={R} T={T}", flush=True)
    got = run_gpu(s, x)
    check_parity(s, got, run_oracle(s, x))
    again = run_gpu(s, x)
    for u, v in zip(got, again):
        assert np.array_equal(u, v)


def test_write_read_narrow_collisions_and_split():
    """64 slots, W = R = 16, chunk 64, bf16 bank: most writes collide; a split call is bitwise equal."""
    s = synth.Shape(1, 192, 2, (8, 8), 4, 32, 16, 16, 64, "bf16", "bf16", name="collide_narrow")
    x = synth.make_inputs(s, seed=22)
    print("write/read narrow collisions", flush=True)
    full = run_gpu(s, x)
    check_parity(s, full, run_oracle(s, x))
    h = 128
    first = {k: (v[:, :h] if k in ("wkeys", "rq", "values", "alpha", "beta") else v) for k, v in x.items()}
    second = {k: (v[:, h:] if k in ("wkeys", "rq", "values", "alpha", "beta") else v) for k, v in x.items()}
    o1, b1, _, _ = run_gpu(s.with_(tokens=h), first)
    o2, b2, _, _ = run_gpu(s.with_(tokens=192 - h), second, bank=b1)
    assert np.array_equal(np.concatenate([o1, o2], 1), full[0])
    assert np.array_equal(b2, full[1])


@pytest.mark.parametrize("pitch", [72, 128])
def test_write_read_narrow_padded_pitch(pitch):
    s = synth.Shape(2, 130, 2, (16, 16), 8, 64, 32, 32, 64, "bf16", "bf16", name="narrow_pitch")
    x = synth.make_inputs(s, seed=23)
    print(f"write/read narrow pitch={pitch}", flush=True)
    got = run_gpu(s, x, pitch=pitch)
    check_parity(s, got, run_oracle(s, x))
    same = run_gpu(s, x)
    for u, v in zip(got, same):
        assert np.array_equal(u, v)


def test_write_read_bank_rows_padding():
    """bank_rows > N: rows past N are never touched."""
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=64, bank_rows=1100)
    x = synth.make_inputs(s, seed=8)
    out, bank, widx, ridx = run_gpu(s, x)
    assert np.array_equal(bank[:, :, 1024:], x["bank"][:, :, 1024:])
    ref = run_oracle(s, x)
    check_parity(s, (out, bank, widx, ridx), ref)


@pytest.mark.parametrize("bank_dt,pitch", [("f32", 96), ("f32", 68), ("bf16", 72), ("bf16", 128)])
def test_write_read_padded_bank_pitch(bank_dt, pitch):
    """A bank whose rows are `pitch` elements apart: same results, padding never touched."""
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=150, batch=2, heads=2, bank=bank_dt, act="bf16", chunk_size=32)
    x = synth.make_inputs(s, seed=12)
    print(f"write/read pitch={pitch} bank={bank_dt}", flush=True)
    got = run_gpu(s, x, pitch=pitch)
    check_parity(s, got, run_oracle(s, x))
    same = run_gpu(s, x)
    for u, v in zip(got, same):
        assert np.array_equal(u, v)  # the pitch does not change the arithmetic


# ------------------------------------------------------------------------------------------------ shared bank
def _disjoint_streams(s, seed):
    """Inputs whose B streams address disjoint slots of each head: factor 0's sub-keys fall into B groups, group g
    near 10 * u_g (u_g = +-e_0, +-e_1, ...), and every query of stream b points along 5 * u_b in factor 0, so the
    best factor-0 score of any tuple outside group b is about 50 below every tuple inside it (the other factors'
    scores are a few units wide). Every written or read slot of stream b then has its factor-0 index in group b."""
    x = synth.make_inputs(s, seed=seed)
    B, dk, n0 = s.batch, s.subkey_dim, s.widths[0]
    assert n0 % B == 0 and B <= 2 * dk
    rng = np.random.default_rng(seed)
    u = np.zeros((B, dk), np.float32)
    for g in range(B):
        u[g, g // 2] = 1.0 if g % 2 == 0 else -1.0
    g = n0 // B
    sub = x["subkeys"].copy()
    for grp in range(B):
        sub[:, grp * g:(grp + 1) * g] = 10.0 * u[grp] + 0.1 * rng.standard_normal((s.heads, g, dk))
    for key in ("wkeys", "rq"):
        q = x[key].copy()
        q[..., :dk] = 5.0 * u[:, None, None, :] + 0.3 * rng.standard_normal(q[..., :dk].shape)
        x[key] = q
    if s.act == "bf16":
        sub = synth.round_bf16_rne(sub)
        x["wkeys"], x["rq"] = synth.round_bf16_rne(x["wkeys"]), synth.round_bf16_rne(x["rq"])
    x["subkeys"] = sub.astype(np.float32)
    x["shared"] = x["bank"][0].copy()  # [H, rows, d]
    return x


def run_gpu_shared(s, x, bank=None, pitch=None, out_fill=None):
    at, bt = TORCH_DT[s.act], TORCH_DT[s.bank]
    t = {k: to_dev(x[k], at) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    src = x["shared"] if bank is None else bank
    g_bank = to_dev(src, bt) if pitch is None else padded_bank(src[None], bt, pitch)[0]
    out = None
    if out_fill is not None:
        out = torch.full((s.batch, s.tokens, s.heads, s.head_dim), out_fill, dtype=at, device=DEV)
    try:
        out, widx, ridx = binding.sdm_write_read(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"],
                                                 t["subkeys"], g_bank, widths=s.widths, num_writes=s.num_writes,
                                                 num_reads=s.num_reads, chunk_size=s.chunk_size, want_index=True,
                                                 out=out, shared_bank=True)
    finally:
        torch.cuda.synchronize()
    if pitch is not None and pitch > s.head_dim:
        assert bool((g_bank._base[..., s.head_dim:] == SENTINEL).all()), "padding columns of the bank were written"
    return to_np(out), to_np(g_bank), to_np(widx), to_np(ridx)


def oracle_shared(s, x):
    """The streams of each head run one after another on the one bank (stream 0 first); with disjoint slots the
    order is immaterial."""
    M = x["shared"][None]
    outs, widx, ridx = [], [], []
    for b in range(s.batch):
        xb = {k: x[k][b:b + 1] for k in ("wkeys", "rq", "values", "alpha", "beta")}
        ref = oracle.write_read(xb["wkeys"], xb["rq"], xb["values"], xb["alpha"], xb["beta"], x["subkeys"], M,
                                s.widths, s.num_writes, s.num_reads, bank_bf16=s.bank == "bf16",
                                act_bf16=s.act == "bf16")
        M = ref["bank"]
        outs.append(ref["out"])
        widx.append(ref["widx"])
        ridx.append(ref["ridx"])
    return {"out": np.concatenate(outs), "bank": M[0], "widx": np.concatenate(widx), "ridx": np.concatenate(ridx)}


# act, bank, chunk, W, R, streams: the held-row loop (float32 bank, pow2 chunk), the 16-byte-slice loop (bf16
# bank), and the general loop (chunk 7, ragged)
SHARED = [
    ("f32", "f32", 16, 8, 8, 4),
    ("bf16", "f32", 64, 64, 64, 2),
    ("bf16", "bf16", 32, 16, 16, 4),
    ("f32", "bf16", 64, 32, 24, 2),
    ("f32", "f32", 7, 5, 6, 4),
]


@pytest.mark.parametrize("act,bank,chunk,W,R,B", SHARED)
def test_shared_bank_disjoint_streams(act, bank, chunk, W, R, B):
    s = synth.Shape(B, 75, 2, (32, 32), 8, 64, W, R, chunk, act, bank, name="shared")
    x = _disjoint_streams(s, seed=31)
    print(f"shared bank act={act} bank={bank} C={chunk} W={W} R={R} B={B}", flush=True)
    ref = oracle_shared(s, x)
    grp = s.widths[0] // B
    for key in ("widx", "ridx"):
        f0 = ref[key] // s.widths[1]
        assert np.array_equal(f0 // grp, np.broadcast_to(np.arange(B)[:, None, None, None], f0.shape)), \
            "the construction did not give disjoint streams"
    got = run_gpu_shared(s, x)
    check_parity(s, got, ref)
    again = run_gpu_shared(s, x)
    for u, v in zip(got, again):
        assert np.array_equal(u, v)


def test_shared_bank_padded_pitch():
    s = synth.Shape(2, 60, 2, (32, 32), 8, 64, 16, 16, 32, "bf16", "bf16", name="shared_pitch")
    x = _disjoint_streams(s, seed=32)
    print("shared bank pitch 72", flush=True)
    got = run_gpu_shared(s, x, pitch=72)
    check_parity(s, got, oracle_shared(s, x))


def test_shared_bank_one_stream_equals_private():
    """B = 1: the shared layout [H, rows, d] is the private one without its batch axis; results are bitwise equal."""
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=100, batch=1, heads=2, chunk_size=32)
    x = synth.make_inputs(s, seed=33)
    x["shared"] = x["bank"][0].copy()
    print("shared bank B=1", flush=True)
    priv = run_gpu(s, x)
    shr = run_gpu_shared(s, x)
    for u, v in zip(priv, shr):
        assert np.array_equal(u.reshape(v.shape), v)


def test_shared_bank_conflict_leaves_bank_and_out_untouched():
    """Random keys over 1024 slots collide across streams: the check fails, SlotConflictError is raised, and neither
    the bank nor out was written. A following disjoint call on the same library state succeeds (the flag and the
    owner table start clear on every call)."""
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=64, batch=2, heads=2, chunk_size=32)
    x = synth.make_inputs(s, seed=34)
    x["shared"] = x["bank"][0].copy()
    ref = oracle.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                            s.widths, s.num_writes, s.num_reads)
    a = set(ref["widx"][0, :, 0].ravel()) | set(ref["ridx"][0, :, 0].ravel())
    b = set(ref["widx"][1, :, 0].ravel()) | set(ref["ridx"][1, :, 0].ravel())
    assert a & b, "the random streams were expected to share a slot"
    print("shared bank conflict", flush=True)
    at, bt = TORCH_DT[s.act], TORCH_DT[s.bank]
    t = {k: to_dev(x[k], at) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    g_bank = to_dev(x["shared"], bt)
    before = g_bank.clone()
    out = torch.full((s.batch, s.tokens, s.heads, s.head_dim), SENTINEL, dtype=at, device=DEV)
    with pytest.raises(binding.SlotConflictError):
        binding.sdm_write_read(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], g_bank,
                               widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
                               chunk_size=s.chunk_size, out=out, shared_bank=True)
    torch.cuda.synchronize()
    assert torch.equal(g_bank, before)
    assert bool((out == SENTINEL).all())
    s2 = synth.Shape(2, 40, 2, (32, 32), 8, 64, 8, 8, 16, name="shared_after")
    x2 = _disjoint_streams(s2, seed=35)
    check_parity(s2, run_gpu_shared(s2, x2), oracle_shared(s2, x2))


def test_write_read_bitwise_repeatable():
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=192, batch=2, heads=2)
    x = synth.make_inputs(s, seed=9)
    a = run_gpu(s, x)
    b = run_gpu(s, x)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_write_read_split_at_chunk_multiple_is_bitwise():
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=256, chunk_size=32)
    x = synth.make_inputs(s, seed=10)
    full = run_gpu(s, x)
    h = 96
    first = {k: (v[:, :h] if k in ("wkeys", "rq", "values", "alpha", "beta") else v) for k, v in x.items()}
    second = {k: (v[:, h:] if k in ("wkeys", "rq", "values", "alpha", "beta") else v) for k, v in x.items()}
    o1, b1, w1, r1 = run_gpu(s.with_(tokens=h), first)
    o2, b2, w2, r2 = run_gpu(s.with_(tokens=256 - h), second, bank=b1)
    assert np.array_equal(np.concatenate([o1, o2], 1), full[0])
    assert np.array_equal(b2, full[1])
    assert np.array_equal(np.concatenate([w1, w2], 1), full[2])


PIPE_CASES = [
    # four streams of 512-byte bf16 rows (the narrow loop's 128 workgroups), three factors, chunk 128
    ("narrow_3f", synth.Shape(1, 1024, 4, (64, 32, 32), 32, 256, 64, 64, 128, "bf16", "bf16", name="pipe_narrow")),
    # two batch rows (windows of whole 16-token multiples), float32 bank on the held-row loop, chunk 32
    ("held_b2", synth.Shape(2, 320, 2, (16, 16), 16, 64, 16, 16, 32, "bf16", "f32", name="pipe_held")),
    # one batch row, chunk 7 (segmented loop) with a ragged last chunk
    ("segmented_c7", synth.Shape(1, 100, 2, (16, 16), 8, 48, 8, 8, 7, "f32", "f32", name="pipe_seg")),
]


@pytest.mark.parametrize("name,s", PIPE_CASES, ids=[c[0] for c in PIPE_CASES])
def test_write_read_pipelined_equals_chunk_calls(name, s):
    """Calls whose chunk loop leaves most compute units free run as pieces, the top-k and plan of the next piece
    beside the loop of this one on a second stream: bitwise equal to one call per chunk (each run in order), and
    within the oracle's tolerance."""
    x = synth.make_inputs(s, seed=61)
    print(f"write/read pipelined {name}", flush=True)
    full = run_gpu(s, x)
    check_parity(s, full, run_oracle(s, x))
    outs, widx, ridx = [], [], []
    bank = None
    for t0 in range(0, s.tokens, s.chunk_size):
        t1 = min(s.tokens, t0 + s.chunk_size)
        part = {k: (np.ascontiguousarray(v[:, t0:t1]) if k in ("wkeys", "rq", "values", "alpha", "beta") else v)
                for k, v in x.items()}
        o, bank, w, r = run_gpu(s.with_(tokens=t1 - t0), part, bank=bank)
        outs.append(o)
        widx.append(w)
        ridx.append(r)
    assert np.array_equal(np.concatenate(outs, 1), full[0])
    assert np.array_equal(bank, full[1])
    assert np.array_equal(np.concatenate(widx, 1), full[2])
    assert np.array_equal(np.concatenate(ridx, 1), full[3])


def test_write_read_pipelined_from_two_threads():
    """Two host threads, each with its own stream, workspace and bank, run pipelined calls at the same time (the
    library's side stream is shared; a call enqueues its pieces under a lock): every result equals the same calls
    run one after another."""
    import threading
    s = PIPE_CASES[0][1].with_(tokens=512)
    jobs = []
    for seed in (63, 64):
        x = synth.make_inputs(s, seed=seed)
        t = {k: to_dev(x[k], torch.bfloat16) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
        jobs.append((t, to_dev(x["bank"], torch.bfloat16)))
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, chunk_size=s.chunk_size)
    print("write/read pipelined from two threads", flush=True)

    def calls(t, bank, n):
        outs = []
        for _ in range(n):
            o, _, _ = binding.sdm_write_read(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"],
                                             bank, **kw)
            outs.append(o)
        return outs

    ref = []
    for t, bank0 in jobs:  # one after another, on the current stream
        bank = bank0.clone()
        outs = calls(t, bank, 3)
        torch.cuda.synchronize()
        ref.append(([to_np(o) for o in outs], to_np(bank)))
    got = [None, None]

    def worker(i):
        t, bank0 = jobs[i]
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            bank = bank0.clone()
            outs = calls(t, bank, 3)
        st.synchronize()
        got[i] = ([to_np(o) for o in outs], to_np(bank))

    torch.cuda.synchronize()
    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    for i in range(2):
        assert got[i] is not None, f"thread {i} failed"
        for a, b in zip(got[i][0], ref[i][0]):
            assert np.array_equal(a, b)
        assert np.array_equal(got[i][1], ref[i][1])


def test_write_read_two_million_slots():
    """2,097,152 slots (factors 1024 x 2048): a slot id and an event index need more than 32 bits together, so the
    chunk plan sorts its events with 64-bit keys (bitonic) instead of the 32-bit radix sort; parity with the oracle."""
    s = synth.Shape(1, 96, 1, (1024, 2048), 16, 16, 8, 8, 32, "f32", "f32", name="slots_2m")
    x = synth.make_inputs(s, seed=62)
    print("write/read 2,097,152 slots", flush=True)
    check_parity(s, run_gpu(s, x), run_oracle(s, x))


@pytest.mark.parametrize("W,R", [(64, 40), (24, 200)])
def test_write_read_filtered_kinds_differ(W, R):
    """bf16 write/read on 1024-sub-key factors (the filtered top-k in block mode) with different write and read k:
    the two kinds' workgroups lay out their score rows and selection buffers differently in one launch (k 200 leaves
    the buffers outside the rows); parity with the oracle."""
    s = synth.Shape(2, 48, 2, (1024, 32), 64, 64, W, R, 16, "bf16", "f32", name="filtered_kinds")
    x = synth.make_inputs(s, seed=63)
    print(f"write/read filtered W={W} R={R}", flush=True)
    check_parity(s, run_gpu(s, x), run_oracle(s, x))


def test_write_read_split_off_the_chunk_grid():
    """Resume at a token that is not a multiple of chunk_size: the chunk grid restarts at the second call, so the
    result may differ from one call only by rounding (chunk size changes results only through rounding); both match
    the oracle, and the ids are exactly one call's."""
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=256, chunk_size=32)
    x = synth.make_inputs(s, seed=65)
    full = run_gpu(s, x)
    h = 100
    first = {k: (np.ascontiguousarray(v[:, :h]) if k in ("wkeys", "rq", "values", "alpha", "beta") else v)
             for k, v in x.items()}
    second = {k: (np.ascontiguousarray(v[:, h:]) if k in ("wkeys", "rq", "values", "alpha", "beta") else v)
              for k, v in x.items()}
    o1, b1, w1, r1 = run_gpu(s.with_(tokens=h), first)
    o2, b2, w2, r2 = run_gpu(s.with_(tokens=256 - h), second, bank=b1)
    split = (np.concatenate([o1, o2], 1), b2, np.concatenate([w1, w2], 1), np.concatenate([r1, r2], 1))
    assert np.array_equal(split[2], full[2]) and np.array_equal(split[3], full[3])
    ref = run_oracle(s, x)
    check_parity(s, split, ref)
    check_parity(s, full, ref)


def test_write_read_empty_tokens():
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=0)
    x = synth.make_inputs(s)
    out, bank, widx, ridx = run_gpu(s, x)
    assert out.shape[1] == 0 and np.array_equal(bank, x["bank"])


# ------------------------------------------------------------------------------------------------ decode
def _decode_inputs(s, step):
    x = synth.make_step_inputs(s, seed=0, step=step)
    return {k: to_dev(v, TORCH_DT[s.act]) for k, v in x.items()}, x


@pytest.mark.parametrize("bank_dt", ["f32", "bf16"])
def test_decode_matches_oracle_and_donated_equals_copied(bank_dt):
    s = synth.WORKLOADS["decode_b128"].with_(batch=16, bank=bank_dt)
    sub_np = synth.make_subkeys(s)
    bank_np = synth.make_bank(s)
    sub = to_dev(sub_np, TORCH_DT[s.act])
    bank_d = to_dev(bank_np, TORCH_DT[bank_dt])   # donated chain
    bank_c = bank_d.clone()                         # copied chain
    ref_bank = bank_np
    print(f"decode bank={bank_dt}", flush=True)
    for step in range(6):
        t, x = _decode_inputs(s, step)
        args = (t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], sub)
        kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, want_index=True)
        od, wd, rd, bd = binding.sdm_decode_step(*args, bank_d, **kw)
        succ = torch.empty_like(bank_c)
        prev = bank_c.clone()
        oc, wc, rc, bc = binding.sdm_decode_step(*args, bank_c, succ, **kw)
        torch.cuda.synchronize()
        assert bd.data_ptr() == bank_d.data_ptr()          # in place
        assert torch.equal(bank_c, prev)                    # predecessor untouched
        assert torch.equal(od, oc) and torch.equal(wd, wc) and torch.equal(rd, rc)
        assert torch.equal(bd, bc)
        bank_c = bc
        ref = oracle.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], sub_np, ref_bank,
                                s.widths, s.num_writes, s.num_reads, bank_bf16=bank_dt == "bf16")
        assert np.array_equal(wd.cpu().numpy(), ref["widx"]) and np.array_equal(rd.cpu().numpy(), ref["ridx"])
        # out is read from bank rows: the coarser of the two tolerances, as in check_parity
        assert rowwise_rel(to_np(od), ref["out"]) <= max(RTOL[s.act], RTOL[bank_dt])
        assert rowwise_rel(to_np(bd), ref["bank"]) <= RTOL[bank_dt]
        ref_bank = ref["bank"]


DECODE_SHAPES = [
    # head_dim, W, R, widths, dk, act, bank: the one-launch step (W, R <= 64, <= 256 sub-keys per factor) with a
    # partial column pass, two column passes and 256-wide factors; the two-kernel step beyond those limits
    (64, 16, 24, (16, 16), 8, "f32", "f32"),
    (1024, 32, 32, (32, 32), 16, "bf16", "bf16"),
    (128, 64, 64, (256, 256), 16, "bf16", "f32"),
    (256, 128, 96, (32, 32), 16, "f32", "f32"),
    (128, 64, 64, (512, 64), 16, "bf16", "f32"),
]


@pytest.mark.parametrize("d,W,R,widths,dk,act,bank", DECODE_SHAPES)
def test_decode_shapes(d, W, R, widths, dk, act, bank):
    s = synth.Shape(4, 1, 2, widths, dk, d, W, R, 1, act, bank, name="decode_shape")
    sub_np = synth.make_subkeys(s, seed=14)
    sub = to_dev(sub_np, TORCH_DT[act])
    ref_bank = synth.make_bank(s, seed=14)
    bank_d = to_dev(ref_bank, TORCH_DT[bank])
    bank_c = bank_d.clone()
    print(f"decode d={d} W={W} R={R} widths={widths} act={act} bank={bank}", flush=True)
    for step in range(3):
        x = synth.make_step_inputs(s, seed=14, step=step)
        t = {k: to_dev(v, TORCH_DT[act]) for k, v in x.items()}
        args = (t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], sub)
        kw = dict(widths=widths, num_writes=W, num_reads=R, want_index=True)
        od, wd, rd, bd = binding.sdm_decode_step(*args, bank_d, **kw)
        succ = torch.empty_like(bank_c)
        oc, wc, rc, bc = binding.sdm_decode_step(*args, bank_c, succ, **kw)
        torch.cuda.synchronize()
        assert torch.equal(od, oc) and torch.equal(wd, wc) and torch.equal(rd, rc) and torch.equal(bd, bc)
        bank_c = bc
        ref = oracle.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], sub_np, ref_bank,
                                widths, W, R, bank_bf16=bank == "bf16", act_bf16=act == "bf16")
        assert np.array_equal(wd.cpu().numpy(), ref["widx"]) and np.array_equal(rd.cpu().numpy(), ref["ridx"])
        assert rowwise_rel(to_np(od), ref["out"]) <= max(RTOL[act], RTOL[bank])
        assert rowwise_rel(to_np(bd), ref["bank"]) <= RTOL[bank]
        ref_bank = ref["bank"]


def test_prepared_decode_step_equals_decode_step():
    """binding.DecodeStep (config and workspace made once) gives the bits of sdm_decode_step, donated and copied."""
    s = synth.WORKLOADS["decode_b128"].with_(batch=8)
    sub = to_dev(synth.make_subkeys(s, seed=15), torch.float32)
    bank0 = to_dev(synth.make_bank(s, seed=15), torch.float32)
    step = binding.DecodeStep(s.batch, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes, s.num_reads,
                              torch.float32, torch.float32, s.rows, DEV)
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads)
    b_ref, b_new, b_cp = bank0.clone(), bank0.clone(), bank0.clone()
    print("prepared decode step", flush=True)
    for i in range(3):
        x = synth.make_step_inputs(s, seed=15, step=i)
        t = {k: to_dev(v, torch.float32) for k, v in x.items()}
        args = (t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], sub)
        o_ref, _, _, _ = binding.sdm_decode_step(*args, b_ref, **kw)
        o_new = step(*args, b_new)
        succ = torch.empty_like(b_cp)
        o_cp = step(*args, b_cp, succ)
        b_cp = succ
        torch.cuda.synchronize()
        assert torch.equal(o_ref, o_new) and torch.equal(o_ref, o_cp)
        assert torch.equal(b_ref, b_new) and torch.equal(b_ref, b_cp)


def test_decode_graph_replay_equals_eager():
    """Decode steps captured into a HIP graph (the C ABI allocates nothing and never synchronises) replay to the
    same bits as the eager calls; several replays with eager work and synchronisations between them."""
    s = synth.WORKLOADS["decode_b128"].with_(batch=8)
    sub = to_dev(synth.make_subkeys(s), torch.float32)
    bank0 = to_dev(synth.make_bank(s), torch.float32)
    steps = [_decode_inputs(s, i)[0] for i in range(4)]
    cfg = binding.make_config(s.batch, 1, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes, s.num_reads, 1)
    ws = torch.empty(binding.workspace_size(cfg, binding.SDM_OP_DECODE), dtype=torch.uint8, device=DEV)
    bank = bank0.clone()
    out = torch.empty((s.batch, 1, s.heads, s.head_dim), dtype=torch.float32, device=DEV)
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, out=out, workspace=ws)

    def run(lo, hi):
        for t in steps[lo:hi]:
            binding.sdm_decode_step(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], sub, bank, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(0, 1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(1, 4)
    bank.copy_(bank0)
    run(1, 4)
    torch.cuda.synchronize()
    ref_out, ref_bank = out.clone(), bank.clone()
    for rep in range(3):
        bank.copy_(bank0)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(bank, ref_bank), f"replay {rep} differs"
        run(0, 1)  # eager work between replays
        torch.cuda.synchronize()


def test_write_read_graph_replay_equals_eager():
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=160, batch=2, heads=2, chunk_size=32, act="bf16")
    x = synth.make_inputs(s, seed=15)
    t = {k: to_dev(x[k], torch.bfloat16) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    bank0 = to_dev(x["bank"], torch.float32)
    cfg = binding.make_config(s.batch, s.tokens, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes,
                              s.num_reads, s.chunk_size, binding.SDM_BF16, binding.SDM_F32)
    ws = torch.empty(binding.workspace_size(cfg, binding.SDM_OP_WRITE_READ), dtype=torch.uint8, device=DEV)
    bank = bank0.clone()
    out = torch.empty((s.batch, s.tokens, s.heads, s.head_dim), dtype=torch.bfloat16, device=DEV)

    def run():
        binding.sdm_write_read(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                               widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
                               chunk_size=s.chunk_size, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    bank.copy_(bank0)
    run()
    torch.cuda.synchronize()
    ref_out, ref_bank = out.clone(), bank.clone()
    for rep in range(3):
        bank.copy_(bank0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(bank, ref_bank), f"replay {rep} differs"
        run()  # eager work between replays (advances the bank)
        torch.cuda.synchronize()


def test_decode_padded_pitch_donated_equals_copied():
    s = synth.WORKLOADS["decode_b128"].with_(batch=8)
    x = synth.make_inputs(s, seed=13)
    t = {k: to_dev(x[k], torch.float32) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, want_index=True)
    args = (t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"])
    b_don = padded_bank(x["bank"], torch.float32, 288)
    b_in = padded_bank(x["bank"], torch.float32, 288)
    b_out = binding.alloc_bank(s.batch, s.heads, s.rows, s.head_dim, torch.float32, DEV, pitch=288)
    o1, w1, r1, _ = binding.sdm_decode_step(*args, b_don, **kw)
    o2, w2, r2, _ = binding.sdm_decode_step(*args, b_in, b_out, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(b_don, b_out) and torch.equal(w1, w2)
    ref = oracle.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                            s.widths, s.num_writes, s.num_reads)
    assert np.array_equal(w1.cpu().numpy(), ref["widx"]) and np.array_equal(r1.cpu().numpy(), ref["ridx"])
    assert rowwise_rel(to_np(o1), ref["out"]) <= 1e-5
    assert rowwise_rel(to_np(b_don), ref["bank"]) <= 1e-5
    assert bool((b_don._base[..., s.head_dim:] == SENTINEL).all())


def test_decode_equals_one_token_write_read():
    s = synth.WORKLOADS["tiny_1k"].with_(tokens=1, batch=3, heads=2)
    x = synth.make_inputs(s, seed=11)
    o1, b1, w1, r1 = run_gpu(s, x)
    t = {k: to_dev(x[k], torch.float32) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    bank = to_dev(x["bank"], torch.float32)
    out, widx, ridx, _ = binding.sdm_decode_step(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"],
                                                 t["subkeys"], bank, widths=s.widths, num_writes=s.num_writes,
                                                 num_reads=s.num_reads, want_index=True)
    torch.cuda.synchronize()
    assert np.array_equal(widx.cpu().numpy(), w1) and np.array_equal(ridx.cpu().numpy(), r1)
    assert rowwise_rel(to_np(out), o1) <= 1e-5
    assert rowwise_rel(to_np(bank), b1) <= 1e-5


# ------------------------------------------------------------------------------------------------ full size
def test_layer_65k_full_size():
    """The 65,536-slot layer workload (B 2, T 4096, H 2, d 1024, W = R = 64, chunk 64, bf16 on a float32 bank),
    every output row and every bank row against the oracle."""
    s = synth.WORKLOADS["layer_65k"]
    print("full-size layer_65k: generating inputs", flush=True)
    x = synth.make_inputs(s)
    print("full-size layer_65k: GPU", flush=True)
    gpu = run_gpu(s, x, pitch=binding.bank_pitch(s.head_dim, torch.float32))
    print("full-size layer_65k: oracle", flush=True)
    ref = run_oracle(s, x)
    e = check_parity(s, gpu, ref)
    print("full-size layer_65k errors", e, flush=True)


def _sub(x, lo, hi):
    """Per-token inputs restricted to tokens [lo, hi)."""
    return {k: (v[:, lo:hi] if k in ("wkeys", "rq", "values", "alpha", "beta") else v) for k, v in x.items()}


def _err_summary(got, ref):
    """Row-wise relative errors: (max, 99.9th percentile, rows above 1e-2) for a diagnostic line."""
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    e = np.abs(got - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float(e.max()), float(np.quantile(e, 0.999)), int((e > 1e-2).sum())


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_three_factor_65k_full_size():
    """Three-factor workload at full size (B 1, T 32768, H 4, d 256, factors 64 x 32 x 32, W = R = 64, chunk 128,
    bf16 activations on a bf16 bank), the whole sequence against the oracle: every write and read id, every output
    row and every final bank row; and a run split at token 2048 equal bit for bit to one run."""
    s = synth.WORKLOADS["three_factor_65k"]
    P = 2048
    print("full-size three_factor_65k: generating inputs", flush=True)
    x = synth.make_inputs(s)
    print("full-size three_factor_65k: GPU, whole sequence", flush=True)
    out, bank, widx, ridx = run_gpu(s, x)
    print("full-size three_factor_65k: oracle, whole sequence (4 streams)", flush=True)
    ref = run_oracle(s, x)
    print("full-size three_factor_65k: out (max, p99.9, rows > 1e-2)", _err_summary(out, ref["out"]),
          "bank", _err_summary(bank, ref["bank"]), flush=True)
    e_out, e_bank = check_parity(s, (out, bank, widx, ridx), ref)
    print("full-size three_factor_65k: GPU prefix and remainder", flush=True)
    sp = s.with_(tokens=P)
    out_p, bank_p, _, _ = run_gpu(sp, _sub(x, 0, P))
    assert np.array_equal(out_p, out[:, :P])
    out_r, bank_r, _, _ = run_gpu(s.with_(tokens=s.tokens - P), _sub(x, P, s.tokens), bank=bank_p)
    assert np.array_equal(out_r, out[:, P:]) and np.array_equal(bank_r, bank)
    print("full-size three_factor_65k errors", e_out, e_bank, flush=True)


@pytest.mark.slow
def test_large_1m_full_size():
    """1,048,576-slot workload at full size (B 4, T 8192, H 4, d 512, W = R = 64, chunk 64, bf16 on a 32 GiB float32
    bank, padded pitch, int64 offsets). Oracle on the first 256 tokens of batch row 0 (its 4 streams); at full
    size: a run split at token 256 equal bit for bit to one run, sampled ids against the oracle's top-k."""
    s = synth.WORKLOADS["large_1m"]
    P = 256
    at = torch.bfloat16
    pitch = binding.bank_pitch(s.head_dim, torch.float32)
    print("full-size large_1m: generating inputs", flush=True)
    x = synth.make_step_inputs(s)
    x["subkeys"] = synth.make_subkeys(s)
    t = {k: to_dev(x[k], at) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, chunk_size=s.chunk_size)

    def call(bank, lo, hi):
        out, wi, ri = binding.sdm_write_read(*(t[k][:, lo:hi].contiguous() for k in ("wkeys", "rq", "values",
                                                                                      "alpha", "beta")),
                                             t["subkeys"], bank, want_index=True, **kw)
        torch.cuda.synchronize()
        return out, wi, ri

    bank = binding.alloc_bank(s.batch, s.heads, s.rows, s.head_dim, torch.float32, DEV, pitch=pitch)
    synth.fill_bank_device(bank, s)
    print("full-size large_1m: GPU, whole sequence", flush=True)
    out, widx, ridx = call(bank, 0, s.tokens)
    print("full-size large_1m: split run", flush=True)
    bank2 = binding.alloc_bank(s.batch, s.heads, s.rows, s.head_dim, torch.float32, DEV, pitch=pitch)
    synth.fill_bank_device(bank2, s)
    out_p, wp, rp = call(bank2, 0, P)
    assert torch.equal(out_p, out[:, :P]) and torch.equal(wp, widx[:, :P]) and torch.equal(rp, ridx[:, :P])
    # the rows the prefix wrote in batch row 0, for the oracle comparison
    touched = [torch.unique(wp[0, :, h].reshape(-1).long()) for h in range(s.heads)]
    got_rows = [bank2[0, h][touched[h]].float().cpu().numpy() for h in range(s.heads)]
    out_r, _, _ = call(bank2, P, s.tokens)
    assert torch.equal(out_r, out[:, P:]), "split run outputs differ"
    assert torch.equal(bank2, bank), "split run bank differs"
    del bank2, out_r
    print("full-size large_1m: oracle on the prefix of batch row 0", flush=True)
    b0 = np.empty((1, s.heads, s.rows, s.head_dim), np.float32)
    tmp = torch.empty((s.rows, s.head_dim), dtype=torch.float32, device=DEV)
    for h in range(s.heads):
        synth.fill_bank_stream_device(tmp, s, 0, h)
        b0[0, h] = tmp.cpu().numpy()
    del tmp
    xp = {k: x[k][0:1, :P] for k in ("wkeys", "rq", "values", "alpha", "beta")}
    ref = oracle.write_read(xp["wkeys"], xp["rq"], xp["values"], xp["alpha"], xp["beta"], x["subkeys"], b0,
                            s.widths, s.num_writes, s.num_reads, act_bf16=True)
    assert np.array_equal(to_np(widx[0:1, :P]), ref["widx"]) and np.array_equal(to_np(ridx[0:1, :P]), ref["ridx"])
    e_out = rowwise_rel(to_np(out[0:1, :P]), ref["out"])
    assert e_out <= RTOL["bf16"], f"out rel err {e_out}"
    e_bank = max(rowwise_rel(got_rows[h], ref["bank"][0, h][touched[h].cpu().numpy()]) for h in range(s.heads))
    assert e_bank <= RTOL["f32"], f"prefix bank rel err {e_bank}"
    rng = np.random.default_rng(6)
    ts = np.sort(rng.choice(s.tokens, 16, replace=False))
    rid, _ = oracle.topk(x["wkeys"][:, ts], x["subkeys"], s.widths, s.num_writes)
    assert np.array_equal(to_np(widx[:, ts]), rid), "sampled write ids differ"
    print("full-size large_1m errors", e_out, e_bank, flush=True)


@pytest.mark.parametrize("kind", ["ternary", "zero_query"])
def test_decode_exact_ties(kind):
    """Decode steps whose slot scores tie exactly (ternary queries and sub-keys; or all-zero queries, where every
    slot scores 0 and the order is by position sums): the one-launch step's merge (radix select started below the
    high bits shared by the keys it can select, tie branch on the low halves) must give the oracle's ids."""
    s = synth.WORKLOADS["decode_b128"].with_(batch=8)
    rng = np.random.default_rng(21 if kind == "ternary" else 22)
    F = len(s.widths)
    sub_np = rng.integers(-1, 2, (s.heads, sum(s.widths), s.subkey_dim)).astype(np.float32)
    sub = to_dev(sub_np, torch.float32)
    bank_np = synth.make_bank(s)
    bank = to_dev(bank_np, torch.float32)
    shape = (s.batch, 1, s.heads, F * s.subkey_dim)
    if kind == "ternary":
        wk = rng.integers(-1, 2, shape).astype(np.float32)
        rq = rng.integers(-1, 2, shape).astype(np.float32)
    else:
        wk = np.zeros(shape, np.float32)
        rq = np.zeros(shape, np.float32)
    x = synth.make_step_inputs(s, seed=5, step=1)
    x["wkeys"], x["rq"] = wk, rq
    t = {k: to_dev(v, torch.float32) for k, v in x.items()}
    o, w, r, b = binding.sdm_decode_step(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], sub, bank,
                                         widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
                                         want_index=True)
    torch.cuda.synchronize()
    ref = oracle.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], sub_np, bank_np, s.widths,
                            s.num_writes, s.num_reads)
    assert np.array_equal(w.cpu().numpy(), ref["widx"]) and np.array_equal(r.cpu().numpy(), ref["ridx"])
    assert rowwise_rel(to_np(o), ref["out"]) <= RTOL["f32"]
    assert rowwise_rel(to_np(b), ref["bank"]) <= RTOL["f32"]


# ------------------------------------------------------------------------------------------------ multi-step decode
STEPS_SHAPES = [  # d, W, R, widths, dk, act, bank, batch
    (256, 64, 64, (32, 32), 32, "f32", "f32", 8),     # the decode workload's shapes (8 streams of 128)
    (512, 48, 40, (32, 16), 16, "bf16", "f32", 3),    # two column passes, W != R
    (256, 64, 64, (16, 8, 8), 16, "bf16", "bf16", 4), # three factors, bf16 bank
    (64, 7, 64, (64, 4), 8, "f32", "f32", 5),         # partial column pass, few writes
]


@pytest.mark.parametrize("d,W,R,widths,dk,act,bank,batch", STEPS_SHAPES)
def test_decode_steps_equal_sequential_steps(d, W, R, widths, dk, act, bank, batch):
    """sdm_decode_steps over K tokens equals K sdm_decode_step calls bit for bit (out, ids, bank; donated and
    copied), and the oracle's recurrence over the K tokens within tolerance with ids exact."""
    K = 12
    s = synth.Shape(batch, K, 2, widths, dk, d, W, R, 1, act, bank, name="steps")
    x = synth.make_inputs(s, seed=71)
    at, bt = TORCH_DT[act], TORCH_DT[bank]
    t = {k: to_dev(x[k], at) for k in ("wkeys", "rq", "values", "alpha", "beta")}
    sub = to_dev(x["subkeys"], at)
    kw = dict(widths=widths, num_writes=W, num_reads=R)
    print(f"decode steps d={d} W={W} R={R} widths={widths} {act}/{bank} B={batch} K={K}", flush=True)
    b_seq = to_dev(x["bank"], bt)
    outs, wis, ris = [], [], []
    for k in range(K):
        one = {n: v[:, k:k + 1].contiguous() for n, v in t.items()}
        o, wi, ri, _ = binding.sdm_decode_step(one["wkeys"], one["rq"], one["values"], one["alpha"], one["beta"],
                                               sub, b_seq, want_index=True, **kw)
        outs.append(o)
        wis.append(wi)
        ris.append(ri)
    b_don = to_dev(x["bank"], bt)
    o_don, w_don, r_don, _ = binding.sdm_decode_steps(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], sub,
                                                      b_don, want_index=True, **kw)
    b_in = to_dev(x["bank"], bt)
    b_out = torch.empty_like(b_in)
    o_cp, _, _, _ = binding.sdm_decode_steps(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], sub, b_in,
                                             b_out, **kw)
    torch.cuda.synchronize()
    seq_out = torch.cat(outs, dim=1)
    assert torch.equal(o_don, seq_out), "multi-step out differs from sequential steps"
    assert torch.equal(w_don, torch.cat(wis, dim=1)) and torch.equal(r_don, torch.cat(ris, dim=1))
    assert torch.equal(b_don, b_seq), "multi-step bank differs from sequential steps"
    assert torch.equal(o_cp, seq_out) and torch.equal(b_out, b_seq), "copied multi-step differs"
    assert torch.equal(b_in, to_dev(x["bank"], bt)), "copied multi-step changed bank_in"
    ref = run_oracle(s, x)
    assert np.array_equal(to_np(w_don), ref["widx"]) and np.array_equal(to_np(r_don), ref["ridx"])
    assert rowwise_rel(to_np(o_don), ref["out"]) <= max(RTOL[act], RTOL[bank])
    assert rowwise_rel(to_np(b_don), ref["bank"]) <= RTOL[bank]


def test_decode_steps_zero_steps_and_graph_replay():
    """K = 0 does nothing; a captured multi-step call replays to the eager bits."""
    s = synth.WORKLOADS["decode_b128"].with_(batch=4, tokens=6)
    x = synth.make_inputs(s, seed=72)
    t = {k: to_dev(x[k], torch.float32) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads)
    bank0 = to_dev(x["bank"], torch.float32)
    bank = bank0.clone()
    z = {k: v[:, :0].contiguous() for k, v in t.items() if k != "subkeys"}
    binding.sdm_decode_steps(z["wkeys"], z["rq"], z["values"], z["alpha"], z["beta"], t["subkeys"], bank, **kw)
    torch.cuda.synchronize()
    assert torch.equal(bank, bank0)
    cfg = binding.make_config(s.batch, s.tokens, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes,
                              s.num_reads, 1, binding.SDM_F32, binding.SDM_F32, s.rows)
    ws = torch.empty(binding.workspace_size(cfg, binding.SDM_OP_DECODE_STEPS), dtype=torch.uint8, device=DEV)
    out = torch.empty((s.batch, s.tokens, s.heads, s.head_dim), device=DEV)

    def run():
        binding.sdm_decode_steps(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                 out=out, workspace=ws, **kw)

    run()
    torch.cuda.synchronize()
    ref_out, ref_bank = out.clone(), bank.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bank.copy_(bank0)
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        bank.copy_(bank0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(bank, ref_bank), f"replay {rep} differs"
        run()  # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------------------------------------------------ large chunks
def test_chunk_256_and_above_the_kernels_chunk():
    """chunk_size 256 (the 7B configuration's) runs as two chunks of 128 with W = 64: the result equals the oracle
    within tolerance and chunk 128's bit for bit; chunk 200 (sub-chunks of 100) equals the oracle, and a call split
    at token 200 gives the bits of one call."""
    s = synth.Shape(2, 600, 2, (32, 32), 16, 64, 64, 64, 256, name="c256")
    x = synth.make_inputs(s, seed=81)
    print("chunk 256 / 128 / 200", flush=True)
    g256 = run_gpu(s, x)
    g128 = run_gpu(s, x, chunk_size=128)
    for a, b in zip(g256, g128):
        assert np.array_equal(a, b), "chunk 256 differs from chunk 128"
    check_parity(s, g256, run_oracle(s, x))
    s200 = s.with_(chunk_size=200)
    g200 = run_gpu(s200, x)
    check_parity(s200, g200, run_oracle(s200, x))
    head = s200.with_(tokens=200)
    o1, b1, w1, r1 = run_gpu(head, _sub(x, 0, 200))
    o2, b2, w2, r2 = run_gpu(s200.with_(tokens=400), _sub(x, 200, 600), bank=b1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), g200[0]) and np.array_equal(b2, g200[1])
