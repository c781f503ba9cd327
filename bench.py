#!/usr/bin/env python
"""SDM benchmark on one MI355X: write/read tokens/s on the 65,536-slot layer workload, decode steps/s at B = 128,
the chunk-loop kernel against the HBM roofline, and the CPU oracle timed beside it.

One step = one sdm_write_read call over the whole batch of the layer workload (B 2 x T 4096 tokens, 2 heads of
1024, 2 factors of 256 sub-keys = 65,536 slots per head, W = R = 64, chunk 64, bf16 activations on a float32 bank),
inputs resident in HBM before the timed region; the bank advances in place from step to step.
Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SDM write/read tokens/s (65536 slots, W=R=64) + decode steps/s at B=128; % HBM roofline"
HBM_PEAK_GBS = 8000.0
PMC_SUMMARY = os.path.join(ROOT, "profiles", "loop_kernel_layer_65k_pmc.txt")
LOOP_SOURCES = ("gated_delta_rule_product_amd/csrc/loop.hip", "gated_delta_rule_product_amd/csrc/sdm_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def loop_sources_sha() -> str:
    h = hashlib.sha256()
    for p in LOOP_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_counters():
    """HBM bytes per chunk-loop launch from the committed rocprofv3 counter summary, if it was taken on the
    current loop-kernel sources (else None)."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    vals = {}
    with open(PMC_SUMMARY) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256") != loop_sources_sha():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def loop_algorithmic_bytes(s, token_heads):
    """Bytes the chunk loop must move per launch: per token-head, W bank rows read and written and R bank rows read
    ((2W + R) d bank elements), the value row read and the output row written (2 d act elements), 2 gates."""
    sb = 2 if s.bank == "bf16" else 4
    sa = 2 if s.act == "bf16" else 4
    return token_heads * ((2 * s.num_writes + s.num_reads) * s.head_dim * sb + 2 * s.head_dim * sa + 2 * sa)


def bwd_algorithmic_bytes(s, token_heads):
    """Bytes the backward must move per call with a float32 snapshot and float32 gradients: per token-head, the read
    rows of the bank and of the adjoint bank, the adjoint rows and snapshot rows of the write terms, loaded; the read
    rows' and write rows' adjoint rows and the restored bank rows, stored ((3R + 4W) d elements with the bank's rows at
    the bank dtype); the output gradient and the values read and their gradient written."""
    sb = 2 if s.bank == "bf16" else 4
    sa = 2 if s.act == "bf16" else 4
    W, R, d = s.num_writes, s.num_reads, s.head_dim
    rows = R * d * (sb + 4) + W * d * (4 + 4) + R * d * 4 + W * d * (4 + sb)
    return token_heads * (rows + 2 * d * sa + d * 4)


def bench_write_read(args, torch, binding, synth):
    s = synth.WORKLOADS["layer_65k"]
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    dev = torch.device("cuda:0")
    log(f"[bench] generating {s.name} inputs")
    x = synth.make_inputs(s)
    t = {k: torch.from_numpy(x[k]).to(dev).to(dt[s.act]) for k in ("wkeys", "rq", "values", "alpha", "beta",
                                                                    "subkeys")}
    pitch = binding.bank_pitch(s.head_dim, dt[s.bank])
    bank = binding.alloc_bank(s.batch, s.heads, s.rows, s.head_dim, dt[s.bank], dev, pitch=pitch)
    bank.copy_(torch.from_numpy(x["bank"]).to(dev).to(dt[s.bank]))
    del x
    cfg = binding.make_config(s.batch, s.tokens, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes,
                              s.num_reads, s.chunk_size, binding.SDM_BF16 if s.act == "bf16" else binding.SDM_F32,
                              binding.SDM_BF16 if s.bank == "bf16" else binding.SDM_F32, s.rows, pitch)
    ws = torch.empty(binding.workspace_size(cfg, binding.SDM_OP_WRITE_READ), dtype=torch.uint8, device=dev)
    out = torch.empty((s.batch, s.tokens, s.heads, s.head_dim), dtype=dt[s.act], device=dev)

    def step():
        binding.sdm_write_read(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                               widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
                               chunk_size=s.chunk_size, out=out, workspace=ws)

    log(f"[bench] write/read warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] write/read timed {args.steps}")
    binding.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = binding.profile_read()
    binding.profile_enable(False)
    ms_step = (t1 - t0) * 1e3 / args.steps
    tokens = s.batch * s.tokens
    kernels = {k: round(v[0] / v[1], 4) for k, v in prof.items() if v[1]}
    loop_ms = prof["loop"][0] / prof["loop"][1]
    # one loop launch per call here (the loop's workgroups fill the chip, so the call is not pipelined); were it
    # pipelined, a launch would cover 1/launches of the call's tokens
    alg = loop_algorithmic_bytes(s, s.batch * s.tokens * s.heads) * args.steps // prof["loop"][1]
    achieved = alg / (loop_ms * 1e-3) / 1e9
    traffic = traffic_from_counters()
    roof = {"kernel": "loop_kernel (chunk loop: gather, solve, read, scatter)", "bound": "hbm",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": alg, "avg_launch_ms": round(loop_ms, 4)}
    step_bytes = loop_algorithmic_bytes(s, s.batch * s.tokens * s.heads)  # the loop's bank traffic dominates
    # the same workload on an unpadded bank (row pitch = head_dim), for comparison
    bank_np = torch.empty((s.batch, s.heads, s.rows, s.head_dim), dtype=dt[s.bank], device=dev)
    bank_np.copy_(bank)
    for _ in range(2):
        binding.sdm_write_read(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank_np,
                               widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
                               chunk_size=s.chunk_size, out=out, workspace=ws)
    torch.cuda.synchronize()
    binding.profile_enable(True)
    for _ in range(5):
        binding.sdm_write_read(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank_np,
                               widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
                               chunk_size=s.chunk_size, out=out, workspace=ws)
    torch.cuda.synchronize()
    p2 = binding.profile_read()
    binding.profile_enable(False)
    unpadded_ms = p2["loop"][0] / p2["loop"][1]
    roof["unpadded_pitch_avg_launch_ms"] = round(unpadded_ms, 4)
    # the same bytes against the loop on a dense [B, H, N, d] bank, and against the whole call's wall time (top-k,
    # plan and loop, launches included)
    roof["unpadded_pitch_frac"] = round(alg / (unpadded_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    roof["whole_call_frac"] = round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    del bank_np
    return {
        "tokens_per_s": tokens / (ms_step * 1e-3), "ms_per_step": ms_step, "kernels_avg_ms": kernels,
        "roofline": roof, "shape": s, "pitch": pitch,
    }


def bench_train(args, torch, binding, synth):
    """Training step of the layer workload: the snapshot-saving forward, then the backward (which steps the bank
    back, so every step starts from the same bank). Context line, not the headline value."""
    s = synth.WORKLOADS["layer_65k"]
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    dev = torch.device("cuda:0")
    log("[bench] train: inputs")
    x = synth.make_inputs(s)
    t = {k: torch.from_numpy(x[k]).to(dev).to(dt[s.act]) for k in ("wkeys", "rq", "values", "alpha", "beta",
                                                                    "subkeys")}
    pitch = binding.bank_pitch(s.head_dim, dt[s.bank])
    bank = binding.alloc_bank(s.batch, s.heads, s.rows, s.head_dim, dt[s.bank], dev, pitch=pitch)
    bank.copy_(torch.from_numpy(x["bank"]).to(dev).to(dt[s.bank]))
    del x
    bank0 = bank.clone()
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    gout = torch.randn((s.batch, s.tokens, s.heads, s.head_dim), generator=gen, device=dev).to(dt[s.act])
    gbank = torch.zeros((s.batch, s.heads, s.rows, pitch), dtype=torch.float32, device=dev)[..., :s.head_dim]
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, chunk_size=s.chunk_size)
    out, _, _, snap = binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"],
                                                  t["subkeys"], bank, **kw)
    cfg = binding.make_config(s.batch, s.tokens, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes,
                              s.num_reads, s.chunk_size, binding.SDM_BF16 if s.act == "bf16" else binding.SDM_F32,
                              binding.SDM_BF16 if s.bank == "bf16" else binding.SDM_F32, s.rows, pitch)
    wsf = torch.empty(binding.workspace_size(cfg, binding.SDM_OP_WRITE_READ), dtype=torch.uint8, device=dev)
    wsb = torch.empty(binding.workspace_size(cfg, binding.SDM_OP_BACKWARD), dtype=torch.uint8, device=dev)
    g = binding.sdm_write_read_backward(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                        snap, gout, gbank, workspace=wsb, **kw)
    torch.cuda.synchronize()
    restored = bool(torch.equal(bank, bank0))
    bank_ref = bank0
    n = max(1, min(args.steps, 5))
    tf = tb = 0.0
    binding.profile_enable(True)
    log(f"[bench] train: {n} steps")
    for _ in range(n):
        gbank.zero_()
        torch.cuda.synchronize()
        a = time.perf_counter()
        binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                    out=out, snapshot=snap, workspace=wsf, **kw)
        torch.cuda.synchronize()
        b = time.perf_counter()
        binding.sdm_write_read_backward(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                        snap, gout, gbank, workspace=wsb, **kw)
        torch.cuda.synchronize()
        c = time.perf_counter()
        tf += b - a
        tb += c - b
    prof = binding.profile_read()
    binding.profile_enable(False)
    ms_f, ms_b = tf * 1e3 / n, tb * 1e3 / n
    # the same step with a bfloat16 snapshot (half the snapshot bytes; the bank comes back rounded where written)
    del snap
    snap_q = torch.empty((s.batch, s.heads, s.tokens, s.num_writes, s.head_dim), dtype=torch.bfloat16, device=dev)
    tqf = tqb = 0.0
    for _ in range(n):
        gbank.zero_()
        torch.cuda.synchronize()
        a = time.perf_counter()
        binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                    out=out, snapshot=snap_q, workspace=wsf, snapshot_quant="bf16", **kw)
        torch.cuda.synchronize()
        b = time.perf_counter()
        binding.sdm_write_read_backward(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                        snap_q, gout, gbank, workspace=wsb, snapshot_quant="bf16", **kw)
        torch.cuda.synchronize()
        c = time.perf_counter()
        tqf += b - a
        tqb += c - b
    snap = snap_q
    ms_qf, ms_qb = tqf * 1e3 / n, tqb * 1e3 / n
    # fp8 and int4 snapshots (groups of 16 columns with power-of-two scales)
    quant = {}
    del snap, snap_q
    for mode in ("fp8", "int4"):
        cfg_q = binding.make_config(s.batch, s.tokens, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes,
                                    s.num_reads, s.chunk_size, binding.SDM_BF16, binding.SDM_F32, s.rows, pitch,
                                    snapshot_dtype=binding._SNAP[mode])
        nbytes = binding._snapshot_shape(cfg_q, binding._SNAP[mode], 0, 0, 0, 0, 0)[0]
        snap_m = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        tf_m = tb_m = 0.0
        for _ in range(n):
            gbank.zero_()
            torch.cuda.synchronize()
            a = time.perf_counter()
            binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                        out=out, snapshot=snap_m, workspace=wsf, snapshot_quant=mode, **kw)
            torch.cuda.synchronize()
            b = time.perf_counter()
            binding.sdm_write_read_backward(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"],
                                            bank, snap_m, gout, gbank, workspace=wsb, snapshot_quant=mode, **kw)
            torch.cuda.synchronize()
            c = time.perf_counter()
            tf_m += b - a
            tb_m += c - b
            bank.copy_(bank_ref)  # the quantized restore leaves the written rows quantized: start every step alike
        quant[mode] = {"tokens_per_s": round(s.batch * s.tokens / ((tf_m + tb_m) / n), 1),
                       "ms_forward_save": round(tf_m * 1e3 / n, 4), "ms_backward": round(tb_m * 1e3 / n, 4),
                       "snapshot_bytes": nbytes}
        del snap_m
    snap = None
    # the backward's kernels (reverse sweep, token grouping, token and sub-key sums) against HBM: a per-token latency
    # chain, so the fraction says how far the round trips keep it from the bandwidth bound
    bwd_bytes = bwd_algorithmic_bytes(s, s.batch * s.heads * s.tokens)
    bwd_ms = prof["bwd"][0] / prof["bwd"][1] if prof.get("bwd", (0, 0))[1] else None
    bwd_roof = None
    if bwd_ms:
        gbps = bwd_bytes / (bwd_ms * 1e-3) / 1e9
        bwd_roof = {"kernel": "bwd (reverse sweep + token grouping, token and sub-key sums)", "bound": "hbm",
                    "achieved": round(gbps, 1), "peak": 8000.0, "unit": "GB/s", "frac": round(gbps / 8000.0, 4),
                    "algorithmic_bytes_per_call": bwd_bytes, "avg_launch_ms": round(bwd_ms, 4),
                    "limit": "one HBM round trip per step of disjoint tokens"}
    res = {"tokens_per_s": round(s.batch * s.tokens / ((ms_f + ms_b) * 1e-3), 1),
           "ms_forward_save": round(ms_f, 4), "ms_backward": round(ms_b, 4), "steps": n,
           "kernels_avg_ms": {k: round(v[0] / v[1], 4) for k, v in prof.items() if v[1]},
           "backward_roofline": bwd_roof,
           "snapshot_bytes": s.batch * s.heads * s.tokens * s.num_writes * s.head_dim * 4,
           "bank_restored_bitwise": restored,
           "bf16_snapshot": {"tokens_per_s": round(s.batch * s.tokens / ((ms_qf + ms_qb) * 1e-3), 1),
                             "ms_forward_save": round(ms_qf, 4), "ms_backward": round(ms_qb, 4),
                             "snapshot_bytes": s.batch * s.heads * s.tokens * s.num_writes * s.head_dim * 2},
           "fp8_snapshot": quant["fp8"], "int4_snapshot": quant["int4"],
           "config": "layer_65k (as the headline), grad_out ~ N(0,1), float32 gradients"}
    log(f"[bench] train: forward+snapshot {ms_f:.3f} ms, backward {ms_b:.3f} ms")
    del g, snap, gbank, bank, bank_ref, wsf, wsb, out, t, gout
    torch.cuda.empty_cache()
    return res


def bench_other(args, torch, binding, synth):
    """The three-factor (65,536 slots, bf16 bank, chunk 128) and 1,048,576-slot (32 GiB float32 bank) workloads at
    full size: tokens/s and the chunk loop's algorithmic bandwidth. Context lines, not the headline value."""
    res = {}
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    dev = torch.device("cuda:0")
    for name in ("three_factor_65k", "large_1m"):
        s = synth.WORKLOADS[name]
        log(f"[bench] {name}: inputs")
        x = synth.make_step_inputs(s)
        x["subkeys"] = synth.make_subkeys(s)
        t = {k: torch.from_numpy(x[k]).to(dev).to(dt[s.act]) for k in ("wkeys", "rq", "values", "alpha", "beta",
                                                                        "subkeys")}
        del x
        pitch = binding.bank_pitch(s.head_dim, dt[s.bank])
        bank = binding.alloc_bank(s.batch, s.heads, s.rows, s.head_dim, dt[s.bank], dev, pitch=pitch)
        synth.fill_bank_device(bank, s)
        cfg = binding.make_config(s.batch, s.tokens, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes,
                                  s.num_reads, s.chunk_size, binding.SDM_BF16 if s.act == "bf16" else binding.SDM_F32,
                                  binding.SDM_BF16 if s.bank == "bf16" else binding.SDM_F32, s.rows, pitch)
        ws = torch.empty(binding.workspace_size(cfg, binding.SDM_OP_WRITE_READ), dtype=torch.uint8, device=dev)
        out = torch.empty((s.batch, s.tokens, s.heads, s.head_dim), dtype=dt[s.act], device=dev)

        def step():
            binding.sdm_write_read(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                   widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
                                   chunk_size=s.chunk_size, out=out, workspace=ws)

        step()
        torch.cuda.synchronize()
        binding.profile_enable(True)
        n = max(1, args.other_steps)
        t0 = time.perf_counter()
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        prof = binding.profile_read()
        binding.profile_enable(False)
        ms = (t1 - t0) * 1e3 / n
        # per call: a pipelined call (the three-factor workload) launches its top-k, plan and loop once per piece,
        # the top-k and plan beside the loop on a second stream, so kernel times are summed over a call's launches
        loop_ms = prof["loop"][0] / n
        alg = loop_algorithmic_bytes(s, s.batch * s.tokens * s.heads)
        topk_ms = prof["topk"][0] / n
        # factor scoring as a dense contraction: both kinds, every query against every sub-key of every factor
        flops = 2 * s.batch * s.tokens * s.heads * sum(s.widths) * s.subkey_dim * 2
        filtered = s.act == "bf16" and min(s.widths) >= 512
        res_mfma = {"kernel": "topk2_kernel (%s factor scoring + exact selection)" % (
                        "bf16 MFMA-filtered" if filtered else "fp64 direct"),
                    "bound": "latency (selection chains)", "scoring_flops_per_call": flops,
                    "achieved": round(flops / (topk_ms * 1e-3) / 1e12, 2), "peak": 2500.0, "unit": "TFLOP/s",
                    "frac": round(flops / (topk_ms * 1e-3) / 1e12 / 2500.0, 5), "ms_per_call": round(topk_ms, 4)}
        res[name] = {"tokens_per_s": round(s.batch * s.tokens / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
                     "topk_scoring_mfma": res_mfma,
                     "steps": n, "kernels_ms_per_call": {k: round(v[0] / n, 4) for k, v in prof.items() if v[1]},
                     "launches_per_call": {k: round(v[1] / n, 2) for k, v in prof.items() if v[1]},
                     "loop_algorithmic_bytes": alg, "loop_achieved_GBps": round(alg / (loop_ms * 1e-3) / 1e9, 1),
                     "loop_frac_of_8TBps": round(alg / (loop_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "bank_bytes": s.batch * s.heads * s.rows * s.head_dim * (2 if s.bank == "bf16" else 4),
                     "config": f"B{s.batch} T{s.tokens} H{s.heads} d{s.head_dim} widths {s.widths} dk {s.subkey_dim} "
                               f"W=R={s.num_writes} chunk {s.chunk_size} {s.act} act / {s.bank} bank"}
        log(f"[bench] {name}: {res[name]['tokens_per_s']} tokens/s, loop {loop_ms:.3f} ms")
        del bank, ws, out, t
        torch.cuda.empty_cache()
    return res


def bench_layer(args, torch, binding, synth):
    """The layer's forward at the layer_65k op shapes and model width 2048 (x [2, 4096, 2048] bf16): input map,
    gates, the op, output map. Context line (tokens/s of the whole layer; the dense maps' MFMA roofline)."""
    s = synth.WORKLOADS["layer_65k"]
    Dm = 2048
    dev = torch.device("cuda:0")
    log("[bench] layer: inputs")
    x = synth.make_layer_inputs(s, Dm)
    t = {k: torch.from_numpy(x[k]).to(dev).to(torch.bfloat16) for k in ("x", "w_in", "w_out", "subkeys")}
    g = {k: torch.from_numpy(x[k]).to(dev) for k in ("a_log", "dt_bias")}
    pitch = binding.bank_pitch(s.head_dim, torch.float32)
    bank = binding.alloc_bank(s.batch, s.heads, s.rows, s.head_dim, torch.float32, dev, pitch=pitch)
    bank.copy_(torch.from_numpy(x["bank"]).to(dev))
    del x
    kw = dict(heads=s.heads, widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
              chunk_size=s.chunk_size)
    y, _, _, ws = binding.sdm_layer_forward(t["x"], t["w_in"], g["a_log"], g["dt_bias"], t["w_out"], t["subkeys"],
                                            bank, return_workspace=True, **kw)
    torch.cuda.synchronize()
    n = max(1, args.other_steps)
    binding.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(n):
        binding.sdm_layer_forward(t["x"], t["w_in"], g["a_log"], g["dt_bias"], t["w_out"], t["subkeys"], bank,
                                  y=y, workspace=ws, **kw)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = binding.profile_read()
    binding.profile_enable(False)
    ms = (t1 - t0) * 1e3 / n
    M = s.batch * s.tokens
    n_in = binding.layer_in_features(s.heads, s.widths, s.subkey_dim, s.head_dim)
    flops = 2 * M * Dm * n_in + 2 * M * s.heads * s.head_dim * Dm
    dense_ms = prof["dense"][0] / n  # both dense maps and the gates, per call
    res = {"tokens_per_s": round(M / (ms * 1e-3), 1), "ms_per_step": round(ms, 4), "steps": n,
           "kernels_ms_per_call": {k: round(v[0] / n, 4) for k, v in prof.items() if v[1]},
           "dense_mfma": {"kernel": "gemm_bf16_kernel (input and output maps) + gates_kernel", "bound": "mfma",
                          "flops_per_call": flops, "achieved": round(flops / (dense_ms * 1e-3) / 1e12, 1),
                          "peak": 2500.0, "unit": "TFLOP/s",
                          "frac": round(flops / (dense_ms * 1e-3) / 1e12 / 2500.0, 4),
                          "ms_per_call": round(dense_ms, 4)},
           "config": f"x [{s.batch}, {s.tokens}, {Dm}] bf16, w_in [{n_in}, {Dm}], w_out [{Dm}, "
                     f"{s.heads * s.head_dim}], op as layer_65k (f32 bank)"}
    log(f"[bench] layer: {res['tokens_per_s']} tokens/s, dense {dense_ms:.3f} ms per call")
    del ws
    # the layer's training step: the snapshot-saving forward and the backward (which steps the bank back)
    gy = torch.randn((s.batch, s.tokens, Dm), generator=torch.Generator(device=dev).manual_seed(5),
                     device=dev).to(torch.bfloat16)
    gbank = torch.zeros((s.batch, s.heads, s.rows, pitch), dtype=torch.float32, device=dev)[..., :s.head_dim]
    bank0 = bank.clone()
    y, snap, wsb, _, _ = binding.sdm_layer_forward_save(t["x"], t["w_in"], g["a_log"], g["dt_bias"], t["w_out"],
                                                        t["subkeys"], bank, **kw)
    binding.sdm_layer_backward(t["x"], t["w_in"], g["a_log"], g["dt_bias"], t["w_out"], t["subkeys"], bank, snap, gy,
                               wsb, gbank, **kw)
    torch.cuda.synchronize()
    restored = bool(torch.equal(bank, bank0))
    tf = tb = 0.0
    binding.profile_enable(True)
    for _ in range(n):
        gbank.zero_()
        torch.cuda.synchronize()
        a = time.perf_counter()
        binding.sdm_layer_forward_save(t["x"], t["w_in"], g["a_log"], g["dt_bias"], t["w_out"], t["subkeys"], bank,
                                       y=y, snapshot=snap, workspace=wsb, **kw)
        torch.cuda.synchronize()
        b = time.perf_counter()
        binding.sdm_layer_backward(t["x"], t["w_in"], g["a_log"], g["dt_bias"], t["w_out"], t["subkeys"], bank, snap,
                                   gy, wsb, gbank, **kw)
        torch.cuda.synchronize()
        tf += b - a
        tb += time.perf_counter() - b
    prof = binding.profile_read()
    binding.profile_enable(False)
    ms_f, ms_b = tf * 1e3 / n, tb * 1e3 / n
    # dense maps of the step: the forward's two, the backward's four (d o, d w_out, d x, d w_in), same shapes
    res["train"] = {"tokens_per_s": round(M / ((ms_f + ms_b) * 1e-3), 1), "ms_forward_save": round(ms_f, 4),
                    "ms_backward": round(ms_b, 4), "bank_restored_bitwise": restored,
                    "dense_ms_per_step": round(prof["dense"][0] / n, 4), "dense_flops_per_step": 3 * flops,
                    "kernels_ms_per_step": {k: round(v[0] / n, 4) for k, v in prof.items() if v[1]},
                    "config": "the layer above; grad_y ~ N(0, 1) bf16, float32 gradients"}
    log(f"[bench] layer train: {res['train']['tokens_per_s']} tokens/s (forward {ms_f:.3f} ms, backward "
        f"{ms_b:.3f} ms)")
    del bank, bank0, wsb, snap, gbank, gy, y, t, g
    torch.cuda.empty_cache()
    return res


def bench_decode(args, torch, binding, synth):
    s = synth.WORKLOADS["decode_b128"]
    dev = torch.device("cuda:0")
    nsteps = args.decode_warmup + args.decode_steps
    log(f"[bench] decode {s.name}: {nsteps} steps of inputs")
    steps = []
    for i in range(nsteps):
        x = synth.make_step_inputs(s, step=i)
        steps.append({k: torch.from_numpy(v).to(dev) for k, v in x.items()})
    sub = torch.from_numpy(synth.make_subkeys(s)).to(dev)
    bank0 = torch.from_numpy(synth.make_bank(s)).to(dev)
    cfg = binding.make_config(s.batch, 1, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes, s.num_reads, 1,
                              binding.SDM_F32, binding.SDM_F32, s.rows)
    ws = torch.empty(binding.workspace_size(cfg, binding.SDM_OP_DECODE), dtype=torch.uint8, device=dev)
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, workspace=ws)
    # the prepared step (config and workspace made once): what a serving loop calls per token
    step_fn = binding.DecodeStep(s.batch, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes, s.num_reads,
                                 torch.float32, torch.float32, s.rows, dev, workspace=ws)
    res = {}
    outs = {}
    for mode in ("donated", "copied"):
        banks = [bank0.clone(), torch.empty_like(bank0)]
        out = torch.empty((s.batch, 1, s.heads, s.head_dim), dtype=torch.float32, device=dev)
        cur = 0

        def one(i):
            nonlocal cur
            a = steps[i]
            if mode == "donated":
                step_fn(a["wkeys"], a["rq"], a["values"], a["alpha"], a["beta"], sub, banks[0], out=out)
            else:
                step_fn(a["wkeys"], a["rq"], a["values"], a["alpha"], a["beta"], sub, banks[cur], banks[1 - cur],
                        out=out)
                cur = 1 - cur

        for i in range(args.decode_warmup):
            one(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.decode_warmup, nsteps):
            one(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = (t1 - t0) * 1e3 / args.decode_steps
        outs[mode] = (out.clone(), (banks[0] if mode == "donated" else banks[cur]).clone())
        # kernel times: the same steps again with timing events on (not part of the steps/s above)
        banks[0].copy_(bank0)
        cur = 0
        torch.cuda.synchronize()
        binding.profile_enable(True)
        for i in range(args.decode_warmup, nsteps):
            one(i)
        torch.cuda.synchronize()
        prof = binding.profile_read()
        binding.profile_enable(False)
        res[mode] = {"steps_per_s": round(1e3 / ms, 1), "ms_per_step": round(ms, 4),
                     "kernels_avg_ms": {k: round(v[0] / v[1], 4) for k, v in prof.items() if v[1]}}
    # graph replay (donated): the timed steps captured once into a HIP graph and replayed; checked bit for bit
    # against the same steps run eagerly from the same bank
    g_bank = bank0.clone()
    g_out = torch.empty((s.batch, 1, s.heads, s.head_dim), dtype=torch.float32, device=dev)

    def eager_step(i):
        a = steps[i]
        binding.sdm_decode_step(a["wkeys"], a["rq"], a["values"], a["alpha"], a["beta"], sub, g_bank, out=g_out,
                                **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(min(3, nsteps)):
            eager_step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.decode_warmup, nsteps):
            eager_step(i)
    g_bank.copy_(bank0)
    for i in range(args.decode_warmup, nsteps):
        eager_step(i)
    torch.cuda.synchronize()
    ref_out, ref_bank = g_out.clone(), g_bank.clone()
    g_bank.copy_(bank0)
    graph.replay()
    torch.cuda.synchronize()
    graph_equal = bool(torch.equal(g_out, ref_out) and torch.equal(g_bank, ref_bank))
    g_bank.copy_(bank0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    res["graph"] = {"steps_per_s": round(args.decode_steps / (t1 - t0), 1),
                    "ms_per_step": round((t1 - t0) * 1e3 / args.decode_steps, 4), "equals_eager_bitwise": graph_equal}
    del graph
    # the same timed steps as one sdm_decode_steps call (inputs [B, K, H, ...]; top-k of every step first, then
    # each stream's steps in one launch), checked bit for bit against the eager donated steps
    K = args.decode_steps
    cat = {k: torch.stack([steps[i][k][:, 0] for i in range(args.decode_warmup, nsteps)], dim=1).contiguous()
           for k in ("wkeys", "rq", "values", "alpha", "beta")}
    m_out = torch.empty((s.batch, K, s.heads, s.head_dim), dtype=torch.float32, device=dev)
    cfg_k = binding.make_config(s.batch, K, s.heads, s.widths, s.subkey_dim, s.head_dim, s.num_writes, s.num_reads, 1,
                                binding.SDM_F32, binding.SDM_F32, s.rows)
    ws_k = torch.empty(binding.workspace_size(cfg_k, binding.SDM_OP_DECODE_STEPS), dtype=torch.uint8, device=dev)
    m_bank = torch.empty_like(bank0)

    def multi():
        binding.sdm_decode_steps(cat["wkeys"], cat["rq"], cat["values"], cat["alpha"], cat["beta"], sub, m_bank,
                                 widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, out=m_out,
                                 workspace=ws_k)

    # reference: the eager donated steps from the bank after the warm-up steps
    r_bank = bank0.clone()
    for i in range(nsteps):
        a = steps[i]
        step_fn(a["wkeys"], a["rq"], a["values"], a["alpha"], a["beta"], sub, r_bank, out=g_out)
        if i == args.decode_warmup - 1:
            warm_bank = r_bank.clone()
    torch.cuda.synchronize()
    m_bank.copy_(warm_bank)
    multi()
    torch.cuda.synchronize()
    multi_equal = bool(torch.equal(m_bank, r_bank) and torch.equal(m_out[:, -1:], g_out))
    reps = 5
    t_m = 0.0
    for _ in range(reps):
        m_bank.copy_(warm_bank)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        multi()
        torch.cuda.synchronize()
        t_m += time.perf_counter() - t0
    binding.profile_enable(True)
    m_bank.copy_(warm_bank)
    multi()
    torch.cuda.synchronize()
    mprof = binding.profile_read()
    binding.profile_enable(False)
    res["multi_step"] = {"steps_per_s": round(K * reps / t_m, 1), "ms_per_call": round(t_m * 1e3 / reps, 4),
                         "steps_per_call": K, "equals_eager_bitwise": multi_equal,
                         "kernels_ms_per_call": {k: round(v[0], 4) for k, v in mprof.items() if v[1]}}
    del cat, m_out, ws_k, m_bank, r_bank, warm_bank
    equal = bool(torch.equal(outs["donated"][0], outs["copied"][0]) and torch.equal(outs["donated"][1],
                                                                                    outs["copied"][1]))
    sb = 4
    per_step = s.batch * s.heads * ((2 * s.num_writes + s.num_reads) * s.head_dim * sb + 2 * s.head_dim * 4 + 8)
    dms = res["donated"]["kernels_avg_ms"].get("decode")
    return {
        "workload": "decode_b128: B128 streams x 1 token, H2 d256 N1024 (2x32) W=R=64, fp32 bank",
        "steps_per_s": res["donated"]["steps_per_s"], "steps_per_s_copied": res["copied"]["steps_per_s"],
        "steps_per_s_graph_replay": res["graph"]["steps_per_s"],
        "steps_per_s_multi_step": res["multi_step"]["steps_per_s"],
        "donated": res["donated"], "copied": res["copied"], "graph_replay": res["graph"],
        "multi_step": res["multi_step"],
        "donated_equals_copied_bitwise": equal,
        "warmup": args.decode_warmup, "steps": args.decode_steps,
        "decode_kernel_hbm_frac": round(per_step / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if dms else None,
    }


def cpu_baseline(args, s, synth):
    """The CPU oracle (sequential per-token fp64; streams spread over threads) on the host cores: the headline
    workload in full with one thread per stream, a single-thread sample of it, and bounded samples of the decode and
    three-factor workloads."""
    import numpy as np

    import oracle

    ncpu = os.cpu_count() or 1
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass

    def run(ss, threads, x=None):
        x = synth.make_inputs(ss) if x is None else x
        t0 = time.perf_counter()
        oracle.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], x["subkeys"], x["bank"],
                          ss.widths, ss.num_writes, ss.num_reads, bank_bf16=ss.bank == "bf16",
                          act_bf16=ss.act == "bf16", nthreads=threads, want_index=False)
        return time.perf_counter() - t0

    threads = min(s.batch * s.heads, ncpu, 16)
    T = args.cpu_tokens or s.tokens
    ss = s.with_(tokens=T)
    log(f"[bench] cpu baseline: oracle on {ss.name} B{ss.batch} T{T} H{ss.heads}, {threads} threads")
    dt = run(ss, threads)
    res = {"value": round(ss.batch * T / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"the full {ss.name} workload (B{ss.batch} x T{T} tokens, H{ss.heads}) in {dt:.1f} s; "
                     f"sequential per-token fp64 oracle, one thread per stream; host CPU {model}, {ncpu} "
                     f"logical CPUs visible"}
    # one thread, a quarter of the sequence
    s1 = s.with_(tokens=max(1, T // 4))
    log(f"[bench] cpu baseline: {s1.name} T{s1.tokens}, 1 thread")
    d1 = run(s1, 1)
    res["single_thread"] = {"value": round(s1.batch * s1.tokens / d1, 2), "unit": "tokens/s", "cores": 1,
                            "sample": f"{s1.name} B{s1.batch} x T{s1.tokens} tokens, H{s1.heads}, in {d1:.1f} s"}
    other = {}
    # decode: consecutive steps of the B = 128 workload, each a one-token write/read of every stream
    sd = synth.WORKLOADS["decode_b128"]
    nsteps = 16
    th = min(sd.batch * sd.heads, ncpu, 16)
    log(f"[bench] cpu baseline: {sd.name} {nsteps} steps, {th} threads")
    bank = synth.make_bank(sd)
    sub = synth.make_subkeys(sd)
    xs = [synth.make_step_inputs(sd, step=i) for i in range(nsteps)]
    t0 = time.perf_counter()
    for x in xs:
        r = oracle.write_read(x["wkeys"], x["rq"], x["values"], x["alpha"], x["beta"], sub, bank, sd.widths,
                              sd.num_writes, sd.num_reads, nthreads=th, want_index=False)
        bank = r["bank"]
    dd = time.perf_counter() - t0
    other["decode_b128"] = {"value": round(nsteps / dd, 2), "unit": "steps/s", "cores": th,
                            "sample": f"{nsteps} consecutive steps of B{sd.batch} x H{sd.heads} streams in {dd:.1f} s"}
    # three-factor workload: the first eighth of the sequence
    s3 = synth.WORKLOADS["three_factor_65k"]
    s3 = s3.with_(tokens=s3.tokens // 8)
    th = min(s3.batch * s3.heads, ncpu, 16)
    log(f"[bench] cpu baseline: {s3.name} T{s3.tokens}, {th} threads")
    d3 = run(s3, th)
    other["three_factor_65k"] = {"value": round(s3.batch * s3.tokens / d3, 2), "unit": "tokens/s", "cores": th,
                                 "sample": f"B{s3.batch} x T{s3.tokens} tokens (an eighth of the sequence), "
                                           f"H{s3.heads}, in {d3:.1f} s"}
    res["other_workloads"] = other
    del np
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--decode-warmup", type=int, default=8)
    ap.add_argument("--cpu-tokens", type=int, default=0, help="tokens of the oracle sample (0: the whole workload)")
    ap.add_argument("--other-steps", type=int, default=3, help="timed calls of each context workload (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-train", dest="train", action="store_false", help="skip the training-step context line")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the SDM hot path here is built and measured on a single MI355X "
              f"(requested --gpus {args.gpus}, WORLD_SIZE {world}); streams shard across GPUs with no exchange, "
              f"so the multi-GPU rate is N times the one-GPU rate by construction and is not measured.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_delta_rule_product_amd import binding, synth

    binding.load()
    wr = bench_write_read(args, torch, binding, synth)
    dec = bench_decode(args, torch, binding, synth)
    train = bench_train(args, torch, binding, synth) if args.train else None
    other = bench_other(args, torch, binding, synth) if args.other_steps > 0 else None
    layer = bench_layer(args, torch, binding, synth) if args.other_steps > 0 else None
    s = wr["shape"]
    line = {
        "metric": METRIC, "value": round(wr["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wr["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded Philox: queries, keys, sub-keys, values ~ N(0,1); gates sigmoid(N(0,1)); "
                "bank ~ N(0, 0.02^2))",
        "config": {"workload": "layer_65k: B2 T4096 H2 d1024, 2 factors x 256 sub-keys (65536 slots/head), dk 64, "
                               "W=R=64, chunk 64, bf16 activations, f32 bank",
                   "global_batch": s.batch, "seq_len": s.tokens, "heads": s.heads, "head_dim": s.head_dim,
                   "slots_per_head": s.slots, "num_writes": s.num_writes, "num_reads": s.num_reads,
                   "chunk_size": s.chunk_size, "act_dtype": s.act, "bank_dtype": s.bank,
                   "bank_row_stride": wr["pitch"], "parallelism": "none (1 GPU)"},
        "kernels_avg_ms": wr["kernels_avg_ms"],
        "roofline": wr["roofline"],
        "decode": dec,
        "train": train,
        "other_workloads": other,
        "layer": layer,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, s, synth)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
