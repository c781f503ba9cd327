"""Bitwise repeatability across fresh processes (CHANGELOG 2.0.0, "Deterministic": outputs, the final bank and
every gradient are bitwise identical across repeated calls, fresh processes and graph replays). Two child
processes, started one after the other, each run the same seeded write/read (with indices), the training step
(saving forward and backward) and a decode step through the C ABI, and print a SHA-256 digest of every result;
the digests must be equal."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import hashlib, json, sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
from gated_delta_rule_product_amd import binding, synth

dev = torch.device("cuda:0")
digest = {}

def put(name, *ts):
    h = hashlib.sha256()
    for t in ts:
        t = t.detach().contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)  # the raw bits
        h.update(t.cpu().numpy().tobytes())
    digest[name] = h.hexdigest()

def dev_t(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)

# write/read: a collision-heavy float32 shape, and bf16 activations on a bf16 bank (three factors)
for name, s in (("f32", synth.Shape(2, 96, 2, (8, 16), 8, 64, 16, 12, 32, name="rep32")),
                ("bf16", synth.Shape(1, 160, 2, (8, 4, 8), 8, 64, 16, 16, 32, "bf16", "bf16", name="rep16"))):
    x = synth.make_inputs(s, seed=61)
    dt = torch.bfloat16 if s.act == "bf16" else torch.float32
    bt = torch.bfloat16 if s.bank == "bf16" else torch.float32
    t = {k: dev_t(x[k], dt) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads, chunk_size=s.chunk_size)
    bank = dev_t(x["bank"], bt)
    out, wi, ri = binding.sdm_write_read(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"],
                                         bank, want_index=True, **kw)
    torch.cuda.synchronize()
    put("write_read_" + name, out, bank, wi, ri)
    # training step from the same initial bank
    bank = dev_t(x["bank"], bt)
    out, _, _, snap = binding.sdm_write_read_save(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"],
                                                  t["subkeys"], bank, **kw)
    gout = dev_t(np.random.default_rng(62).standard_normal(out.shape).astype(np.float32), dt)
    g = binding.sdm_write_read_backward(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"],
                                        bank, snap, gout, **kw)
    torch.cuda.synchronize()
    put("train_" + name, out, snap, *[g[k] for k in sorted(g)])

# decode step, donated
s = synth.WORKLOADS["decode_b128"].with_(batch=16)
x = synth.make_inputs(s, seed=63)
t = {k: dev_t(x[k], torch.float32) for k in ("wkeys", "rq", "values", "alpha", "beta", "subkeys")}
bank = dev_t(x["bank"], torch.float32)
out, wi, ri, _ = binding.sdm_decode_step(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], t["subkeys"], bank,
                                         widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads,
                                         want_index=True)
torch.cuda.synchronize()
put("decode", out, bank, wi, ri)
print("DIGESTS " + json.dumps(digest), flush=True)
'''


def _run_child():
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("DIGESTS ")]
    assert line, r.stdout[-2000:]
    return json.loads(line[-1][len("DIGESTS "):])


def test_results_bitwise_equal_across_fresh_processes():
    print("fresh process 1", flush=True)
    a = _run_child()
    print("fresh process 2", flush=True)
    b = _run_child()
    assert a.keys() == b.keys() and len(a) == 5
    diff = [k for k in a if a[k] != b[k]]
    assert not diff, f"results differ between fresh processes: {diff}"
