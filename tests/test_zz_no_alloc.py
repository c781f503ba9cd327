"""sdm_decode_step_noalloc (include/sdm.h): the decode step for callers that cannot allocate device memory, with
the library's per-GPU scratch array in place of the workspace. Through the C ABI it must give the bits of
sdm_decode_step with a caller workspace, donated and copied, on both step kernels (the one-launch step, which needs
no temporary storage, and the two-kernel step, whose candidate tables, ids and weights live in the scratch), over
two calls in a row with the second on fewer streams, and refuse a step whose workspace exceeds the scratch before
any work."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_product_amd import binding, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _step_pair(s, sub, bank, seed, step):
    """One step with sdm_decode_step (workspace) and with sdm_decode_step_noalloc, donated and copied, from the
    same bank; returns (reference results, no-alloc results) as tensors."""
    x = synth.make_step_inputs(s, seed=seed, step=step)
    t = {k: _dev(v) for k, v in x.items()}
    args = (t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], sub)
    kw = dict(widths=s.widths, num_writes=s.num_writes, num_reads=s.num_reads)
    # reference: the existing entry point, donated
    b_ref = bank.clone()
    o_ref, w_ref, r_ref, _ = binding.sdm_decode_step(*args, b_ref, want_index=True, **kw)
    # no-alloc, donated
    b_na = bank.clone()
    o_na = torch.empty_like(o_ref)
    w_na = torch.empty_like(w_ref)
    r_na = torch.empty_like(r_ref)
    binding.sdm_decode_step_noalloc(*args, b_na, out=o_na, write_idx=w_na, read_idx=r_na, **kw)
    # no-alloc, copied successor (bank_in left unchanged)
    b_in = bank.clone()
    b_out = torch.empty_like(bank)
    o_cp = torch.empty_like(o_ref)
    binding.sdm_decode_step_noalloc(*args, b_in, b_out, out=o_cp, **kw)
    torch.cuda.synchronize()
    return x, (o_ref, w_ref, r_ref, b_ref), (o_na, w_na, r_na, b_na), (o_cp, b_out, b_in)


@pytest.mark.parametrize("W,R,widths", [(64, 64, (32, 32)),      # one-launch step (no temporary storage)
                                        (128, 96, (32, 32)),     # two-kernel step (scratch: tables, ids, weights)
                                        (64, 64, (512, 16))])    # two-kernel step, 512 sub-keys in factor 0
def test_noalloc_equals_decode_step(W, R, widths):
    base = synth.WORKLOADS["decode_b128"].with_(num_writes=W, num_reads=R, widths=widths)
    for call, batch in enumerate((12, 5)):  # the second call on fewer streams
        s = base.with_(batch=batch)
        print(f"noalloc decode W={W} R={R} widths={widths} B={batch}", flush=True)
        sub_np = synth.make_subkeys(s, seed=21)
        sub = _dev(sub_np)
        bank0_np = synth.make_bank(s, seed=21 + call)
        bank0 = _dev(bank0_np)
        x, ref, na, cp = _step_pair(s, sub, bank0, seed=21, step=call)
        for a, b in zip(ref, na):
            assert torch.equal(a, b), "no-alloc step differs from sdm_decode_step"
        assert torch.equal(cp[0], ref[0]) and torch.equal(cp[1], ref[3]), "copied no-alloc step differs"
        assert torch.equal(cp[2], bank0), "copied no-alloc step changed bank_in"
        ids = oracle.topk(x["wkeys"], sub_np, s.widths, W)[0]
        assert np.array_equal(ref[1].cpu().numpy(), ids), "write ids differ from the oracle's top-k"


def test_noalloc_refuses_a_step_beyond_the_scratch():
    # 4096 streams x (512 + 512) ids and weights: 32 MiB of temporary storage, above the 8 MiB scratch
    s = synth.WORKLOADS["decode_b128"].with_(batch=2048, num_writes=512, num_reads=512, widths=(32, 32),
                                             head_dim=16)
    cfg = binding.make_config(s.batch, 1, s.heads, s.widths, s.subkey_dim, s.head_dim, 512, 512, 1)
    assert binding.workspace_size(cfg, binding.SDM_OP_DECODE) > binding.NOALLOC_SCRATCH_BYTES
    x = synth.make_step_inputs(s, seed=3, step=0)
    t = {k: _dev(v) for k, v in x.items()}
    sub = _dev(synth.make_subkeys(s, seed=3))
    bank = torch.zeros((s.batch, s.heads, s.rows, s.head_dim), dtype=torch.float32, device=DEV)
    out = torch.full((s.batch, 1, s.heads, s.head_dim), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(binding.UnsupportedConfigurationError) as e:
        binding.sdm_decode_step_noalloc(t["wkeys"], t["rq"], t["values"], t["alpha"], t["beta"], sub, bank,
                                        widths=s.widths, num_writes=512, num_reads=512, out=out)
    assert e.value.status == binding.SDM_ERR_RANGE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((bank == 0).all()), "a refused call wrote its outputs"
