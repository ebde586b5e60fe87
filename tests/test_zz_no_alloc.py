"""The allocation-free block step (nh_mamba_block_step_noalloc) against nh_mamba_block_step,
through the C ABI: two calls in a row, the second at a smaller batch, each compared with the
workspace entry point run on an identical copy of the same inputs and state.  Both run the
same kernels on the same bytes, so outputs and states must agree bit for bit."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _run_pair(nh, gu, torch, W, d, batch, seed):
    x = gu.to_dev(synth.block_input(seed, batch, 1)[:, 0])
    cs0, ss0 = synth.prefilled_state(seed, batch)
    st_a, cs_a, ss_a = gu.state_dev(cs0, ss0)
    st_b, cs_b, ss_b = gu.state_dev(cs0, ss0)
    ws = gu.workspace(nh.nh_block_workspace_bytes(d, batch, 1, nh.NH_MODE_STEP))
    out_a = gu.empty_f32(batch, 4480)
    out_b = gu.empty_f32(batch, 4480)
    nh.nh_mamba_block_step(d, W, st_a, x, nh.NH_BF16, out_a, nh.NH_F32, batch, ws, ws.numel())
    nh.nh_mamba_block_step_noalloc(d, W, st_b, x, nh.NH_BF16, out_b, nh.NH_F32, batch)
    torch.cuda.synchronize()
    print(f"[no-alloc batch {batch}] compared", flush=True)
    assert torch.equal(out_a, out_b)
    assert torch.equal(ss_a, ss_b)
    assert torch.equal(cs_a, cs_b)
    assert bool(torch.isfinite(out_b).all())


def test_noalloc_step_matches_workspace_step_twice():
    import torch
    import hybrid_mamba2_decode_amd as nh
    from tests import gpu_util as gu
    lw = synth.layer_weights(5)
    W = gu.layer_dev(lw)
    d = nh.dims()
    print("[case] no-alloc step: batch 3, then batch 1", flush=True)
    _run_pair(nh, gu, torch, W, d, 3, 31)
    _run_pair(nh, gu, torch, W, d, 1, 32)
