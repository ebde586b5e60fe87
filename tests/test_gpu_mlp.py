"""GPU parity of one MLP layer of the hybrid stack (nh_mlp_step) against the CPU oracle,
through the C ABI.

Tolerances: the block's bars (rel-L2 <= 5e-3 and max-abs <= 3e-2 on the fp32 output), also
held on the layer's own update (output - input), which the residual would otherwise hide.  The
two bf16 storage points (the normalised input and the squared-ReLU activation) flip by one
unit where fp32 and fp64 sums fall on either side of a rounding boundary."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import hybrid_mamba2_decode_amd as nh
    import oracle
    from tests import gpu_util as gu
    oracle.build(force=False)
    assert torch.cuda.is_available()
    mw = synth.mlp_weights(1)
    dev = (gu.to_dev(mw.norm_w), gu.w4_dev(mw.up), gu.w4_dev(mw.down))
    return nh, oracle, gu, torch, mw, dev


@pytest.mark.parametrize("B,xf32,of32", [(1, False, True), (1, True, True), (2, False, False), (3, True, True),
                                         (4, False, True)])
def test_mlp_step_matches_oracle(env, B, xf32, of32):
    nh, oracle, gu, torch, mw, (nw, up, down) = env
    print("[case] mlp step batch", B, "x", "f32" if xf32 else "bf16", "out", "f32" if of32 else "bf16", flush=True)
    xb = synth.block_input(21, B, 1)[:, 0]
    xd = synth.bf16_to_f32(xb).astype(np.float64)
    xin = gu.to_dev(xd.astype(np.float32)) if xf32 else gu.to_dev(xb)
    out = gu.empty_f32(B, 4480) if of32 else gu.empty_u16(B, 4480)
    ws = gu.workspace(nh.nh_mlp_workspace_bytes(synth.MLP_INTER, B))
    nh.nh_mlp_step(nw, up, down, 1e-5, xin, nh.NH_F32 if xf32 else nh.NH_BF16, out,
                   nh.NH_F32 if of32 else nh.NH_BF16, B, ws, ws.numel())
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64) if of32 else gu.bf16_bits_to_f64(gu.from_dev_u16(out))
    ref = oracle.mlp(xd, mw.norm_w, mw.up, mw.down, 1e-5)
    r, m = gu.rel_l2(got, ref), gu.max_abs(got, ref)
    rd = gu.rel_l2(got - xd, ref - xd)
    print(f"[mlp b{B}] rel-L2 {r:.3e} max-abs {m:.3e} update rel-L2 {rd:.3e}", flush=True)
    assert r <= 5e-3 and rd <= 5e-3
    assert m <= (3e-2 if of32 else 6e-2)    # a bf16 output near |8| has an ulp of 0.0625


@pytest.mark.parametrize("B", [1, 2, 4])
def test_mlp_step_large_activations(env, B):
    # a norm weight of 160 makes the up projection reach several hundred, so the squared-ReLU
    # activations that feed the down projection reach 1e5 (beyond fp16 without the chunk scaling)
    nh, oracle, gu, torch, mw0, _ = env
    print("[case] mlp step, up outputs above 256, batch", B, flush=True)
    nwb = synth.f32_to_bf16(np.full(4480, 160.0, np.float32))
    mw = synth.MlpWeights(nwb, mw0.up, mw0.down)
    nw, up, down = gu.to_dev(nwb), gu.w4_dev(mw.up), gu.w4_dev(mw.down)
    xb = synth.block_input(22, B, 1)[:, 0]
    xd = synth.bf16_to_f32(xb).astype(np.float64)
    out = gu.empty_f32(B, 4480)
    ws = gu.workspace(nh.nh_mlp_workspace_bytes(synth.MLP_INTER, B))
    nh.nh_mlp_step(nw, up, down, 1e-5, gu.to_dev(xb), nh.NH_BF16, out, nh.NH_F32, B, ws, ws.numel())
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    # the activations themselves, to confirm the case: max relu(up)^2 well above 65504
    u = oracle.round_bf16(oracle.rmsnorm(xd, nwb, 1e-5))
    upv = oracle.w4_matvec(mw.up, u)
    hmax = float(np.max(np.maximum(upv, 0.0) ** 2))
    ref = oracle.mlp(xd, nwb, mw.up, mw.down, 1e-5)
    rd = gu.rel_l2(got - xd, ref - xd)
    print(f"[mlp large b{B}] max h {hmax:.3g}, update rel-L2 {rd:.3e}", flush=True)
    assert hmax > 65504.0 * 4
    assert np.isfinite(got).all()
    assert rd <= 5e-3
