"""GPU parity of the whole Mamba2 block (per-position step and full-history seq) against
the CPU oracle in CONTRACT mode, through the C ABI.

Bars (the stated tolerances): block outputs rel-L2 <= 5e-3 and max-abs <= 3e-2, read on the
fp32 block output before any output rounding (a bf16 output near |4| has a unit in the last
place of 0.03125, so a single rounding-boundary flip would break max-abs 3e-2 on bf16 bits);
the fp32 SSM state rel-L2 <= 1e-3.  The bf16 output is also checked by rel-L2 and its
rounding flips are counted.
Workloads: one block with seeded synthetic weights (the layer-0 draw): batch 1, T = 16 both
ways; one step from a prefilled state; batch 1, T = 413 with chunk 128."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

OUT_REL, OUT_MAX, STATE_REL = 5e-3, 3e-2, 1e-3


@pytest.fixture(scope="module")
def env():
    import torch
    import hybrid_mamba2_decode_amd as nh
    import oracle
    from tests import gpu_util as gu
    oracle.build(force=False)
    lw = synth.layer_weights(0)
    return nh, oracle, gu, torch, lw, gu.layer_dev(lw)


def _say(*a):
    print("[case]", *a, flush=True)


def _check_out(gu, got, ref, what):
    r, m = gu.rel_l2(got, ref), gu.max_abs(got, ref)
    print(f"[{what}] rel-L2 {r:.3e} max-abs {m:.3e}", flush=True)
    assert r <= OUT_REL and m <= OUT_MAX, (r, m)


def _check_state(gu, got, ref, what):
    r = gu.rel_l2(got, ref)
    print(f"[{what}] state rel-L2 {r:.3e}", flush=True)
    assert r <= STATE_REL, r


def test_block_step_prefilled_b1(env):
    nh, oracle, gu, torch, lw, W = env
    _say("block step, batch 1, prefilled state")
    B = 1
    x = synth.block_input(1, B, 1)
    cs0, ss0 = synth.prefilled_state(1, B)
    st, csd, ssd = gu.state_dev(cs0, ss0)
    d = nh.dims()
    ws = gu.workspace(nh.nh_block_workspace_bytes(d, B, 1, nh.NH_MODE_STEP))
    out = gu.empty_f32(B, 4480)
    nh.nh_mamba_block_step(d, W, st, gu.to_dev(x[:, 0]), nh.NH_BF16, out, nh.NH_F32, B, ws, ws.numel())
    ref = oracle.block(synth.REAL, lw, gu.bf16_bits_to_f64(x), gu.bf16_bits_to_f64(cs0), ss0,
                       mode=oracle.CONTRACT, stepwise=True)
    _check_out(gu, out.cpu().numpy(), ref.out[:, 0], "step b1")
    _check_state(gu, ssd.cpu().numpy(), ref.ssm_state, "step b1")
    cs_got = gu.bf16_bits_to_f64(gu.from_dev_u16(csd))
    assert np.array_equal(cs_got[:, :2], gu.bf16_bits_to_f64(cs0)[:, 1:])   # shifted rows are copies
    assert gu.rel_l2(cs_got, ref.conv_state) < 4e-3                     # new row: bf16 in_proj output


@pytest.mark.parametrize("B,xf32", [(1, False), (2, False), (3, False), (4, False), (1, True), (4, True)])
def test_inproj_conv_step_matches_oracle(env, B, xf32):
    """The fused front of the step (pre-norm, in_proj, split, conv step + SiLU) against the
    oracle's storage points of the same step (z and dt_raw from zxbcdt, xc after the conv).
    Batch 3 and 4 run the matrix-core kernel; an fp32 input is the residual stream of a stack."""
    nh, oracle, gu, torch, lw, W = env
    _say("in_proj + conv step, batch", B, "fp32 x" if xf32 else "bf16 x")
    x = synth.block_input(11, B, 1)
    cs0, ss0 = synth.prefilled_state(11, B)
    st, csd, ssd = gu.state_dev(cs0, ss0)
    z, xc, dtr = gu.empty_u16(B, 10240), gu.empty_u16(B, synth.CONV_DIM), gu.empty_u16(B, 128)
    xin = gu.to_dev(gu.bf16_bits_to_f64(x[:, 0]).astype(np.float32)) if xf32 else gu.to_dev(x[:, 0])
    nh.nh_inproj_conv_step(nh.dims(), W, st, xin, nh.NH_F32 if xf32 else nh.NH_BF16, z, xc, dtr, B)
    ref = oracle.block(synth.REAL, lw, gu.bf16_bits_to_f64(x), gu.bf16_bits_to_f64(cs0), ss0,
                       mode=oracle.CONTRACT, stepwise=True, debug=True)
    zx = ref.debug["zxbcdt"][:, 0]
    for name, got, want in [("z", z, zx[:, :10240]), ("dt_raw", dtr, zx[:, 22528:]),
                            ("xc", xc, ref.debug["xc"][:, 0])]:
        g = gu.bf16_bits_to_f64(gu.from_dev_u16(got))
        r = gu.rel_l2(g, want)
        for b in range(B):
            print(f"[inproj step b{B}] {name} row {b}: rel-L2 {gu.rel_l2(g[b], want[b]):.3e} "
                  f"non-finite {int((~np.isfinite(g[b])).sum())}", flush=True)
        print(f"[inproj step b{B}] {name} rel-L2 {r:.3e} flips {gu.bf16_ulp_flips(gu.from_dev_u16(got), want)}",
              flush=True)
        assert r < 4e-3, (name, r)
    cs_got = gu.bf16_bits_to_f64(gu.from_dev_u16(csd))
    assert np.array_equal(cs_got[:, :2], gu.bf16_bits_to_f64(cs0)[:, 1:])
    assert gu.rel_l2(cs_got, ref.conv_state) < 4e-3
    assert np.array_equal(ssd.cpu().numpy(), ss0)                         # the SSM state is not touched


@pytest.mark.parametrize("B", [3, 4])
def test_block_step_batch3_4(env, B):
    # the step kernels are specialised per batch size up to 4
    nh, oracle, gu, torch, lw, W = env
    _say("block step, batch", B)
    x = synth.block_input(9, B, 1)
    cs0, ss0 = synth.prefilled_state(9, B)
    st, csd, ssd = gu.state_dev(cs0, ss0)
    d = nh.dims()
    ws = gu.workspace(nh.nh_block_workspace_bytes(d, B, 1, nh.NH_MODE_STEP))
    out = gu.empty_f32(B, 4480)
    nh.nh_mamba_block_step(d, W, st, gu.to_dev(x[:, 0]), nh.NH_BF16, out, nh.NH_F32, B, ws, ws.numel())
    ref = oracle.block(synth.REAL, lw, gu.bf16_bits_to_f64(x), gu.bf16_bits_to_f64(cs0), ss0,
                       mode=oracle.CONTRACT, stepwise=True)
    _check_out(gu, out.cpu().numpy(), ref.out[:, 0], f"step b{B}")
    _check_state(gu, ssd.cpu().numpy(), ref.ssm_state, f"step b{B}")
    assert gu.rel_l2(gu.bf16_bits_to_f64(gu.from_dev_u16(csd)), ref.conv_state) < 4e-3


def test_block_step_batch2_bf16_out(env):
    nh, oracle, gu, torch, lw, W = env
    _say("block step, batch 2, bf16 out")
    B = 2
    x = synth.block_input(7, B, 1)
    cs0, ss0 = synth.prefilled_state(7, B)
    st, csd, ssd = gu.state_dev(cs0, ss0)
    d = nh.dims()
    ws = gu.workspace(nh.nh_block_workspace_bytes(d, B, 1, nh.NH_MODE_STEP))
    out = gu.empty_u16(B, 4480)
    nh.nh_mamba_block_step(d, W, st, gu.to_dev(x[:, 0]), nh.NH_BF16, out, nh.NH_BF16, B, ws, ws.numel())
    ref = oracle.block(synth.REAL, lw, gu.bf16_bits_to_f64(x), gu.bf16_bits_to_f64(cs0), ss0,
                       mode=oracle.CONTRACT, stepwise=True)
    got = gu.bf16_bits_to_f64(gu.from_dev_u16(out))
    r = gu.rel_l2(got, ref.out[:, 0])
    print(f"[step b2 bf16] rel-L2 {r:.3e} flips {gu.bf16_ulp_flips(gu.from_dev_u16(out), ref.out[:, 0])}")
    assert r <= OUT_REL
    _check_state(gu, ssd.cpu().numpy(), ref.ssm_state, "step b2")


@pytest.mark.parametrize("Q", [128, 4, 8])
def test_block_seq_and_step_b1_t16(env, Q):
    nh, oracle, gu, torch, lw, W = env
    _say("block batch 1, T=16, Q", Q)
    B, T = 1, 16
    x = synth.block_input(0, B, T)
    xf = gu.bf16_bits_to_f64(x)
    ref = oracle.block(synth.REAL, lw, xf, np.zeros((B, 3, synth.CONV_DIM)), None, mode=oracle.CONTRACT)
    d = nh.dims(chunk=Q)
    # full history (seq) from zero state
    fin, fcs, fss = gu.state_dev(np.zeros((B, 3, synth.CONV_DIM), np.uint16), np.zeros((B, 128, 80, 128), np.float32))
    ws = gu.workspace(nh.nh_block_workspace_bytes(d, B, T, nh.NH_MODE_SEQ))
    out = gu.empty_f32(B, T, 4480)
    nh.nh_mamba_block_seq(d, W, None, fin, gu.to_dev(x), nh.NH_BF16, T, out, nh.NH_F32, B, ws, ws.numel())
    seq_out = out.cpu().numpy()
    _check_out(gu, seq_out, ref.out, f"seq t16 Q={Q}")
    _check_state(gu, fss.cpu().numpy(), ref.ssm_state, f"seq t16 Q={Q}")
    assert gu.rel_l2(gu.bf16_bits_to_f64(gu.from_dev_u16(fcs)), ref.conv_state) < 4e-3
    # cached per-position steps from zero state
    st, csd, ssd = gu.state_dev(np.zeros((B, 3, synth.CONV_DIM), np.uint16), np.zeros((B, 128, 80, 128), np.float32))
    wss = gu.workspace(nh.nh_block_workspace_bytes(d, B, 1, nh.NH_MODE_STEP))
    xd = gu.to_dev(x)
    step_out = np.empty((B, T, 4480), np.float32)
    o1 = gu.empty_f32(B, 4480)
    for t in range(T):
        nh.nh_mamba_block_step(d, W, st, xd[:, t].contiguous(), nh.NH_BF16, o1, nh.NH_F32, B, wss, wss.numel())
        step_out[:, t] = o1.cpu().numpy()
    _check_out(gu, step_out, ref.out, "step t16")
    _check_state(gu, ssd.cpu().numpy(), ref.ssm_state, "step t16")
    # the two GPU modes agree with each other (the pages' cached == full-history claim)
    assert gu.rel_l2(step_out, seq_out) <= OUT_REL


def test_block_seq_b1_t413_q128(env):
    nh, oracle, gu, torch, lw, W = env
    _say("block batch 1, T=413, Q=128")
    B, T = 1, 413
    x = synth.block_input(2, B, T)
    d = nh.dims(chunk=128)
    fin, fcs, fss = gu.state_dev(np.zeros((B, 3, synth.CONV_DIM), np.uint16), np.zeros((B, 128, 80, 128), np.float32))
    ws = gu.workspace(nh.nh_block_workspace_bytes(d, B, T, nh.NH_MODE_SEQ))
    out = gu.empty_f32(B, T, 4480)
    nh.nh_mamba_block_seq(d, W, None, fin, gu.to_dev(x), nh.NH_BF16, T, out, nh.NH_F32, B, ws, ws.numel())
    ref = oracle.block(synth.REAL, lw, gu.bf16_bits_to_f64(x), np.zeros((B, 3, synth.CONV_DIM)), None,
                       mode=oracle.CONTRACT)
    _check_out(gu, out.cpu().numpy(), ref.out, "seq t413")
    _check_state(gu, fss.cpu().numpy(), ref.ssm_state, "seq t413")


def test_block_resume_seq_then_steps(env):
    nh, oracle, gu, torch, lw, W = env
    _say("resume: seq prefix then steps")
    B, T, t0 = 1, 12, 7
    x = synth.block_input(9, B, T)
    d = nh.dims(chunk=4)
    st, csd, ssd = gu.state_dev(np.zeros((B, 3, synth.CONV_DIM), np.uint16), np.zeros((B, 128, 80, 128), np.float32))
    ws = gu.workspace(nh.nh_block_workspace_bytes(d, B, T, nh.NH_MODE_SEQ))
    xd = gu.to_dev(x)
    out = gu.empty_f32(B, t0, 4480)
    nh.nh_mamba_block_seq(d, W, st, st, xd[:, :t0].contiguous(), nh.NH_BF16, t0, out, nh.NH_F32, B, ws, ws.numel())
    outs = [out.cpu().numpy()]
    o1 = gu.empty_f32(B, 4480)
    for t in range(t0, T):
        nh.nh_mamba_block_step(d, W, st, xd[:, t].contiguous(), nh.NH_BF16, o1, nh.NH_F32, B, ws, ws.numel())
        outs.append(o1.cpu().numpy()[:, None])
    got = np.concatenate(outs, axis=1)
    ref = oracle.block(synth.REAL, lw, gu.bf16_bits_to_f64(x), np.zeros((B, 3, synth.CONV_DIM)), None,
                       mode=oracle.CONTRACT)
    _check_out(gu, got, ref.out, "resume")
    _check_state(gu, ssd.cpu().numpy(), ref.ssm_state, "resume")


def test_block_step_is_deterministic(env):
    nh, oracle, gu, torch, lw, W = env
    _say("determinism")
    B = 1
    x = gu.to_dev(synth.block_input(1, B, 1)[:, 0])
    cs0, ss0 = synth.prefilled_state(1, B)
    d = nh.dims()
    ws = gu.workspace(nh.nh_block_workspace_bytes(d, B, 1, nh.NH_MODE_STEP))
    res = []
    for _ in range(2):
        st, csd, ssd = gu.state_dev(cs0, ss0)
        out = gu.empty_f32(B, 4480)
        nh.nh_mamba_block_step(d, W, st, x, nh.NH_BF16, out, nh.NH_F32, B, ws, ws.numel())
        res.append((out.cpu().numpy(), ssd.cpu().numpy(), gu.from_dev_u16(csd)))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)
