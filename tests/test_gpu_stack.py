"""GPU parity of the 27-layer Mamba2 stack through nh_mamba_stack, at the full workload sizes.

* 27 blocks, batch 1, 413 cached per-position steps (stepwise, state carried): every layer's
  output is read back; layers 0 and 26 are recomputed by the oracle over all 413 positions with
  the GPU's own input to that layer (teacher forcing, so a layer is judged on its own error),
  and compared in full, outputs and final conv/SSM state.
* 27 blocks, batch 2, T = 3750, chunk 256 (full-history seq): the scan alone at this shape is
  compared in full with the oracle's recurrence, also row by row (every (position, head) row
  of 80 outputs); layers 0, 13 and 26 of the seq stack are held to the oracle over two
  windows of both sequences, each fed the stack's own input to that layer (teacher forcing):
  positions 0..299 from the zero state (across the chunk boundary at 256), and positions
  3456..3749 from the GPU's own state at 3456 (across the chunk boundary at 3584 and through
  the 166-row last chunk), where the final conv and SSM states are also compared with the
  full run's; and the property the method rests on, full-history recompute == cached
  per-position steps, is checked per layer on identical input (layers 0, 1, 13, 26 stepped
  through 3750 positions on the seq stack's own input to that layer: block outputs and final
  state), and for the freely stepped 27-layer stack on its residual stream.

Bars as in the block tests: block outputs rel-L2 <= 5e-3 and max-abs <= 3e-2 (fp32 outputs),
SSM state rel-L2 <= 1e-3.  With the synthetic 4-bit weights (q uniform on 0..15, bias -8 s,
so every weight has mean -s/2) each block shifts the residual stream by a common offset, and
after 27 blocks the stream sits near -240, where an absolute bar says nothing about a block:
there the stream is held to the rel-L2 bar and a block's own contribution (its output minus
its input) to both bars.  Two GPU results compared with each other (seq
vs steps) are each held to the bars against the exact result, so by the triangle inequality
they may differ by twice the bars; mode-vs-mode checks use 2x (states included)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

OUT_REL, OUT_MAX, STATE_REL = 5e-3, 3e-2, 1e-3
N_LAYERS = 27


@pytest.fixture(scope="module")
def env():
    import torch
    import hybrid_mamba2_decode_amd as nh
    import oracle
    from tests import gpu_util as gu
    oracle.build(force=False)
    print("[case] drawing 27 layers of weights", flush=True)
    lws = [synth.layer_weights(l) for l in range(N_LAYERS)]
    devs = [gu.layer_dev(lw) for lw in lws]
    return nh, oracle, gu, torch, lws, devs, devs


def _say(*a):
    print("[case]", *a, flush=True)


def _check(gu, got, ref, what, state=False, scale=1.0):
    r = gu.rel_l2(got, ref)
    if state:
        print(f"[{what}] state rel-L2 {r:.3e}", flush=True)
        assert r <= scale * STATE_REL, r
    else:
        m = gu.max_abs(got, ref)
        print(f"[{what}] rel-L2 {r:.3e} max-abs {m:.3e}", flush=True)
        assert r <= scale * OUT_REL and m <= scale * OUT_MAX, (r, m)


def _zero_states(nh, gu, B):
    keep, sts = [], []
    for _ in range(N_LAYERS):
        st, cs, ss = gu.state_dev(np.zeros((B, 3, synth.CONV_DIM), np.uint16),
                                  np.zeros((B, 128, 80, 128), np.float32))
        keep.append((cs, ss))
        sts.append(st)
    return sts, keep


def _run_steps(nh, gu, torch, arr, x_dev, B, T):
    """The stack stepwise over T positions; returns per-layer outputs [L][B][T][hidden] (host)."""
    d = nh.dims()
    states, keep = _zero_states(nh, gu, B)
    ws = gu.workspace(nh.nh_block_workspace_bytes(d, B, 1, nh.NH_MODE_STEP))
    outs = gu.empty_f32(N_LAYERS, B, 1, 4480)
    allo = torch.empty((N_LAYERS, B, T, 4480), dtype=torch.float32, device="cuda")
    for t in range(T):
        nh.nh_mamba_stack(d, arr, states, N_LAYERS, nh.NH_MODE_STEP, x_dev[:, t].contiguous(), nh.NH_BF16, 1,
                          outs, B, ws, ws.numel())
        allo[:, :, t] = outs[:, :, 0]
        if t % 100 == 0:
            _say("step", t)
    torch.cuda.synchronize()
    return allo, keep


def test_stack_steps_t413_teacher_forced(env):
    nh, oracle, gu, torch, lws, devs, arr = env
    _say("stack: 27 layers, batch 1, 413 steps")
    B, T = 1, 413
    x = synth.block_input(3, B, T)
    allo, keep = _run_steps(nh, gu, torch, arr, gu.to_dev(x), B, T)
    outs = allo.cpu().numpy()
    assert np.all(np.isfinite(outs))
    for layer in (0, N_LAYERS - 1):
        inp = gu.bf16_bits_to_f64(x) if layer == 0 else outs[layer - 1].astype(np.float64)
        _say("oracle layer", layer)
        ref = oracle.block(synth.REAL, lws[layer], inp, np.zeros((B, 3, synth.CONV_DIM)), None,
                           mode=oracle.CONTRACT)
        _check(gu, outs[layer], ref.out, f"stack step layer {layer}")
        cs, ss = keep[layer]
        _check(gu, ss.cpu().numpy(), ref.ssm_state, f"stack step layer {layer}", state=True)
        assert gu.rel_l2(gu.bf16_bits_to_f64(gu.from_dev_u16(cs)), ref.conv_state) < 4e-3


def test_scan_full_size_b2_t3750(env):
    nh, oracle, gu, torch, lws, devs, arr = env
    _say("scan at B=2, T=3750, Q=256")
    B, T, Q = 2, 3750, 256
    rng = np.random.default_rng(3750)
    xc = synth.f32_to_bf16(rng.normal(0, 0.6, (B, T, synth.CONV_DIM)).astype(np.float32))
    dtr = synth.f32_to_bf16(rng.normal(0, 1.25, (B, T, 128)).astype(np.float32))
    lw = lws[4]
    d = nh.dims(chunk=Q)
    n = nh.nh_ssd_scan_workspace_bytes(d, B, T)
    ws = gu.workspace(n)
    y = gu.empty_f32(B, T, 10240)
    hT = gu.empty_f32(B, 128, 80, 128)
    nh.nh_ssd_chunk_scan(d, gu.to_dev(xc), gu.to_dev(dtr), 128, T, gu.to_dev(lw.dt_bias), gu.to_dev(lw.A_log),
                         gu.to_dev(lw.D), None, hT, y, nh.NH_F32, B, ws, n)
    yg, Sg = y.cpu().numpy(), hT.cpu().numpy()
    for b in range(B):
        xcd = gu.bf16_bits_to_f64(xc[b])
        dt, A = oracle.discretize(gu.bf16_bits_to_f64(dtr[b]), lw.dt_bias, lw.A_log)
        ry, rS = oracle.ssm_recurrence(xcd[:, :10240], xcd[:, 10240:11264], xcd[:, 11264:], dt, A, lw.D,
                                       np.zeros((128, 80, 128)), G=8)
        r = gu.rel_l2(yg[b], ry)
        worst, mabs, top = gu.row_errors(yg[b], ry)
        print(f"[scan full b{b}] y rel-L2 {r:.3e}; worst row rel {worst:.3e}, max-abs {mabs:.3e} of {top:.3e}",
              flush=True)
        assert r < 2e-3
        assert worst <= 1e-2 and mabs <= 1e-2 * top, (worst, mabs, top)
        _check(gu, Sg[b], rS, f"scan full b{b}", state=True)


T4, B4, Q4 = 3750, 2, 256
LATE = 3456          # window start: 13.5 chunks in, so the window crosses 3584 and the last chunk
EARLY = 300          # positions 0..299 cross the chunk boundary at 256


@pytest.fixture(scope="module")
def seq_run(env):
    """The 27-layer full-history stack at batch 2, T = 3750, chunk 256, run once."""
    nh, oracle, gu, torch, lws, devs, arr = env
    _say("stack: 27 layers, batch 2, T=3750, chunk 256 (seq)")
    x = synth.block_input(4, B4, T4)
    xd = gu.to_dev(x)
    d = nh.dims(chunk=Q4)
    states, keep = _zero_states(nh, gu, B4)
    ws = gu.workspace(nh.nh_block_workspace_bytes(d, B4, T4, nh.NH_MODE_SEQ))
    outs = gu.empty_f32(N_LAYERS, B4, T4, 4480)
    nh.nh_mamba_stack(d, arr, states, N_LAYERS, nh.NH_MODE_SEQ, xd, nh.NH_BF16, T4, outs, B4, ws, ws.numel())
    torch.cuda.synchronize()
    assert bool(torch.isfinite(outs).all())
    return x, xd, outs, keep, ws


def _layer_input(gu, x, outs, layer, t0, t1):
    """The seq stack's input to `layer` over positions [t0, t1), as doubles."""
    if layer == 0:
        return gu.bf16_bits_to_f64(x[:, t0:t1])
    return outs[layer - 1, :, t0:t1].cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("layer", [0, 13, N_LAYERS - 1])
def test_stack_seq_oracle_windows_b2_t3750(env, seq_run, layer):
    nh, oracle, gu, torch, lws, devs, arr = env
    x, xd, outs, keep, ws = seq_run
    d = nh.dims(chunk=Q4)
    # early window from the zero state
    _say("oracle window", layer, 0, EARLY)
    inp = _layer_input(gu, x, outs, layer, 0, EARLY)
    ref = oracle.block(synth.REAL, lws[layer], inp, np.zeros((B4, 3, synth.CONV_DIM)), None, mode=oracle.CONTRACT)
    got = outs[layer, :, :EARLY].cpu().numpy()
    _check(gu, got - inp, ref.out - inp, f"seq layer {layer} t<{EARLY}, block output")
    _check(gu, got, ref.out, f"seq layer {layer} t<{EARLY}, residual stream")
    # late window: the GPU's state at LATE from a full-history run over [0, LATE) on the same
    # input, then the oracle's recurrence over [LATE, T)
    _say("GPU state at", LATE, "layer", layer)
    st, cs, ss = gu.state_dev(np.zeros((B4, 3, synth.CONV_DIM), np.uint16), np.zeros((B4, 128, 80, 128), np.float32))
    part = gu.empty_f32(B4, LATE, 4480)
    if layer == 0:
        xin, xt = xd[:, :LATE].contiguous(), nh.NH_BF16
    else:
        xin, xt = outs[layer - 1, :, :LATE].contiguous(), nh.NH_F32
    nh.nh_mamba_block_seq(d, arr[layer], None, st, xin, xt, LATE, part, nh.NH_F32, B4, ws, ws.numel())
    torch.cuda.synchronize()
    del part
    _say("oracle window", layer, LATE, T4)
    inp = _layer_input(gu, x, outs, layer, LATE, T4)
    ref = oracle.block(synth.REAL, lws[layer], inp, gu.bf16_bits_to_f64(gu.from_dev_u16(cs)),
                       ss.cpu().numpy().astype(np.float64), mode=oracle.CONTRACT)
    got = outs[layer, :, LATE:].cpu().numpy()
    _check(gu, got - inp, ref.out - inp, f"seq layer {layer} t>={LATE}, block output")
    _check(gu, got, ref.out, f"seq layer {layer} t>={LATE}, residual stream")
    fcs, fss = keep[layer]
    _check(gu, fss.cpu().numpy(), ref.ssm_state, f"seq layer {layer} final", state=True)
    rc = gu.rel_l2(gu.bf16_bits_to_f64(gu.from_dev_u16(fcs)), ref.conv_state)
    print(f"[seq layer {layer} final] conv state rel-L2 {rc:.3e}", flush=True)
    assert rc < 4e-3


def test_stack_seq_equals_steps_b2_t3750(env, seq_run):
    nh, oracle, gu, torch, lws, devs, arr = env
    x, xd, outs, seq_keep, _ = seq_run
    B, T = B4, T4
    d = nh.dims(chunk=Q4)
    # cached == full history, per layer on identical input: the seq stack's input to layer l
    # is stepped through layer l alone
    wss = gu.workspace(nh.nh_block_workspace_bytes(d, B, 1, nh.NH_MODE_STEP))
    o1 = gu.empty_f32(B, 4480)
    for layer in (0, 1, 13, N_LAYERS - 1):
        _say("steps through layer", layer)
        st, cs, ss = gu.state_dev(np.zeros((B, 3, synth.CONV_DIM), np.uint16), np.zeros((B, 128, 80, 128), np.float32))
        got = torch.empty((B, T, 4480), dtype=torch.float32, device="cuda")
        for t in range(T):
            if layer == 0:
                nh.nh_mamba_block_step(d, arr[layer], st, xd[:, t].contiguous(), nh.NH_BF16, o1, nh.NH_F32, B,
                                       wss, wss.numel())
            else:
                nh.nh_mamba_block_step(d, arr[layer], st, outs[layer - 1, :, t].contiguous(), nh.NH_F32, o1,
                                       nh.NH_F32, B, wss, wss.numel())
            got[:, t] = o1
        inp = gu.bf16_bits_to_f64(x) if layer == 0 else outs[layer - 1].cpu().numpy().astype(np.float64)
        seq_l = outs[layer].cpu().numpy()
        _check(gu, got.cpu().numpy() - inp, seq_l - inp, f"layer {layer} steps vs seq, block output", scale=2.0)
        _check(gu, ss.cpu().numpy(), seq_keep[layer][1].cpu().numpy(), f"layer {layer} steps vs seq", state=True,
               scale=2.0)
    # the whole stack stepped freely: each mode carries its own rounding into the next layer's
    # input, and slowly decaying heads integrate that difference (about 3e-3 in the state after
    # 27 layers, against 5e-4 to 7e-4 per layer on identical input), so the states are held to
    # 1e-2 here; the residual stream to twice the rel-L2 bar
    seq_last = outs[N_LAYERS - 1].cpu().numpy()
    allo, step_keep = _run_steps(nh, gu, torch, arr, xd, B, T)
    r = gu.rel_l2(allo[N_LAYERS - 1].cpu().numpy(), seq_last)
    print(f"[stack seq vs steps] residual stream rel-L2 {r:.3e}", flush=True)
    assert r <= 2 * OUT_REL
    worst = max(gu.rel_l2(seq_keep[l][1].cpu().numpy(), step_keep[l][1].cpu().numpy()) for l in range(N_LAYERS))
    print(f"[stack seq vs steps] worst final-state rel-L2 over 27 free-running layers {worst:.3e}", flush=True)
    assert worst <= 1e-2
