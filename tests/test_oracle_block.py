"""Block-level pins for the oracle.

* An independent composition of the block from torch library routines (rms_norm,
  conv1d with groups, softplus, silu, matmul) plus the brute-force SSD dual-form sum
  must agree with oracle.block in EXACT mode.
* The docs page "Nemotron VoiceChat", section "Offline timeline", states that the
  full-history recompute and the cached per-position mode give the same result: the
  per-position (step) and the whole-sequence (seq) evaluations must agree, and so must a
  seq prefix resumed by steps.
* Causality: position t of a seq over [0, T) equals the last output of a seq over [0, t].
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from tests.test_oracle_pins import TINY, _brute_force_dual, _byte_split_dequant


def _tiny_weights(layer=0, seed=0):
    return synth.layer_weights(layer, seed=seed, d=TINY)


def _x(T, B=1, seed=0, d=TINY):
    return synth.bf16_to_f32(synth.block_input(0, B, T, seed=seed, d=d)).astype(np.float64)


def _torch_block_exact(d, w, x, conv_state, ssm_state):
    """Independent EXACT-mode block for one sequence built from library routines."""
    xt = torch.from_numpy(x)
    bf = lambda a: torch.from_numpy(synth.bf16_to_f32(a).astype(np.float64))  # noqa: E731
    u = F.rms_norm(xt, (d.hidden,), weight=bf(w.norm_w), eps=d.eps)
    Win = torch.from_numpy(_byte_split_dequant(w.in_proj)[1])
    zx = u @ Win.T
    DI, G, N, H, P, K = d.d_inner, d.n_groups, d.d_state, d.n_heads, d.head_dim, d.conv_k
    CD = d.conv_dim
    z, xbc, dt_raw = zx[:, :DI], zx[:, DI:DI + CD], zx[:, DI + CD:]
    hist = torch.cat([torch.from_numpy(conv_state), xbc], dim=0)          # [K-1+T][CD]
    conv = F.conv1d(hist.T.unsqueeze(0), bf(w.conv_w).reshape(CD, 1, K), bf(w.conv_b), groups=CD)
    xc = F.silu(conv[0].T)
    dt = F.softplus(dt_raw + torch.from_numpy(w.dt_bias.astype(np.float64)))
    A = -np.exp(w.A_log.astype(np.float64))
    y = _brute_force_dual(xc[:, :DI].numpy(), xc[:, DI:DI + G * N].numpy(),
                          xc[:, DI + G * N:].numpy(), dt.numpy(), A, w.D, ssm_state, G)
    g = torch.from_numpy(y) * F.silu(z)
    grp = DI // G
    gw = bf(w.gnorm_w)
    o = torch.cat([F.rms_norm(g[:, j * grp:(j + 1) * grp], (grp,), weight=gw[j * grp:(j + 1) * grp],
                              eps=d.eps) for j in range(G)], dim=1)
    Wout = torch.from_numpy(_byte_split_dequant(w.out_proj)[1])
    return (xt + o @ Wout.T).numpy()


def test_block_matches_independent_library_composition(oracle_lib):
    w = _tiny_weights()
    T = 6
    x = _x(T)
    rng = np.random.default_rng(9)
    cs = rng.normal(size=(1, TINY.conv_k - 1, TINY.conv_dim))
    ss = 0.1 * rng.normal(size=(1, TINY.n_heads, TINY.head_dim, TINY.d_state))
    r = oracle_lib.block(TINY, w, x, cs, ss, mode=oracle_lib.EXACT)
    ref = _torch_block_exact(TINY, w, x[0], cs[0], ss[0])
    assert np.allclose(r.out[0], ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("mode", [0, 1])
def test_step_equals_seq(oracle_lib, mode):
    w = _tiny_weights(1)
    T = 16
    x = _x(T, B=2, seed=3)
    seq = oracle_lib.block(TINY, w, x, np.zeros((2, 3, TINY.conv_dim)), None, mode=mode)
    step = oracle_lib.block_stepwise(TINY, w, x, None, None, mode=mode)
    if mode == oracle_lib.EXACT:
        assert np.allclose(step.out, seq.out, rtol=1e-12, atol=1e-12)
        assert np.allclose(step.ssm_state, seq.ssm_state, rtol=1e-12, atol=1e-13)
        assert np.array_equal(step.conv_state, seq.conv_state)
    else:
        # CONTRACT: step stores the state in float32 between positions; the only
        # difference from seq is that rounding, far below the bf16 storage points.
        assert np.allclose(step.out, seq.out, rtol=1e-4, atol=1e-4)
        rel = np.linalg.norm(step.ssm_state - seq.ssm_state) / np.linalg.norm(seq.ssm_state)
        assert rel < 1e-5


def test_step_equals_seq_real_dims(oracle_lib):
    w = synth.layer_weights(0)
    x = synth.bf16_to_f32(synth.block_input(0, 1, 3)).astype(np.float64)
    seq = oracle_lib.block(synth.REAL, w, x, np.zeros((1, 3, synth.CONV_DIM)), None,
                           mode=oracle_lib.EXACT)
    step = oracle_lib.block_stepwise(synth.REAL, w, x, None, None, mode=oracle_lib.EXACT)
    assert np.allclose(step.out, seq.out, rtol=1e-12, atol=1e-12)
    rel = np.linalg.norm(step.ssm_state - seq.ssm_state) / np.linalg.norm(seq.ssm_state)
    assert rel < 1e-12


def test_resume_seq_prefix_then_steps(oracle_lib):
    w = _tiny_weights(2)
    T, t0 = 12, 5
    x = _x(T, seed=4)
    full = oracle_lib.block(TINY, w, x, np.zeros((1, 3, TINY.conv_dim)), None, mode=oracle_lib.EXACT)
    pre = oracle_lib.block(TINY, w, x[:, :t0], np.zeros((1, 3, TINY.conv_dim)), None,
                           mode=oracle_lib.EXACT)
    rest = oracle_lib.block_stepwise(TINY, w, x[:, t0:], pre.conv_state, pre.ssm_state,
                                     mode=oracle_lib.EXACT)
    assert np.allclose(np.concatenate([pre.out, rest.out], axis=1), full.out, rtol=1e-12, atol=1e-12)
    assert np.allclose(rest.ssm_state, full.ssm_state, rtol=1e-12, atol=1e-13)


def test_full_history_prefix_causality(oracle_lib):
    w = _tiny_weights(3)
    T = 16
    x = _x(T, seed=5)
    full = oracle_lib.block(TINY, w, x, None, None, mode=oracle_lib.CONTRACT)
    for t in [1, 5, 16]:
        pre = oracle_lib.block(TINY, w, x[:, :t], None, None, mode=oracle_lib.CONTRACT)
        assert np.array_equal(pre.out[:, -1], full.out[:, t - 1])


def test_contract_storage_points_are_bf16(oracle_lib):
    w = _tiny_weights(4)
    x = _x(5, seed=6)
    r = oracle_lib.block(TINY, w, x, None, None, mode=oracle_lib.CONTRACT, debug=True)
    for k in ("u", "zxbcdt", "xc", "y", "o"):
        v = r.debug[k]
        assert np.array_equal(oracle_lib.round_bf16(v), v), k
    e = oracle_lib.block(TINY, w, x, None, None, mode=oracle_lib.EXACT)
    rel = np.linalg.norm(r.out - e.out) / np.linalg.norm(e.out)
    assert rel < 1e-2


def test_stack_composes_blocks_in_pattern_order(oracle_lib):
    n_m = len(oracle_lib.layers_of_kind("M"))
    ws = [_tiny_weights(i) for i in range(n_m)]
    x = _x(3, seed=7)
    outs, _, _ = oracle_lib.stack(TINY, ws, x, mode=oracle_lib.EXACT)
    h = x
    for i in range(n_m):
        h = oracle_lib.block(TINY, ws[i], h, None, None, mode=oracle_lib.EXACT).out
        assert np.array_equal(outs[i], h)
