"""GPU parity of the attention layers (nh_attention_decode, nh_attention_step) against the
oracle's attention_core and attention, through the C ABI.

Cases: caches of 0, 1, 16 and 413 earlier positions at batch 1; ragged batches (each sequence
its own position, one of them past a split boundary); long caches that spread each key/value
head over many work-groups (4096 and 10000 positions); a peaked softmax (q scaled by 16); a
position outside the cache (its row must be NaN and the cache untouched, the other rows
exact); three consecutive positions appended by the kernels themselves.

Cache rows past the attended range are filled with NaN, so any read beyond positions[b]
would surface as a NaN output.

Tolerances.  The attention output o is rounded to bf16 on both sides; the GPU sums in fp32
(scores, softmax weights, the weighted value sums), so o differs from the oracle's fp64 value
by its half-ulp rounding plus fp32 sums over at most 10^4 positions: every 128-value head row
is held to 4e-3 of its own norm (1 bf16 ulp is 2^-8 = 3.9e-3 of a value), and no more than 2%
of the bf16 values may round differently.  The new k and v rows are single W4 rows of fp32
sums of 4480 terms rounded to bf16: at most 1% of them may round differently and none by more
than one ulp.  The layer's contribution out - x (the o_proj product) is held to rel-L2 5e-3
per row, the block bar."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

NAN16 = 0x7FC0
HEADS, KVH, HD = 40, 8, 128


@pytest.fixture(scope="module")
def env():
    import torch
    import hybrid_mamba2_decode_amd as nh
    import oracle
    from tests import gpu_util as gu
    oracle.build(force=False)
    assert torch.cuda.is_available()
    return nh, oracle, gu, torch


def _cache(batch, lens, max_len, seed=0):
    """bf16 caches [batch][8][max_len][128]: sequence b's first lens[b] rows from synth.kv_cache,
    the rest NaN."""
    k = np.full((batch, KVH, max_len, HD), NAN16, np.uint16)
    v = np.full((batch, KVH, max_len, HD), NAN16, np.uint16)
    for b, L in enumerate(lens):
        if L > 0:
            kb, vb = synth.kv_cache(100 * seed + b, 1, L, seed=seed)
            k[b, :, :L], v[b, :, :L] = kb[0], vb[0]
    return k, v


def _attn_dev(nh, gu, aw):
    return nh.attention_weights(gu.to_dev(aw.norm_w), gu.w4_dev(aw.q_proj), gu.w4_dev(aw.k_proj),
                                gu.w4_dev(aw.v_proj), gu.w4_dev(aw.o_proj))


def _check_o(gu, oracle, got_bits, ref, what):
    got = gu.bf16_bits_to_f64(got_bits)
    worst, mabs, mref = gu.row_errors(got, ref, row=HD)
    flips = gu.bf16_ulp_flips(got_bits, ref)
    print(f"[{what}] o head-row rel {worst:.2e} max-abs {mabs:.2e} (max |o| {mref:.2f}) "
          f"flips {flips}/{ref.size}", flush=True)
    assert np.isfinite(got).all()
    assert worst <= 4e-3
    assert flips <= 0.02 * ref.size


@pytest.mark.parametrize("lens,max_len,qscale", [
    ((1,), 16, 1.0),
    ((2,), 64, 1.0),
    ((17,), 17, 1.0),
    ((64,), 200, 1.0),
    ((65,), 200, 1.0),
    ((414,), 1024, 1.0),
    ((414,), 1024, 16.0),
    ((4096,), 4096, 1.0),
    ((10000,), 12000, 1.0),
    ((1, 17, 414, 131), 500, 1.0),
    ((4097, 64), 5000, 1.0),
])
def test_attention_decode_core(env, lens, max_len, qscale):
    nh, oracle, gu, torch = env
    B = len(lens)
    print(f"[case] attention core lens {lens} max_len {max_len} qscale {qscale}", flush=True)
    k, v = _cache(B, lens, max_len, seed=1)
    qf = synth.rng(3, len(lens), max_len).normal(0.0, 1.2 * qscale, (B, HEADS, HD)).astype(np.float32)
    q = oracle.to_bf16(qf)
    pos = np.array([L - 1 for L in lens], np.int32)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    cache = nh.kv_cache(kd, vd, max_len)
    o = gu.empty_u16(B, HEADS, HD)
    ws = gu.workspace(nh.nh_attention_decode_workspace_bytes(B))
    nh.nh_attention_decode(gu.to_dev(q), cache, gu.to_dev(pos), o, B, ws, ws.numel())
    torch.cuda.synchronize()
    got = gu.from_dev_u16(o)
    for b, L in enumerate(lens):
        ref = oracle.attention_core(oracle.bf16_to_double(q[b]), oracle.bf16_to_double(k[b, :, :L]),
                                    oracle.bf16_to_double(v[b, :, :L]), KVH)
        _check_o(gu, oracle, got[b], ref, f"core L={L} b={b}")
    # the caches are read only
    assert np.array_equal(gu.from_dev_u16(kd), k) and np.array_equal(gu.from_dev_u16(vd), v)


def test_attention_decode_invalid_position(env):
    nh, oracle, gu, torch = env
    print("[case] attention core with a position outside the cache", flush=True)
    lens, max_len = (30, 1, 5), 64
    k, v = _cache(3, lens, max_len, seed=2)
    q = oracle.to_bf16(synth.rng(4, 0, 0).normal(0.0, 1.2, (3, HEADS, HD)).astype(np.float32))
    for bad in (max_len, -1):
        pos = np.array([lens[0] - 1, bad, lens[2] - 1], np.int32)
        o = gu.empty_u16(3, HEADS, HD)
        ws = gu.workspace(nh.nh_attention_decode_workspace_bytes(3))
        nh.nh_attention_decode(gu.to_dev(q), nh.kv_cache(gu.to_dev(k), gu.to_dev(v), max_len), gu.to_dev(pos), o, 3,
                               ws, ws.numel())
        torch.cuda.synchronize()
        got = gu.from_dev_u16(o)
        assert np.isnan(gu.bf16_bits_to_f64(got[1])).all()
        for b in (0, 2):
            L = lens[b]
            ref = oracle.attention_core(oracle.bf16_to_double(q[b]), oracle.bf16_to_double(k[b, :, :L]),
                                        oracle.bf16_to_double(v[b, :, :L]), KVH)
            _check_o(gu, oracle, got[b], ref, f"core invalid-neighbour b={b}")


def _check_step(gu, oracle, out, x64, ref_out, k_dev, v_dev, k_before, v_before, pos, ref_k, ref_v, what):
    for b in range(out.shape[0]):
        d_got, d_ref = out[b] - x64[b], ref_out[b] - x64[b]
        r = gu.rel_l2(d_got, d_ref)
        print(f"[{what} b={b}] out - x rel-L2 {r:.2e}", flush=True)
        assert r <= 5e-3
    kg, vg = gu.from_dev_u16(k_dev), gu.from_dev_u16(v_dev)
    for b, p in enumerate(pos):
        for name, got_c, ref_new, before in (("k", kg, ref_k, k_before), ("v", vg, ref_v, v_before)):
            new = got_c[b, :, p]
            flips = gu.bf16_ulp_flips(new, ref_new[b])
            err = np.abs(gu.bf16_bits_to_f64(new) - ref_new[b])
            assert flips <= 0.01 * new.size, (name, b, flips)
            assert np.all(err <= 2.0 ** -6 * np.abs(ref_new[b]) + 1e-5), (name, b, err.max())
            # every other cache row unchanged
            other = np.ones(got_c.shape[2], bool)
            other[p] = False
            assert np.array_equal(got_c[b][:, other], before[b][:, other]), (name, b)


@pytest.mark.parametrize("lens,max_len,xt,ot", [
    ((0,), 16, 0, 1),
    ((1,), 16, 0, 1),
    ((16,), 64, 1, 1),
    ((413,), 1024, 0, 1),
    ((413, 16), 500, 1, 0),
    ((1, 16, 413, 130), 448, 0, 1),
    ((7, 300, 2), 320, 1, 1),
])
def test_attention_step(env, lens, max_len, xt, ot):
    nh, oracle, gu, torch = env
    B = len(lens)
    print(f"[case] attention step lens {lens} max_len {max_len} x {'f32' if xt else 'bf16'} "
          f"out {'f32' if ot else 'bf16'}", flush=True)
    aw = synth.attention_weights(len(lens), seed=5)
    w = _attn_dev(nh, gu, aw)
    k, v = _cache(B, lens, max_len, seed=3)
    xb = synth.block_input(7, B, 1)[:, 0]
    if xt == nh.NH_F32:
        x64 = synth.rng(8, B, 0).normal(0.0, 1.0, (B, 4480)).astype(np.float32).astype(np.float64)
        x_dev = gu.to_dev(x64.astype(np.float32))
    else:
        x64 = oracle.bf16_to_double(xb)
        x_dev = gu.to_dev(xb)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    pos = np.array(lens, np.int32)
    out = gu.empty_f32(B, 4480) if ot == nh.NH_F32 else gu.empty_u16(B, 4480)
    ws = gu.workspace(nh.nh_attention_workspace_bytes(B))
    nh.nh_attention_step(w, nh.kv_cache(kd, vd, max_len), gu.to_dev(pos), x_dev, xt, out, ot, B, 1e-5, ws,
                         ws.numel())
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64) if ot == nh.NH_F32 else gu.bf16_bits_to_f64(gu.from_dev_u16(out))
    ref_out = np.empty((B, 4480))
    ref_k = np.empty((B, KVH, HD))
    ref_v = np.empty((B, KVH, HD))
    for b, L in enumerate(lens):
        r = oracle.attention(x64[b:b + 1], aw, oracle.bf16_to_double(k[b:b + 1, :, :L]),
                             oracle.bf16_to_double(v[b:b + 1, :, :L]), 1e-5)
        ref_out[b], ref_k[b], ref_v[b] = r[0][0], r[1][0], r[2][0]
    if ot == nh.NH_BF16:
        # bf16 out: the rounding of x + delta adds up to half an ulp of |out| per value
        for b in range(B):
            assert np.all(np.abs(got[b] - ref_out[b]) <= 2.0 ** -8 * np.abs(ref_out[b]) + 0.02)
        ref_out = oracle.bf16_to_double(oracle.to_bf16(ref_out))
    _check_step(gu, oracle, got, x64, ref_out, kd, vd, k, v, lens, ref_k, ref_v, f"step lens {lens}")


def test_attention_step_invalid_position(env):
    nh, oracle, gu, torch = env
    print("[case] attention step with a position outside the cache", flush=True)
    B, max_len, lens = 2, 32, (5, 32)
    aw = synth.attention_weights(9, seed=5)
    w = _attn_dev(nh, gu, aw)
    k, v = _cache(B, lens, max_len, seed=4)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    xb = synth.block_input(9, B, 1)[:, 0]
    out = gu.empty_f32(B, 4480)
    ws = gu.workspace(nh.nh_attention_workspace_bytes(B))
    nh.nh_attention_step(w, nh.kv_cache(kd, vd, max_len), gu.to_dev(np.array(lens, np.int32)), gu.to_dev(xb),
                         nh.NH_BF16, out, nh.NH_F32, B, 1e-5, ws, ws.numel())
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isnan(got[1]).all()
    assert np.array_equal(gu.from_dev_u16(kd)[1], k[1]) and np.array_equal(gu.from_dev_u16(vd)[1], v[1])
    x64 = oracle.bf16_to_double(xb)
    r = oracle.attention(x64[:1], aw, oracle.bf16_to_double(k[:1, :, :5]), oracle.bf16_to_double(v[:1, :, :5]), 1e-5)
    assert gu.rel_l2(got[0] - x64[0], r[0][0] - x64[0]) <= 5e-3


def test_attention_step_consecutive_positions(env):
    # three positions in a row; each step's k and v come from the kernels' own appends, and the
    # oracle is fed the GPU's cache of the earlier positions (teacher forcing)
    nh, oracle, gu, torch = env
    print("[case] attention step: three consecutive positions, batch 2", flush=True)
    B, max_len, lens = 2, 128, [15, 62]
    aw = synth.attention_weights(11, seed=5)
    w = _attn_dev(nh, gu, aw)
    k, v = _cache(B, lens, max_len, seed=6)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    cache = nh.kv_cache(kd, vd, max_len)
    ws = gu.workspace(nh.nh_attention_workspace_bytes(B))
    for step in range(3):
        xb = synth.block_input(20 + step, B, 1)[:, 0]
        x64 = oracle.bf16_to_double(xb)
        k_before, v_before = gu.from_dev_u16(kd), gu.from_dev_u16(vd)
        out = gu.empty_f32(B, 4480)
        pos = np.array(lens, np.int32)
        nh.nh_attention_step(w, cache, gu.to_dev(pos), gu.to_dev(xb), nh.NH_BF16, out, nh.NH_F32, B, 1e-5, ws,
                             ws.numel())
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        ref_out = np.empty((B, 4480))
        ref_k = np.empty((B, KVH, HD))
        ref_v = np.empty((B, KVH, HD))
        for b, L in enumerate(lens):
            r = oracle.attention(x64[b:b + 1], aw, oracle.bf16_to_double(k_before[b:b + 1, :, :L]),
                                 oracle.bf16_to_double(v_before[b:b + 1, :, :L]), 1e-5)
            ref_out[b], ref_k[b], ref_v[b] = r[0][0], r[1][0], r[2][0]
        _check_step(gu, oracle, got, x64, ref_out, kd, vd, k_before, v_before, lens, ref_k, ref_v,
                    f"consecutive step {step}")
        lens = [L + 1 for L in lens]
