"""Pins for the CPU oracle: each oracle function is checked against something other
than itself -- printed facts from the pages, closed forms, special cases that reduce
to library routines, brute-force sums on tiny inputs, and invariants of the method.

Sources: the issue page "feat(nemotron_voicechat): ... offline duplex inference #1374"
(section "config.json" for the constants, quantization and layer pattern; "Network 2"
for the conv weight layout) and the docs page "Nemotron VoiceChat" (section "Offline
timeline": full-history recompute and the cached mode agree).  The Mamba2 equations
are the standard selective-SSM mixer (Dao & Gu 2024).
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# A tiny block with every structural feature of the real one (groups of heads, two
# quantization groups per input row, K=4 conv, several heads per B/C group).
TINY = synth.Dims(hidden=128, n_heads=4, head_dim=16, d_state=16, n_groups=2, conv_k=4,
                  group_size=64, eps=1e-5)


# --------------------------------------------------------------------- bf16

def test_bf16_rounding_matches_torch(oracle_lib):
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.normal(0, 1, 5000), rng.normal(0, 1e-3, 2000),
                        rng.uniform(-300, 300, 2000)]).astype(np.float32)
    ours = oracle_lib.to_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_ties_to_even(oracle_lib):
    # bf16 spacing in [1, 2) is 2^-7.  1 + 2^-8 is halfway between 1 (even mantissa) and
    # 1 + 2^-7 (odd): it rounds to 1.  1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and
    # 1 + 2^-6 (even): it rounds up.
    assert oracle_lib.to_bf16([1 + 2 ** -8])[0] == 0x3F80
    assert oracle_lib.to_bf16([1 + 3 * 2 ** -8])[0] == 0x3F82
    assert oracle_lib.to_bf16([-(1 + 3 * 2 ** -8)])[0] == 0xBF82
    assert oracle_lib.to_bf16([1 + 2 ** -8 + 2 ** -30])[0] == 0x3F81
    assert oracle_lib.to_bf16([0.0])[0] == 0
    assert oracle_lib.to_bf16([2.0 ** -130])[0] == 0x0008  # 8 steps of the subnormal grid 2^-133
    assert oracle_lib.to_bf16([3 * 2.0 ** -134])[0] == 0x0002  # 1.5 steps: tie -> even (2)


# ------------------------------------------------------------ scalar maps

def test_silu_softplus_closed_forms(oracle_lib):
    assert oracle_lib.silu(0.0) == 0.0
    assert abs(oracle_lib.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle_lib.silu(1.0) - 1.0 / (1.0 + math.e ** -1)) < 1e-15
    assert abs(oracle_lib.softplus(0.0) - math.log(2.0)) < 1e-15
    for v in [-30.0, -3.0, -0.5, 0.1, 2.0, 25.0, 700.0]:
        # softplus(v) - softplus(-v) = v
        assert abs(oracle_lib.softplus(v) - oracle_lib.softplus(-v) - v) < 1e-12 * max(1, abs(v))
    # round trip with the inverse used to draw dt_bias: softplus(ln(expm1(v))) = v
    for v in np.linspace(1e-3, 0.1, 17):
        assert abs(oracle_lib.softplus(math.log(math.expm1(v))) - v) < 1e-15


# ------------------------------------------------------------ layer map

def _golden_kv(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or not line.strip():
            continue
        k, *vals = line.split()
        out[k] = [int(v) for v in vals]
    return out


def test_layer_pattern_matches_printed_facts(oracle_lib):
    g = _golden_kv("layer_pattern.txt")
    p = oracle_lib.hybrid_pattern()
    assert len(p) == g["num_hidden_layers"][0]
    assert oracle_lib.layers_of_kind("*") == g["attention_layers"]
    assert len(oracle_lib.layers_of_kind("M")) == g["mamba_count"][0]
    assert len(oracle_lib.layers_of_kind("*")) == g["attention_count"][0]
    assert len(oracle_lib.layers_of_kind("-")) == g["mlp_count"][0]
    assert oracle_lib.layers_of_kind("M") == g["mamba_layers"]


# ------------------------------------------------------------------- W4

def test_nibble_unpack_handpacked(oracle_lib):
    for line in open(os.path.join(GOLDEN, "w4_handpacked.txt")):
        if line.startswith("#") or not line.strip():
            continue
        word, *nibs = line.split()
        w = np.array([int(word, 16)], dtype=np.uint32)
        assert [oracle_lib.w4_nibble(w, k) for k in range(8)] == [int(n) for n in nibs]


def _byte_split_dequant(W):
    """Independent decoding: view the packed words as little-endian bytes; each byte
    holds two consecutive k, the low nibble first."""
    b = W.qweight.view(np.uint8).reshape(W.n_out, W.k_in // 2)
    q = np.empty((W.n_out, W.k_in), dtype=np.int64)
    q[:, 0::2] = b & 0xF
    q[:, 1::2] = b >> 4
    s = np.repeat(synth.bf16_to_f32(W.scales).astype(np.float64), W.group_size, axis=1)
    bi = np.repeat(synth.bf16_to_f32(W.biases).astype(np.float64), W.group_size, axis=1)
    return q, s * q + bi


def test_dequant_handpacked_rows(oracle_lib):
    # row 0: every word 0x76543210 -> q = k % 8; row 1: 0xFEDCBA98 -> q = 8 + k % 8.
    qw = np.array([[0x76543210] * 16, [0xFEDCBA98] * 16], dtype=np.uint32)
    sc = synth.f32_to_bf16(np.array([[0.25, 0.5], [0.125, 1.0]], dtype=np.float32))
    bi = synth.f32_to_bf16(np.array([[-2.0, 0.0], [1.0, -8.0]], dtype=np.float32))
    W = synth.W4Matrix(qw, sc, bi, 2, 128, 64)
    got = oracle_lib.w4_dequant(W)
    k = np.arange(128)
    exp0 = np.where(k < 64, 0.25 * (k % 8) - 2.0, 0.5 * (k % 8))
    exp1 = np.where(k < 64, 0.125 * (8 + k % 8) + 1.0, 1.0 * (8 + k % 8) - 8.0)
    assert np.array_equal(got[0], exp0) and np.array_equal(got[1], exp1)


def test_gemv_all_ones_closed_form(oracle_lib):
    W = synth.w4_random(7, 0, 1, 2, 96, 256)
    q, _ = _byte_split_dequant(W)
    qsum = q.reshape(96, 4, 64).sum(axis=2)                     # integer group sums
    s = synth.bf16_to_f32(W.scales).astype(np.float64)
    b = synth.bf16_to_f32(W.biases).astype(np.float64)
    expect = (s * qsum + 64.0 * b).sum(axis=1)
    got = oracle_lib.w4_matvec(W, np.ones(256))
    assert np.allclose(got, expect, rtol=0, atol=1e-12)


def test_gemv_one_hot_and_library_matmul(oracle_lib):
    W = synth.w4_random(3, 1, 1, 2, 64, 192)
    _, Wd = _byte_split_dequant(W)
    # one-hot inputs select single columns exactly
    for k in [0, 1, 7, 8, 63, 64, 191]:
        e = np.zeros(192)
        e[k] = 1.0
        assert np.array_equal(oracle_lib.w4_matvec(W, e), Wd[:, k])
    x = np.random.default_rng(0).normal(size=(5, 192))
    assert np.allclose(oracle_lib.w4_matvec(W, x), x @ Wd.T, rtol=1e-13, atol=1e-12)


# ----------------------------------------------------------- output head

def test_greedy_ids_brute_force_rules(oracle_lib):
    # small integer-valued rows full of ties, with NaN and infinities mixed in
    rng = np.random.default_rng(11)
    rows = rng.integers(-3, 4, size=(200, 9)).astype(np.float64)
    rows[rng.random(rows.shape) < 0.15] = np.nan
    rows[rng.random(rows.shape) < 0.05] = -np.inf
    rows[rng.random(rows.shape) < 0.02] = np.inf
    rows[0] = np.nan
    rows[1] = -np.inf
    got = oracle_lib.greedy_ids(rows)
    for r, row in enumerate(rows):
        best, bi = None, -1
        for i, v in enumerate(row):
            if math.isnan(v):
                continue
            if best is None or v > best:
                best, bi = v, i
        assert got[r] == bi, (r, row)
    assert got[0] == -1 and got[1] == 0


def test_head_planted_maximum_closed_form(oracle_lib):
    # every nibble 9 and bias -8 s: row r of W is the constant s_r; a constant positive x
    # normalises to 1/sqrt(1 + eps/c^2), which rounds to 1.0 in bf16 for c = 3
    n, k, eps = 40, 4480, 1e-5
    q = np.full((n, k // 8), 0x99999999, dtype=np.uint32)
    s32 = np.linspace(0.002, 0.006, n).astype(np.float32)
    s32[[7, 23]] = np.float32(0.0075)                    # tied largest rows: 7 wins
    sb = synth.f32_to_bf16(np.repeat(s32[:, None], k // 64, axis=1))
    bb = synth.f32_to_bf16(synth.bf16_to_f32(sb) * np.float32(-8.0))
    W = synth.W4Matrix(q, sb, bb, n, k)
    sd = synth.bf16_to_f32(sb[:, 0]).astype(np.float64)
    x = np.full((2, k), 3.0)
    x[1] *= -1.0                                          # negative x: h = -1, smallest s wins
    wn = synth.f32_to_bf16(np.ones(k, dtype=np.float32))
    logits, ids = oracle_lib.head(W, x, wn, eps)
    assert np.allclose(logits[0], k * sd, rtol=1e-14) and np.allclose(logits[1], -k * sd, rtol=1e-14)
    assert ids[0] == 7 and ids[1] == int(np.argmin(sd))
    ex, _ = oracle_lib.head(W, x, wn, eps, mode=oracle_lib.EXACT)
    assert np.allclose(ex[0], k * sd / math.sqrt(1 + eps / 9.0), rtol=1e-14)


def test_head_matches_library_pieces(oracle_lib):
    # EXACT mode is torch's rms_norm followed by a matmul with the byte-split dequantised W
    rng = np.random.default_rng(12)
    W = synth.w4_random(5, 2, 1, 2, 96, 4480)
    _, Wd = _byte_split_dequant(W)
    x = rng.normal(size=(3, 4480))
    wn = synth.f32_to_bf16((1 + 0.05 * rng.normal(size=4480)).astype(np.float32))
    wd = torch.from_numpy(synth.bf16_to_f32(wn).astype(np.float64))
    h = F.rms_norm(torch.from_numpy(x), (4480,), weight=wd, eps=1e-5).numpy()
    logits, ids = oracle_lib.head(W, x, wn, 1e-5, mode=oracle_lib.EXACT)
    assert np.allclose(logits, h @ Wd.T, rtol=1e-12, atol=1e-12)
    assert np.array_equal(ids, np.argmax(h @ Wd.T, axis=1))


def test_fused_embedding_handpacked_closed_form(oracle_lib):
    # row 0: every word 0x76543210 (q = k % 8), scale 0.25, bias -2 -> 0.25 (k % 8) - 2;
    # row 1: every word 0xFEDCBA98 (q = 8 + k % 8), scale 0.5, bias 1 -> 0.5 (8 + k % 8) + 1
    k = 128
    qw = np.array([[0x76543210] * 16, [0xFEDCBA98] * 16], dtype=np.uint32)
    s = synth.f32_to_bf16(np.array([[0.25, 0.25], [0.5, 0.5]], dtype=np.float32))
    b = synth.f32_to_bf16(np.array([[-2.0, -2.0], [1.0, 1.0]], dtype=np.float32))
    E = synth.W4Matrix(qw, s, b, 2, k)
    kk = np.arange(k)
    e0, e1 = 0.25 * (kk % 8) - 2.0, 0.5 * (8 + kk % 8) + 1.0
    audio = np.stack([np.linspace(-1, 1, k), np.full(k, 0.5), np.zeros(k)])
    got = oracle_lib.fused_embedding(E, [0, 1, 1], [1, 0, 1], audio, 2.0)
    assert np.array_equal(got[0], e0 + audio[0] + 2 * e1)
    assert np.array_equal(got[1], e1 + audio[1] + 2 * e0)
    assert np.array_equal(got[2], 3 * e1)
    assert np.array_equal(oracle_lib.fused_embedding(E, [1], [0], audio[:1], 0.0)[0], e1 + audio[0])


def test_fused_embedding_independent_decode_and_bad_ids(oracle_lib):
    rng = np.random.default_rng(13)
    E = synth.w4_random(9, 3, 1, 2, 50, 4480)
    _, Ed = _byte_split_dequant(E)
    t, f = np.array([0, 49, 12, 7]), np.array([12, 0, 49, 7])
    audio = rng.normal(size=(4, 4480))
    got = oracle_lib.fused_embedding(E, t, f, audio)
    assert np.allclose(got, Ed[t] + audio + 2.0 * Ed[f], rtol=0, atol=1e-15)
    bad = oracle_lib.fused_embedding(E, [-1, 3, 50], [3, 50, 3], audio[:3])
    assert np.isnan(bad).all()


def _const_w4(vals, k):
    """Rows of constant value v (every nibble 9, bias -8 s, scale s = v): W[n][k] = v_n."""
    n = len(vals)
    q = np.full((n, k // 8), 0x99999999, dtype=np.uint32)
    sb = synth.f32_to_bf16(np.repeat(np.asarray(vals, np.float32)[:, None], k // 64, axis=1))
    bb = synth.f32_to_bf16(synth.bf16_to_f32(sb) * np.float32(-8.0))
    return synth.W4Matrix(q, sb, bb, n, k)


def test_mlp_closed_form(oracle_lib):
    # up rows: +0.25 (kept) and -0.25 (cut by the ReLU); down rows constant 0.5 and -1;
    # x = 3 everywhere normalises to h0 = 1/sqrt(1 + eps/9) (EXACT mode)
    k, inter, eps = 128, 192, 1e-5
    up = _const_w4([0.25] * 100 + [-0.25] * 92, k)
    down = _const_w4([0.5] * 64 + [-1.0] * 64, inter)
    wn = synth.f32_to_bf16(np.ones(k, dtype=np.float32))
    x = np.full((1, k), 3.0)
    h0 = 1.0 / math.sqrt(1 + eps / 9.0)
    a = 0.25 * k * h0                      # each kept unit
    m = 100 * a * a                        # sum over the kept units of relu(a)^2
    got = oracle_lib.mlp(x, wn, up, down, eps, mode=oracle_lib.EXACT)[0]
    want = np.r_[np.full(64, 3.0 + 0.5 * m), np.full(64, 3.0 - m)]
    assert np.allclose(got, want, rtol=1e-13)


def test_mlp_matches_library_pieces(oracle_lib):
    # EXACT mode is torch's rms_norm, two independently decoded matmuls and relu^2
    rng = np.random.default_rng(14)
    up = synth.w4_random(4, 5, 1, 2, 192, 256)
    down = synth.w4_random(4, 5, 3, 4, 256, 192)
    _, Ud = _byte_split_dequant(up)
    _, Dd = _byte_split_dequant(down)
    x = rng.normal(size=(3, 256))
    wn = synth.f32_to_bf16((1 + 0.05 * rng.normal(size=256)).astype(np.float32))
    wd = torch.from_numpy(synth.bf16_to_f32(wn).astype(np.float64))
    u = F.rms_norm(torch.from_numpy(x), (256,), weight=wd, eps=1e-5)
    h = torch.relu(u @ torch.from_numpy(Ud).T) ** 2
    want = (torch.from_numpy(x) + h @ torch.from_numpy(Dd).T).numpy()
    got = oracle_lib.mlp(x, wn, up, down, 1e-5, mode=oracle_lib.EXACT)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- norms

def test_rmsnorm_constant_vector_closed_form(oracle_lib):
    d, eps = 64, 1e-5
    w = synth.f32_to_bf16(np.linspace(0.5, 1.5, d).astype(np.float32))
    wd = synth.bf16_to_f32(w).astype(np.float64)
    for c in [3.0, -0.25, 1e-3]:
        got = oracle_lib.rmsnorm(np.full(d, c), w, eps)
        assert np.allclose(got, np.sign(c) * wd / math.sqrt(1 + eps / c ** 2), rtol=1e-14)


def test_rmsnorm_matches_torch_library(oracle_lib):
    x = np.random.default_rng(2).normal(size=(3, 4480))
    w = synth.f32_to_bf16(1 + 0.05 * np.random.default_rng(3).normal(size=4480).astype(np.float32))
    wd = torch.from_numpy(synth.bf16_to_f32(w).astype(np.float64))
    ref = F.rms_norm(torch.from_numpy(x), (4480,), weight=wd, eps=1e-5).numpy()
    assert np.allclose(oracle_lib.rmsnorm(x, w, 1e-5), ref, rtol=1e-13, atol=1e-14)


def test_gated_norm_groups_and_library(oracle_lib):
    rng = np.random.default_rng(4)
    d, grp = 1280 * 2, 1280
    y, z = rng.normal(size=(2, d)), rng.normal(size=(2, d))
    w = synth.f32_to_bf16(1 + 0.05 * rng.normal(size=d).astype(np.float32))
    got = oracle_lib.rmsnorm_gated(y, z, w, grp, 1e-5)
    # library composition: silu gate, then rms_norm per group
    g = torch.from_numpy(y) * F.silu(torch.from_numpy(z))
    wd = torch.from_numpy(synth.bf16_to_f32(w).astype(np.float64))
    ref = torch.cat([F.rms_norm(g[:, j * grp:(j + 1) * grp], (grp,), weight=wd[j * grp:(j + 1) * grp],
                                eps=1e-5) for j in range(d // grp)], dim=1).numpy()
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-14)
    # group independence: perturbing group 1 leaves group 0 unchanged
    y2 = y.copy()
    y2[:, grp + 5] += 3.0
    got2 = oracle_lib.rmsnorm_gated(y2, z, w, grp, 1e-5)
    assert np.array_equal(got2[:, :grp], got[:, :grp])
    assert not np.allclose(got2[:, grp:], got[:, grp:])


# ----------------------------------------------------------------- conv

def test_conv_single_tap_kernels(oracle_lib):
    rng = np.random.default_rng(5)
    T, Cn, K = 7, 6, 4
    x = rng.normal(size=(T, Cn))
    st = rng.normal(size=(K - 1, Cn))
    zero_b = np.zeros(Cn, dtype=np.uint16)
    one = np.uint16(0x3F80)
    w3 = np.zeros((Cn, K), dtype=np.uint16)
    w3[:, 3] = one     # newest tap only -> silu(x_t)
    out, st_out = oracle_lib.conv1d(x, w3, zero_b, st)
    assert np.allclose(out, x / (1 + np.exp(-x)), rtol=1e-15)
    assert np.array_equal(st_out, x[-3:])
    w0 = np.zeros((Cn, K), dtype=np.uint16)
    w0[:, 0] = one     # oldest tap only -> silu(x_{t-3}), the first three read the state
    out0, _ = oracle_lib.conv1d(x, w0, zero_b, st)
    src = np.concatenate([st, x])[:T]
    assert np.allclose(out0, src / (1 + np.exp(-src)), rtol=1e-15)


def test_conv_matches_torch_library_and_continuation(oracle_lib):
    rng = np.random.default_rng(6)
    T, Cn, K = 11, 12, 4
    x = rng.normal(size=(T, Cn))
    w = synth.f32_to_bf16(rng.normal(0, 0.25, (Cn, K)).astype(np.float32))
    b = synth.f32_to_bf16(rng.normal(0, 0.1, Cn).astype(np.float32))
    out, st = oracle_lib.conv1d(x, w, b, None)
    wt = torch.from_numpy(synth.bf16_to_f32(w).astype(np.float64)).reshape(Cn, 1, K)
    bt = torch.from_numpy(synth.bf16_to_f32(b).astype(np.float64))
    xt = F.pad(torch.from_numpy(x.T.copy()).unsqueeze(0), (K - 1, 0))
    ref = F.silu(F.conv1d(xt, wt, bt, groups=Cn))[0].T.numpy()
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-15)
    # carrying the state across a split gives the unsplit result
    for t in [1, 2, 3, 5]:
        o1, s1 = oracle_lib.conv1d(x[:t], w, b, None)
        o2, s2 = oracle_lib.conv1d(x[t:], w, b, s1)
        assert np.allclose(np.concatenate([o1, o2]), out, rtol=1e-14, atol=1e-15)
        assert np.array_equal(s2, st)


def test_discretize(oracle_lib):
    H = 5
    v = np.linspace(1e-3, 0.1, H)
    dt_bias = np.log(np.expm1(v)).astype(np.float32)
    A_log = np.log(np.arange(1, H + 1, dtype=np.float64)).astype(np.float32)
    dt, A = oracle_lib.discretize(np.zeros((1, H)), dt_bias, A_log)
    assert np.allclose(dt[0], v, rtol=1e-6)           # float32 dt_bias
    assert np.allclose(A, -np.exp(A_log.astype(np.float64)), rtol=1e-15)
    assert np.allclose(A, -np.arange(1, H + 1), rtol=1e-6)


# ------------------------------------------------------------------ SSM

def _ssm_problem(rng, T, H=4, P=3, N=5, G=2, s0_scale=0.3):
    x = rng.normal(size=(T, H * P))
    Bm = rng.normal(size=(T, G * N))
    Cm = rng.normal(size=(T, G * N))
    dt = rng.uniform(0.01, 0.5, size=(T, H))
    A = -rng.uniform(0.5, 4.0, size=H)
    D = rng.uniform(0.5, 1.5, size=H).astype(np.float32)
    S0 = s0_scale * rng.normal(size=(H, P, N))
    return x, Bm, Cm, dt, A, D, S0


def _brute_force_dual(x, Bm, Cm, dt, A, D, S0, G):
    """Explicit sums of the SSD 'dual' (attention-like) form:
    y_t = sum_{s<=t} (C_t.B_s) exp(A sum_{r=s+1..t} dt_r) dt_s x_s
          + C_t.(exp(A sum_{r<=t} dt_r) S0) + D x_t."""
    T = x.shape[0]
    H, P, N = S0.shape
    hpg = H // G
    y = np.zeros((T, H * P))
    for t in range(T):
        for h in range(H):
            g = h // hpg
            Ct = Cm[t, g * N:(g + 1) * N]
            for p in range(P):
                acc = 0.0
                for s in range(t + 1):
                    decay = math.exp(A[h] * sum(dt[r, h] for r in range(s + 1, t + 1)))
                    acc += float(Ct @ Bm[s, g * N:(g + 1) * N]) * decay * dt[s, h] * x[s, h * P + p]
                decay0 = math.exp(A[h] * sum(dt[r, h] for r in range(t + 1)))
                acc += float(Ct @ (decay0 * S0[h, p]))
                y[t, h * P + p] = acc + float(D[h]) * x[t, h * P + p]
    return y


@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_recurrence_equals_brute_force_dual_form(oracle_lib, T):
    rng = np.random.default_rng(10 + T)
    x, Bm, Cm, dt, A, D, S0 = _ssm_problem(rng, T)
    y, _ = oracle_lib.ssm_recurrence(x, Bm, Cm, dt, A, D, S0, G=2)
    ref = _brute_force_dual(x, Bm, Cm, dt, A, D, S0, G=2)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_recurrence_special_cases(oracle_lib):
    rng = np.random.default_rng(20)
    x, Bm, Cm, dt, A, D, S0 = _ssm_problem(rng, 1)
    H, P, N = S0.shape
    # T = 1 from zero state: y = dt (C.B) x + D x
    y, S = oracle_lib.ssm_recurrence(x, Bm, Cm, dt, A, D, np.zeros_like(S0), G=2)
    for h in range(H):
        g = h // 2
        cb = float(Cm[0, g * N:(g + 1) * N] @ Bm[0, g * N:(g + 1) * N])
        assert np.allclose(y[0, h * P:(h + 1) * P],
                           dt[0, h] * cb * x[0, h * P:(h + 1) * P] + D[h] * x[0, h * P:(h + 1) * P],
                           rtol=1e-13)
    # dt = 0 leaves the state unchanged and reads it out through C
    y, S = oracle_lib.ssm_recurrence(x, Bm, Cm, np.zeros_like(dt), A, D, S0, G=2)
    assert np.array_equal(S, S0)
    for h in range(H):
        g = h // 2
        assert np.allclose(y[0, h * P:(h + 1) * P],
                           S0[h] @ Cm[0, g * N:(g + 1) * N] + D[h] * x[0, h * P:(h + 1) * P],
                           rtol=1e-13)
    # A -> -inf: memoryless, S_t = dt x (outer) B
    x5, B5, C5, dt5, _, D5, S05 = _ssm_problem(rng, 5)
    _, S = oracle_lib.ssm_recurrence(x5, B5, C5, dt5, np.full(H, -1e30), D5, S05, G=2)
    for h in range(H):
        g = h // 2
        assert np.allclose(S[h], dt5[-1, h] * np.outer(x5[-1, h * P:(h + 1) * P],
                                                         B5[-1, g * N:(g + 1) * N]), rtol=1e-14)


@pytest.mark.parametrize("Q", [1, 2, 3, 5, 8, 16])
def test_chunked_ssd_equals_recurrence(oracle_lib, Q):
    for T in range(1, 18):
        rng = np.random.default_rng(100 * Q + T)
        x, Bm, Cm, dt, A, D, S0 = _ssm_problem(rng, T)
        y, S = oracle_lib.ssm_recurrence(x, Bm, Cm, dt, A, D, S0, G=2)
        yc, Sc = oracle_lib.ssd_chunked(x, Bm, Cm, dt, A, D, S0, G=2, Q=Q)
        assert np.allclose(yc, y, rtol=1e-11, atol=1e-11)
        assert np.allclose(Sc, S, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("T,Q", [(413, 128), (300, 256), (256, 256), (129, 128)])
def test_chunked_ssd_equals_recurrence_long(oracle_lib, T, Q):
    rng = np.random.default_rng(T + Q)
    x, Bm, Cm, dt, A, D, S0 = _ssm_problem(rng, T, H=4, P=8, N=16, G=2)
    dt *= 0.2
    y, S = oracle_lib.ssm_recurrence(x, Bm, Cm, dt, A, D, S0, G=2)
    yc, Sc = oracle_lib.ssd_chunked(x, Bm, Cm, dt, A, D, S0, G=2, Q=Q)
    assert np.allclose(yc, y, rtol=1e-10, atol=1e-10)
    assert np.allclose(Sc, S, rtol=1e-10, atol=1e-10)
