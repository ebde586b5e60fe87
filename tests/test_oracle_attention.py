"""Pins for the oracle's grouped-query attention (the '*' layers of the hybrid stack).

Constants: the issue page "feat(nemotron_voicechat): ... offline duplex inference #1374",
section "config.json" (num_attention_heads 40, num_key_value_heads 8, head_dim 128,
attention_bias false, attention at layers 14, 21, 30, 39); the docs page "Nemotron
VoiceChat", section "Online session" (attention key/value caches persist across positions).
Each check compares the oracle with something other than itself: closed forms (equal keys give
the mean of the values, one position gives its value, a dominant key gives its value), the
grouping of query heads onto key/value heads, torch's scaled_dot_product_attention on
repeated key/value heads, and the whole layer against a composition of torch library ops on
independently decoded 4-bit weights."""
import numpy as np
import torch
import torch.nn.functional as F

import synth


def _byte_split_dequant(W):
    """Independent decoding of the 4-bit matrix: bytes hold two consecutive k, low nibble first."""
    b = W.qweight.view(np.uint8).reshape(W.n_out, W.k_in // 2)
    q = np.empty((W.n_out, W.k_in), dtype=np.int64)
    q[:, 0::2] = b & 0xF
    q[:, 1::2] = b >> 4
    s = np.repeat(synth.bf16_to_f32(W.scales).astype(np.float64), W.group_size, axis=1)
    bi = np.repeat(synth.bf16_to_f32(W.biases).astype(np.float64), W.group_size, axis=1)
    return s * q + bi


def test_equal_keys_give_the_mean_of_the_values(oracle_lib):
    rng = np.random.default_rng(1)
    heads, n_kv, T, hd = 10, 2, 7, 16
    q = rng.normal(size=(heads, hd))
    K = np.repeat(rng.normal(size=(n_kv, 1, hd)), T, axis=1)     # every position the same key
    V = rng.normal(size=(n_kv, T, hd))
    o = oracle_lib.attention_core(q, K, V, n_kv)
    for h in range(heads):
        assert np.allclose(o[h], V[h // 5].mean(axis=0), rtol=1e-13, atol=1e-13)


def test_one_position_gives_its_value_and_a_dominant_key_wins(oracle_lib):
    rng = np.random.default_rng(2)
    heads, n_kv, hd = 8, 4, 16
    q = rng.normal(size=(heads, hd))
    V1 = rng.normal(size=(n_kv, 1, hd))
    o = oracle_lib.attention_core(q, rng.normal(size=(n_kv, 1, hd)), V1, n_kv)
    for h in range(heads):
        assert np.allclose(o[h], V1[h // 2, 0], rtol=0, atol=1e-15)
    # a key equal to 60 sqrt(hd) q / |q|^2 scores 60 above the others (scores of 0): its
    # value carries weight 1 / (1 + (T - 1) e^-60)
    T = 9
    K = np.zeros((n_kv, T, hd))
    V = rng.normal(size=(n_kv, T, hd))
    for g in range(n_kv):
        qa = q[2 * g]
        K[g, 4] = 60.0 * np.sqrt(hd) * qa / (qa @ qa)
    o = oracle_lib.attention_core(q, K, V, n_kv)
    for g in range(n_kv):
        w = 1.0 / (1.0 + (T - 1) * np.exp(-60.0))
        want = w * V[g, 4] + (1 - w) / (T - 1) * (V[g].sum(axis=0) - V[g, 4])
        assert np.allclose(o[2 * g], want, rtol=1e-12, atol=1e-12)


def test_query_heads_group_onto_key_value_heads(oracle_lib):
    # perturbing key/value head g changes exactly the query heads 5g .. 5g + 4 (40 onto 8)
    rng = np.random.default_rng(3)
    heads, n_kv, T, hd = 40, 8, 5, 8
    q, K, V = rng.normal(size=(heads, hd)), rng.normal(size=(n_kv, T, hd)), rng.normal(size=(n_kv, T, hd))
    base = oracle_lib.attention_core(q, K, V, n_kv)
    for g in (0, 3, 7):
        K2, V2 = K.copy(), V.copy()
        K2[g] += 0.5
        V2[g] -= 0.25
        o = oracle_lib.attention_core(q, K2, V2, n_kv)
        changed = np.flatnonzero(np.abs(o - base).max(axis=1) > 0)
        assert list(changed) == list(range(5 * g, 5 * g + 5))


def test_matches_torch_sdpa_on_repeated_kv_heads(oracle_lib):
    rng = np.random.default_rng(4)
    heads, n_kv, T, hd = 40, 8, 33, 128
    q = rng.normal(size=(heads, hd))
    K, V = rng.normal(size=(n_kv, T, hd)), rng.normal(size=(n_kv, T, hd))
    Kt = torch.from_numpy(K).repeat_interleave(heads // n_kv, dim=0)   # [heads][T][hd]
    Vt = torch.from_numpy(V).repeat_interleave(heads // n_kv, dim=0)
    want = F.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], Kt, Vt)[:, 0, :].numpy()
    got = oracle_lib.attention_core(q, K, V, n_kv)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_layer_matches_library_pieces(oracle_lib):
    # EXACT mode is torch's rms_norm, independently decoded matmuls, torch SDPA on repeated
    # key/value heads over [cache; new], and the residual.  Small heads keep it quick.
    rng = np.random.default_rng(5)
    hidden, heads, n_kv, hd, T, m = 128, 8, 2, 16, 6, 2
    aw = synth.AttentionWeights(
        synth.f32_to_bf16((1 + 0.05 * rng.normal(size=hidden)).astype(np.float32)),
        synth.w4_random(7, 1, 1, 2, heads * hd, hidden), synth.w4_random(7, 1, 3, 4, n_kv * hd, hidden),
        synth.w4_random(7, 1, 5, 6, n_kv * hd, hidden), synth.w4_random(7, 1, 7, 8, hidden, heads * hd))
    x = rng.normal(size=(m, hidden))
    kc, vc = rng.normal(size=(m, n_kv, T, hd)), rng.normal(size=(m, n_kv, T, hd))
    out, k_new, v_new = oracle_lib.attention(x, aw, kc, vc, 1e-5, mode=oracle_lib.EXACT)
    wd = torch.from_numpy(synth.bf16_to_f32(aw.norm_w).astype(np.float64))
    u = F.rms_norm(torch.from_numpy(x), (hidden,), weight=wd, eps=1e-5)
    Wq, Wk, Wv, Wo = (torch.from_numpy(_byte_split_dequant(W)) for W in (aw.q_proj, aw.k_proj, aw.v_proj, aw.o_proj))
    q = (u @ Wq.T).reshape(m, heads, 1, hd)
    k = (u @ Wk.T).reshape(m, n_kv, 1, hd)
    v = (u @ Wv.T).reshape(m, n_kv, 1, hd)
    K = torch.cat([torch.from_numpy(kc), k], dim=2).repeat_interleave(heads // n_kv, dim=1)
    V = torch.cat([torch.from_numpy(vc), v], dim=2).repeat_interleave(heads // n_kv, dim=1)
    o = F.scaled_dot_product_attention(q, K, V).reshape(m, heads * hd)
    want = (torch.from_numpy(x) + o @ Wo.T).numpy()
    assert np.allclose(out, want, rtol=1e-11, atol=1e-11)
    assert np.allclose(k_new, k[:, :, 0, :].numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(v_new, v[:, :, 0, :].numpy(), rtol=1e-12, atol=1e-12)


def test_empty_cache_attends_to_the_new_position_only(oracle_lib):
    # T = 0: the single key is the new one, so o is v repeated over each group of query heads
    rng = np.random.default_rng(6)
    hidden, heads, n_kv, hd = 128, 4, 2, 16
    aw = synth.AttentionWeights(
        synth.f32_to_bf16(np.ones(hidden, np.float32)),
        synth.w4_random(8, 1, 1, 2, heads * hd, hidden), synth.w4_random(8, 1, 3, 4, n_kv * hd, hidden),
        synth.w4_random(8, 1, 5, 6, n_kv * hd, hidden), synth.w4_random(8, 1, 7, 8, hidden, heads * hd))
    x = rng.normal(size=(1, hidden))
    empty = np.zeros((1, n_kv, 0, hd))
    out, _, v_new = oracle_lib.attention(x, aw, empty, empty, 1e-5, mode=oracle_lib.CONTRACT)
    o = oracle_lib.round_bf16(np.repeat(v_new[0], heads // n_kv, axis=0).reshape(1, -1))
    want = x + oracle_lib.w4_matvec(aw.o_proj, o)
    assert np.allclose(out, want, rtol=1e-14, atol=1e-14)
