"""GPU parity of one language-model position (nh_lm_step) against a composition of the CPU
oracle's functions, through the C ABI: the fused input row, all 56 layers in the order of the
hybrid pattern (27 Mamba2 blocks, 25 MLP layers, 4 attention layers with their key/value
caches), norm_f and both heads with their greedy ids.  Three positions in a row, each fed the
previous one's ids as the pages' greedy loop does, so the carried block states and the
caches the attention layers append to are exercised too.

Tolerances: the stream before norm_f is held to rel-L2 <= 5e-3 (the block bar; the 56 layers
each add about 3e-5).  Ids are checked as in the head test: each GPU id must be the greedy id
of the oracle's logits computed on the GPU's own stream, within 4e-3 of their maximum (a
vocabulary of 1000 rows keeps the oracle heads quick)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

VOCAB_T = 1000


@pytest.fixture(scope="module")
def env():
    import torch
    import hybrid_mamba2_decode_amd as nh
    import oracle
    from tests import gpu_util as gu
    oracle.build(force=False)
    assert torch.cuda.is_available()
    return nh, oracle, gu, torch


def test_lm_step_three_positions(env):
    nh, oracle, gu, torch = env
    pat = nh.hybrid_pattern()
    m_layers = [i for i, c in enumerate(pat) if c == "M"]
    f_layers = [i for i, c in enumerate(pat) if c == "-"]
    a_layers = [i for i, c in enumerate(pat) if c == "*"]
    print("[case] lm step: layers", len(m_layers), "mamba", len(f_layers), "mlp", len(a_layers), "attention",
          flush=True)
    lws = [synth.layer_weights(l) for l in range(len(m_layers))]
    mws = [synth.mlp_weights(l) for l in f_layers]
    aws = [synth.attention_weights(l) for l in a_layers]
    hw = synth.head_weights(seed=6, n_out=VOCAB_T)
    E = synth.embed_tokens(seed=6, n_out=VOCAB_T)
    mamba = [gu.layer_dev(lw) for lw in lws]
    mlp = [nh.mlp_weights(gu.to_dev(mw.norm_w), gu.w4_dev(mw.up), gu.w4_dev(mw.down)) for mw in mws]
    attn = [nh.attention_weights(gu.to_dev(aw.norm_w), gu.w4_dev(aw.q_proj), gu.w4_dev(aw.k_proj),
                                 gu.w4_dev(aw.v_proj), gu.w4_dev(aw.o_proj)) for aw in aws]
    w = nh.lm_weights(gu.w4_dev(E), mamba, mlp, attn, gu.to_dev(hw.norm_f), gu.w4_dev(hw.lm_head),
                      gu.w4_dev(hw.function_head), 2.0)
    d = nh.dims()
    states = [gu.state_dev(np.zeros((1, 3, synth.CONV_DIM), np.uint16),
                           np.zeros((1, 128, 80, 128), np.float32)) for _ in m_layers]
    max_len = 8
    kv = [(gu.empty_u16(1, 8, max_len, 128), gu.empty_u16(1, 8, max_len, 128)) for _ in a_layers]
    caches = [nh.kv_cache(k, v, max_len) for k, v in kv]
    o_kc = [np.zeros((1, 8, 0, 128)) for _ in a_layers]
    o_vc = [np.zeros((1, 8, 0, 128)) for _ in a_layers]
    ws = gu.workspace(nh.nh_lm_workspace_bytes(d, synth.MLP_INTER, 1))
    hid = gu.empty_f32(1, 4480)
    t_out = torch.empty(1, dtype=torch.int32, device=gu.DEV)
    f_out = torch.empty(1, dtype=torch.int32, device=gu.DEV)

    o_cs = [np.zeros((1, 3, synth.CONV_DIM)) for _ in m_layers]
    o_ss = [np.zeros((1, 128, 80, 128)) for _ in m_layers]
    t_id, f_id = np.array([12], np.int32), np.array([12], np.int32)   # pad for the first position
    for pos in range(3):
        audio = synth.rng(6, 4000 + pos, 0).normal(0.0, 1.0, (1, 4480)).astype(np.float32)
        positions = torch.tensor([pos], dtype=torch.int32, device=gu.DEV)
        nh.nh_lm_step(d, w, [s[0] for s in states], caches, positions, torch.tensor(t_id, device=gu.DEV),
                      torch.tensor(f_id, device=gu.DEV), gu.to_dev(audio), nh.NH_F32, 1, hid, t_out, f_out,
                      ws, ws.numel())
        torch.cuda.synchronize()
        # oracle: the same position through the oracle's functions, fp32 stream between layers
        x = oracle.fused_embedding(E, t_id, f_id, audio.astype(np.float64)).astype(np.float32).astype(np.float64)
        mi = li = ai = 0
        for c in pat:
            if c == "M":
                r = oracle.block(synth.REAL, lws[mi], x[:, None, :], o_cs[mi], o_ss[mi], stepwise=True)
                o_cs[mi], o_ss[mi] = r.conv_state, r.ssm_state
                x = r.out[:, 0].astype(np.float32).astype(np.float64)
                mi += 1
            elif c == "-":
                x = oracle.mlp(x, mws[li].norm_w, mws[li].up, mws[li].down, 1e-5).astype(np.float32).astype(np.float64)
                li += 1
            else:
                x, k_new, v_new = oracle.attention(x, aws[ai], o_kc[ai], o_vc[ai], 1e-5)
                x = x.astype(np.float32).astype(np.float64)
                o_kc[ai] = np.concatenate([o_kc[ai], k_new[:, :, None, :]], axis=2)
                o_vc[ai] = np.concatenate([o_vc[ai], v_new[:, :, None, :]], axis=2)
                ai += 1
        got = hid.cpu().numpy().astype(np.float64)
        r = gu.rel_l2(got, x)
        print(f"[lm pos {pos}] stream rel-L2 {r:.3e}", flush=True)
        assert r <= 5e-3
        ids = []
        for W, out in ((hw.lm_head, t_out), (hw.function_head, f_out)):
            ref_l, _ = oracle.head(W, got, hw.norm_f, 1e-5)
            gid = int(out.cpu().numpy()[0])
            assert ref_l[0, gid] >= ref_l.max() - 4e-3, (gid, ref_l.max() - ref_l[0, gid])
            ids.append(gid)
        print(f"[lm pos {pos}] ids {ids}", flush=True)
        t_id, f_id = np.array([ids[0]], np.int32), np.array([ids[1]], np.int32)


def test_lm_step_batch2_rows_match_batch1(env):
    # two sessions in one call (batch-2 kernels) against each session alone (batch-1 kernels):
    # both are held to the oracle bar, so the rows agree within twice it; ids must agree where
    # the oracle's top two logits are apart by more than the head tolerance
    nh, oracle, gu, torch = env
    pat = nh.hybrid_pattern()
    m_layers = [i for i, c in enumerate(pat) if c == "M"]
    f_layers = [i for i, c in enumerate(pat) if c == "-"]
    print("[case] lm step batch 2 vs batch 1", flush=True)
    mamba = [gu.layer_dev(synth.layer_weights(l)) for l in range(len(m_layers))]
    mws = [synth.mlp_weights(l) for l in f_layers]
    mlp = [nh.mlp_weights(gu.to_dev(mw.norm_w), gu.w4_dev(mw.up), gu.w4_dev(mw.down)) for mw in mws]
    attn = []
    for l in [i for i, c in enumerate(pat) if c == "*"]:
        aw = synth.attention_weights(l)
        attn.append(nh.attention_weights(gu.to_dev(aw.norm_w), gu.w4_dev(aw.q_proj), gu.w4_dev(aw.k_proj),
                                         gu.w4_dev(aw.v_proj), gu.w4_dev(aw.o_proj)))
    hw = synth.head_weights(seed=7, n_out=VOCAB_T)
    w = nh.lm_weights(gu.w4_dev(synth.embed_tokens(seed=7, n_out=VOCAB_T)), mamba, mlp, attn, gu.to_dev(hw.norm_f),
                      gu.w4_dev(hw.lm_head), gu.w4_dev(hw.function_head), 2.0)
    # pre-filled caches: sequence 0 at position 20, sequence 1 at position 5
    max_len, pos2 = 32, np.array([20, 5], np.int32)
    kv_fill = [synth.kv_cache(30 + a, 2, max_len) for a in range(4)]
    d = nh.dims()
    t_ids, f_ids, audio = synth.embed_inputs(8, 2, n_out=VOCAB_T)

    def run(rows):
        B = len(rows)
        states = [gu.state_dev(np.zeros((B, 3, synth.CONV_DIM), np.uint16),
                               np.zeros((B, 128, 80, 128), np.float32))[0] for _ in m_layers]
        ws = gu.workspace(nh.nh_lm_workspace_bytes(d, synth.MLP_INTER, B))
        hid = gu.empty_f32(B, 4480)
        to = torch.empty(B, dtype=torch.int32, device=gu.DEV)
        fo = torch.empty(B, dtype=torch.int32, device=gu.DEV)
        caches = [nh.kv_cache(gu.to_dev(np.ascontiguousarray(k[rows])), gu.to_dev(np.ascontiguousarray(v[rows])),
                              max_len) for k, v in kv_fill]
        nh.nh_lm_step(d, w, states, caches, torch.tensor(pos2[rows], device=gu.DEV),
                      torch.tensor(t_ids[rows], device=gu.DEV), torch.tensor(f_ids[rows], device=gu.DEV),
                      gu.to_dev(np.ascontiguousarray(audio[rows])), nh.NH_F32, B, hid, to, fo, ws, ws.numel())
        torch.cuda.synchronize()
        return hid.cpu().numpy().astype(np.float64), to.cpu().numpy(), fo.cpu().numpy()

    h2, t2, f2 = run([0, 1])
    for r in (0, 1):
        h1, t1, f1 = run([r])
        rel = gu.rel_l2(h2[r], h1[0])
        print(f"[lm b2 row {r}] rel-L2 vs batch 1 {rel:.3e} ids {t2[r]},{f2[r]} vs {t1[0]},{f1[0]}", flush=True)
        assert rel <= 1e-2
        for W, a, b in ((hw.lm_head, t2[r], t1[0]), (hw.function_head, f2[r], f1[0])):
            ref_l, _ = oracle.head(W, h1[:1], hw.norm_f, 1e-5)
            top = np.sort(ref_l[0])[-2:]
            if top[1] - top[0] > 8e-3:
                assert a == b
