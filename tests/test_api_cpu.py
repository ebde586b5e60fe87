"""The C ABI without a GPU: the library loads, exports every entry point that
include/nhmamba.h declares, and rejects bad arguments before touching the device
(no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nhmamba.h")


@pytest.fixture(scope="module")
def nh():
    import hybrid_mamba2_decode_amd as m
    return m


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nh_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_exports(nh):
    assert _declared() == sorted(nh.EXPORTS)


def test_library_exports_every_declared_symbol(nh):
    for name in _declared():
        assert hasattr(nh.lib, name), name


def test_info_strings(nh):
    assert "gfx950" in nh.version()
    p = nh.hybrid_pattern()
    assert len(p) == 56 and p.count("M") == 27 and p.count("*") == 4 and p.count("-") == 25


def _fake_w4(n=64, k=128, gs=64, base=0x10000):
    return nh_w4(base, base + 0x1000, base + 0x2000, n, k, gs)


def nh_w4(q, s, b, n, k, gs):
    import hybrid_mamba2_decode_amd as m
    return m.nh_w4_matrix(q, s, b, n, k, gs)


def _status(fn):
    import hybrid_mamba2_decode_amd as m
    with pytest.raises(m.NhError) as e:
        fn()
    return e.value.status


def test_gemv_rejects_bad_arguments(nh):
    A = 0x20000  # aligned fake addresses: validation fails before any use
    assert _status(lambda: nh.nh_w4_gemv(_fake_w4(gs=32), A, 0, 1, None, 0, A, 0, 0)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_w4_gemv(_fake_w4(k=96), A, 0, 1, None, 0, A, 0, 0)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_w4_gemv(_fake_w4(), None, 0, 1, None, 0, A, 0, 0)) == nh.NH_ERR_INVALID_ARGUMENT
    assert _status(lambda: nh.nh_w4_gemv(_fake_w4(), A + 2, 0, 1, None, 0, A, 0, 0)) == nh.NH_ERR_MISALIGNED
    assert _status(lambda: nh.nh_w4_gemv(_fake_w4(), A, 0, 5, None, 0, A, 0, 0)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_w4_gemv(_fake_w4(), A, 0, 1, None, 0, A, 7, 0)) == nh.NH_ERR_INVALID_ARGUMENT
    assert _status(lambda: nh.nh_w4_gemv(_fake_w4(), A, 2, 1, None, 0, A, 0, 0)) == nh.NH_ERR_INVALID_ARGUMENT
    assert "batch" in nh.lib.nh_last_error().decode() or "dtype" in nh.lib.nh_last_error().decode()


def test_packed_matrix_over_2gib_rejected(nh):
    A = 0x20000
    big = nh_w4(A, A + 0x1000, A + 0x2000, 1 << 18, 16384, 64)   # 2 GiB of packed words
    assert _status(lambda: nh.nh_w4_gemv(big, A, 0, 1, None, 0, A, 0, 0)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert "2 GiB" in nh.lib.nh_last_error().decode()


def test_head_rejects_bad_arguments(nh):
    A = 0x20000
    ws = nh.nh_head_workspace_bytes(1)
    assert ws == 256 * 8 and nh.nh_head_workspace_bytes(4) == 4 * 256 * 8
    assert nh.nh_head_workspace_bytes(0) == 0 and nh.nh_head_workspace_bytes(5) == 0
    W = _fake_w4(n=131072, k=4480)
    ok = dict(W=W, x=A, x_dtype=0, norm_w=A, eps=1e-5, batch=1, logits=None, ids=A, ws=A, ws_bytes=ws)

    def call(**kw):
        a = dict(ok, **kw)
        return _status(lambda: nh.nh_head_argmax(a["W"], a["x"], a["x_dtype"], a["norm_w"], a["eps"],
                                                 a["batch"], a["logits"], a["ids"], a["ws"], a["ws_bytes"], 0))
    assert call(W=_fake_w4(n=1000, k=4096)) == nh.NH_ERR_UNSUPPORTED_SHAPE        # k_in != hidden
    assert call(W=_fake_w4(n=(1 << 19) + 1, k=4480)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(batch=0) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(batch=5) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(ws_bytes=ws - 1) == nh.NH_ERR_WORKSPACE_TOO_SMALL
    assert call(ids=None) == nh.NH_ERR_INVALID_ARGUMENT
    assert call(norm_w=A + 2) == nh.NH_ERR_MISALIGNED
    assert call(logits=A + 4) == nh.NH_ERR_MISALIGNED
    assert call(x_dtype=3) == nh.NH_ERR_INVALID_ARGUMENT
    assert call(eps=0.0) == nh.NH_ERR_INVALID_ARGUMENT


def test_fused_embedding_rejects_bad_arguments(nh):
    A = 0x20000
    E = _fake_w4(n=131072, k=4480)

    def call(**kw):
        a = dict(E=E, t=A, f=A, audio=A, at=0, w=2.0, batch=1, out=A)
        a.update(kw)
        return _status(lambda: nh.nh_fused_embedding(a["E"], a["t"], a["f"], a["audio"], a["at"], a["w"],
                                                     a["batch"], a["out"], 0))
    assert call(batch=0) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(batch=4097) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(t=None) == nh.NH_ERR_INVALID_ARGUMENT
    assert call(f=A + 4) == nh.NH_ERR_MISALIGNED
    assert call(at=2) == nh.NH_ERR_INVALID_ARGUMENT
    assert call(w=float("nan")) == nh.NH_ERR_INVALID_ARGUMENT
    assert call(E=_fake_w4(gs=32)) == nh.NH_ERR_UNSUPPORTED_SHAPE


def test_mlp_rejects_bad_arguments(nh):
    A = 0x20000
    assert nh.nh_mlp_workspace_bytes(15680, 1) == 31488 and nh.nh_mlp_workspace_bytes(15680, 5) == 0
    assert nh.nh_mlp_workspace_bytes(100, 1) == 0
    up, down = _fake_w4(n=15680, k=4480), _fake_w4(n=4480, k=15680)
    ws = nh.nh_mlp_workspace_bytes(15680, 1)

    def call(**kw):
        a = dict(up=up, down=down, batch=1, ws_bytes=ws, x=A, xt=0)
        a.update(kw)
        return _status(lambda: nh.nh_mlp_step(A, a["up"], a["down"], 1e-5, a["x"], a["xt"], A, 0, a["batch"], A,
                                              a["ws_bytes"], 0))
    assert call(down=_fake_w4(n=4480, k=15616)) == nh.NH_ERR_UNSUPPORTED_SHAPE   # inner sizes differ
    assert call(up=_fake_w4(n=15680, k=4096)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(batch=5) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(ws_bytes=ws - 1) == nh.NH_ERR_WORKSPACE_TOO_SMALL
    assert call(x=A + 8) == nh.NH_ERR_MISALIGNED
    assert call(xt=5) == nh.NH_ERR_INVALID_ARGUMENT


def test_lm_step_rejects_bad_arguments(nh):
    A = 0x40000
    d = nh.dims()
    need = nh.nh_lm_workspace_bytes(d, 15680, 1)
    assert need >= 2 * 4480 * 4 + nh.nh_mlp_workspace_bytes(15680, 1)
    assert nh.nh_lm_workspace_bytes(d, 15680, 5) == 0 and nh.nh_lm_workspace_bytes(d, 100, 1) == 0
    emb = _fake_w4(n=131072, k=4480)
    m = nh.nh_mamba_weights(A, _fake_w4(n=22656, k=4480), A, A, A, A, A, A, _fake_w4(n=4480, k=10240))
    f = nh.nh_mlp_weights(A, _fake_w4(n=15680, k=4480), _fake_w4(n=4480, k=15680))
    at = _fake_attention(nh, A)
    assert need >= nh.nh_attention_workspace_bytes(1)
    w = nh.lm_weights(emb, [m] * 27, [f] * 25, [at] * 4, A, emb, emb, 2.0)
    st = [nh.nh_mamba_state(A, A)] * 27
    kv = [nh.nh_kv_cache(A, A, 512)] * 4

    def call(w=w, batch=1, ws_bytes=need, t=A, kv=kv, pos=A):
        return _status(lambda: nh.nh_lm_step(d, w, st, kv, pos, t, A, A, 0, batch, None, A, A, A, ws_bytes, 0))
    assert call(batch=5) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(ws_bytes=need - 1) == nh.NH_ERR_WORKSPACE_TOO_SMALL
    assert call(t=None) == nh.NH_ERR_INVALID_ARGUMENT
    assert call(pos=None) == nh.NH_ERR_INVALID_ARGUMENT
    assert call(kv=[nh.nh_kv_cache(A, A, 512)] * 3 + [nh.nh_kv_cache(A, A, 0)]) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(kv=[nh.nh_kv_cache(A, A + 8, 512)] * 4) == nh.NH_ERR_MISALIGNED
    bad_f = nh.nh_mlp_weights(A, _fake_w4(n=15680, k=4480), _fake_w4(n=4480, k=15616))
    assert call(w=nh.lm_weights(emb, [m] * 27, [f] * 24 + [bad_f], [at] * 4, A, emb, emb, 2.0)) == \
        nh.NH_ERR_UNSUPPORTED_SHAPE
    bad_a = _fake_attention(nh, A, kv_rows=512)
    assert call(w=nh.lm_weights(emb, [m] * 27, [f] * 25, [at] * 3 + [bad_a], A, emb, emb, 2.0)) == \
        nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(w=nh.lm_weights(emb, [m] * 27, [f] * 25, [at] * 4, A, emb, emb, float("inf"))) == \
        nh.NH_ERR_INVALID_ARGUMENT


def _fake_attention(nh, A, kv_rows=1024):
    return nh.nh_attention_weights(A, _fake_w4(n=5120, k=4480), _fake_w4(n=kv_rows, k=4480),
                                   _fake_w4(n=1024, k=4480), _fake_w4(n=4480, k=5120))


def test_attention_step_rejects_bad_arguments(nh):
    A = 0x40000
    need = nh.nh_attention_workspace_bytes(2)
    assert need >= 2 * 2 * 5120 * 2
    assert nh.nh_attention_workspace_bytes(0) == 0 and nh.nh_attention_workspace_bytes(5) == 0
    at = _fake_attention(nh, A)

    def call(w=at, kv=nh.nh_kv_cache(A, A, 413), pos=A, x=A, out=A + 0x1000, batch=2, eps=1e-5, ws=need, xt=0):
        return _status(lambda: nh.nh_attention_step(w, kv, pos, x, xt, out, 0, batch, eps, A, ws, 0))
    assert call(w=_fake_attention(nh, A, kv_rows=512)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(kv=nh.nh_kv_cache(A, A, 0)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(kv=nh.nh_kv_cache(A, A, (1 << 22) + 1)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(kv=nh.nh_kv_cache(None, A, 16)) == nh.NH_ERR_INVALID_ARGUMENT
    assert call(pos=None) == nh.NH_ERR_INVALID_ARGUMENT
    assert call(pos=A + 4) == nh.NH_ERR_MISALIGNED
    assert call(out=A) == nh.NH_ERR_INVALID_ARGUMENT   # out aliases x
    assert call(batch=0) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(batch=5) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert call(eps=0.0) == nh.NH_ERR_INVALID_ARGUMENT
    assert call(ws=need - 1) == nh.NH_ERR_WORKSPACE_TOO_SMALL
    assert call(xt=3) == nh.NH_ERR_INVALID_ARGUMENT


def test_gemm_workspace_check(nh):
    A = 0x20000
    need = nh.nh_w4_gemm_workspace_bytes(100, 128)
    assert need >= 100 * 128 * 2
    assert _status(lambda: nh.nh_w4_gemm(_fake_w4(), A, 100, None, 0, A, 0, A, need - 1, 0)) == \
        nh.NH_ERR_WORKSPACE_TOO_SMALL
    assert _status(lambda: nh.nh_w4_gemm(_fake_w4(), A, 0, None, 0, A, 0, A, need, 0)) == \
        nh.NH_ERR_UNSUPPORTED_SHAPE


def test_block_dims_and_workspace_checks(nh):
    A = 0x40000
    d = nh.dims(chunk=128)
    lw = nh.mamba_weights(A, _fake_w4(22656, 4480), A, A, A, A, A, A, _fake_w4(4480, 10240))
    st = nh.mamba_state(A, A)
    step_ws = nh.nh_block_workspace_bytes(d, 1, 1, nh.NH_MODE_STEP)
    seq_ws = nh.nh_block_workspace_bytes(d, 2, 100, nh.NH_MODE_SEQ)
    assert step_ws > 0 and seq_ws > step_ws
    assert nh.nh_block_workspace_bytes(d, 5, 1, nh.NH_MODE_STEP) == 0
    bad = nh.dims(chunk=128, head_dim=64)
    assert _status(lambda: nh.nh_mamba_block_step(bad, lw, st, A, 0, A + 0x100, 0, 1, A, step_ws, 0)) == \
        nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_mamba_block_step(d, lw, st, A, 0, A + 0x100, 0, 1, A, step_ws - 1, 0)) == \
        nh.NH_ERR_WORKSPACE_TOO_SMALL
    assert _status(lambda: nh.nh_mamba_block_step(d, lw, st, A, 0, A, 0, 1, A, step_ws, 0)) == \
        nh.NH_ERR_INVALID_ARGUMENT  # out aliases x
    wrong = nh.mamba_weights(A, _fake_w4(22656, 4416), A, A, A, A, A, A, _fake_w4(4480, 10240))
    assert _status(lambda: nh.nh_mamba_block_step(d, wrong, st, A, 0, A + 0x100, 0, 1, A, step_ws, 0)) == \
        nh.NH_ERR_UNSUPPORTED_SHAPE
    for q in (0, 257):
        assert _status(lambda: nh.nh_mamba_block_seq(nh.dims(chunk=q), lw, None, None, A, 0, 100, A + 0x100,
                                                     0, 2, A, seq_ws, 0)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_mamba_block_seq(d, lw, None, None, A, 0, 100, A + 0x100, 0, 2, A,
                                                 seq_ws - 1, 0)) == nh.NH_ERR_WORKSPACE_TOO_SMALL
    assert _status(lambda: nh.nh_mamba_stack(d, [lw], [st], 1, nh.NH_MODE_STEP, A, 0, 2, A + 0x100, 1, A,
                                             step_ws, 0)) == nh.NH_ERR_UNSUPPORTED_SHAPE


def test_noalloc_step_checks(nh):
    """The allocation-free step validates like the workspace step, and rejects batches beyond
    its scratch array's limit, before any device call."""
    A = 0x40000
    d = nh.dims(chunk=128)
    lw = nh.mamba_weights(A, _fake_w4(22656, 4480), A, A, A, A, A, A, _fake_w4(4480, 10240))
    st = nh.mamba_state(A, A)
    for b in (0, 5):
        assert _status(lambda: nh.nh_mamba_block_step_noalloc(d, lw, st, A, 0, A + 0x100, 0, b, 0)) == \
            nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_mamba_block_step_noalloc(d, lw, st, A, 0, A, 0, 1, 0)) == \
        nh.NH_ERR_INVALID_ARGUMENT  # out aliases x
    assert _status(lambda: nh.nh_mamba_block_step_noalloc(nh.dims(head_dim=64), lw, st, A, 0, A + 0x100, 0, 1,
                                                          0)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_mamba_block_step_noalloc(d, lw, st, A + 8, 0, A + 0x100, 0, 1, 0)) == \
        nh.NH_ERR_MISALIGNED


def test_primitive_checks(nh):
    A = 0x40000
    d = nh.dims(chunk=64)
    assert _status(lambda: nh.nh_conv1d_step(A, 16, A, A, A, A, 1, 16, 3, 0)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_conv1d_seq(A, 16, 4, A, A, A, A, A, 1, 16, 4, 0)) == nh.NH_ERR_INVALID_ARGUMENT
    assert _status(lambda: nh.nh_ssm_step(d, A, A, 128, A, A, A, A, A, 0, 0, 0)) == nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_ssd_chunk_scan(d, A, A, 22656, 0, A, A, A, None, None, A, 0, 1, A, 1 << 20, 0)) == \
        nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_rmsnorm_gated(A, 0, A, 10240, A, A, 1, 10240, 1000, 1e-5, 0)) == \
        nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_rmsnorm(A, 0, A, A, 1, 4480, 0.0, 0)) == nh.NH_ERR_INVALID_ARGUMENT


def test_scan_workspace_size_and_checks(nh):
    A = 0x40000
    # chunk 256: the causal 16 x 16 fp16 tiles of C.B^T per (chunk, sequence, group) in pairs of
    # 2 x 512 B; row block I holds ceil((I+1)/2) pairs, 72 for 16 row blocks; a partial last
    # chunk of 166 rows has 11 row blocks, 36 pairs
    d256 = nh.dims(chunk=256)
    tiles = 2 * 8 * 1024 * (14 * 72 + 36)
    # chunks of at least 128 rows in sequences of at least 64 positions add, per (chunk,
    # sequence, group), B as ceil(L/32) steps x 8 state blocks of 1 KiB and C as ceil(L/16) row
    # blocks x 4 steps of 1 KiB, and per (chunk, sequence, head) the decay tables, 14 bytes per
    # position over 32 ceil(L/32) positions (rounded up to 64 bytes): 3584 at 256 rows, 2688 at 166
    bfr = 2 * 8 * (14 * 64 + 6 * 8) * 1024
    cfr = 2 * 8 * (14 * 64 + 11 * 4) * 1024
    tab = 2 * 128 * (14 * 3584 + 2688)
    assert nh.nh_ssd_scan_workspace_bytes(d256, 2, 3750) == tiles + bfr + cfr + tab
    assert nh.nh_ssd_scan_workspace_bytes(d256, 1, 1) == 8 * 1024          # short: tiles only
    # 63 positions (short): 4 row blocks of 1 + 1 + 2 + 2 pairs of 1 KiB per group
    assert nh.nh_ssd_scan_workspace_bytes(d256, 1, 63) == 8 * 1024 * 6
    for B, T, Q in [(1, 1, 1), (2, 413, 128), (3, 17, 16), (1, 300, 7), (2, 3750, 256), (1, 130, 129)]:
        n = nh.nh_ssd_scan_workspace_bytes(nh.dims(chunk=Q), B, T)
        # the block gives the scan its gated-norm output region, 20 KiB per position
        assert 0 < n <= (10240 if Q >= 128 and T >= 64 else 8192) * B * T
    assert nh.nh_ssd_scan_workspace_bytes(nh.dims(chunk=0), 1, 10) == 0
    assert nh.nh_ssd_scan_workspace_bytes(nh.dims(chunk=257), 1, 10) == 0
    assert nh.nh_ssd_scan_workspace_bytes(d256, 0, 10) == 0
    n = nh.nh_ssd_scan_workspace_bytes(d256, 1, 100)
    assert _status(lambda: nh.nh_ssd_chunk_scan(d256, A, A, 128, 100, A, A, A, None, None, A, 0, 1, A, n - 1, 0)) == \
        nh.NH_ERR_WORKSPACE_TOO_SMALL
    assert _status(lambda: nh.nh_ssd_chunk_scan(d256, A, A, 128, 100, A, A, A, None, None, A, 0, 1, None, n, 0)) == \
        nh.NH_ERR_INVALID_ARGUMENT
    assert _status(lambda: nh.nh_ssd_chunk_scan(d256, A, A, 128, 100, A, A, A, None, None, A, 0, 1, A + 2, n, 0)) == \
        nh.NH_ERR_MISALIGNED


def test_inproj_conv_step_checks(nh):
    A = 0x40000
    d = nh.dims()
    lw = nh.mamba_weights(A, _fake_w4(22656, 4480), A, A, A, A, A, A, _fake_w4(4480, 10240))
    st = nh.mamba_state(A, A)
    assert _status(lambda: nh.nh_inproj_conv_step(d, lw, st, A, 0, A + 0x100, A + 0x200, A + 0x300, 5, 0)) == \
        nh.NH_ERR_UNSUPPORTED_SHAPE
    assert _status(lambda: nh.nh_inproj_conv_step(d, lw, st, A, 0, A, A + 0x200, A + 0x300, 1, 0)) == \
        nh.NH_ERR_INVALID_ARGUMENT  # z aliases x
    assert _status(lambda: nh.nh_inproj_conv_step(d, lw, st, A, 0, None, A + 0x200, A + 0x300, 1, 0)) == \
        nh.NH_ERR_INVALID_ARGUMENT
    assert _status(lambda: nh.nh_inproj_conv_step(d, lw, st, A, 0, A + 0x100, A + 0x208, A + 0x300, 1, 0)) == \
        nh.NH_ERR_MISALIGNED
    wrong = nh.mamba_weights(A, _fake_w4(22656, 4416), A, A, A, A, A, A, _fake_w4(4480, 10240))
    assert _status(lambda: nh.nh_inproj_conv_step(d, wrong, st, A, 0, A + 0x100, A + 0x200, A + 0x300, 1, 0)) == \
        nh.NH_ERR_UNSUPPORTED_SHAPE
