"""GPU parity of each libnhmamba primitive against the CPU oracle, through the C ABI.

Tolerances: integer / indexing work (nibble unpack and dequantisation) is bit-exact;
fp32 outputs of exact-arithmetic kernels agree to fp32 accumulation error; bf16 outputs
agree up to a rounding-boundary flip of one bf16 unit; the scan, whose matrix-core
operands are fp16, agrees to rel-L2 2e-3 on y and 1e-3 on the fp32 state (the stated
state tolerance), and row by row: every (position, head) row of 80 outputs within ROW_REL of
its own norm (floored at a tenth of the RMS row norm) and every element within ROW_ABS of
max |y|, so that one wrong row cannot hide in a whole-tensor norm."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

# Row-wise scan bars: the fp16 operands round each computed product term to 2^-11 relative,
# so a row's error is of the order of 1e-3 of its norm; ten times that still flags a single
# wrong (position, head) row, whose error is of the order of its whole norm.
ROW_REL, ROW_ABS = 1e-2, 1e-2


@pytest.fixture(scope="module")
def env():
    import torch
    import hybrid_mamba2_decode_amd as nh
    import oracle
    from tests import gpu_util as gu
    oracle.build(force=False)
    assert torch.cuda.is_available()
    return nh, oracle, gu, torch


def _say(*a):
    print("[case]", *a, flush=True)


def _asym(W, seed, exact_offset=False):
    """Same matrix with arbitrary (non-symmetric) bf16 biases.  exact_offset: biases that are
    tiny next to 8 s, so that beta + 8 s is not an fp32 number, are set to 0 (still not
    symmetric): the matrix product adds the offset term (beta + 8 s) * sum x in fp32, so only
    then is its result the single rounding of the exact value."""
    rng = np.random.default_rng(seed)
    b = synth.f32_to_bf16(rng.uniform(-0.05, 0.05, W.biases.shape).astype(np.float32))
    if exact_offset:
        s64 = synth.bf16_to_f32(W.scales).astype(np.float64)
        b64 = synth.bf16_to_f32(b).astype(np.float64)
        b = np.where(np.float32(8 * s64 + b64).astype(np.float64) == 8 * s64 + b64, b, np.uint16(0)).astype(np.uint16)
    return synth.W4Matrix(W.qweight, W.scales, b, W.n_out, W.k_in, W.group_size)


def _x(rng, m, k):
    return synth.f32_to_bf16(rng.normal(0, 1, (m, k)).astype(np.float32))


# ------------------------------------------------------------------------ GEMV

@pytest.mark.parametrize("asym", [False, True])
def test_gemv_one_hot_is_bit_exact(env, asym):
    nh, oracle, gu, torch = env
    W = synth.w4_random(11, 0, 1, 2, 300, 4480)
    if asym:
        W = _asym(W, 5)
    ks = [0, 1, 7, 8, 63, 64, 2345, 4479]
    _say("gemv one-hot", asym)
    Wd = oracle.w4_dequant(W)
    for b0 in range(0, len(ks), 4):
        kk = ks[b0:b0 + 4]
        x = np.zeros((len(kk), 4480), dtype=np.uint16)
        for i, k in enumerate(kk):
            x[i, k] = 0x3F80  # 1.0
        y = gu.empty_f32(len(kk), 300)
        nh.nh_w4_gemv(gu.w4_dev(W), gu.to_dev(x), nh.NH_BF16, len(kk), None, 0, y, nh.NH_F32)
        got = y.cpu().numpy()
        for i, k in enumerate(kk):
            assert np.array_equal(got[i], Wd[:, k].astype(np.float32)), k


@pytest.mark.parametrize("n,k,batch", [(22656, 4480, 1), (22656, 4480, 2), (4480, 10240, 1),
                                       (4480, 10240, 2), (37, 64, 3), (130, 16384, 1), (7, 2048, 4)])
def test_gemv_matches_oracle(env, n, k, batch):
    nh, oracle, gu, torch = env
    _say("gemv", n, k, batch)
    rng = np.random.default_rng(n + k + batch)
    W = synth.w4_random(3, n, 1, 2, n, k)
    x = _x(rng, batch, k)
    y = gu.empty_f32(batch, n)
    nh.nh_w4_gemv(gu.w4_dev(W), gu.to_dev(x), nh.NH_BF16, batch, None, 0, y, nh.NH_F32)
    ref = oracle.w4_matvec(W, gu.bf16_bits_to_f64(x))
    got = y.cpu().numpy()
    assert gu.rel_l2(got, ref) < 1e-5
    assert gu.max_abs(got, ref) < 1e-4 * max(1.0, np.abs(ref).max())


# K = 4480 at batch 3 and 4 runs the batched in_proj's matrix-core kernel: ceil(n / 4) four-row
# stages split evenly over the 8 XCDs and then over 1024 waves, two stages per loop iteration
# (loads past a wave's last stage re-read it; only the second compute is conditional).  These
# n_out give waves of {0,1}, {1,2}, {2,3}, {3,4}, {4,5} and {5,6} stages (odd and even counts,
# idle waves) and last stages with 1, 2, 3 and 4 rows inside the matrix.
MF_TAILS = [1, 3, 66, 4100, 8594, 14339, 16385, 22656]


@pytest.mark.parametrize("batch", [3, 4])
def test_gemv_matrix_core_stage_tails(env, batch):
    nh, oracle, gu, torch = env
    rng = np.random.default_rng(40 + batch)
    for n in MF_TAILS:
        _say("gemv matrix-core tails", n, batch)
        W = _asym(synth.w4_random(5, n, 1, 2, n, 4480), n)
        x = _x(rng, batch, 4480)
        res = rng.normal(size=(batch, n)).astype(np.float32)
        y = gu.empty_f32(batch, n)
        nh.nh_w4_gemv(gu.w4_dev(W), gu.to_dev(x), nh.NH_BF16, batch, gu.to_dev(res), nh.NH_F32, y, nh.NH_F32)
        ref = oracle.w4_matvec(W, gu.bf16_bits_to_f64(x)) + res
        got = y.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), n
        assert gu.rel_l2(got, ref) < 1e-5, n
        assert gu.max_abs(got, ref) < 1e-4 * max(1.0, np.abs(ref).max()), n


# Activations far outside the fp16 range: each 32-value chunk is staged in fp16 after an exact
# power-of-two scaling, so bf16 inputs of any magnitude are multiplied exactly.  Rows mix
# magnitudes 1e3..1e5 (the chunk maxima overflow fp16 unscaled), with some chunks of tiny values
# (1e-3) and some exact zeros; every kernel of nh_w4_gemv is covered (per-row kernel, K = 4480
# matrix-core kernel at batch 3-4, LDS matrix-core kernel above K = 10240 or at batch 4).
@pytest.mark.parametrize("n,k,batch", [(300, 4480, 1), (300, 4480, 2), (1000, 4480, 3), (1000, 4480, 4),
                                       (4480, 5120, 4), (4480, 10240, 1), (4480, 10240, 3), (4480, 10240, 4),
                                       (4480, 15680, 1), (4480, 15680, 2), (4480, 15680, 4)])
def test_gemv_large_activations(env, n, k, batch):
    nh, oracle, gu, torch = env
    _say("gemv large activations", n, k, batch)
    rng = np.random.default_rng(7 * n + k + batch)
    W = _asym(synth.w4_random(8, n, 1, 2, n, k), n + 1)
    mag = 10.0 ** rng.uniform(3, 5, (batch, k))
    xf = rng.normal(0, 1, (batch, k)) * mag
    xf[:, 64:96] = rng.normal(0, 1e-3, (batch, 32))     # a chunk of tiny values
    xf[:, 160:192] = 0.0                                  # an all-zero chunk
    x = synth.f32_to_bf16(xf.astype(np.float32))
    y = gu.empty_f32(batch, n)
    nh.nh_w4_gemv(gu.w4_dev(W), gu.to_dev(x), nh.NH_BF16, batch, None, 0, y, nh.NH_F32)
    ref = oracle.w4_matvec(W, gu.bf16_bits_to_f64(x))
    got = y.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert gu.rel_l2(got, ref) < 1e-5
    assert gu.max_abs(got, ref) < 1e-4 * np.abs(ref).max()


@pytest.mark.parametrize("n,k,batch", [(300, 4480, 1), (300, 4480, 2), (1000, 4480, 3), (1000, 4480, 4),
                                       (4480, 10240, 1), (4480, 15680, 2), (4480, 10240, 4)])
def test_gemv_f32_input(env, n, k, batch):
    # x given as fp32 (not bf16-exact): the GEMV rounds it to bf16, its activation precision
    nh, oracle, gu, torch = env
    _say("gemv f32 input", n, k, batch)
    rng = np.random.default_rng(11 * n + k + batch)
    W = _asym(synth.w4_random(10, n, 1, 2, n, k), n + 2)
    xf = rng.normal(0, 1, (batch, k)).astype(np.float32)
    y = gu.empty_f32(batch, n)
    nh.nh_w4_gemv(gu.w4_dev(W), gu.to_dev(xf), nh.NH_F32, batch, None, 0, y, nh.NH_F32)
    ref = oracle.w4_matvec(W, oracle.round_bf16(xf.astype(np.float64)))
    got = y.cpu().numpy().astype(np.float64)
    assert gu.rel_l2(got, ref) < 1e-5
    assert gu.max_abs(got, ref) < 1e-4 * max(1.0, np.abs(ref).max())


def test_gemv_residual_bf16_out(env):
    nh, oracle, gu, torch = env
    _say("gemv residual bf16")
    rng = np.random.default_rng(1)
    W = _asym(synth.w4_random(4, 0, 1, 2, 4480, 10240), 9)
    x = _x(rng, 2, 10240)
    res = rng.normal(size=(2, 4480)).astype(np.float32)
    y = gu.empty_u16(2, 4480)
    nh.nh_w4_gemv(gu.w4_dev(W), gu.to_dev(x), nh.NH_BF16, 2, gu.to_dev(res), nh.NH_F32, y, nh.NH_BF16)
    ref = oracle.w4_matvec(W, gu.bf16_bits_to_f64(x)) + res
    got = gu.bf16_bits_to_f64(gu.from_dev_u16(y))
    # half a bf16 unit of the value plus the fp32 accumulation error (a rounding-boundary flip)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8 + 2e-5 * np.abs(ref).max())


# ------------------------------------------------------------------------ GEMM

# 200 columns run the split-role kernel, 17000 the wide-tile one (on 256 compute units: 266
# split tiles, two rounds, against 134 wide tiles, one round)
@pytest.mark.parametrize("N", [200, 17000])
@pytest.mark.parametrize("asym", [False, True])
def test_gemm_identity_probe_is_bit_exact(env, asym, N):
    nh, oracle, gu, torch = env
    _say("gemm identity", asym, N)
    K = 512
    W = synth.w4_random(13, 0, 1, 2, N, K)
    if asym:
        W = _asym(W, 6, exact_offset=True)
    X = np.zeros((K, K), dtype=np.uint16)
    X[np.arange(K), np.arange(K)] = 0x3F80
    Y = gu.empty_f32(K, N)
    ws = gu.workspace(nh.nh_w4_gemm_workspace_bytes(K, K))
    nh.nh_w4_gemm(gu.w4_dev(W), gu.to_dev(X), K, None, 0, Y, nh.NH_F32, ws, ws.numel())
    assert np.array_equal(Y.cpu().numpy(), oracle.w4_dequant(W).T.astype(np.float32))


@pytest.mark.parametrize("M,n,k,asym", [(1, 300, 4480, False), (16, 300, 4480, True), (130, 260, 4480, False),
                                        (413, 4480, 10240, True), (257, 64, 128, False),
                                        # odd group counts (the split-role kernel): one, three and
                                        # five groups of 64, fewer than the loaders' three-step lead,
                                        # several tiles in both directions
                                        (37, 129, 64, True), (300, 520, 192, False), (600, 1000, 320, True),
                                        # even group counts, few tiles (the split-role kernel): two,
                                        # four, six and sixteen groups, ragged rows and columns
                                        (37, 129, 128, True), (300, 520, 256, False), (600, 1000, 384, True),
                                        (513, 600, 1024, True),
                                        # even group counts, many columns (the wide-tile kernel on 256
                                        # compute units): ragged rows and columns, four and two groups
                                        (300, 17000, 256, True), (520, 16500, 128, False),
                                        # one row on the wide kernel (255 of the tile's rows past the
                                        # end; 313 split tiles against 157 wide ones)
                                        (1, 40000, 128, True)])
def test_gemm_matches_oracle(env, M, n, k, asym):
    nh, oracle, gu, torch = env
    _say("gemm", M, n, k, asym)
    rng = np.random.default_rng(M * 7 + n)
    W = synth.w4_random(5, M, 1, 2, n, k)
    if asym:
        W = _asym(W, M)
    X = _x(rng, M, k)
    Y = gu.empty_f32(M, n)
    ws = gu.workspace(nh.nh_w4_gemm_workspace_bytes(M, k))
    nh.nh_w4_gemm(gu.w4_dev(W), gu.to_dev(X), M, None, 0, Y, nh.NH_F32, ws, ws.numel())
    got = Y.cpu().numpy()
    rows = np.arange(M) if M <= 64 else np.unique(np.r_[0, 1, M // 2, M - 2, M - 1, rng.integers(0, M, 8)])
    ref = oracle.w4_matvec(W, gu.bf16_bits_to_f64(X[rows]))
    assert gu.rel_l2(got[rows], ref) < 1e-5
    assert gu.max_abs(got[rows], ref) < 1e-4 * max(1.0, np.abs(ref).max())


def test_gemm_in_proj_full_size_sampled_rows(env):
    nh, oracle, gu, torch = env
    _say("gemm in_proj 413 rows")
    rng = np.random.default_rng(2)
    W = synth.layer_weights(0).in_proj
    M = 413
    X = _x(rng, M, 4480)
    res = synth.f32_to_bf16(rng.normal(size=(M, W.n_out)).astype(np.float32))
    Y = gu.empty_u16(M, W.n_out)
    ws = gu.workspace(nh.nh_w4_gemm_workspace_bytes(M, 4480))
    nh.nh_w4_gemm(gu.w4_dev(W), gu.to_dev(X), M, gu.to_dev(res), nh.NH_BF16, Y, nh.NH_BF16, ws, ws.numel())
    got = gu.bf16_bits_to_f64(gu.from_dev_u16(Y))
    rows = [0, 127, 128, 255, 256, 412]
    ref = oracle.w4_matvec(W, gu.bf16_bits_to_f64(X[rows])) + gu.bf16_bits_to_f64(res[rows])
    assert np.all(np.abs(got[rows] - ref) <= np.abs(ref) * 2 ** -8 + 1e-4)


# ------------------------------------------------------------------------ conv

def test_conv_step_and_seq(env):
    nh, oracle, gu, torch = env
    rng = np.random.default_rng(3)
    C, B, ld = synth.CONV_DIM, 2, synth.IN_PROJ_OUT
    w = synth.f32_to_bf16(rng.normal(0, 0.25, (C, 4)).astype(np.float32))
    b = synth.f32_to_bf16(rng.normal(0, 0.1, C).astype(np.float32))
    for T in [1, 2, 3, 17, 413]:
        for with_state in [False, True]:
            _say("conv seq", T, with_state)
            xbc = synth.f32_to_bf16(rng.normal(0, 1.2, (B, T, ld)).astype(np.float32))
            st = synth.f32_to_bf16(rng.normal(0, 1, (B, 3, C)).astype(np.float32)) if with_state else None
            out = gu.empty_u16(B, T, C)
            so = gu.empty_u16(B, 3, C)
            xd = gu.to_dev(xbc)
            nh.nh_conv1d_seq(xd[:, :, 10240:], ld, T, None if st is None else gu.to_dev(st), so,
                             gu.to_dev(w), gu.to_dev(b), out, B, C)
            got = gu.bf16_bits_to_f64(gu.from_dev_u16(out))
            for bb in range(B):
                ref, ref_st = oracle.conv1d(gu.bf16_bits_to_f64(xbc[bb, :, 10240:10240 + C]), w, b,
                                            None if st is None else gu.bf16_bits_to_f64(st[bb]))
                assert np.all(np.abs(got[bb] - ref) <= np.abs(ref) * 2 ** -8 + 1e-6)
                assert np.array_equal(gu.bf16_bits_to_f64(gu.from_dev_u16(so)[bb]), ref_st)
    _say("conv step")
    st = synth.f32_to_bf16(rng.normal(0, 1, (B, 3, C)).astype(np.float32))
    xs = synth.f32_to_bf16(rng.normal(0, 1.2, (B, ld)).astype(np.float32))
    std = gu.to_dev(st)
    out = gu.empty_u16(B, C)
    xsd = gu.to_dev(xs)
    nh.nh_conv1d_step(xsd[:, 10240:], ld, std, gu.to_dev(w), gu.to_dev(b), out, B, C)
    got = gu.bf16_bits_to_f64(gu.from_dev_u16(out))
    for bb in range(B):
        ref, ref_st = oracle.conv1d(gu.bf16_bits_to_f64(xs[bb:bb + 1, 10240:10240 + C]), w, b,
                                    gu.bf16_bits_to_f64(st[bb]))
        assert np.all(np.abs(got[bb] - ref[0]) <= np.abs(ref[0]) * 2 ** -8 + 1e-6)
        assert np.array_equal(gu.bf16_bits_to_f64(gu.from_dev_u16(std)[bb]), ref_st)


@pytest.mark.parametrize("C,ld,T", [(100, 103, 40), (96, 96, 64), (12288, 22656, 33)])
def test_conv_seq_other_shapes(env, C, ld, T):
    # channel counts and row strides that are not multiples of 8 take the one-channel kernel;
    # the others the 8-channel one, here with a full and a one-position last block
    nh, oracle, gu, torch = env
    _say("conv seq shape", C, ld, T)
    rng = np.random.default_rng(C + T)
    w = synth.f32_to_bf16(rng.normal(0, 0.25, (C, 4)).astype(np.float32))
    b = synth.f32_to_bf16(rng.normal(0, 0.1, C).astype(np.float32))
    for with_state in [False, True]:
        xbc = synth.f32_to_bf16(rng.normal(0, 1.2, (1, T, ld)).astype(np.float32))
        st = synth.f32_to_bf16(rng.normal(0, 1, (1, 3, C)).astype(np.float32)) if with_state else None
        out = gu.empty_u16(1, T, C)
        so = gu.empty_u16(1, 3, C)
        nh.nh_conv1d_seq(gu.to_dev(xbc), ld, T, None if st is None else gu.to_dev(st), so,
                         gu.to_dev(w), gu.to_dev(b), out, 1, C)
        got = gu.bf16_bits_to_f64(gu.from_dev_u16(out))[0]
        ref, ref_st = oracle.conv1d(gu.bf16_bits_to_f64(xbc[0, :, :C]), w, b,
                                    None if st is None else gu.bf16_bits_to_f64(st[0]))
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8 + 1e-6)
        assert np.array_equal(gu.bf16_bits_to_f64(gu.from_dev_u16(so)[0]), ref_st)


# ------------------------------------------------------------------- SSM step

def _scan_inputs(rng, B, T):
    """xc ~ N(0, 0.6^2) and dt_raw ~ N(0, 1.25^2) in bf16: the magnitudes the block produces."""
    xc = synth.f32_to_bf16(rng.normal(0, 0.6, (B, T, synth.CONV_DIM)).astype(np.float32))
    dtr = synth.f32_to_bf16(rng.normal(0, 1.25, (B, T, synth.N_HEADS)).astype(np.float32))
    return xc, dtr


def _oracle_scan(oracle, gu, lw, xc, dtr, S0):
    xcd = gu.bf16_bits_to_f64(xc)
    dt, A = oracle.discretize(gu.bf16_bits_to_f64(dtr), lw.dt_bias, lw.A_log)
    return oracle.ssm_recurrence(xcd[:, :10240], xcd[:, 10240:11264], xcd[:, 11264:], dt, A, lw.D, S0, G=8)


@pytest.mark.parametrize("B", [1, 2])
def test_ssm_step_matches_oracle(env, B):
    nh, oracle, gu, torch = env
    _say("ssm step", B)
    rng = np.random.default_rng(40 + B)
    lw = synth.layer_weights(0)
    xc, dtr = _scan_inputs(rng, B, 1)
    S0 = (0.1 * rng.normal(size=(B, 128, 80, 128))).astype(np.float32)
    Sd = gu.to_dev(S0)
    y = gu.empty_f32(B, 10240)
    nh.nh_ssm_step(nh.dims(), gu.to_dev(xc), gu.to_dev(dtr), 128, gu.to_dev(lw.dt_bias), gu.to_dev(lw.A_log),
                   gu.to_dev(lw.D), Sd, y, nh.NH_F32, B)
    for b in range(B):
        ry, rS = _oracle_scan(oracle, gu, lw, xc[b], dtr[b], S0[b].astype(np.float64))
        assert gu.rel_l2(y.cpu().numpy()[b], ry[0]) < 1e-5
        assert gu.rel_l2(Sd.cpu().numpy()[b], rS) < 1e-6


# ----------------------------------------------------------------------- scan

def _rows(gu, got, ref, what, bf16=False):
    """Row-wise bars on a scan output (bf16 outputs add one bf16 rounding, 2^-9 relative)."""
    worst, mabs, top = gu.row_errors(got, ref)
    slack = 2.0 if bf16 else 1.0
    print(f"[{what}] worst row rel {worst:.3e}, max-abs {mabs:.3e} of max |y| {top:.3e}", flush=True)
    assert worst <= slack * ROW_REL, worst
    assert mabs <= slack * ROW_ABS * top, (mabs, top)


def _scan_ws(nh, gu, Q, B, T):
    n = nh.nh_ssd_scan_workspace_bytes(nh.dims(chunk=Q), B, T)
    # at most 8 KiB per position for short chunks (C.B^T tiles; chunks under 17 rows at worst),
    # 10 KiB for long ones (tiles, B and C fragments, decay tables)
    assert 0 < n <= (10240 if Q >= 128 and T >= 64 else 8192) * B * T
    return gu.workspace(n), n


@pytest.mark.parametrize("T,Q,h0,B", [(1, 128, False, 1), (5, 4, True, 1), (16, 128, False, 1), (17, 16, True, 2),
                                      (40, 7, False, 1), (129, 128, True, 1), (300, 256, False, 1),
                                      (413, 128, False, 1), (413, 256, True, 2), (64, 1, False, 1),
                                      # chunks of at least 128 rows in sequences of at least 64
                                      # positions take the long-chunk kernel: its threshold (one
                                      # 64-row chunk), chunk lengths that are not powers of two, and
                                      # a last chunk of one row
                                      (64, 128, True, 1), (200, 160, True, 2), (300, 200, False, 1),
                                      (257, 256, False, 1), (511, 255, True, 1)])
def test_scan_matches_recurrence(env, T, Q, h0, B):
    nh, oracle, gu, torch = env
    _say("scan", T, Q, h0, B)
    rng = np.random.default_rng(T * 31 + Q)
    lw = synth.layer_weights(1)
    xc, dtr = _scan_inputs(rng, B, T)
    S0 = (0.1 * rng.normal(size=(B, 128, 80, 128))).astype(np.float32) if h0 else None
    y = gu.empty_f32(B, T, 10240)
    hT = gu.empty_f32(B, 128, 80, 128)
    nh.nh_ssd_chunk_scan(nh.dims(chunk=Q), gu.to_dev(xc), gu.to_dev(dtr), 128, T, gu.to_dev(lw.dt_bias),
                         gu.to_dev(lw.A_log), gu.to_dev(lw.D), None if S0 is None else gu.to_dev(S0), hT, y,
                         nh.NH_F32, B, *_scan_ws(nh, gu, Q, B, T))
    yg, Sg = y.cpu().numpy(), hT.cpu().numpy()
    for b in range(B):
        s0 = np.zeros((128, 80, 128)) if S0 is None else S0[b].astype(np.float64)
        ry, rS = _oracle_scan(oracle, gu, lw, xc[b], dtr[b], s0)
        assert gu.rel_l2(yg[b], ry) < 2e-3, gu.rel_l2(yg[b], ry)
        assert gu.rel_l2(Sg[b], rS) < 1e-3, gu.rel_l2(Sg[b], rS)
        _rows(gu, yg[b], ry, f"scan T={T} Q={Q} b{b}")


@pytest.mark.parametrize("T,Q", [(100, 32), (300, 256)])
def test_scan_bf16_output_and_alias(env, T, Q):
    nh, oracle, gu, torch = env
    _say("scan bf16 + aliased state", T, Q)
    rng = np.random.default_rng(77 + T)
    lw = synth.layer_weights(2)
    xc, dtr = _scan_inputs(rng, 1, T)
    S0 = (0.1 * rng.normal(size=(1, 128, 80, 128))).astype(np.float32)
    Sd = gu.to_dev(S0)
    y = gu.empty_u16(1, T, 10240)
    nh.nh_ssd_chunk_scan(nh.dims(chunk=Q), gu.to_dev(xc), gu.to_dev(dtr), 128, T, gu.to_dev(lw.dt_bias),
                         gu.to_dev(lw.A_log), gu.to_dev(lw.D), Sd, Sd, y, nh.NH_BF16, 1, *_scan_ws(nh, gu, Q, 1, T))
    ry, rS = _oracle_scan(oracle, gu, lw, xc[0], dtr[0], S0[0].astype(np.float64))
    yb = gu.bf16_bits_to_f64(gu.from_dev_u16(y)[0])
    assert gu.rel_l2(yb, ry) < 4e-3
    _rows(gu, yb, ry, "scan bf16", bf16=True)
    assert gu.rel_l2(Sd.cpu().numpy()[0], rS) < 1e-3


@pytest.mark.parametrize("T,Q", [(413, 128), (29, 256), (7, 4), (257, 256), (190, 160)])
def test_scan_stores_stay_inside_the_sequence(env, T, Q):
    """Rows past T in the last, partial chunk are computed as padding and must never be stored:
    the memory right after y (and before it) keeps its contents."""
    nh, oracle, gu, torch = env
    _say("scan bounds", T, Q)
    rng = np.random.default_rng(5 + T)
    lw = synth.layer_weights(3)
    xc, dtr = _scan_inputs(rng, 1, T)
    pad = 64
    buf = torch.full(((T + 2 * pad) * 10240,), 0x7E5A, dtype=torch.int16, device="cuda")
    y = buf[pad * 10240:(pad + T) * 10240]
    nh.nh_ssd_chunk_scan(nh.dims(chunk=Q), gu.to_dev(xc), gu.to_dev(dtr), 128, T, gu.to_dev(lw.dt_bias),
                         gu.to_dev(lw.A_log), gu.to_dev(lw.D), None, None, y, nh.NH_BF16, 1, *_scan_ws(nh, gu, Q, 1, T))
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:pad * 10240] == 0x7E5A)
    assert np.all(host[(pad + T) * 10240:] == 0x7E5A)
    ry, _ = _oracle_scan(oracle, gu, lw, xc[0], dtr[0], np.zeros((128, 80, 128)))
    got = gu.bf16_bits_to_f64(host[pad * 10240:(pad + T) * 10240].view(np.uint16).reshape(T, 10240))
    assert gu.rel_l2(got, ry) < 4e-3
    _rows(gu, got, ry, f"scan bounds T={T} Q={Q}", bf16=True)


# ---------------------------------------------------------------------- norms

def test_rmsnorm_and_gated_norm(env):
    nh, oracle, gu, torch = env
    rng = np.random.default_rng(8)
    rows = 33
    _say("rmsnorm")
    x = rng.normal(size=(rows, 4480)).astype(np.float32)
    w = synth.f32_to_bf16((1 + 0.05 * rng.normal(size=4480)).astype(np.float32))
    u = gu.empty_u16(rows, 4480)
    nh.nh_rmsnorm(gu.to_dev(x), nh.NH_F32, gu.to_dev(w), u, rows, 4480, 1e-5)
    ref = oracle.rmsnorm(x.astype(np.float64), w, 1e-5)
    got = gu.bf16_bits_to_f64(gu.from_dev_u16(u))
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8 + 1e-7)
    assert gu.bf16_ulp_flips(gu.from_dev_u16(u), ref) <= rows * 4480 * 1e-3
    _say("gated norm")
    y = synth.f32_to_bf16(rng.normal(size=(rows, 10240)).astype(np.float32))
    z = synth.f32_to_bf16(rng.normal(size=(rows, 22656)).astype(np.float32))
    gw = synth.f32_to_bf16((1 + 0.05 * rng.normal(size=10240)).astype(np.float32))
    o = gu.empty_u16(rows, 10240)
    nh.nh_rmsnorm_gated(gu.to_dev(y), nh.NH_BF16, gu.to_dev(z), 22656, gu.to_dev(gw), o, rows, 10240, 1280, 1e-5)
    ref = oracle.rmsnorm_gated(gu.bf16_bits_to_f64(y), gu.bf16_bits_to_f64(z)[:, :10240], gw, 1280, 1e-5)
    got = gu.bf16_bits_to_f64(gu.from_dev_u16(o))
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8 + 1e-7)


@pytest.mark.parametrize("rows,d,group,ld_z", [(33, 10240, 1280, 22656), (5, 8192, 4096, 8200)])
def test_gated_norm_f32_y(env, rows, d, group, ld_z):
    # y given as fp32 (the SSM's own precision): used as it is, with z bf16
    nh, oracle, gu, torch = env
    rng = np.random.default_rng(rows + group)
    _say(f"gated norm f32 y rows={rows} d={d} group={group}")
    y = rng.normal(size=(rows, d)).astype(np.float32)
    z = synth.f32_to_bf16(rng.normal(size=(rows, ld_z)).astype(np.float32))
    gw = synth.f32_to_bf16((1 + 0.05 * rng.normal(size=d)).astype(np.float32))
    o = gu.empty_u16(rows, d)
    nh.nh_rmsnorm_gated(gu.to_dev(y), nh.NH_F32, gu.to_dev(z), ld_z, gu.to_dev(gw), o, rows, d, group, 1e-5)
    ref = oracle.rmsnorm_gated(y.astype(np.float64), gu.bf16_bits_to_f64(z)[:, :d], gw, group, 1e-5)
    got = gu.bf16_bits_to_f64(gu.from_dev_u16(o))
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8 + 1e-7)


@pytest.mark.gpu
@pytest.mark.parametrize("rows,d,group,ld_z", [(5, 8192, 4096, 8200), (7, 96, 8, 96), (3, 2048, 2048, 2048)])
def test_gated_norm_other_groups(env, rows, d, group, ld_z):
    # groups above 2048 channels take the work-group-per-group kernel, the rest the
    # wave-per-group one; ragged 16-byte tails (group / 8 not a multiple of 64) included
    nh, oracle, gu, torch = env
    rng = np.random.default_rng(rows * 31 + group)
    _say(f"gated norm rows={rows} d={d} group={group}")
    y = synth.f32_to_bf16(rng.normal(size=(rows, d)).astype(np.float32))
    z = synth.f32_to_bf16(rng.normal(size=(rows, ld_z)).astype(np.float32))
    gw = synth.f32_to_bf16((1 + 0.05 * rng.normal(size=d)).astype(np.float32))
    o = gu.empty_u16(rows, d)
    nh.nh_rmsnorm_gated(gu.to_dev(y), nh.NH_BF16, gu.to_dev(z), ld_z, gu.to_dev(gw), o, rows, d, group, 1e-5)
    ref = oracle.rmsnorm_gated(gu.bf16_bits_to_f64(y), gu.bf16_bits_to_f64(z)[:, :d], gw, group, 1e-5)
    got = gu.bf16_bits_to_f64(gu.from_dev_u16(o))
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8 + 1e-7)
