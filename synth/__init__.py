"""Seeded synthetic inputs for the Nemotron-H Mamba2 mixer block.

This module only draws numbers and lays them out; it holds none of the
block's arithmetic.  Both the oracle-side tests and the GPU-side tests and
benchmark take their inputs from here, so the two implementations are
compared on identical bytes.

Shapes follow the text_config of the Nemotron-H language model printed on the
issue page "feat(nemotron_voicechat): ... offline duplex inference #1374",
section "config.json" (hidden_size 4480, mamba_num_heads 128, mamba_head_dim
80, ssm_state_size 128, n_groups 8, conv_kernel 4), and the 4-bit group-64
quantization of the mixer projections stated in the same section.

Distributions (the workload recipe, identical for every consumer):
  in_proj / out_proj: q ~ U{0..15} per nibble, scale ~ U(0.002, 0.006) rounded
      to bf16, bias = -8 * scale (exact in bf16);
  A_log = ln U(1, 16); dt_bias = softplus^-1(U(1e-3, 0.1)); D ~ U(0.5, 1.5)
      (all float32);
  conv weight ~ N(0, 0.25^2), conv bias ~ N(0, 0.1^2), both norm weights
      1 + N(0, 0.05^2) (all bf16);
  block input x ~ N(0, 1) (bf16); pre-filled conv state ~ N(0, 1) (bf16);
  pre-filled SSM state ~ N(0, 0.1^2) (float32);
  attention layers (the '*' layers): norm weight 1 + N(0, 0.05^2) (bf16); q_proj
      (5120 x 4480), k_proj, v_proj (1024 x 4480 each) and o_proj (4480 x 5120) drawn like
      in_proj; a pre-filled KV cache ~ N(0, 1.3^2) (bf16), the magnitude of k = W_k u;
  output heads (lm_head, function_head, 131072 x 4480 each, the vocab_size of the
      same config) and the input embedding embed_tokens (same shape): drawn like in_proj;
      norm_f ~ 1 + N(0, 0.05^2) (bf16); previous text / function ids ~ U{0..131071};
      projected audio frame ~ N(0, 1) (float32).

Random streams: numpy PCG64 seeded by SeedSequence([seed, layer, tensor_id])
for weights and SeedSequence([seed, 1000 + stream, tensor_id]) for inputs (stream: a
small integer naming the input draw), so any tensor can be regenerated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Nemotron-H mixer dimensions.
HIDDEN = 4480
N_HEADS = 128
HEAD_DIM = 80
D_STATE = 128
N_GROUPS = 8
CONV_K = 4
GROUP_SIZE = 64
D_INNER = N_HEADS * HEAD_DIM                    # 10240
CONV_DIM = D_INNER + 2 * N_GROUPS * D_STATE     # 12288
IN_PROJ_OUT = 2 * D_INNER + 2 * N_GROUPS * D_STATE + N_HEADS  # 22656
EPS = 1e-5

# Stable tensor ids (part of the seeding recipe; never renumber).
_T_NORM_W, _T_IN_Q, _T_IN_S, _T_CONV_W, _T_CONV_B = 0, 1, 2, 3, 4
_T_DT_BIAS, _T_A_LOG, _T_D, _T_GNORM_W, _T_OUT_Q, _T_OUT_S = 5, 6, 7, 8, 9, 10
_I_X, _I_CONV_STATE, _I_SSM_STATE = 0, 1, 2
# The final norm and the two output heads sit outside the 56 layers; they draw from
# pseudo-layer HEADS_LAYER with their own tensor ids.
HEADS_LAYER = 100
_T_NORM_F, _T_LMH_Q, _T_LMH_S, _T_FNH_Q, _T_FNH_S = 11, 12, 13, 14, 15
_T_EMB_Q, _T_EMB_S = 16, 17
# MLP layers use their own layer index of the hybrid pattern and these tensor ids
_T_MLP_NORM, _T_UP_Q, _T_UP_S, _T_DOWN_Q, _T_DOWN_S = 20, 21, 22, 23, 24
MLP_INTER = 15680
_I_AUDIO, _I_IDS = 3, 4
# attention layers: 40 query heads and 8 key/value heads of 128 (text_config)
ATT_HEADS, ATT_KV_HEADS, ATT_HEAD_DIM = 40, 8, 128
_T_ATT_NORM, _T_Q_Q, _T_Q_S, _T_K_Q, _T_K_S, _T_V_Q, _T_V_S, _T_O_Q, _T_O_S = 30, 31, 32, 33, 34, 35, 36, 37, 38
_I_KV = 5
VOCAB = 131072


@dataclass
class Dims:
    hidden: int = HIDDEN
    n_heads: int = N_HEADS
    head_dim: int = HEAD_DIM
    d_state: int = D_STATE
    n_groups: int = N_GROUPS
    conv_k: int = CONV_K
    group_size: int = GROUP_SIZE
    eps: float = EPS

    @property
    def d_inner(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def conv_dim(self) -> int:
        return self.d_inner + 2 * self.n_groups * self.d_state

    @property
    def in_proj_out(self) -> int:
        return 2 * self.d_inner + 2 * self.n_groups * self.d_state + self.n_heads


REAL = Dims()


def rng(seed: int, *path: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, *path]))


def f32_to_bf16(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class W4Matrix:
    """MLX-style affine 4-bit matrix: W[n][k] = scale[n][k//gs] * q[n][k] + bias[n][k//gs].

    qweight[n][j] packs nibbles k = 8j .. 8j+7, the lowest nibble holding k = 8j.
    """
    qweight: np.ndarray   # uint32 [n_out][k_in/8]
    scales: np.ndarray    # uint16 (bf16 bits) [n_out][k_in/gs]
    biases: np.ndarray    # uint16 (bf16 bits) [n_out][k_in/gs]
    n_out: int
    k_in: int
    group_size: int = GROUP_SIZE


def w4_random(seed: int, layer: int, tid_q: int, tid_s: int, n: int, k: int,
              gs: int = GROUP_SIZE) -> W4Matrix:
    assert k % gs == 0 and k % 8 == 0
    # Eight i.i.d. U{0..15} nibbles packed into one word are one uniform 32-bit word.
    qw = rng(seed, layer, tid_q).integers(0, 1 << 32, size=(n, k // 8), dtype=np.uint32)
    s32 = rng(seed, layer, tid_s).uniform(0.002, 0.006, size=(n, k // gs)).astype(np.float32)
    sb = f32_to_bf16(s32)
    bb = f32_to_bf16(bf16_to_f32(sb) * np.float32(-8.0))  # exact: a power-of-two multiple
    return W4Matrix(qw, sb, bb, n, k, gs)


@dataclass
class LayerWeights:
    norm_w: np.ndarray      # bf16 [hidden]
    in_proj: W4Matrix       # [in_proj_out][hidden]
    conv_w: np.ndarray      # bf16 [conv_dim][conv_k], tap conv_k-1 multiplies the newest input
    conv_b: np.ndarray      # bf16 [conv_dim]
    dt_bias: np.ndarray     # f32 [n_heads]
    A_log: np.ndarray       # f32 [n_heads]
    D: np.ndarray           # f32 [n_heads]
    gnorm_w: np.ndarray     # bf16 [d_inner]
    out_proj: W4Matrix      # [hidden][d_inner]


def layer_weights(layer: int, seed: int = 0, d: Dims = REAL) -> LayerWeights:
    g = lambda tid: rng(seed, layer, tid)  # noqa: E731
    f32 = np.float32
    norm_w = f32_to_bf16(1.0 + g(_T_NORM_W).normal(0.0, 0.05, d.hidden).astype(f32))
    in_proj = w4_random(seed, layer, _T_IN_Q, _T_IN_S, d.in_proj_out, d.hidden, d.group_size)
    conv_w = f32_to_bf16(g(_T_CONV_W).normal(0.0, 0.25, (d.conv_dim, d.conv_k)).astype(f32))
    conv_b = f32_to_bf16(g(_T_CONV_B).normal(0.0, 0.1, d.conv_dim).astype(f32))
    dt0 = g(_T_DT_BIAS).uniform(1e-3, 0.1, d.n_heads)
    dt_bias = np.log(np.expm1(dt0)).astype(f32)
    A_log = np.log(g(_T_A_LOG).uniform(1.0, 16.0, d.n_heads)).astype(f32)
    D = g(_T_D).uniform(0.5, 1.5, d.n_heads).astype(f32)
    gnorm_w = f32_to_bf16(1.0 + g(_T_GNORM_W).normal(0.0, 0.05, d.d_inner).astype(f32))
    out_proj = w4_random(seed, layer, _T_OUT_Q, _T_OUT_S, d.hidden, d.d_inner, d.group_size)
    return LayerWeights(norm_w, in_proj, conv_w, conv_b, dt_bias, A_log, D, gnorm_w, out_proj)


@dataclass
class HeadWeights:
    norm_f: np.ndarray          # bf16 [hidden]
    lm_head: W4Matrix           # [n_out][hidden]
    function_head: W4Matrix     # [n_out][hidden]


def head_weights(seed: int = 0, n_out: int = VOCAB, d: Dims = REAL) -> HeadWeights:
    """norm_f ~ 1 + N(0, 0.05^2) (bf16); both heads drawn like the mixer projections."""
    g = rng(seed, HEADS_LAYER, _T_NORM_F)
    norm_f = f32_to_bf16(1.0 + g.normal(0.0, 0.05, d.hidden).astype(np.float32))
    lm = w4_random(seed, HEADS_LAYER, _T_LMH_Q, _T_LMH_S, n_out, d.hidden, d.group_size)
    fn = w4_random(seed, HEADS_LAYER, _T_FNH_Q, _T_FNH_S, n_out, d.hidden, d.group_size)
    return HeadWeights(norm_f, lm, fn)


@dataclass
class MlpWeights:
    norm_w: np.ndarray      # bf16 [hidden]
    up: W4Matrix            # [15680][hidden]
    down: W4Matrix          # [hidden][15680]


def mlp_weights(layer: int, seed: int = 0, inter: int = MLP_INTER, d: Dims = REAL) -> MlpWeights:
    """norm weight 1 + N(0, 0.05^2); up and down drawn like in_proj.  The down scales are
    divided by 8 (U(0.00025, 0.00075)): the squared-ReLU activations reach tens, and the
    mixer's scale range would make each MLP layer add O(100) to the residual stream."""
    g = rng(seed, layer, _T_MLP_NORM)
    norm_w = f32_to_bf16(1.0 + g.normal(0.0, 0.05, d.hidden).astype(np.float32))
    up = w4_random(seed, layer, _T_UP_Q, _T_UP_S, inter, d.hidden, d.group_size)
    dq = rng(seed, layer, _T_DOWN_Q).integers(0, 1 << 32, size=(d.hidden, inter // 8), dtype=np.uint32)
    s32 = rng(seed, layer, _T_DOWN_S).uniform(0.00025, 0.00075, size=(d.hidden, inter // d.group_size)).astype(np.float32)
    sb = f32_to_bf16(s32)
    bb = f32_to_bf16(bf16_to_f32(sb) * np.float32(-8.0))
    return MlpWeights(norm_w, up, W4Matrix(dq, sb, bb, d.hidden, inter, d.group_size))


@dataclass
class AttentionWeights:
    norm_w: np.ndarray      # bf16 [hidden]
    q_proj: W4Matrix        # [heads * head_dim][hidden]
    k_proj: W4Matrix        # [kv_heads * head_dim][hidden]
    v_proj: W4Matrix        # [kv_heads * head_dim][hidden]
    o_proj: W4Matrix        # [hidden][heads * head_dim]


def attention_weights(layer: int, seed: int = 0, d: Dims = REAL) -> AttentionWeights:
    """One attention layer ('*' of the pattern): norm weight 1 + N(0, 0.05^2); q, k, v and o
    projections drawn like in_proj (q U{0..15}, scales U(0.002, 0.006), bias -8 scale)."""
    g = rng(seed, layer, _T_ATT_NORM)
    norm_w = f32_to_bf16(1.0 + g.normal(0.0, 0.05, d.hidden).astype(np.float32))
    qd, kd = ATT_HEADS * ATT_HEAD_DIM, ATT_KV_HEADS * ATT_HEAD_DIM
    return AttentionWeights(norm_w,
                            w4_random(seed, layer, _T_Q_Q, _T_Q_S, qd, d.hidden, d.group_size),
                            w4_random(seed, layer, _T_K_Q, _T_K_S, kd, d.hidden, d.group_size),
                            w4_random(seed, layer, _T_V_Q, _T_V_S, kd, d.hidden, d.group_size),
                            w4_random(seed, layer, _T_O_Q, _T_O_S, d.hidden, qd, d.group_size))


def kv_cache(stream: int, batch: int, T: int, seed: int = 0):
    """A pre-filled KV cache of T positions: keys and values ~ N(0, 1.3^2) rounded to bf16,
    layout [batch][kv_heads][T][head_dim] (uint16 bits) each."""
    g = rng(seed, 1000 + stream, _I_KV)
    shape = (batch, ATT_KV_HEADS, T, ATT_HEAD_DIM)
    k = g.normal(0.0, 1.3, shape).astype(np.float32)
    v = g.normal(0.0, 1.3, shape).astype(np.float32)
    return f32_to_bf16(k), f32_to_bf16(v)


def embed_tokens(seed: int = 0, n_out: int = VOCAB, d: Dims = REAL) -> W4Matrix:
    """The 4-bit input embedding [n_out][hidden], drawn like in_proj."""
    return w4_random(seed, HEADS_LAYER, _T_EMB_Q, _T_EMB_S, n_out, d.hidden, d.group_size)


def embed_inputs(stream: int, batch: int, n_out: int = VOCAB, seed: int = 0, d: Dims = REAL):
    """Per position: previous text id and function id ~ U{0..n_out-1} (int32) and the projected
    audio frame ~ N(0, 1) (float32, [batch][hidden])."""
    ids = rng(seed, 1000 + stream, _I_IDS).integers(0, n_out, size=(2, batch)).astype(np.int32)
    audio = rng(seed, 1000 + stream, _I_AUDIO).normal(0.0, 1.0, (batch, d.hidden)).astype(np.float32)
    return ids[0], ids[1], audio


def block_input(stream: int, batch: int, T: int, seed: int = 0, d: Dims = REAL) -> np.ndarray:
    """x ~ N(0, 1) rounded to bf16, layout [batch][T][hidden] (uint16 bits)."""
    x = rng(seed, 1000 + stream, _I_X).normal(0.0, 1.0, (batch, T, d.hidden)).astype(np.float32)
    return f32_to_bf16(x)


def prefilled_state(stream: int, batch: int, seed: int = 0, d: Dims = REAL):
    """Pre-filled decode state: conv [batch][K-1][conv_dim] bf16 ~ N(0,1), SSM [batch][H][P][N] f32 ~ N(0, 0.1^2)."""
    cs = rng(seed, 1000 + stream, _I_CONV_STATE).normal(
        0.0, 1.0, (batch, d.conv_k - 1, d.conv_dim)).astype(np.float32)
    ss = rng(seed, 1000 + stream, _I_SSM_STATE).normal(
        0.0, 0.1, (batch, d.n_heads, d.head_dim, d.d_state)).astype(np.float32)
    return f32_to_bf16(cs), ss


# The five workloads: (name, layers, batch, T, chunk, mode).
@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    layers: int
    batch: int
    T: int
    chunk: int
    mode: str
    prefilled: bool = False


CONFIGS = [
    Config(0, "block_b1_t16_seq_and_step", 1, 1, 16, 128, "both"),
    Config(1, "block_b1_step_prefilled", 1, 1, 1, 128, "step", prefilled=True),
    Config(2, "block_b1_t413_seq_q128", 1, 1, 413, 128, "seq"),
    Config(3, "stack27_b1_t413_step", 27, 1, 413, 128, "step"),
    Config(4, "stack27_b2_t3750_seq_q256", 27, 2, 3750, 256, "seq"),
]
