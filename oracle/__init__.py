"""CPU oracle for the Nemotron-H Mamba2 mixer block (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the GPU library and
its Python binding) never imports, links or runs anything under ``oracle/``.

The arithmetic lives in ``nh_oracle.c`` (plain C, fp64); this module builds it
with gcc, wraps it with ctypes and adds these numpy-level pieces:

* ``ssd_chunked`` -- the chunked state-space-duality form of the same scan
  (Dao & Gu 2024, "Transformers are SSMs", the SSD algorithm: intra-chunk
  quadratic form, chunk states, state passing, state-to-output), in fp64.  It
  is not used to produce expected values; it is pinned against the recurrence
  for many chunk lengths and documents the decomposition the GPU scan uses.
* ``stack`` -- composition of blocks over the hybrid layer pattern.
* ``head`` and ``greedy_ids`` -- the final norm, one 4-bit output head and the
  greedy id (smallest index of the largest logit, NaN never chosen).
* ``fused_embedding`` -- the language model's input row: two 4-bit embedding rows
  and the audio frame.
* ``mlp`` -- one MLP layer of the hybrid stack (pre-norm, 4-bit up, squared ReLU,
  4-bit down, residual).
* ``attention_core`` and ``attention`` -- one grouped-query attention layer of the hybrid
  stack at one position with its key/value cache (pre-norm, 4-bit q/k/v, softmax attention
  over the cached and the new position, 4-bit o, residual).

Readings of the pages that the oracle fixes (no mixer equations are printed
on the pages; see the header of nh_oracle.c):
  split order z | x | B | C | dt_raw; head h uses B/C group h // (H/G);
  conv = cross-correlation, tap K-1 newest, SiLU on all x|B|C channels;
  softplus without threshold, no dt clamp; D skip on the post-conv x;
  RMSNorm with a plain weight and eps inside the root; gate before the norm.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nh_oracle.c")
_LIB = os.path.join(_HERE, "libnhoracle.so")

EXACT = 0
CONTRACT = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP for the outer loops)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        dp = C.POINTER(C.c_double)
        u16p = C.POINTER(C.c_uint16)
        u32p = C.POINTER(C.c_uint32)
        f32p = C.POINTER(C.c_float)
        L.nho_bf16_to_double.restype = C.c_double
        L.nho_bf16_to_double.argtypes = [C.c_uint16]
        L.nho_double_to_bf16.restype = C.c_uint16
        L.nho_double_to_bf16.argtypes = [C.c_double]
        L.nho_double_to_bf16_array.argtypes = [dp, u16p, C.c_long]
        L.nho_silu.restype = C.c_double
        L.nho_silu.argtypes = [C.c_double]
        L.nho_softplus.restype = C.c_double
        L.nho_softplus.argtypes = [C.c_double]
        L.nho_hybrid_pattern.restype = C.c_char_p
        L.nho_layers_of_kind.restype = C.c_int
        L.nho_layers_of_kind.argtypes = [C.c_char, C.POINTER(C.c_int), C.c_int]
        L.nho_w4_nibble.restype = C.c_int
        L.nho_w4_nibble.argtypes = [u32p, C.c_int]
        L.nho_w4_dequant.argtypes = [u32p, u16p, u16p, C.c_int, C.c_int, C.c_int, dp]
        L.nho_w4_matvec.argtypes = [u32p, u16p, u16p, C.c_int, C.c_int, C.c_int, dp, C.c_int,
                                    dp, C.c_int]
        L.nho_rmsnorm.argtypes = [dp, C.c_int, C.c_int, u16p, C.c_double, dp]
        L.nho_rmsnorm_gated.argtypes = [dp, dp, C.c_int, C.c_int, C.c_int, u16p, C.c_double, dp]
        L.nho_conv1d.argtypes = [dp, C.c_long, C.c_int, C.c_int, C.c_int, dp, u16p, u16p, dp, dp]
        L.nho_discretize.argtypes = [dp, C.c_long, C.c_int, C.c_int, f32p, f32p, dp, dp]
        L.nho_ssm_recurrence.argtypes = [C.c_int] * 5 + [dp, C.c_long, dp, C.c_long, dp, C.c_long,
                                                         dp, dp, f32p, dp, dp, C.c_int, C.c_int]
        L.nho_block.restype = C.c_int
        L.nho_block.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, dp, dp, dp, dp,
                                C.c_int, C.c_int, C.c_int, C.c_void_p]
        L.nho_max_threads.restype = C.c_int
        _lib = L
    return _lib


# ------------------------------------------------------------------ helpers

def _p(a, t):
    return a.ctypes.data_as(C.POINTER(t))


def _d(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def _u32(a):
    return np.ascontiguousarray(a, dtype=np.uint32)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def bf16_to_double(bits) -> np.ndarray:
    b = _u16(bits)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16(v) -> np.ndarray:
    """Round doubles to bf16 (nearest, ties to even) with the oracle's own rounding; uint16 bits."""
    v = _d(v)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().nho_double_to_bf16_array(_p(v, C.c_double), _p(out, C.c_uint16), v.size)
    return out


def round_bf16(v) -> np.ndarray:
    return bf16_to_double(to_bf16(v))


def silu(v: float) -> float:
    return lib().nho_silu(float(v))


def softplus(v: float) -> float:
    return lib().nho_softplus(float(v))


def hybrid_pattern() -> str:
    return lib().nho_hybrid_pattern().decode()


def layers_of_kind(c: str) -> list[int]:
    L = lib()
    n = L.nho_layers_of_kind(c.encode(), None, 0)
    idx = (C.c_int * max(n, 1))()
    L.nho_layers_of_kind(c.encode(), idx, n)
    return list(idx[:n])


def w4_nibble(qrow, k: int) -> int:
    q = _u32(qrow)
    return lib().nho_w4_nibble(_p(q, C.c_uint32), k)


def w4_dequant(W) -> np.ndarray:
    q, s, b = _u32(W.qweight), _u16(W.scales), _u16(W.biases)
    out = np.empty((W.n_out, W.k_in), dtype=np.float64)
    lib().nho_w4_dequant(_p(q, C.c_uint32), _p(s, C.c_uint16), _p(b, C.c_uint16),
                         W.n_out, W.k_in, W.group_size, _p(out, C.c_double))
    return out


def w4_matvec(W, x, nthreads: int = 0) -> np.ndarray:
    """y[m][n] = sum_k W[n][k] x[m][k] in fp64 (x given as doubles, [m][k])."""
    x = _d(x)
    squeeze = x.ndim == 1
    x2 = x.reshape(-1, W.k_in)
    q, s, b = _u32(W.qweight), _u16(W.scales), _u16(W.biases)
    y = np.empty((x2.shape[0], W.n_out), dtype=np.float64)
    lib().nho_w4_matvec(_p(q, C.c_uint32), _p(s, C.c_uint16), _p(b, C.c_uint16), W.n_out, W.k_in,
                        W.group_size, _p(x2, C.c_double), x2.shape[0], _p(y, C.c_double), nthreads)
    return y[0] if squeeze else y


def rmsnorm(x, w_bf16, eps: float) -> np.ndarray:
    x = _d(x)
    x2 = x.reshape(-1, x.shape[-1])
    w = _u16(w_bf16)
    out = np.empty_like(x2)
    lib().nho_rmsnorm(_p(x2, C.c_double), x2.shape[0], x2.shape[1], _p(w, C.c_uint16), eps,
                      _p(out, C.c_double))
    return out.reshape(x.shape)


def greedy_ids(logits) -> np.ndarray:
    """Greedy choice per row of logits [m][n]: the smallest index among those holding the
    largest value.  NaN entries never win; a row of NaN only gives -1."""
    l = _d(logits)
    l2 = l.reshape(-1, l.shape[-1])
    ids = np.full(l2.shape[0], -1, dtype=np.int64)
    for r in range(l2.shape[0]):
        ok = ~np.isnan(l2[r])
        if ok.any():
            best = l2[r][ok].max()
            ids[r] = int(np.flatnonzero(ok & (l2[r] == best))[0])
    return ids


def mlp(x, norm_w, W_up, W_down, eps: float, mode: int = CONTRACT) -> np.ndarray:
    """One MLP layer of the hybrid stack: out = x + down(relu(up(u))^2), u = RMSNorm(x) w.

    The issue page "feat(nemotron_voicechat): ... offline duplex inference #1374", section
    "config.json": the '-' layers of hybrid_override_pattern are MLPs with intermediate_size
    15680 and mlp_bias false, quantized like the mixer projections; the pages do not name the
    activation, and the squared ReLU of the Nemotron-H architecture is the reading taken here.
    CONTRACT rounds u and the activation h = relu(up(u))^2 to bf16 (the storage points the GPU
    kernels use); sums are fp64.  x: [m][hidden] doubles.  Returns out [m][hidden]."""
    x2 = _d(x).reshape(-1, W_up.k_in)
    u = rmsnorm(x2, norm_w, eps)
    if mode == CONTRACT:
        u = round_bf16(u)
    a = w4_matvec(W_up, u)
    h = np.maximum(a, 0.0) ** 2
    if mode == CONTRACT:
        h = round_bf16(h)
    return x2 + w4_matvec(W_down, h)


def attention_core(q, K, V, n_kv: int) -> np.ndarray:
    """Softmax attention of one query position per head over T key/value positions, with
    query heads grouped onto key/value heads (grouped-query attention).

    The issue page "feat(nemotron_voicechat): ... offline duplex inference #1374", section
    "config.json": num_attention_heads 40, num_key_value_heads 8, head_dim 128.  Query head h
    reads key/value head h // (heads / n_kv) (consecutive query heads share one key/value
    head), scores are q . k / sqrt(head_dim), and the weights are the softmax of the scores over
    all T positions (the query sits at the last position, so every cached position is visible).
    q: [heads][hd]; K, V: [n_kv][T][hd] (doubles).  Returns o [heads][hd] in fp64."""
    q, K, V = _d(q), _d(K), _d(V)
    heads, hd = q.shape
    rep = heads // n_kv
    o = np.empty((heads, hd))
    for h in range(heads):
        g = h // rep
        s = K[g] @ q[h] / np.sqrt(hd)        # [T]
        w = np.exp(s - s.max())
        w /= w.sum()
        o[h] = w @ V[g]
    return o


def attention(x, aw, k_cache, v_cache, eps: float, mode: int = CONTRACT):
    """One attention layer of the hybrid stack at one position per sequence, with its cache.

    The '*' layers of hybrid_override_pattern (issue page, section "config.json": attention at
    layers 14, 21, 30, 39, attention_bias false; q/k/v/o are Nemotron-H mixer projections and
    so 4-bit group-64 like the others).  No positional encoding enters (text_config names none):
        u = RMSNorm(x) w,  q = W_q u,  k = W_k u,  v = W_v u,
        o = attention_core(q, [K_cache; k], [V_cache; v]),  out = x + W_o o.
    The docs page "Nemotron VoiceChat", section "Online session": the attention key/value
    caches persist across positions; the new position's k and v are appended to them.
    CONTRACT rounds u, q, k, v and o to bf16 (the points where the GPU kernels store them).
    x: [m][hidden]; k_cache, v_cache: [m][n_kv][T][hd] doubles (T may be 0).
    Returns (out [m][hidden], k_new [m][n_kv][hd], v_new [m][n_kv][hd])."""
    x2 = _d(x).reshape(-1, aw.q_proj.k_in)
    m = x2.shape[0]
    kc, vc = _d(k_cache), _d(v_cache)
    n_kv = kc.shape[1]
    hd = kc.shape[3]
    heads = aw.q_proj.n_out // hd
    rnd = round_bf16 if mode == CONTRACT else (lambda a: a)
    u = rnd(rmsnorm(x2, aw.norm_w, eps))
    q = rnd(w4_matvec(aw.q_proj, u)).reshape(m, heads, hd)
    k = rnd(w4_matvec(aw.k_proj, u)).reshape(m, n_kv, hd)
    v = rnd(w4_matvec(aw.v_proj, u)).reshape(m, n_kv, hd)
    o = np.empty((m, heads * hd))
    for r in range(m):
        K = np.concatenate([kc[r], k[r][:, None, :]], axis=1)
        V = np.concatenate([vc[r], v[r][:, None, :]], axis=1)
        o[r] = attention_core(q[r], K, V, n_kv).reshape(-1)
    o = rnd(o)
    return x2 + w4_matvec(aw.o_proj, o), k, v


def fused_embedding(E, text_ids, function_ids, audio, function_weight: float = 2.0) -> np.ndarray:
    """The language model's input row per position, in fp64.

    The issue page "feat(nemotron_voicechat): ... offline duplex inference #1374", section
    "Network 2": the input at a timeline position is the 4-bit embed_tokens row of the
    previous text id, plus the projected audio frame, plus function_channel_weight (2.0 in
    the config) times the embed_tokens row of the previous function id; the LLM then runs on
    it with no lookup of its own.  E[id][k] = s q + b (the W4 affine map).
    text_ids, function_ids: [m] ints; audio: [m][k_in] doubles.  An id outside 0..n_out-1
    gives a row of NaN (a reading: the pages never feed such ids)."""
    a = _d(audio).reshape(-1, E.k_in)
    t = np.asarray(text_ids, dtype=np.int64).reshape(-1)
    f = np.asarray(function_ids, dtype=np.int64).reshape(-1)
    out = np.empty_like(a)
    for r in range(a.shape[0]):
        if not (0 <= t[r] < E.n_out and 0 <= f[r] < E.n_out):
            out[r] = np.nan
            continue
        et = _w4_row(E, int(t[r]))
        ef = _w4_row(E, int(f[r]))
        out[r] = et + a[r] + function_weight * ef
    return out


def _w4_row(E, n: int) -> np.ndarray:
    """Row n of dequant(E), through the oracle's W4 decode."""
    sub = type(E)(E.qweight[n:n + 1], E.scales[n:n + 1], E.biases[n:n + 1], 1, E.k_in, E.group_size)
    return w4_dequant(sub)[0]


def head(W, x, norm_w, eps: float, mode: int = CONTRACT):
    """Final norm and one greedy output head of the language model.

    The issue page "feat(nemotron_voicechat): ... offline duplex inference #1374", section
    "Network 2": the final hidden state is normalised by norm_f and fed to two 4-bit heads
    of shape [4480 -> 131072] (lm_head, function_head) with no linear bias; each head's id
    is chosen greedily from its logits at the newest position.
    h = x / rms(x) * norm_w (rounded to bf16 in CONTRACT mode, the point where the GPU
    kernel stores it); logits = dequant(W) h in fp64; ids = greedy_ids(logits).
    x: [m][k_in] doubles.  Returns (logits [m][n_out], ids [m])."""
    x2 = _d(x).reshape(-1, W.k_in)
    h = rmsnorm(x2, norm_w, eps)
    if mode == CONTRACT:
        h = round_bf16(h)
    logits = w4_matvec(W, h)
    return logits, greedy_ids(logits)


def rmsnorm_gated(y, z, w_bf16, group: int, eps: float) -> np.ndarray:
    y, z = _d(y), _d(z)
    y2, z2 = y.reshape(-1, y.shape[-1]), z.reshape(-1, z.shape[-1])
    w = _u16(w_bf16)
    out = np.empty_like(y2)
    lib().nho_rmsnorm_gated(_p(y2, C.c_double), _p(z2, C.c_double), y2.shape[0], y2.shape[1], group,
                            _p(w, C.c_uint16), eps, _p(out, C.c_double))
    return out.reshape(y.shape)


def conv1d(xbc, w_bf16, b_bf16, state_in=None):
    """xbc: [T][C] doubles (pre-conv).  Returns (out [T][C], state_out [K-1][C])."""
    xbc = _d(xbc)
    T, Cn = xbc.shape
    w = _u16(w_bf16)
    K = w.shape[1]
    b = _u16(b_bf16)
    out = np.empty((T, Cn), dtype=np.float64)
    st = np.empty((K - 1, Cn), dtype=np.float64)
    si = None if state_in is None else _d(state_in)
    lib().nho_conv1d(_p(xbc, C.c_double), Cn, T, Cn, K, None if si is None else _p(si, C.c_double),
                     _p(w, C.c_uint16), _p(b, C.c_uint16), _p(out, C.c_double), _p(st, C.c_double))
    return out, st


def discretize(dt_raw, dt_bias, A_log):
    dt_raw = _d(dt_raw)
    T, H = dt_raw.shape
    db, al = _f32(dt_bias), _f32(A_log)
    dt = np.empty((T, H), dtype=np.float64)
    A = np.empty(H, dtype=np.float64)
    lib().nho_discretize(_p(dt_raw, C.c_double), H, T, H, _p(db, C.c_float), _p(al, C.c_float),
                         _p(dt, C.c_double), _p(A, C.c_double))
    return dt, A


def ssm_recurrence(x, Bm, Cm, dt, A, D, S0, G: int, round_state_f32: bool = False,
                   nthreads: int = 0):
    """x [T][H*P], Bm/Cm [T][G*N], dt [T][H], A [H], D [H] (f32), S0 [H][P][N].

    Returns (y [T][H*P], S [H][P][N]) in fp64."""
    x, Bm, Cm, dt, A = _d(x), _d(Bm), _d(Cm), _d(dt), _d(A)
    Dv = _f32(D)
    S = np.array(S0, dtype=np.float64, copy=True, order="C")
    H, P, N = S.shape
    T = x.shape[0]
    y = np.empty((T, H * P), dtype=np.float64)
    lib().nho_ssm_recurrence(T, H, P, N, G, _p(x, C.c_double), x.shape[1], _p(Bm, C.c_double),
                             Bm.shape[1], _p(Cm, C.c_double), Cm.shape[1], _p(dt, C.c_double),
                             _p(A, C.c_double), _p(Dv, C.c_float), _p(S, C.c_double),
                             _p(y, C.c_double), int(round_state_f32), nthreads)
    return y, S


# ---------------------------------------------------------------- the block

class _Dims(C.Structure):
    _fields_ = [("hidden", C.c_int), ("n_heads", C.c_int), ("head_dim", C.c_int),
                ("d_state", C.c_int), ("n_groups", C.c_int), ("conv_k", C.c_int),
                ("group_size", C.c_int), ("eps", C.c_double)]


class _Weights(C.Structure):
    _fields_ = [("norm_w", C.c_void_p), ("in_q", C.c_void_p), ("in_s", C.c_void_p),
                ("in_b", C.c_void_p), ("conv_w", C.c_void_p), ("conv_b", C.c_void_p),
                ("dt_bias", C.c_void_p), ("A_log", C.c_void_p), ("D", C.c_void_p),
                ("gnorm_w", C.c_void_p), ("out_q", C.c_void_p), ("out_s", C.c_void_p),
                ("out_b", C.c_void_p)]


class _Debug(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("u", "zxbcdt", "xc", "dt", "y", "o", "m")]


@dataclass
class BlockResult:
    out: np.ndarray               # [B][T][hidden] fp64, before output rounding
    conv_state: np.ndarray | None  # [B][K-1][conv_dim]
    ssm_state: np.ndarray         # [B][H][P][N]
    debug: dict


def block(dims, w, x, conv_state=None, ssm_state=None, mode: int = CONTRACT,
          stepwise: bool = False, nthreads: int = 0, debug: bool = False) -> BlockResult:
    """Run one block over x [B][T][hidden] (doubles; widen bf16/f32 inputs first).

    conv_state [B][K-1][conv_dim] or None (zeros, nothing returned);
    ssm_state [B][H][P][N] or None (zeros)."""
    x = _d(x)
    Bn, T, Hd = x.shape
    H, P, N = dims.n_heads, dims.head_dim, dims.d_state
    cd = dims.d_inner + 2 * dims.n_groups * dims.d_state
    keep = [x]
    arrs = dict(norm_w=_u16(w.norm_w), in_q=_u32(w.in_proj.qweight), in_s=_u16(w.in_proj.scales),
                in_b=_u16(w.in_proj.biases), conv_w=_u16(w.conv_w), conv_b=_u16(w.conv_b),
                dt_bias=_f32(w.dt_bias), A_log=_f32(w.A_log), D=_f32(w.D),
                gnorm_w=_u16(w.gnorm_w), out_q=_u32(w.out_proj.qweight),
                out_s=_u16(w.out_proj.scales), out_b=_u16(w.out_proj.biases))
    keep += list(arrs.values())
    cw = _Weights(**{k: v.ctypes.data for k, v in arrs.items()})
    cdims = _Dims(dims.hidden, H, P, N, dims.n_groups, dims.conv_k, dims.group_size, dims.eps)
    cs = None if conv_state is None else np.array(conv_state, dtype=np.float64, copy=True, order="C")
    ss = (np.zeros((Bn, H, P, N)) if ssm_state is None
          else np.array(ssm_state, dtype=np.float64, copy=True, order="C"))
    out = np.empty_like(x)
    dbg = None
    dbg_arrs = {}
    if debug:
        widths = dict(u=Hd, zxbcdt=dims.in_proj_out, xc=cd, dt=H, y=dims.d_inner, o=dims.d_inner,
                      m=Hd)
        dbg_arrs = {k: np.empty((Bn, T, v)) for k, v in widths.items()}
        dbg = _Debug(**{k: v.ctypes.data for k, v in dbg_arrs.items()})
    rc = lib().nho_block(C.byref(cdims), C.byref(cw), Bn, T, _p(x, C.c_double),
                         None if cs is None else _p(cs, C.c_double), _p(ss, C.c_double),
                         _p(out, C.c_double), mode, int(stepwise), nthreads,
                         None if dbg is None else C.byref(dbg))
    if rc != 0:
        raise ValueError("oracle block rejected its arguments")
    return BlockResult(out, cs, ss, dbg_arrs)


def block_stepwise(dims, w, x, conv_state, ssm_state, mode: int = CONTRACT, nthreads: int = 0,
                   debug: bool = False) -> BlockResult:
    """The cached per-position mode: one block call per position, state carried between calls."""
    x = _d(x)
    Bn, T, Hd = x.shape
    cd = dims.d_inner + 2 * dims.n_groups * dims.d_state
    cs = (np.zeros((Bn, dims.conv_k - 1, cd)) if conv_state is None
          else np.array(conv_state, dtype=np.float64))
    ss = ssm_state
    outs, dbgs = [], []
    for t in range(T):
        r = block(dims, w, x[:, t:t + 1], cs, ss, mode=mode, stepwise=True, nthreads=nthreads,
                  debug=debug)
        cs, ss = r.conv_state, r.ssm_state
        outs.append(r.out)
        dbgs.append(r.debug)
    dbg = {k: np.concatenate([d[k] for d in dbgs], axis=1) for k in (dbgs[0] if debug else {})}
    return BlockResult(np.concatenate(outs, axis=1), cs, ss, dbg)


def stack(dims, layer_weights: list, x, mode: int = CONTRACT, stepwise: bool = False,
          conv_states=None, ssm_states=None, nthreads: int = 0):
    """The Mamba2 layers of the hybrid pattern in order; attention and MLP layers are identity.

    The residual stream between blocks is rounded to float32 in CONTRACT mode.
    Returns (per-layer outputs, final conv states, final ssm states)."""
    m_layers = layers_of_kind("M")
    assert len(layer_weights) == len(m_layers)
    h = _d(x)
    outs, css, sss = [], [], []
    for i, w in enumerate(layer_weights):
        cs = None if conv_states is None else conv_states[i]
        ss = None if ssm_states is None else ssm_states[i]
        if stepwise:
            r = block_stepwise(dims, w, h, cs, ss, mode=mode, nthreads=nthreads)
        else:
            r = block(dims, w, h, cs, ss, mode=mode, nthreads=nthreads)
        h = r.out.astype(np.float32).astype(np.float64) if mode == CONTRACT else r.out
        outs.append(h)
        css.append(r.conv_state)
        sss.append(r.ssm_state)
    return outs, css, sss


# ------------------------------------------------- chunked SSD (numpy, fp64)

def ssd_chunked(x, Bm, Cm, dt, A, D, S0, G: int, Q: int):
    """The same scan as ssm_recurrence, computed chunk by chunk (SSD form).

    Per chunk of length L <= Q and head h (group g):
      (i)   cum_t = sum_{s<=t in chunk} dt_s A_h
      (ii)  Gm = C B^T over the chunk (group g)
      (iii) Y_diag[i] = sum_{j<=i} Gm[i,j] exp(cum_i - cum_j) dt_j x_j
      (iv)  S_c = sum_j exp(cum_{L-1} - cum_j) dt_j x_j (outer) B_j
      (v)   S_next = exp(cum_{L-1}) S_in + S_c
      (vi)  Y_off[i] = exp(cum_i) C_i S_in
      (vii) y = Y_diag + Y_off + D x
    Shapes as in ssm_recurrence.  Returns (y, S_final)."""
    x, Bm, Cm, dt, A = _d(x), _d(Bm), _d(Cm), _d(dt), _d(A)
    D = _d(D)
    S = np.array(S0, dtype=np.float64, copy=True)
    H, P, N = S.shape
    T = x.shape[0]
    hpg = H // G
    y = np.zeros((T, H * P))
    for c0 in range(0, T, Q):
        c1 = min(T, c0 + Q)
        for h in range(H):
            g = h // hpg
            xs = x[c0:c1, h * P:(h + 1) * P]          # [L][P]
            Bs = Bm[c0:c1, g * N:(g + 1) * N]          # [L][N]
            Cs = Cm[c0:c1, g * N:(g + 1) * N]
            a = dt[c0:c1, h] * A[h]
            cum = np.cumsum(a)
            Gm = Cs @ Bs.T
            seg = cum[:, None] - cum[None, :]
            mask = np.tril(np.ones((c1 - c0, c1 - c0), dtype=bool))
            Lm = np.where(mask, np.exp(np.where(mask, seg, 0.0)), 0.0)
            Y_diag = (Gm * Lm * dt[c0:c1, h][None, :]) @ xs
            w_end = np.exp(cum[-1] - cum) * dt[c0:c1, h]
            S_c = (xs * w_end[:, None]).T @ Bs
            Y_off = np.exp(cum)[:, None] * (Cs @ S[h].T)
            y[c0:c1, h * P:(h + 1) * P] = Y_diag + Y_off + D[h] * xs
            S[h] = np.exp(cum[-1]) * S[h] + S_c
    return y, S
