"""Python binding of libnhmamba (the Nemotron-H Mamba2 mixer block on MI355X / gfx950).

Argument marshalling only: every step of the block runs in the library's HIP kernels.
Functions carry the names of the C entry points in include/nhmamba.h and take torch
tensors (device memory) or raw integer addresses; PyTorch supplies memory and streams.

The library must be built first (``__graft_entry__.build()`` or
``python hybrid_mamba2_decode_amd/build.py``); importing this package without it raises.
There is no fallback path of any kind.
"""
from __future__ import annotations

import ctypes as C
import os

# PyTorch provides device memory and streams; load it first so that this library binds to
# the same HIP runtime instance (a second runtime would not see torch's allocations).
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnhmamba.so")

NH_OK = 0
NH_ERR_INVALID_ARGUMENT = 1
NH_ERR_UNSUPPORTED_SHAPE = 2
NH_ERR_MISALIGNED = 3
NH_ERR_WORKSPACE_TOO_SMALL = 4
NH_ERR_HIP = 5
NH_BF16 = 0
NH_F32 = 1
NH_MODE_STEP = 0
NH_MODE_SEQ = 1

# Entry points declared in include/nhmamba.h.
EXPORTS = (
    "nh_last_error", "nh_version", "nh_hybrid_pattern", "nh_profile_events",
    "nh_w4_gemv", "nh_w4_gemm_workspace_bytes", "nh_w4_gemm", "nh_rmsnorm", "nh_inproj_conv_step",
    "nh_conv1d_step", "nh_conv1d_seq", "nh_ssm_step", "nh_ssd_scan_workspace_bytes", "nh_ssd_chunk_scan",
    "nh_rmsnorm_gated", "nh_block_workspace_bytes", "nh_mamba_block_step", "nh_mamba_block_step_noalloc", "nh_mamba_block_seq",
    "nh_mamba_stack", "nh_head_workspace_bytes", "nh_head_argmax", "nh_fused_embedding",
    "nh_mlp_workspace_bytes", "nh_mlp_step", "nh_attention_workspace_bytes", "nh_attention_step",
    "nh_attention_decode_workspace_bytes", "nh_attention_decode",
    "nh_lm_workspace_bytes", "nh_lm_step",
)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950); there is no fallback implementation")
lib = C.CDLL(LIB_PATH)


class NhError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"nh status {status}: {message}")
        self.status = status
        self.message = message


class nh_mamba_dims(C.Structure):
    _fields_ = [("hidden", C.c_int), ("n_heads", C.c_int), ("head_dim", C.c_int),
                ("d_state", C.c_int), ("n_groups", C.c_int), ("conv_k", C.c_int),
                ("chunk", C.c_int), ("eps", C.c_float)]


class nh_w4_matrix(C.Structure):
    _fields_ = [("qweight", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p),
                ("n_out", C.c_int), ("k_in", C.c_int), ("group_size", C.c_int)]


class nh_mamba_weights(C.Structure):
    _fields_ = [("norm_w", C.c_void_p), ("in_proj", nh_w4_matrix), ("conv_w", C.c_void_p),
                ("conv_b", C.c_void_p), ("dt_bias", C.c_void_p), ("A_log", C.c_void_p),
                ("D", C.c_void_p), ("gnorm_w", C.c_void_p), ("out_proj", nh_w4_matrix)]


class nh_mamba_state(C.Structure):
    _fields_ = [("conv_state", C.c_void_p), ("ssm_state", C.c_void_p)]


class nh_mlp_weights(C.Structure):
    _fields_ = [("norm_w", C.c_void_p), ("up", nh_w4_matrix), ("down", nh_w4_matrix)]


class nh_attention_weights(C.Structure):
    _fields_ = [("norm_w", C.c_void_p), ("q_proj", nh_w4_matrix), ("k_proj", nh_w4_matrix),
                ("v_proj", nh_w4_matrix), ("o_proj", nh_w4_matrix)]


class nh_kv_cache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("max_len", C.c_int)]


class nh_lm_weights(C.Structure):
    _fields_ = [("embed", nh_w4_matrix), ("mamba", C.POINTER(nh_mamba_weights)),
                ("mlp", C.POINTER(nh_mlp_weights)), ("attn", C.POINTER(nh_attention_weights)),
                ("norm_f", C.c_void_p), ("lm_head", nh_w4_matrix),
                ("function_head", nh_w4_matrix), ("function_weight", C.c_float)]


_vp, _i, _l, _sz = C.c_void_p, C.c_int, C.c_long, C.c_size_t
_sigs = {
    "nh_last_error": (C.c_char_p, []),
    "nh_version": (C.c_char_p, []),
    "nh_hybrid_pattern": (C.c_char_p, []),
    "nh_w4_gemv": (_i, [_vp, _vp, _i, _i, _vp, _i, _vp, _i, _vp]),
    "nh_w4_gemm_workspace_bytes": (_sz, [_i, _i]),
    "nh_w4_gemm": (_i, [_vp, _vp, _i, _vp, _i, _vp, _i, _vp, _sz, _vp]),
    "nh_rmsnorm": (_i, [_vp, _i, _vp, _vp, _i, _i, C.c_float, _vp]),
    "nh_inproj_conv_step": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _vp]),
    "nh_conv1d_step": (_i, [_vp, _l, _vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "nh_conv1d_seq": (_i, [_vp, _l, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "nh_ssm_step": (_i, [_vp, _vp, _vp, _l, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp]),
    "nh_ssd_scan_workspace_bytes": (_sz, [_vp, _i, _i]),
    "nh_ssd_chunk_scan": (_i, [_vp, _vp, _vp, _l, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _sz, _vp]),
    "nh_rmsnorm_gated": (_i, [_vp, _i, _vp, _l, _vp, _vp, _i, _i, _i, C.c_float, _vp]),
    "nh_block_workspace_bytes": (_sz, [_vp, _i, _i, _i]),
    "nh_mamba_block_step": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _i, _i, _vp, _sz, _vp]),
    "nh_mamba_block_step_noalloc": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _i, _i, _vp]),
    "nh_mamba_block_seq": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _i, _i, _vp, _sz, _vp]),
    "nh_mamba_stack": (_i, [_vp, _vp, _vp, _i, _i, _vp, _i, _i, _vp, _i, _vp, _sz, _vp]),
    "nh_profile_events": (_i, [_vp, _i]),
    "nh_head_workspace_bytes": (_sz, [_i]),
    "nh_head_argmax": (_i, [_vp, _vp, _i, _vp, C.c_float, _i, _vp, _vp, _vp, _sz, _vp]),
    "nh_fused_embedding": (_i, [_vp, _vp, _vp, _vp, _i, C.c_float, _i, _vp, _vp]),
    "nh_mlp_workspace_bytes": (_sz, [_i, _i]),
    "nh_mlp_step": (_i, [_vp, _vp, _vp, C.c_float, _vp, _i, _vp, _i, _i, _vp, _sz, _vp]),
    "nh_lm_workspace_bytes": (_sz, [_vp, _i, _i]),
    "nh_attention_workspace_bytes": (_sz, [_i]),
    "nh_attention_step": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _i, _i, C.c_float, _vp, _sz, _vp]),
    "nh_attention_decode_workspace_bytes": (_sz, [_i]),
    "nh_attention_decode": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _sz, _vp]),
    "nh_lm_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


# ------------------------------------------------------------------ marshalling

def _ptr(t):
    """Device address of a torch tensor, an int address, a ctypes struct, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, C.Structure):
        return C.addressof(t)
    if isinstance(t, C.Array):
        return C.addressof(t)
    return t.data_ptr()


def _stream(s):
    if s is not None:
        return s if isinstance(s, int) else s.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(rc: int):
    if rc != NH_OK:
        raise NhError(rc, lib.nh_last_error().decode())


def dims(chunk: int = 128, eps: float = 1e-5, hidden: int = 4480, n_heads: int = 128,
         head_dim: int = 80, d_state: int = 128, n_groups: int = 8, conv_k: int = 4) -> nh_mamba_dims:
    return nh_mamba_dims(hidden, n_heads, head_dim, d_state, n_groups, conv_k, chunk, eps)


def w4_matrix(qweight, scales, biases, n_out: int, k_in: int, group_size: int = 64) -> nh_w4_matrix:
    m = nh_w4_matrix(_ptr(qweight), _ptr(scales), _ptr(biases), n_out, k_in, group_size)
    m._keep = (qweight, scales, biases)
    return m


def mamba_weights(norm_w, in_proj: nh_w4_matrix, conv_w, conv_b, dt_bias, A_log, D, gnorm_w,
                  out_proj: nh_w4_matrix) -> nh_mamba_weights:
    w = nh_mamba_weights(_ptr(norm_w), in_proj, _ptr(conv_w), _ptr(conv_b), _ptr(dt_bias),
                         _ptr(A_log), _ptr(D), _ptr(gnorm_w), out_proj)
    w._keep = (norm_w, in_proj, conv_w, conv_b, dt_bias, A_log, D, gnorm_w, out_proj)
    return w


def mamba_state(conv_state, ssm_state) -> nh_mamba_state:
    s = nh_mamba_state(_ptr(conv_state), _ptr(ssm_state))
    s._keep = (conv_state, ssm_state)
    return s


def version() -> str:
    return lib.nh_version().decode()


def hybrid_pattern() -> str:
    return lib.nh_hybrid_pattern().decode()


# ------------------------------------------------------------------ entry points

def nh_w4_gemv(W, x, x_dtype, batch, residual, res_dtype, y, y_dtype, stream=None):
    _check(lib.nh_w4_gemv(C.byref(W), _ptr(x), x_dtype, batch, _ptr(residual), res_dtype, _ptr(y), y_dtype,
                          _stream(stream)))


def mlp_weights(norm_w, up: nh_w4_matrix, down: nh_w4_matrix) -> nh_mlp_weights:
    w = nh_mlp_weights(_ptr(norm_w), up, down)
    w._keep = (norm_w, up, down)
    return w


def attention_weights(norm_w, q_proj: nh_w4_matrix, k_proj: nh_w4_matrix, v_proj: nh_w4_matrix,
                      o_proj: nh_w4_matrix) -> nh_attention_weights:
    w = nh_attention_weights(_ptr(norm_w), q_proj, k_proj, v_proj, o_proj)
    w._keep = (norm_w, q_proj, k_proj, v_proj, o_proj)
    return w


def kv_cache(k, v, max_len: int) -> nh_kv_cache:
    c = nh_kv_cache(_ptr(k), _ptr(v), max_len)
    c._keep = (k, v)
    return c


def lm_weights(embed: nh_w4_matrix, mamba: list, mlp: list, attn: list, norm_f, lm_head: nh_w4_matrix,
               function_head: nh_w4_matrix, function_weight: float = 2.0) -> nh_lm_weights:
    """mamba: nh_mamba_weights per 'M' layer; mlp: nh_mlp_weights per '-' layer; attn:
    nh_attention_weights per '*' layer (pattern order)."""
    ma = (nh_mamba_weights * len(mamba))(*mamba)
    ml = (nh_mlp_weights * len(mlp))(*mlp)
    at = (nh_attention_weights * len(attn))(*attn)
    w = nh_lm_weights(embed, ma, ml, at, _ptr(norm_f), lm_head, function_head, function_weight)
    w._keep = (embed, mamba, mlp, attn, ma, ml, at, norm_f, lm_head, function_head)
    return w


def nh_lm_workspace_bytes(d, inter, batch) -> int:
    return lib.nh_lm_workspace_bytes(C.byref(d), inter, batch)


def nh_lm_step(d, w, states, caches, positions, text_ids, function_ids, audio, audio_dtype, batch, hidden_out,
               text_out, function_out, ws, ws_bytes, stream=None):
    st = (nh_mamba_state * len(states))(*states)
    kc = (nh_kv_cache * len(caches))(*caches)
    _check(lib.nh_lm_step(C.byref(d), C.byref(w), st, kc, _ptr(positions), _ptr(text_ids), _ptr(function_ids),
                          _ptr(audio), audio_dtype, batch, _ptr(hidden_out), _ptr(text_out), _ptr(function_out),
                          _ptr(ws), ws_bytes, _stream(stream)))


def nh_attention_workspace_bytes(batch) -> int:
    return lib.nh_attention_workspace_bytes(batch)


def nh_attention_step(w, cache, positions, x, x_dtype, out, out_dtype, batch, eps, ws, ws_bytes, stream=None):
    _check(lib.nh_attention_step(C.byref(w), C.byref(cache), _ptr(positions), _ptr(x), x_dtype, _ptr(out),
                                 out_dtype, batch, eps, _ptr(ws), ws_bytes, _stream(stream)))


def nh_mlp_workspace_bytes(inter, batch) -> int:
    return lib.nh_mlp_workspace_bytes(inter, batch)


def nh_mlp_step(norm_w, up, down, eps, x, x_dtype, out, out_dtype, batch, ws, ws_bytes, stream=None):
    _check(lib.nh_mlp_step(_ptr(norm_w), C.byref(up), C.byref(down), eps, _ptr(x), x_dtype, _ptr(out),
                           out_dtype, batch, _ptr(ws), ws_bytes, _stream(stream)))


def nh_fused_embedding(E, text_ids, function_ids, audio, audio_dtype, function_weight, batch, out,
                       stream=None):
    _check(lib.nh_fused_embedding(C.byref(E), _ptr(text_ids), _ptr(function_ids), _ptr(audio), audio_dtype,
                                  function_weight, batch, _ptr(out), _stream(stream)))


def nh_head_workspace_bytes(batch) -> int:
    return lib.nh_head_workspace_bytes(batch)


def nh_head_argmax(W, x, x_dtype, norm_w, eps, batch, logits, ids, ws, ws_bytes, stream=None):
    _check(lib.nh_head_argmax(C.byref(W), _ptr(x), x_dtype, _ptr(norm_w), eps, batch, _ptr(logits),
                              _ptr(ids), _ptr(ws), ws_bytes, _stream(stream)))


def nh_w4_gemm_workspace_bytes(M, k_in) -> int:
    return lib.nh_w4_gemm_workspace_bytes(M, k_in)


def nh_w4_gemm(W, X, M, residual, res_dtype, Y, y_dtype, ws, ws_bytes, stream=None):
    _check(lib.nh_w4_gemm(C.byref(W), _ptr(X), M, _ptr(residual), res_dtype, _ptr(Y), y_dtype,
                          _ptr(ws), ws_bytes, _stream(stream)))


def nh_rmsnorm(x, x_dtype, w, u, rows, d, eps, stream=None):
    _check(lib.nh_rmsnorm(_ptr(x), x_dtype, _ptr(w), _ptr(u), rows, d, eps, _stream(stream)))


def nh_conv1d_step(xbc, ld, conv_state, w, b, out, batch, channels, k=4, stream=None):
    _check(lib.nh_conv1d_step(_ptr(xbc), ld, _ptr(conv_state), _ptr(w), _ptr(b), _ptr(out), batch,
                              channels, k, _stream(stream)))


def nh_conv1d_seq(xbc, ld, T, state_in, state_out, w, b, out, batch, channels, k=4, stream=None):
    _check(lib.nh_conv1d_seq(_ptr(xbc), ld, T, _ptr(state_in), _ptr(state_out), _ptr(w), _ptr(b),
                             _ptr(out), batch, channels, k, _stream(stream)))


def nh_ssm_step(d, xc, dt_raw, ld_dt, dt_bias, A_log, D, ssm_state, y, y_dtype, batch, stream=None):
    _check(lib.nh_ssm_step(C.byref(d), _ptr(xc), _ptr(dt_raw), ld_dt, _ptr(dt_bias), _ptr(A_log),
                           _ptr(D), _ptr(ssm_state), _ptr(y), y_dtype, batch, _stream(stream)))


def nh_ssd_scan_workspace_bytes(d, batch, T) -> int:
    return lib.nh_ssd_scan_workspace_bytes(C.byref(d), batch, T)


def nh_ssd_chunk_scan(d, xc, dt_raw, ld_dt, T, dt_bias, A_log, D, h0, h_final, y, y_dtype, batch,
                      ws, ws_bytes, stream=None):
    _check(lib.nh_ssd_chunk_scan(C.byref(d), _ptr(xc), _ptr(dt_raw), ld_dt, T, _ptr(dt_bias),
                                 _ptr(A_log), _ptr(D), _ptr(h0), _ptr(h_final), _ptr(y), y_dtype,
                                 batch, _ptr(ws), ws_bytes, _stream(stream)))


def nh_rmsnorm_gated(y, y_dtype, z, ld_z, w, out, rows, d, group, eps, stream=None):
    _check(lib.nh_rmsnorm_gated(_ptr(y), y_dtype, _ptr(z), ld_z, _ptr(w), _ptr(out), rows, d, group, eps,
                                _stream(stream)))


def nh_block_workspace_bytes(d, batch, T, mode) -> int:
    return lib.nh_block_workspace_bytes(C.byref(d), batch, T, mode)


def nh_inproj_conv_step(d, w, state, x, x_dtype, z, xc, dt_raw, batch, stream=None):
    _check(lib.nh_inproj_conv_step(C.byref(d), C.byref(w), C.byref(state), _ptr(x), x_dtype, _ptr(z), _ptr(xc),
                                   _ptr(dt_raw), batch, _stream(stream)))


def nh_mamba_block_step(d, w, state, x, x_dtype, out, out_dtype, batch, ws, ws_bytes, stream=None):
    _check(lib.nh_mamba_block_step(C.byref(d), C.byref(w), C.byref(state), _ptr(x), x_dtype,
                                   _ptr(out), out_dtype, batch, _ptr(ws), ws_bytes, _stream(stream)))


def nh_mamba_block_step_noalloc(d, w, state, x, x_dtype, out, out_dtype, batch, stream=None):
    _check(lib.nh_mamba_block_step_noalloc(C.byref(d), C.byref(w), C.byref(state), _ptr(x), x_dtype,
                                           _ptr(out), out_dtype, batch, _stream(stream)))


def nh_mamba_block_seq(d, w, init, final_state, x, x_dtype, T, out, out_dtype, batch, ws, ws_bytes,
                       stream=None):
    _check(lib.nh_mamba_block_seq(C.byref(d), C.byref(w), None if init is None else C.byref(init),
                                  None if final_state is None else C.byref(final_state), _ptr(x),
                                  x_dtype, T, _ptr(out), out_dtype, batch, _ptr(ws), ws_bytes,
                                  _stream(stream)))


def nh_mamba_stack(d, weights, states, n_layers, mode, x, x_dtype, T, outs, batch, ws, ws_bytes,
                   stream=None):
    """weights / states: sequences of nh_mamba_weights / nh_mamba_state (or None for states)."""
    warr = (nh_mamba_weights * n_layers)(*weights)
    sarr = None if states is None else (nh_mamba_state * n_layers)(*states)
    _check(lib.nh_mamba_stack(C.byref(d), warr, sarr, n_layers, mode, _ptr(x), x_dtype, T, _ptr(outs),
                              batch, _ptr(ws), ws_bytes, _stream(stream)))


def nh_profile_events(events):
    """events: None (off) or a sequence of 4 hipEvent_t handles (ints)."""
    if events is None:
        _check(lib.nh_profile_events(None, 0))
    else:
        arr = (C.c_void_p * len(events))(*events)
        _check(lib.nh_profile_events(arr, len(events)))


def nh_attention_decode_workspace_bytes(batch) -> int:
    return lib.nh_attention_decode_workspace_bytes(batch)


def nh_attention_decode(q, cache, positions, o, batch, ws, ws_bytes, stream=None):
    _check(lib.nh_attention_decode(_ptr(q), C.byref(cache), _ptr(positions), _ptr(o), batch, _ptr(ws), ws_bytes,
                                   _stream(stream)))
