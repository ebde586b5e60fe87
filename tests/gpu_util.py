"""Helpers shared by the GPU tests and the benchmark: device upload of the synthetic
inputs and comparison metrics.  Marshalling and measurement only -- no block arithmetic."""
from __future__ import annotations

import numpy as np
import torch

import hybrid_mamba2_decode_amd as nh

DEV = "cuda:0"


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    else:
        t = torch.from_numpy(a)
    return t.to(DEV)


def from_dev_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def empty_u16(*shape) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.int16, device=DEV)


def empty_f32(*shape) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.float32, device=DEV)


def workspace(nbytes: int) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def w4_dev(W):
    q, s, b = to_dev(W.qweight), to_dev(W.scales), to_dev(W.biases)
    return nh.w4_matrix(q, s, b, W.n_out, W.k_in, W.group_size)


def layer_dev(lw):
    """Upload a synth.LayerWeights and build the nh_mamba_weights struct."""
    return nh.mamba_weights(to_dev(lw.norm_w), w4_dev(lw.in_proj), to_dev(lw.conv_w), to_dev(lw.conv_b),
                            to_dev(lw.dt_bias), to_dev(lw.A_log), to_dev(lw.D), to_dev(lw.gnorm_w),
                            w4_dev(lw.out_proj))


def state_dev(conv_state: np.ndarray, ssm_state: np.ndarray):
    cs, ss = to_dev(conv_state), to_dev(np.ascontiguousarray(ssm_state, dtype=np.float32))
    return nh.mamba_state(cs, ss), cs, ss


def rel_l2(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(a, ref) -> float:
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(ref, dtype=np.float64))))


def bf16_ulp_flips(gpu_bits: np.ndarray, ref: np.ndarray) -> int:
    """How many bf16 outputs differ from the oracle's value rounded to bf16."""
    import oracle
    return int(np.count_nonzero(np.asarray(gpu_bits, dtype=np.uint16) != oracle.to_bf16(ref)))


def row_errors(got, ref, row: int = 80):
    """Per-row view of a scan or block output, rows of `row` values (one (position, head) of
    the scan's y, 80 channels).  Returns (worst row error relative to the row's own norm, with
    the norm floored at a tenth of the RMS row norm so that near-zero rows do not divide by
    ~0; max-abs error; max |ref|).  A wrong row gives a relative error near 1 here, whatever
    the size of the tensor, where a whole-tensor rel-L2 would dilute it."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, row)
    r = np.asarray(ref, dtype=np.float64).reshape(-1, row)
    en = np.linalg.norm(g - r, axis=1)
    rn = np.linalg.norm(r, axis=1)
    floor = 0.1 * float(np.sqrt(np.mean(rn * rn)))
    worst = float(np.max(en / np.maximum(rn, max(floor, 1e-300))))
    return worst, float(np.max(np.abs(g - r))), float(np.max(np.abs(r)))
