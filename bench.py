#!/usr/bin/env python3
"""Benchmark of libnhmamba (the Nemotron-H Mamba2 mixer block) on one MI355X.

Headline (the JSON line's `value`): the cached per-position block step at batch 1 with a
pre-filled state, in microseconds per layer-step, against the HBM roofline.  The
timed loop rotates over `--copies` independent weight + state sets (27 x 93.7 MB by default,
the stack's layers, ten times the 256 MB last-level cache; with fewer copies the cache keeps
part of the rotation and the figure flatters), so every step streams its weights from HBM; a
single-copy (cache-resident) figure is reported separately and labelled as such.

Also measured in the same run, each in its own object of the JSON line:
  * the chunked SSD scan at batch 2, T = 3750, chunk 256 (27 layers' parameters), in
    position-layers per second against the matrix-core roofline (and the HBM one);
  * the 27-layer stack stepwise over T = 413 at batch 1, and the 27-layer full-history
    stack at batch 2, T = 3750, chunk 256;
  * the block step with 4 sessions sharing one weight stream;
  * one MLP layer step and one attention layer step (the hybrid stack's other layer kinds),
    over the 25 MLP and 4 attention layers' weights, and one whole language-model position
    (input row, all 56 layers, both heads);
  * the final norm + both output heads (W4 131072 x 4480 each) + greedy ids at batch 1,
    and the fused input row (two W4 embedding rows + the audio frame);
  * the CPU oracle on the host cores (a bounded sample of the batch-1 block step), as a
    reported baseline.

The roofline's kernel (the fused pre-norm / in_proj / conv step, 61% of the step's bytes) is
timed alone: back-to-back launches of nh_inproj_conv_step over the same rotating copies, with
two HIP events on the launch stream around the loop.  The per-kernel split of the block step
comes from the library's nh_profile_events hook (an event recorded before each kernel, and
one stamped at its end), so each of those figures also holds that kernel's dispatch.
All inputs are seeded synthetic data (synth package); nothing is read from disk except the
committed HBM-traffic counter summary under profiles/.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_F16_PEAK = 2.5e15     # flop/s, dense bf16/fp16 matrix cores
H, P, N, G, HID = 128, 80, 128, 8, 4480
DI, CD, NIN = 10240, 12288, 22656
VOCAB = 131072             # vocab_size: rows of each output head


# ------------------------------------------------------- algorithmic work

def pattern_layers(kind: str):
    """Layer indices of one kind in the hybrid pattern, read from the library."""
    import hybrid_mamba2_decode_amd as nh
    return [i for i, c in enumerate(nh.hybrid_pattern()) if c == kind]


def w4_bytes(n, k):
    return n * k // 2 + 2 * 2 * n * (k // 64)   # packed nibbles + bf16 scales + bf16 biases


def step_kernel_bytes(B=1, out_bytes=4):
    """Algorithmic HBM bytes of the three kernels of one block step (batch B)."""
    k1 = (w4_bytes(NIN, HID) + 2 * HID            # weights, norm weight
          + B * 2 * HID                           # x (bf16)
          + 12288 * 4 * 2 + 12288 * 2             # conv weight, bias
          + B * 2 * 3 * CD * 2                    # conv state read + write
          + B * 2 * (DI + CD + H))                # z, xc, dt_raw written
    k2 = (B * H * P * N * 4 * 2                   # fp32 state read + write
          + B * 2 * (2 * 1024 + DI)               # B, C, x (bf16)
          + B * 2 * H + 4 * 3 * H                 # dt_raw, dt_bias, A_log, D
          + B * 2 * DI * 3 + 2 * DI)              # y written, z read, o written, gated-norm weight
    k3 = (w4_bytes(HID, DI) + B * 2 * DI          # weights, o
          + B * 2 * HID + B * out_bytes * HID)    # residual x, output
    return k1, k2, k3


def scan_bytes_per_position():
    return 2 * CD + 2 * H + 2 * DI                # xc + dt_raw read, y written (bf16)


def scan_flops_per_position(Q):
    """Causal-count flops per position of the chunked scan (all heads), chunk Q."""
    hpg = H // G
    per_head = ((Q + 1) / 2 * P * 2            # Y_diag = (G o L) X
                + P * N * 2                    # chunk state
                + N * P * 2                    # state -> output
                + (Q + 1) / 2 * N * 2 / hpg)   # C B^T, once per group
    return per_head * H


# ------------------------------------------------------------- HIP events

class Hip:
    def __init__(self):
        # bind to the HIP runtime already mapped by torch (one runtime per process)
        path = "libamdhip64.so"
        for line in open("/proc/self/maps"):
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
        self.lib = C.CDLL(path)
        self.lib.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.lib.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [C.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.lib.hipEventDestroy.argtypes = [C.c_void_p]

    def event(self):
        e = C.c_void_p()
        assert self.lib.hipEventCreate(C.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, stream) == 0

    def ms(self, a, b):
        self.lib.hipEventSynchronize(b)
        f = C.c_float()
        assert self.lib.hipEventElapsedTime(C.byref(f), a, b) == 0
        return f.value

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


# ------------------------------------------------------ counter summaries

def _source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "hybrid_mamba2_decode_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str, *sources: str):
    """HBM bytes per dispatch from the committed PMC summary, or None when absent or when
    the kernel's source changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    key = kernel.replace(" ", "")
    for line in open(path):
        f = line.split()
        if len(f) >= 4 and f[0] == key:
            sha, nbytes = f[1], float(f[2])
            return nbytes if sha == _source_sha(*sources) else None
    return None


def _sum_or_none(*v):
    return None if any(x is None for x in v) else float(sum(v))


def counters_from_profile(kernel: str, *sources: str):
    """MFMA busy fraction, matrix-core TFLOP/s and LDS bank-conflict share of one kernel from the
    committed counter summary, or None when absent or when the kernel's source changed after
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", "scan_gemm_counters.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        f = line.split()
        if len(f) >= 5 and f[0] == kernel:
            if f[1] != _source_sha(*sources):
                return None
            return {"file": "profiles/scan_gemm_counters.md", "mfma_busy": float(f[2]),
                    "matrix_core_tflops": float(f[3]), "lds_bank_conflict_share": float(f[4])}
    return None


# ------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000, help="timed batch-1 block steps")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=27,
                    help="rotating weight+state sets (27: the stack's layers, 2.4 GB)")
    ap.add_argument("--skip-step", action="store_true",
                    help="skip the block-step legs (batch 1 and 4); the line then has no value (profiling runs)")
    ap.add_argument("--skip-seq", action="store_true", help="skip the batch-2 T=3750 scan and stack")
    ap.add_argument("--skip-stack", action="store_true", help="skip the 27-layer stacks")
    ap.add_argument("--skip-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--skip-heads", action="store_true",
                    help="skip the legs outside the block: MLP layer, output heads, input row")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); the block "
              "has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import hybrid_mamba2_decode_amd as nh
    from tests import gpu_util as gu

    assert torch.cuda.is_available(), "no GPU visible"
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)  # noqa: E731

    n_layers = 27
    need_layers = n_layers if not (args.skip_stack and args.skip_seq) else args.copies
    t0 = time.time()
    host_layers = [synth.layer_weights(l) for l in range(max(need_layers, args.copies))]
    dev_layers = [gu.layer_dev(lw) for lw in host_layers]
    log(f"weights for {len(dev_layers)} layers ready in {time.time() - t0:.1f} s")

    d128 = nh.dims(chunk=128)
    out = {"metric": "Mamba2 block step us/layer (% HBM peak); SSD scan positions/s (% MFMA peak)"}

    e0, e1 = hip.event(), hip.event()
    B = 1
    cs0, ss0 = synth.prefilled_state(1, B)           # the pre-filled state (also the CPU baseline's)
    ws_step = gu.workspace(nh.nh_block_workspace_bytes(d128, B, 1, nh.NH_MODE_STEP))
    total_bytes = sum(step_kernel_bytes(B))
    if args.skip_step:
        out["value"] = None
    else:
        # ------------------------------------- block step, batch 1, pre-filled state
        x1 = gu.to_dev(synth.block_input(1, B, 1)[:, 0])
        states = [gu.state_dev(cs0, ss0) for _ in range(args.copies)]
        o1 = gu.empty_f32(B, HID)

        def step(i):
            nh.nh_mamba_block_step(d128, dev_layers[i], states[i][0], x1, nh.NH_BF16, o1, nh.NH_F32, B,
                                   ws_step, ws_step.numel(), stream)

        for i in range(args.warmup):
            step(i % args.copies)
        torch.cuda.synchronize()
        hip.record(e0, stream)
        t_wall = time.perf_counter()
        for i in range(args.steps):
            step(i % args.copies)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t_wall) * 1e3
        ms_total = hip.ms(e0, e1)
        us_layer = ms_total * 1e3 / args.steps
        log(f"block step: {us_layer:.2f} us/layer ({args.copies} rotating copies), host wall {wall_ms:.1f} ms")

        # per-kernel durations of the block step (events between its three kernels)
        nprof = min(args.steps, 400)
        evs = [[hip.event() for _ in range(6)] for _ in range(nprof)]
        for i in range(nprof):
            nh.nh_profile_events(evs[i])
            step(i % args.copies)
        nh.nh_profile_events(None)
        torch.cuda.synchronize()
        kt = np.array([[hip.ms(e[2 * j], e[2 * j + 1]) for j in range(3)] for e in evs]) * 1e3  # us
        k_avg = kt.mean(axis=0)
        k_med = np.median(kt, axis=0)
        for e in evs:
            for x in e:
                hip.destroy(x)
        kb = step_kernel_bytes(B)
        names = ["k_inproj_step<1, 0>", "k_ssm_step<true, 1>", "k_outproj_step"]  # batch 1, bf16 input
        kernels = [{"kernel": names[j], "avg_us": round(float(k_avg[j]), 3), "median_us": round(float(k_med[j]), 3),
                    "algorithmic_bytes": int(kb[j]), "GBps": round(kb[j] / (k_avg[j] * 1e-6) / 1e9, 1),
                    "hbm_frac": round(kb[j] / (k_avg[j] * 1e-6) / HBM_PEAK, 4)} for j in range(3)]
        log("kernels:", kernels)

        # the dominant kernel alone (fused pre-norm / in_proj / conv step): back-to-back launches
        # over the same rotating weight + state copies, two events around the loop
        zb, xcb, dtb = gu.empty_u16(B, DI), gu.empty_u16(B, CD), gu.empty_u16(B, H)

        def inproj(i):
            nh.nh_inproj_conv_step(d128, dev_layers[i], states[i][0], x1, nh.NH_BF16, zb, xcb, dtb, B, stream)

        for i in range(args.warmup):
            inproj(i % args.copies)
        hip.record(e0, stream)
        for i in range(args.steps):
            inproj(i % args.copies)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        dom_us = hip.ms(e0, e1) * 1e3 / args.steps
        log(f"k_inproj_step alone: {dom_us:.2f} us per launch")

        # cache-resident (single copy) figure, labelled
        for i in range(args.warmup):
            step(0)
        hip.record(e0, stream)
        for i in range(args.steps):
            step(0)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        us_hot = hip.ms(e0, e1) * 1e3 / args.steps

        total_bytes = sum(kb)
        out.update({
            "value": round(us_layer, 3), "unit": "us/layer", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(us_layer / 1e3, 6), "higher_is_better": False,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded; pages' shapes and distributions)",
            "config": {"workload": "one Mamba2 block (hidden 4480, 128 heads x 80, state 128), batch 1, one "
                                   "cached step with a pre-filled state, timed over rotating weight/state copies",
                       "batch": B, "hidden": HID, "heads": H, "head_dim": P, "d_state": N, "groups": G,
                       "weights": "W4 group-64 affine (in_proj 22656x4480, out_proj 4480x10240)",
                       "rotating_copies": args.copies},
            "hbm_frac": round(total_bytes / (us_layer * 1e-6) / HBM_PEAK, 4),
            "step_algorithmic_bytes": int(total_bytes),
            "step_us_cache_resident": round(us_hot, 3),
            "kernels": kernels,
        })
        dom = 0
        out["roofline"] = {
            "kernel": names[dom], "bound": "hbm",
            "achieved": round(kb[dom] / (dom_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": round(kb[dom] / (dom_us * 1e-6) / HBM_PEAK, 4),
            "traffic": traffic_from_profile(names[dom], "gemv.hip", "nh_device.hpp"),
            "bytes_per_launch": int(kb[dom]), "avg_launch_us": round(dom_us, 3),
            "timing": f"{args.steps} back-to-back launches over {args.copies} rotating weight/state copies, "
                      "two HIP events on the launch stream",
        }

        # --------------- batched step: 4 sessions share one weight stream (27 rotating copies)
        B4s = 4
        x4s = gu.to_dev(synth.block_input(1, B4s, 1)[:, 0])
        cs4, ss4 = synth.prefilled_state(1, B4s)
        st4 = [gu.state_dev(cs4, ss4) for _ in range(args.copies)]
        ws4s = gu.workspace(nh.nh_block_workspace_bytes(d128, B4s, 1, nh.NH_MODE_STEP))
        o4s = gu.empty_f32(B4s, HID)

        def step4(i):
            nh.nh_mamba_block_step(d128, dev_layers[i], st4[i][0], x4s, nh.NH_BF16, o4s, nh.NH_F32, B4s, ws4s,
                                   ws4s.numel(), stream)

        for i in range(args.warmup):
            step4(i % args.copies)
        nb4 = max(args.steps // 4, 50)
        hip.record(e0, stream)
        for i in range(nb4):
            step4(i % args.copies)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        us4 = hip.ms(e0, e1) * 1e3 / nb4
        b4 = sum(step_kernel_bytes(B4s))
        out["step_batch4"] = {
            "workload": f"one Mamba2 block, {B4s} independent sessions per step (pre-filled states), "
                        f"{args.copies} rotating weight/state copies",
            "us_per_layer_step": round(us4, 3), "us_per_session_layer": round(us4 / B4s, 3),
            "algorithmic_bytes": int(b4), "hbm_frac": round(b4 / (us4 * 1e-6) / HBM_PEAK, 4),
        }
        log("batch-4 step:", out["step_batch4"])
        del st4, ws4s

    # ----------------------- MLP layer step, batch 1, over the model's 25 MLP layers' weights
    if not args.skip_heads:
        t0 = time.time()
        mlps = []
        for l in pattern_layers("-"):
            mw = synth.mlp_weights(l)
            mlps.append((gu.to_dev(mw.norm_w), gu.w4_dev(mw.up), gu.w4_dev(mw.down)))
            del mw
        log(f"{len(mlps)} MLP layers ready in {time.time() - t0:.1f} s")
        wsm_n = nh.nh_mlp_workspace_bytes(synth.MLP_INTER, 1)
        wsm = gu.workspace(wsm_n)
        xm = gu.to_dev(np.random.default_rng(78).normal(0, 1, (1, HID)).astype(np.float32))
        om = gu.empty_f32(1, HID)

        def mlp_step(i):
            nw_, up_, dn_ = mlps[i % len(mlps)]
            nh.nh_mlp_step(nw_, up_, dn_, 1e-5, xm, nh.NH_F32, om, nh.NH_F32, 1, wsm, wsm_n, stream)

        for i in range(100):
            mlp_step(i)
        nm = 500
        hip.record(e0, stream)
        for i in range(nm):
            mlp_step(i)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        us_m = hip.ms(e0, e1) * 1e3 / nm
        mb = w4_bytes(synth.MLP_INTER, HID) + w4_bytes(HID, synth.MLP_INTER) + 2 * HID + 4 * HID * 2 + 2 * synth.MLP_INTER * 2
        out["mlp_step"] = {
            "workload": f"one MLP layer (pre-norm, W4 up 4480->15680, squared ReLU, W4 down 15680->4480, residual), "
                        f"batch 1, rotating over the {len(mlps)} MLP layers' weights",
            "us_per_layer_step": round(us_m, 3), "algorithmic_bytes": int(mb),
            "hbm_frac": round(mb / (us_m * 1e-6) / HBM_PEAK, 4),
        }
        log("mlp step:", out["mlp_step"])

        # one attention layer at batch 1 over a cache of T_att earlier positions (the 33 s
        # timeline, and the 5 min one), rotating over the 4 attention layers' weights and caches
        t0 = time.time()
        atts = []
        for l in pattern_layers("*"):
            aw = synth.attention_weights(l)
            atts.append(nh.attention_weights(gu.to_dev(aw.norm_w), gu.w4_dev(aw.q_proj), gu.w4_dev(aw.k_proj),
                                             gu.w4_dev(aw.v_proj), gu.w4_dev(aw.o_proj)))
            del aw
        log(f"{len(atts)} attention layers ready in {time.time() - t0:.1f} s")
        att_w_bytes = w4_bytes(5120, HID) + 2 * w4_bytes(1024, HID) + w4_bytes(HID, 5120) + 2 * HID
        wsa_n = nh.nh_attention_workspace_bytes(1)
        wsa = gu.workspace(wsa_n)
        xa = gu.to_dev(np.random.default_rng(79).normal(0, 1, (1, HID)).astype(np.float32))
        oa = gu.empty_f32(1, HID)
        att_out = {}
        for T_att in (413, 3750):
            caches = []
            for a in range(len(atts)):
                kk, vv = synth.kv_cache(40 + a, 1, T_att + 1)
                caches.append(nh.kv_cache(gu.to_dev(kk), gu.to_dev(vv), T_att + 1))
            pos_a = torch.tensor([T_att], dtype=torch.int32, device="cuda")

            def att_step(i):
                j = i % len(atts)
                nh.nh_attention_step(atts[j], caches[j], pos_a, xa, nh.NH_F32, oa, nh.NH_F32, 1, 1e-5, wsa, wsa_n,
                                     stream)

            for i in range(50):
                att_step(i)
            na = 500
            hip.record(e0, stream)
            for i in range(na):
                att_step(i)
            hip.record(e1, stream)
            torch.cuda.synchronize()
            us_a = hip.ms(e0, e1) * 1e3 / na
            ab = (att_w_bytes + 2 * (T_att + 1) * 8 * 128 * 2     # weights; k and v cache rows read
                  + 2 * 8 * 128 * 2 + 4 * HID * 2)               # new k, v rows; x read, out written
            att_out[f"cache_{T_att}"] = {
                "us_per_layer_step": round(us_a, 3), "algorithmic_bytes": int(ab),
                "hbm_frac": round(ab / (us_a * 1e-6) / HBM_PEAK, 4),
            }
            del caches
        out["attention_step"] = {
            "workload": "one attention layer (pre-norm, W4 q/k/v 4480->5120/1024/1024, k/v appended to the cache, "
                        "40-head grouped-query attention over the 8 key/value heads of 128, W4 o_proj 5120->4480, "
                        "residual), batch 1, over a cache of 413 and of 3750 earlier positions, rotating over the 4 "
                        "attention layers' weights and caches",
            **att_out,
        }
        log("attention step:", out["attention_step"])

        # one language-model position: input row, all 56 layers in pattern order (27 Mamba2,
        # 25 MLP, 4 attention over caches of 413 earlier positions), norm_f, both heads and ids
        hw = synth.head_weights(seed=9)
        lmw = nh.lm_weights(gu.w4_dev(synth.embed_tokens(seed=9)), dev_layers[:n_layers],
                            [nh.mlp_weights(*m) for m in mlps], atts, gu.to_dev(hw.norm_f), gu.w4_dev(hw.lm_head),
                            gu.w4_dev(hw.function_head), 2.0)
        del hw
        st_lm = [gu.state_dev(np.zeros((1, 3, CD), np.uint16), np.zeros((1, H, P, N), np.float32))[0]
                 for _ in range(n_layers)]
        T_lm = 413
        kv_lm = []
        for a in range(len(atts)):
            kk, vv = synth.kv_cache(50 + a, 1, T_lm + 1)
            kv_lm.append(nh.kv_cache(gu.to_dev(kk), gu.to_dev(vv), T_lm + 1))
        pos_lm = torch.tensor([T_lm], dtype=torch.int32, device="cuda")
        wsl_n = nh.nh_lm_workspace_bytes(d128, synth.MLP_INTER, 1)
        wsl = gu.workspace(wsl_n)
        ti, fi, au = synth.embed_inputs(200, 1)
        ti, fi, au = (torch.tensor(ti, device="cuda"), torch.tensor(fi, device="cuda"), gu.to_dev(au))
        ot, of = (torch.empty(1, dtype=torch.int32, device="cuda") for _ in range(2))

        def lm_pos():
            nh.nh_lm_step(d128, lmw, st_lm, kv_lm, pos_lm, ti, fi, au, nh.NH_F32, 1, None, ot, of, wsl, wsl_n,
                          stream)

        for _ in range(5):
            lm_pos()
        npos = 50
        hip.record(e0, stream)
        for _ in range(npos):
            lm_pos()
        hip.record(e1, stream)
        torch.cuda.synchronize()
        us_lm = hip.ms(e0, e1) * 1e3 / npos
        lm_bytes = (n_layers * sum(step_kernel_bytes(1)) + len(mlps) * mb + 2 * (w4_bytes(VOCAB, HID) + 6 * HID)
                    + len(atts) * att_out["cache_413"]["algorithmic_bytes"])
        out["lm_step"] = {
            "workload": "one language-model position at batch 1: input row, all 56 layers in pattern order "
                        "(27 Mamba2 blocks, 25 MLP layers, 4 attention layers over caches of 413 earlier "
                        "positions), norm_f, lm_head + function_head (W4 131072x4480) and greedy ids",
            "ms_per_position": round(us_lm / 1e3, 4), "algorithmic_bytes": int(lm_bytes),
            "hbm_frac": round(lm_bytes / (us_lm * 1e-6) / HBM_PEAK, 4),
        }
        log("lm step:", out["lm_step"])
        del mlps, lmw, st_lm, kv_lm, atts

    # ------------------------------- 27-layer stack, batch 1, stepwise over T=413
    if not args.skip_stack:
        T3 = 413
        x3 = gu.to_dev(synth.block_input(3, 1, T3))
        st3 = [gu.state_dev(np.zeros((1, 3, CD), np.uint16), np.zeros((1, H, P, N), np.float32))
               for _ in range(n_layers)]
        outs3 = gu.empty_f32(n_layers, 1, HID)
        s3 = [s[0] for s in st3]
        xs = [x3[:, t].contiguous() for t in range(T3)]
        torch.cuda.synchronize()
        hip.record(e0, stream)
        for t in range(T3):
            nh.nh_mamba_stack(d128, dev_layers[:n_layers], s3, n_layers, nh.NH_MODE_STEP, xs[t], nh.NH_BF16, 1,
                              outs3, 1, ws_step, ws_step.numel(), stream)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        ms3 = hip.ms(e0, e1)
        out["stack_step"] = {
            "workload": "27 Mamba2 blocks, batch 1, stepwise over T=413 carrying conv+SSM state",
            "total_ms": round(ms3, 3), "us_per_layer_step": round(ms3 * 1e3 / (T3 * n_layers), 3),
            "hbm_frac": round(total_bytes / (ms3 * 1e-3 / (T3 * n_layers)) / HBM_PEAK, 4),
        }
        log("stack steps:", out["stack_step"])
        del st3, outs3

    # ----------- final norm + lm_head + function_head + greedy ids, batch 1, vocab 131072
    if not args.skip_heads:
        heads = []
        nsets = 4
        for seed in range(nsets):   # four rotating sets of both heads: 2.6 GB, ten times the last-level cache
            hw = synth.head_weights(seed=seed)
            heads.append((gu.to_dev(hw.norm_f), gu.w4_dev(hw.lm_head), gu.w4_dev(hw.function_head)))
            del hw
        xh1 = gu.to_dev(np.random.default_rng(77).normal(0, 1, (1, HID)).astype(np.float32))
        hws_n = nh.nh_head_workspace_bytes(1)
        hws = gu.workspace(hws_n)
        ids = [torch.empty(1, dtype=torch.int32, device="cuda") for _ in range(2)]

        def head_pair(i):
            nf, lm, fn = heads[i % nsets]
            nh.nh_head_argmax(lm, xh1, nh.NH_F32, nf, 1e-5, 1, None, ids[0], hws, hws_n, stream)
            nh.nh_head_argmax(fn, xh1, nh.NH_F32, nf, 1e-5, 1, None, ids[1], hws, hws_n, stream)

        for i in range(300):   # also lets the clocks settle after the host-side weight generation
            head_pair(i)
        reps = 100
        hip.record(e0, stream)
        for i in range(reps):
            head_pair(i)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        pair_us = hip.ms(e0, e1) * 1e3 / reps
        head_bytes = w4_bytes(VOCAB, HID) + HID * 4 + HID * 2
        out["heads"] = {
            "workload": "final norm + lm_head + function_head (W4 131072x4480 each) + greedy ids, batch 1, "
                        f"{nsets} rotating sets",
            "us_per_position": round(pair_us, 2), "us_per_head": round(pair_us / 2, 2),
            "algorithmic_bytes_per_head": int(head_bytes),
            "hbm_frac": round(2 * head_bytes / (pair_us * 1e-6) / HBM_PEAK, 4),
            "timing": f"{reps} back-to-back pairs of calls (head kernel + id kernel each), two HIP events",
        }
        log("heads:", out["heads"])
        del heads

        # the fused input row at batch 1: two random rows of the W4 embedding table + audio
        E = gu.w4_dev(synth.embed_tokens())
        nemb = 1000
        ids_t = [torch.tensor(synth.embed_inputs(100 + i, 1)[0], device="cuda") for i in range(16)]
        ids_f = [torch.tensor(synth.embed_inputs(100 + i, 1)[1], device="cuda") for i in range(16)]
        aud = gu.to_dev(synth.embed_inputs(99, 1)[2])
        emb = gu.empty_f32(1, HID)

        def embed(i):
            nh.nh_fused_embedding(E, ids_t[i % 16], ids_f[i % 16], aud, nh.NH_F32, 2.0, 1, emb, stream)

        for i in range(100):
            embed(i)
        hip.record(e0, stream)
        for i in range(nemb):
            embed(i)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        out["embedding"] = {
            "workload": "fused input row E[text] + audio + 2 E[function] (W4 table 131072x4480), batch 1",
            "us_per_position": round(hip.ms(e0, e1) * 1e3 / nemb, 3),
            "bound": "latency (two 2.5 KB table rows, 36 KB in all)",
            "timing": f"{nemb} back-to-back calls over 16 id pairs, two HIP events",
        }
        log("embedding:", out["embedding"])
        del E

    # ------------------------- scan and 27-layer stack, batch 2, T=3750, chunk 256
    if not args.skip_seq:
        B4, T4, Q4 = 2, 3750, 256
        d256 = nh.dims(chunk=Q4)
        rng = np.random.default_rng(4004)
        sets = []
        for _ in range(3):   # rotating inputs: 3 x 184 MB, beyond the last-level cache
            xc = synth.f32_to_bf16(rng.normal(0, 0.6, (B4, T4, CD)).astype(np.float32))
            dtr = synth.f32_to_bf16(rng.normal(0, 1.25, (B4, T4, H)).astype(np.float32))
            sets.append((gu.to_dev(xc), gu.to_dev(dtr)))
        y4 = gu.empty_u16(B4, T4, DI)
        hT = gu.empty_f32(B4, H, P, N)
        sws_n = nh.nh_ssd_scan_workspace_bytes(d256, B4, T4)
        sws = gu.workspace(sws_n)

        def scan(l):
            xcd, dtd = sets[l % 3]
            lw = dev_layers[l % len(dev_layers)]
            nh.nh_ssd_chunk_scan(d256, xcd, dtd, H, T4, lw.dt_bias, lw.A_log, lw.D, None, hT, y4, nh.NH_BF16,
                                 B4, sws, sws_n, stream)

        for l in range(3):
            scan(l)
        sev = [hip.event() for _ in range(n_layers + 1)]
        hip.record(sev[0], stream)
        for l in range(n_layers):
            scan(l)
            hip.record(sev[l + 1], stream)
        torch.cuda.synchronize()
        per = np.array([hip.ms(sev[l], sev[l + 1]) for l in range(n_layers)])
        for e in sev:
            hip.destroy(e)
        pos = B4 * T4
        sec = per.sum() * 1e-3
        pps = pos * n_layers / sec
        fl = scan_flops_per_position(Q4)
        by = scan_bytes_per_position()
        out["scan"] = {
            "workload": "chunked SSD scan (pre-pass + scan), batch 2, T=3750, chunk 256, 27 layers' "
                        "parameters, 3 rotating input sets",
            "metric": "SSD scan positions/s", "value": round(pps, 1), "unit": "position-layers/s",
            "avg_launch_us": round(float(per.mean() * 1e3), 2),
            "mfma_frac": round(pps * fl / MFMA_F16_PEAK, 4),
            "hbm_frac": round(pps * by / HBM_PEAK, 4),
            "roofline": {"kernel": "k_ssd_scanx + k_ssd_cb", "bound": "mfma",
                         "achieved": round(pps * fl / 1e12, 1), "peak": MFMA_F16_PEAK / 1e12, "unit": "TFLOP/s",
                         "frac": round(pps * fl / MFMA_F16_PEAK, 4),
                         # HBM bytes of one scan call: the scan kernel and its pre-pass
                         "traffic": _sum_or_none(traffic_from_profile("k_ssd_scanx", "scan.hip", "nh_device.hpp"),
                                                 traffic_from_profile("k_ssd_cb", "scan.hip", "nh_device.hpp")),
                         "counters": counters_from_profile("k_ssd_scanx", "scan.hip", "nh_device.hpp"),
                         "flops_per_position": round(fl), "bytes_per_position": by,
                         "achieved_GBps": round(pps * by / 1e9, 1), "hbm_peak_GBps": HBM_PEAK / 1e9},
        }
        log("scan:", out["scan"])
        del sets

        # ------- the W4 GEMM alone: in_proj and out_proj of the full-history block at M = 7500
        # rows (batch 2 x T 3750), rotating over the 27 layers' weights
        M = pos
        Xi = gu.to_dev(synth.f32_to_bf16(rng.normal(0, 1, (M, HID)).astype(np.float32)))
        Xo = gu.to_dev(synth.f32_to_bf16(rng.normal(0, 1, (M, DI)).astype(np.float32)))
        Yi, Yo = gu.empty_u16(M, NIN), gu.empty_u16(M, HID)
        gws_n = max(nh.nh_w4_gemm_workspace_bytes(M, HID), nh.nh_w4_gemm_workspace_bytes(M, DI))
        gws = gu.workspace(gws_n)
        gemm_out = {}
        for name, X, Y, n_out, k_in in (("in_proj", Xi, Yi, NIN, HID), ("out_proj", Xo, Yo, HID, DI)):
            def gemm(l):
                W = getattr(dev_layers[l % len(dev_layers)], name)
                nh.nh_w4_gemm(W, X, M, None, 0, Y, nh.NH_BF16, gws, gws_n, stream)

            for l in range(3):
                gemm(l)
            hip.record(e0, stream)
            for l in range(n_layers):
                gemm(l)
            hip.record(e1, stream)
            torch.cuda.synchronize()
            ms_g = hip.ms(e0, e1) / n_layers
            fl_g = 2.0 * M * n_out * k_in
            gemm_out[name] = {"ms": round(ms_g, 3), "tflops": round(fl_g / (ms_g * 1e-3) / 1e12, 1),
                              "mfma_frac": round(fl_g / (ms_g * 1e-3) / MFMA_F16_PEAK, 4)}
        out["gemm"] = {
            "workload": "W4 GEMM Y = X W^T of the full-history block, M = 7500 rows (batch 2 x T 3750): "
                        "in_proj 4480->22656 and out_proj 10240->4480, bf16 output, 27 layers' weights",
            **gemm_out,
            "counters": counters_from_profile("k_w4_gemm_wide", "gemm.hip", "nh_device.hpp"),
        }
        log("gemm:", out["gemm"])
        del Xi, Xo, Yi, Yo, gws

        if not args.skip_stack:
            x4 = gu.to_dev(synth.block_input(4, B4, T4))
            ws4 = gu.workspace(nh.nh_block_workspace_bytes(d256, B4, T4, nh.NH_MODE_SEQ))
            outs4 = gu.empty_f32(n_layers, B4, T4, HID)

            def stack4():
                nh.nh_mamba_stack(d256, dev_layers[:n_layers], None, n_layers, nh.NH_MODE_SEQ, x4, nh.NH_BF16,
                                  T4, outs4, B4, ws4, ws4.numel(), stream)

            stack4()
            torch.cuda.synchronize()
            reps = 2
            hip.record(e0, stream)
            for _ in range(reps):
                stack4()
            hip.record(e1, stream)
            torch.cuda.synchronize()
            ms4 = hip.ms(e0, e1) / reps
            gemm_flops = 2 * pos * (NIN * HID + HID * DI) * n_layers
            out["stack_seq"] = {
                "workload": "27 Mamba2 blocks, batch 2, full-history T=3750, chunk 256",
                "ms": round(ms4, 2), "position_layers_per_s": round(pos * n_layers / (ms4 * 1e-3), 1),
                "w4_gemm_tflops": round(gemm_flops / (ms4 * 1e-3) / 1e12, 1),
            }
            log("stack seq:", out["stack_seq"])
            del outs4, ws4

    if args.calib_copy_mib > 0:
        a = torch.empty(args.calib_copy_mib * (1 << 20), dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = a.numel()

    # ------------------------------------------------- CPU oracle baseline
    if not args.skip_cpu:
        import oracle
        oracle.build(force=False)
        cores = oracle.lib().nho_max_threads()
        cpu_model = "unknown"
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        xh = gu.bf16_bits_to_f64(synth.block_input(1, 1, 1))
        csh = gu.bf16_bits_to_f64(cs0)
        lw0 = host_layers[0]

        def timed(fn, budget, min_reps=2):
            reps, t = 0, 0.0
            while t < budget or reps < min_reps:
                ts = time.perf_counter()
                fn()
                t += time.perf_counter() - ts
                reps += 1
            return t / reps, reps, t

        # C1: one batch-1 step with a pre-filled state, every host thread
        c1, c1_reps, c1_t = timed(lambda: oracle.block(synth.REAL, lw0, xh, csh, ss0, mode=oracle.CONTRACT,
                                                       stepwise=True, nthreads=cores), args.cpu_seconds)
        # C2: the batch-1 full-history recompute, a 32-position prefix of its T = 413 input
        x2 = gu.bf16_bits_to_f64(synth.block_input(2, 1, 32))
        c2, _, c2_t = timed(lambda: oracle.block(synth.REAL, lw0, x2, nthreads=cores), 0.0, 1)
        # C4: batch 2 full history, one layer over a 16-position prefix of its T = 3750 input
        x4 = gu.bf16_bits_to_f64(synth.block_input(4, 2, 16))
        c4, _, c4_t = timed(lambda: oracle.block(synth.REAL, lw0, x4, nthreads=cores), 0.0, 1)
        # C1 on one thread
        c1s, _, c1s_t = timed(lambda: oracle.block(synth.REAL, lw0, xh, csh, ss0, mode=oracle.CONTRACT,
                                                   stepwise=True, nthreads=1), 0.0, 2)
        oracle.block(synth.REAL, lw0, xh, csh, ss0, stepwise=True, nthreads=cores)  # restore the thread count
        out["cpu_baseline"] = {
            "value": round(c1 * 1e6, 1), "unit": "us/layer", "cores": cores, "cpu_model": cpu_model,
            "kind": "oracle",
            "sample": f"one batch-1 block step with a pre-filled state, fp64 oracle on {cores} threads, "
                      f"{c1_reps} repeats, {c1_t:.1f} s of host time",
            "single_thread_us_per_layer": round(c1s * 1e6, 1),
            "c2_positions_per_s": round(32 / c2, 2),
            "c4_position_layers_per_s": round(2 * 16 / c4, 2),
            "legs": "C1 step on all threads (value) and on one thread; C2 full history over the first 32 of "
                    "its 413 positions (batch 1); C4 full history over the first 16 of its 3750 positions "
                    "(batch 2, one layer); positions/s are position-layers per second",
            "host_seconds": round(c1_t + c2_t + c4_t + c1s_t, 1),
        }
        log("cpu baseline:", out["cpu_baseline"])

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
