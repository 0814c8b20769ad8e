#!/usr/bin/env python3
"""Benchmark of the MoT token-routed projection on one MI355X.

Headline: routed-GEMM TFLOP/s (and % of the bf16 MFMA peak) of the BAGEL
fused QKV projection, T=4096 packed rows (77 und + 1024 gen rows cycled:
308 und / 3788 gen) after the routed RMSNorm (X is the library's fused
add-RMSNorm of a seeded residual stream), K=3584 -> N=4608 (3584 q + 512 k +
512 v).  One step is
one mot_routed_gemm call on inputs already resident in HBM: the routing plan
(segment list) and the routed GEMM with its bf16 epilogue.  FLOPs count real
rows only: 2*T*K*N.

Beside it, on the same line:
  roofline      dominant kernel (the routed GEMM) against the bf16 MFMA peak,
                its average duration from HIP events on the launch stream;
  cpu_baseline  the CPU oracle timed on a bounded row sample on this host;
  components    the other hot-path steps, each against its own roofline:
                routed fused add-RMSNorm and the QK norm + rotary (GB/s), the
                routed-RMSNorm prologue, small weight-bound packs, the
                backward's dX and dW, the QKV GEMM with the QK norm + rotary
                in its epilogue, shared joint attention, the MLP, one GPU's
                share under 4-way tensor parallelism, a whole layer on the
                CFG pack and on a 16384-row pack, and the latent step (CFG
                combine, SDE step with its log-probability).  --only picks
                some of them (one rocprofv3 run per kernel family).

Inputs are synthetic and seeded (CPU generators, then copied to the GPU).
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-GEMM TFLOP/s and % bf16 MFMA peak at T=4096, 3584->4608 QKV"
# MI355X: 256 CUs x 2.4 GHz x 4096 dense bf16 flop/clk/CU (published 2.5 PFLOP/s).
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--soak-s", type=float, default=1.0,
                   help="seconds of untimed launches before the warm-up (clock settling)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-components", action="store_true")
    p.add_argument("--only", default="",
                   help="comma-separated components to run (for one rocprofv3 run per kernel family): norm, "
                        "prologue, small_packs, down_small_packs, backward, qk_norm_rope, qkv_qk_fused, attention, "
                        "context_blas, "
                        "mlp, tp4, layer_chain, gen_step, latent")
    p.add_argument("--copy-probe", action="store_true",
                   help="run one 1 GiB device copy first (HBM counter calibration under rocprofv3)")
    p.add_argument("--cpu-rows", type=int, default=4096,
                   help="oracle row sample for cpu_baseline (stratified, with every segment boundary)")
    return p.parse_args()


def git_rev():
    info = os.path.join(ROOT, "mixture_transformers_token_amd", "BUILD_INFO.json")
    if os.path.exists(info):
        with open(info) as f:
            d = json.load(f)
        return d.get("commit", "unknown"), d.get("dirty")
    try:
        rev = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                             text=True).stdout.strip()
        dirty = subprocess.run(["git", "status", "--porcelain"], cwd=ROOT, capture_output=True,
                               text=True).stdout.strip() != ""
        return rev or "unknown", dirty if rev else None
    except Exception:
        return "unknown", None


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "qkv_routed_gemm_T4096_hbm_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "mixture_transformers_token_amd", "csrc", "mot_kernels.hip")


def measured_traffic():
    """HBM-side bytes per launch of the QKV routed GEMM from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary -- only while the kernel source
    is the one those counters were taken on (else None)."""
    import hashlib
    try:
        kv = dict(line.strip().split("=", 1) for line in open(TRAFFIC_SUMMARY) if "=" in line
                  and not line.startswith(("|", "-", "`", "#")) and " " not in line.strip())
        h = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]
        if kv.get("kernel_source_sha256_16") != h:
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def time_calls(fn, iters, stream):
    """Average duration of `fn` launches, HIP events on the launch stream."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters * 1e-3  # seconds


def time_each(fn, n, stream):
    """Per-launch durations (seconds) of n launches, an event pair around
    each on the launch stream."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)


def time_component(fn, iters, stream, blocks=5, warmup=3):
    """Median over `blocks` blocks of `iters` launches (after `warmup`
    untimed launches) of the per-launch duration, HIP events on the stream."""
    for _ in range(warmup):
        fn()
    ts = sorted(time_calls(fn, iters, stream) for _ in range(blocks))
    return ts[len(ts) // 2]


def time_component_graph(fn, calls, stream, reps=9, warmup=3):
    """Per-call time of `fn` from HIP-graph replays of `calls` captured
    launches (median of `reps` replays), for kernels shorter than the host's
    per-call launch cost: eager launches of such kernels measure the host,
    not the GPU.  The library's calls allocate nothing, so they capture."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3 / calls)
    ts.sort()
    return ts[len(ts) // 2]


def n_gen_rows(m):
    return int((m == 1).sum())


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the "
              "routed projection is row-local and would shard by rows", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_transformers_token_amd as mot
    import workloads as W

    torch.cuda.init()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.copy_probe:
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # ---- headline workload: BAGEL fused QKV, T=4096 --------------------------
    T, K, N = 4096, W.HIDDEN, W.QKV_DIM
    x, wu, wg, m = W.qkv(T)
    wud, wgd = wu.to(dev), wg.to(dev)
    md = torch.from_numpy(m).to(dev)
    # X as the workload has it: the routed RMSNorm of a seeded residual
    # stream, made by the library's fused add-RMSNorm (the CPU leg below
    # times the oracle on generator rows of the same shape: its time does
    # not depend on the values)
    xr0, r0 = W.residual_inputs(T, K, base=77)
    nw0 = tuple(t.to(dev) for t in W.norm_weights(K, base=77))
    xd = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    mot.fused_add_rmsnorm(xr0.to(dev), r0.to(dev), nw0[0], nw0[1], md, out=xd, rstd=None)
    torch.cuda.synchronize()
    del xr0, r0
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    ws = mot.new_workspace(T, dev)
    flops = 2.0 * T * K * N

    def step():
        mot.routed_gemm(xd, wud, wgd, md, out=y, workspace=ws)

    # untimed soak before the requested warm-up: the chip's clock settles
    # under sustained MFMA load within about a second, so the timed steps and
    # the per-kernel event times below measure the steady state, not the
    # faster first milliseconds
    soak_launches = 0
    t_soak = time.perf_counter()
    while time.perf_counter() - t_soak < args.soak_s:
        for _ in range(50):
            step()
        soak_launches += 50
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = flops * args.steps / elapsed / 1e12
    if mot.read_device_error(ws) != 0:
        raise RuntimeError("device error word set during the benchmark")

    # dominant kernel: packs of up to 8192 rows are one launch of the routed
    # GEMM (segment list built in-kernel), timed with HIP events on its stream
    gemm_s = time_calls(step, max(args.steps, 50), stream)
    achieved = flops / gemm_s / 1e12
    each = time_each(step, 100, stream)
    pct = {f"p{q}": round(each[min(len(each) - 1, q * len(each) // 100)] * 1e6, 2) for q in (10, 50, 90)}
    n_und, n_gen = int((m == 0).sum()), int((m == 1).sum())
    traffic = measured_traffic()
    roofline = {
        "kernel": "gemm_kernel<false,false,true,false,false,false,false,false,false> (routed QKV GEMM, in-kernel segment list)",
        "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
        "avg_kernel_us": round(gemm_s * 1e6, 2),
        "launch_us_percentiles": pct,
        "flop_per_launch": flops,
        "alg_bytes_per_launch": 2 * (2 * N * K + T * K + T * N) + T,
    }

    def small_packs(components):
        """Small, weight-bound packs (HBM roofline) at the QKV shape, weights
        rotated over eight copies of both sets (528 MB, twice the last-level
        cache) so that they come from HBM.  Two variants per size: the BAGEL
        pattern's prefix (a prompt of 77 und rows, then latents) and a pack of
        generation rows only.  Timed per call from HIP-graph replays (the
        kernels are shorter than an eager launch's host cost; eager_us is the
        eager figure)."""
        copies = [(W.normal_bf16((N, K), 90 + i, 0.02).to(dev), W.normal_bf16((N, K), 190 + i, 0.02).to(dev))
                  for i in range(8)]
        for Ts in (1, 8, 64, 77, 128, 256):
            for variant in ("prefix", "gen"):
                ms = W.pattern(Ts) if variant == "prefix" else np.ones(Ts, np.uint8)
                xs_s = W.normal_bf16((Ts, K), 9).to(dev)
                mds = torch.from_numpy(ms).to(dev)
                ys = torch.empty((Ts, N), dtype=torch.bfloat16, device=dev)
                wss = mot.new_workspace(Ts, dev)
                ctr = [0]

                def small():
                    a, b = copies[ctr[0] % 8]
                    ctr[0] += 1
                    mot.routed_gemm(xs_s, a, b, mds, out=ys, workspace=wss)
                s_small = time_component_graph(small, 16, stream)
                s_eager = time_component(small, 40, stream)
                sets = int((ms == 0).any()) + int((ms == 1).any())
                nb = sets * N * K * 2 + Ts * K * 2 + Ts * N * 2 + Ts
                components[f"qkv_small_T{Ts}_{variant}"] = {
                    "us": round(s_small * 1e6, 2), "GB/s": round(nb / s_small / 1e9, 1),
                    "frac_hbm": round(nb / s_small / 1e9 / PEAK_HBM_GBS, 3), "sets": sets,
                    "eager_us": round(s_eager * 1e6, 2)}
        del copies

    def down_small_packs(components):
        """Small packs at the down projection's shape (K = 18944 -> N = 3584):
        a chain of 1184 dependent MFMAs per output element and only 112
        32-column blocks, so the paired small-pack kernel spreads a set's rows
        over all four slots of a block.  Weights rotated over two copies of
        both sets (543 MB, twice the last-level cache); HIP-graph timed."""
        Kd, Nd = W.FFN, W.HIDDEN
        copies = [(W.normal_bf16((Nd, Kd), 290 + i, 0.02).to(dev), W.normal_bf16((Nd, Kd), 390 + i, 0.02).to(dev))
                  for i in range(2)]
        for Ts in (1, 64, 128, 256):
            for variant in ("prefix", "gen"):
                ms = W.pattern(Ts) if variant == "prefix" else np.ones(Ts, np.uint8)
                xs_d = W.normal_bf16((Ts, Kd), 19).to(dev)
                mds = torch.from_numpy(ms).to(dev)
                ys = torch.empty((Ts, Nd), dtype=torch.bfloat16, device=dev)
                wss = mot.new_workspace(Ts, dev)
                ctr = [0]

                def small():
                    a, b = copies[ctr[0] % 2]
                    ctr[0] += 1
                    mot.routed_gemm(xs_d, a, b, mds, out=ys, workspace=wss)
                s_small = time_component_graph(small, 16, stream)
                sets = int((ms == 0).any()) + int((ms == 1).any())
                nb = sets * Nd * Kd * 2 + Ts * Kd * 2 + Ts * Nd * 2 + Ts
                components[f"down_small_T{Ts}_{variant}"] = {
                    "us": round(s_small * 1e6, 2), "GB/s": round(nb / s_small / 1e9, 1),
                    "frac_hbm": round(nb / s_small / 1e9 / PEAK_HBM_GBS, 3), "sets": sets}
        del copies

    def joint_attention(components, qkv_buf, iters):
        # shared joint attention over QKV rows (28 q / 4 kv heads, causal,
        # bottom-right aligned; q, k, v read as column ranges of the buffer):
        # MFMA-bound; useful flops count only the visible keys
        q_v, k_v = qkv_buf[:, :W.Q_DIM], qkv_buf[:, W.Q_DIM:W.Q_DIM + W.KV_DIM]
        v_v = qkv_buf[:, W.Q_DIM + W.KV_DIM:]
        att = torch.empty((T, W.Q_DIM), dtype=torch.bfloat16, device=dev)
        s_att = time_component(lambda: mot.joint_attention(q_v, k_v, v_v, W.N_Q_HEADS, W.N_K_HEADS, causal=True,
                                                           out=att), iters, stream)
        f_att = 4.0 * W.N_Q_HEADS * 128 * T * (T + 1) / 2
        components["joint_attention_causal_T4096"] = {
            "us": round(s_att * 1e6, 1), "TFLOP/s": round(f_att / s_att / 1e12, 1),
            "frac_mfma": round(f_att / s_att / 1e12 / PEAK_BF16_TFLOPS, 3),
            "note": "one kernel (V read in place); flops of visible keys only"}

    def latent_step(components):
        """The per-step latent work of a batch of 16 rollouts of 1024 latent
        rows x 64 fp32 channels (512x512 images): the three-branch CFG
        combine with the per-request norm-ratio rescale, then the SDE step
        sampling x_next with its log-probability, and the evaluation of a
        given x_next.  HBM-bound, small: timed from HIP-graph replays."""
        B, R, Cl = 16, 1024, 64
        g = torch.Generator().manual_seed(77)
        br = [torch.randn((B * R, Cl), generator=g).to(dev) for _ in range(6)]
        vc, vt, vi, xl, nz, xn = br
        cul = torch.arange(0, B * R + 1, R, dtype=torch.int32).to(dev)
        tl = torch.full((B,), 0.6, dtype=torch.float32, device=dev)
        tn = torch.full((B,), 0.55, dtype=torch.float32, device=dev)
        vg = torch.empty_like(vc)
        xo = torch.empty_like(vc)
        lp = torch.empty(B, dtype=torch.float32, device=dev)
        wsl = torch.empty(mot.latent_workspace_bytes(B, R), dtype=torch.uint8, device=dev)
        cfg = lambda: mot.cfg_combine_renorm(vc, vt, vi, cul, R, tl, 4.0, 1.5, 0.0, 1.0, 0.0, "global", out=vg,
                                             workspace=wsl)
        sde = lambda: mot.flow_sde_step_logp(xl, vg, cul, R, tl, tn, 1.0, noise=nz, out=xo, logp=lp, workspace=wsl)
        ev = lambda: mot.flow_sde_step_logp(xl, vg, cul, R, tl, tn, 1.0, x_next=xn, logp=lp, workspace=wsl)
        ent = {}
        for nm, fn, arrays in (("cfg_combine_renorm", cfg, 4), ("sde_step_sample_logp", sde, 4),
                               ("sde_step_eval_logp", ev, 3)):
            st = time_component_graph(fn, 16, stream)
            nb = arrays * B * R * Cl * 4
            ent[nm] = {"us": round(st * 1e6, 2), "GB/s": round(nb / st / 1e9, 1),
                       "frac_hbm": round(nb / st / 1e9 / PEAK_HBM_GBS, 3)}
        if mot.read_device_error(wsl) != 0:
            raise RuntimeError("latent step raised its error word")
        components["latent_step_16x1024x64_fp32"] = ent

    # ---- other hot-path steps ------------------------------------------------
    # Each component is a function of the dict it fills; --only picks some
    # (one rocprofv3 run per kernel family), --no-components none.
    iters = 30
    nwu, nwg = (t.to(dev) for t in W.norm_weights(K))
    qn, kn = W.qk_norm_weights()
    qn, kn = tuple(t.to(dev) for t in qn), tuple(t.to(dev) for t in kn)
    cos_t, sin_t, pos = (t.to(dev) for t in W.rope_inputs(T, 4096))
    xs, rs = W.residual_inputs(T, K)
    xsd, rsd = xs.to(dev), rs.to(dev)

    def c_norm(components):
        # routed fused add-RMSNorm, T=4096, H=3584 (x, residual in; residual,
        # y out); eight input copies rotated (x, residual, out: 8 x 3 x 29 MB,
        # above the 256 MB last-level cache), so every byte comes from HBM
        yn = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
        rstd = torch.empty(T, dtype=torch.float32, device=dev)
        norm_sets = [(xsd.clone(), rsd.clone(), torch.empty_like(yn)) for _ in range(8)]
        nctr = [0]

        def norm_rot():
            xa, ra, ya = norm_sets[nctr[0] % 8]
            nctr[0] += 1
            mot.fused_add_rmsnorm(xa, ra, nwu, nwg, md, out=ya, rstd=rstd)
        s_norm = time_component(norm_rot, iters, stream)
        s_norm_hot = time_component(lambda: mot.fused_add_rmsnorm(xsd, rsd, nwu, nwg, md, out=yn, rstd=rstd),
                                    iters, stream)
        nbytes = 4 * T * K * 2 + T * 4 + T
        components["fused_add_rmsnorm_T4096_H3584"] = {
            "us": round(s_norm * 1e6, 2), "GB/s": round(nbytes / s_norm / 1e9, 1),
            "frac_hbm": round(nbytes / s_norm / 1e9 / PEAK_HBM_GBS, 3),
            "us_same_inputs": round(s_norm_hot * 1e6, 2),
            "note": "inputs rotated over eight copies (from HBM); us_same_inputs reuses one set (cache-served)"}

    def c_prologue(components):
        # QKV with the routed-RMSNorm prologue (reads h + rstd instead of y)
        rstd = torch.empty(T, dtype=torch.float32, device=dev)
        yn = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
        h = rsd.clone()
        mot.fused_add_rmsnorm(xsd, h, nwu, nwg, md, out=yn, rstd=rstd)
        s_pro = time_component(lambda: mot.routed_gemm(h, wud, wgd, md, out=y, workspace=ws,
                                                       norm=(rstd, nwu, nwg)), iters, stream)
        components["qkv_prologue_T4096"] = {"us": round(s_pro * 1e6, 2),
                                            "TFLOP/s": round(flops / s_pro / 1e12, 1)}

    def c_backward(components):
        # routed backward of the QKV projection: dX = dY W_m with the weights
        # read as they lie (and, for comparison, on transposed weights made
        # once per weight update), and the generation
        # set's dW over its 3788 rows (one kernel over dY and X as they lie;
        # the contraction runs over all T rows, the und rows read as zeros)
        dyd = W.normal_bf16((T, N), 11).to(dev)
        wt = (mot.transpose(wud), mot.transpose(wgd))
        dx = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
        s_dx = time_component(lambda: mot.routed_gemm_dx(dyd, wud, wgd, md, out=dx, workspace=ws), iters, stream)
        s_dx_wt = time_component(lambda: mot.routed_gemm_dx(dyd, wud, wgd, md, wt=wt, out=dx, workspace=ws),
                                 iters, stream)
        s_wt = time_component(lambda: mot.transpose(wgd), iters, stream)
        s_dw = time_component(lambda: mot.grad_w(dyd, xd, md, keep=1), 10, stream)
        s_dw32 = time_component(lambda: mot.grad_w(dyd, xd, md, keep=1, out_dtype=torch.float32), 10, stream)
        f_dw = 2.0 * n_gen_rows(m) * N * K
        components["qkv_backward_T4096"] = {
            "dx_us": round(s_dx * 1e6, 1), "dx_TFLOP/s": round(flops / s_dx / 1e12, 1),
            "dx_pretransposed_weights_us": round(s_dx_wt * 1e6, 1),
            "weight_transpose_us": round(s_wt * 1e6, 1),
            "dw_gen_us": round(s_dw * 1e6, 1), "dw_gen_TFLOP/s": round(f_dw / s_dw / 1e12, 1),
            "dw_gen_fp32_us": round(s_dw32 * 1e6, 1), "dw_gen_fp32_TFLOP/s": round(f_dw / s_dw32 / 1e12, 1),
            "dw_gen_rows": n_gen_rows(m),
            "note": "dw_gen: one mot_grad_w call (token-major operands, no transposes); flops count the gen rows"}

    wsq = mot.new_workspace(0, dev)

    def c_qk_norm_rope(components):
        # routed per-head QK RMSNorm + rotary embedding, in place on the QKV
        # output (28 q + 4 k heads of 128; rotary tables as data, 4096
        # positions): HBM-bound, reads and writes the q and k columns
        qkv_buf = y.clone()
        s_qk = time_component(lambda: mot.qk_norm_rope(qkv_buf, W.N_Q_HEADS, W.N_K_HEADS, md, qn, kn, pos, cos_t,
                                                       sin_t, workspace=wsq), iters, stream)
        if mot.read_device_error(wsq) != 0:
            raise RuntimeError("qk_norm_rope raised its error word")
        qk_cols = 128 * (W.N_Q_HEADS + W.N_K_HEADS)
        nb_qk = 2 * T * qk_cols * 2 + T * (1 + 4 + 2 * 64 * 2)
        components["qk_norm_rope_T4096"] = {"us": round(s_qk * 1e6, 2), "GB/s": round(nb_qk / s_qk / 1e9, 1),
                                            "frac_hbm": round(nb_qk / s_qk / 1e9 / PEAK_HBM_GBS, 3)}

    def c_qkv_qk_fused(components):
        # the QKV GEMM with the QK norm + rotary in its epilogue, against the
        # two calls (same bytes)
        yq = torch.empty_like(y)
        s_fused = time_component(lambda: mot.routed_gemm_qk_norm_rope(xd, wud, wgd, md, W.N_Q_HEADS, W.N_K_HEADS, qn,
                                                                       kn, pos, cos_t, sin_t, out=yq, workspace=ws),
                                 iters, stream)

        def two_calls():
            mot.routed_gemm(xd, wud, wgd, md, out=yq, workspace=ws)
            mot.qk_norm_rope(yq, W.N_Q_HEADS, W.N_K_HEADS, md, qn, kn, pos, cos_t, sin_t, workspace=wsq)
        s_two = time_component(two_calls, iters, stream)
        components["qkv_qk_norm_rope_fused_T4096"] = {
            "us": round(s_fused * 1e6, 2), "TFLOP/s": round(flops / s_fused / 1e12, 1),
            "two_calls_us": round(s_two * 1e6, 2)}
        del yq

    def c_attention(components):
        joint_attention(components, y.clone(), iters)

    def c_context_blas(components):
        # context only: the vendor library's dense GEMM of one weight set at
        # the same shape (hipBLASLt via torch.matmul; not batch-invariant,
        # not a target)
        wg_t = wgd.t()
        s_blas = time_component(lambda: torch.matmul(xd, wg_t), iters, stream)
        components["context_dense_one_set_torch_matmul_T4096"] = {
            "us": round(s_blas * 1e6, 1), "TFLOP/s": round(flops / s_blas / 1e12, 1),
            "note": "hipBLASLt dense x @ W_gen^T, one set, for context; not batch-invariant"}

    mlp_w = []

    def mlp_dev():
        if not mlp_w:
            mlp_w.extend(t.to(dev) for t in W.mlp_weights())
        return mlp_w

    def c_mlp(components):
        # MLP: gate/up+SwiGLU 3584 -> 2x18944, down 18944 -> 3584
        gu_u, gu_g, dn_u, dn_g = mlp_dev()
        act = torch.empty((T, W.FFN), dtype=torch.bfloat16, device=dev)
        yd = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
        s_gu = time_component(lambda: mot.routed_gemm_swiglu(xd, gu_u, gu_g, md, out=act, workspace=ws),
                              5, stream)
        s_dn = time_component(lambda: mot.routed_gemm(act, dn_u, dn_g, md, out=yd, workspace=ws), 5, stream)
        f_gu = 2.0 * T * K * 2 * W.FFN
        f_dn = 2.0 * T * W.FFN * K
        components["gate_up_swiglu_T4096"] = {"us": round(s_gu * 1e6, 1),
                                              "TFLOP/s": round(f_gu / s_gu / 1e12, 1)}
        components["down_T4096"] = {"us": round(s_dn * 1e6, 1), "TFLOP/s": round(f_dn / s_dn / 1e12, 1)}

    def c_tp4(components):
        # one GPU's share under 4-way tensor parallelism (28 q / 4 kv heads:
        # TP2 and TP4 are valid, TP8 is not): column-parallel QKV and gate/up
        # (N / 4 of both sets), row-parallel O and down (K / 4); the partial
        # sums' reduction across GPUs is not part of this measurement
        tp = {}
        for name, (Kt, Nt, sw) in {"qkv_tp4": (K, N // 4, False), "o_tp4": (W.Q_DIM // 4, K, False),
                                   "gate_up_swiglu_tp4": (K, W.FFN // 4, True),
                                   "down_tp4": (W.FFN // 4, K, False)}.items():
            xt = W.normal_bf16((T, Kt), 31).to(dev)
            rows_w = 2 * Nt if sw else Nt
            wa = W.normal_bf16((rows_w, Kt), 32, 0.02).to(dev)
            wb = W.normal_bf16((rows_w, Kt), 33, 0.02).to(dev)
            yt = torch.empty((T, Nt), dtype=torch.bfloat16, device=dev)
            fn = (lambda: mot.routed_gemm_swiglu(xt, wa, wb, md, out=yt, workspace=ws)) if sw else \
                 (lambda: mot.routed_gemm(xt, wa, wb, md, out=yt, workspace=ws))
            st = time_component(fn, 10, stream)
            ft = 2.0 * T * Kt * rows_w
            tp[name] = {"K": Kt, "N": Nt, "us": round(st * 1e6, 1), "TFLOP/s": round(ft / st / 1e12, 1),
                        "frac_mfma": round(ft / st / 1e12 / PEAK_BF16_TFLOPS, 3)}
            del xt, wa, wb, yt
        components["tp4_shard_shapes_T4096"] = tp

    def c_layer_chain(components):
        gu_u, gu_g, dn_u, dn_g = mlp_dev()
        # per-layer chain: fused add-RMSNorm -> QKV -> QK norm + rotary ->
        # shared joint attention (causal within each request: the CFG pack's
        # seven, the 16384-row pack as one) -> O ->
        # fused add-RMSNorm -> gate/up+SwiGLU -> down, on the three-branch CFG
        # pack and on a 16384-row pack; "TFLOP/s" counts the routed linear
        # steps over real rows only (the CFG pack's 562 padding rows
        # excluded), the attention's time is in the layer time
        ou, og = (t.to(dev) for t in W.o_weights())
        for name, mc, real, lens in (("cfg_pack_T4096", W.cfg_pack_modality(), 3534, W.cfg_pack_lengths()),
                                     ("pack_T16384", W.pattern(16384), 16384, [16384])):
            Tc = mc.size
            mcd = torch.from_numpy(mc).to(dev)
            xc, rc = (t.to(dev) for t in W.residual_inputs(Tc, K, base=5))
            res_c = rc.clone()
            y1 = torch.empty((Tc, K), dtype=torch.bfloat16, device=dev)
            qkv_c = torch.empty((Tc, N), dtype=torch.bfloat16, device=dev)
            o_c = torch.empty((Tc, K), dtype=torch.bfloat16, device=dev)
            att_c = torch.empty((Tc, W.Q_DIM), dtype=torch.bfloat16, device=dev)
            cu_c = torch.from_numpy(W.cu_lengths(lens)).to(dev)
            ws_att_c = torch.empty(mot.attention_varlen_workspace_bytes(Tc, len(lens), W.N_K_HEADS),
                                   dtype=torch.uint8, device=dev)
            act_c = torch.empty((Tc, W.FFN), dtype=torch.bfloat16, device=dev)
            out_c = torch.empty((Tc, K), dtype=torch.bfloat16, device=dev)
            wsc = mot.new_workspace(Tc, dev)
            cos_c, sin_c, pos_c = (t.to(dev) for t in W.rope_inputs(Tc, 4096, base=5))
            ops = {
                "norm1": lambda: mot.fused_add_rmsnorm(xc, res_c, nwu, nwg, mcd, out=y1, rstd=None),
                "qkv_qk_norm_rope": lambda: mot.routed_gemm_qk_norm_rope(y1, wud, wgd, mcd, W.N_Q_HEADS, W.N_K_HEADS,
                                                                         qn, kn, pos_c, cos_c, sin_c, out=qkv_c,
                                                                         workspace=wsc),
                "attention": lambda: mot.joint_attention_varlen(
                    qkv_c[:, :W.Q_DIM], qkv_c[:, W.Q_DIM:W.Q_DIM + W.KV_DIM], qkv_c[:, W.Q_DIM + W.KV_DIM:], cu_c,
                    cu_c, max(lens), W.N_Q_HEADS, W.N_K_HEADS, causal=True, out=att_c, workspace=ws_att_c),
                "o": lambda: mot.routed_gemm(att_c, ou, og, mcd, out=o_c, workspace=wsc),
                "norm2": lambda: mot.fused_add_rmsnorm(o_c, res_c, nwu, nwg, mcd, out=y1, rstd=None),
                "gate_up_swiglu": lambda: mot.routed_gemm_swiglu(y1, gu_u, gu_g, mcd, out=act_c, workspace=wsc),
                "down": lambda: mot.routed_gemm(act_c, dn_u, dn_g, mcd, out=out_c, workspace=wsc),
            }

            def layer():
                for f in ops.values():
                    f()
            s_layer = time_component(layer, 2, stream)
            per_op = {k: round(time_component(f, 3, stream) * 1e6, 1) for k, f in ops.items()}
            if name == "cfg_pack_T4096":
                # the generation step's attention: each branch's 1024 latent
                # rows query its 77 prompt rows and its latents without a mask
                # (the prompt's keys and values come from the cache in a real
                # step; here they are the pack's own rows)
                # One packed call over the three branches (their prompt
                # rows ride along as queries: 7% more work, not counted)
                cu_gen = torch.from_numpy(W.cu_lengths([1101, 1101, 1101])).to(dev)
                ws_gen = torch.empty(mot.attention_varlen_workspace_bytes(3303, 3, W.N_K_HEADS), dtype=torch.uint8,
                                     device=dev)

                def gen_step_attention():
                    mot.joint_attention_varlen(qkv_c[:3303, :W.Q_DIM], qkv_c[:3303, W.Q_DIM:W.Q_DIM + W.KV_DIM],
                                               qkv_c[:3303, W.Q_DIM + W.KV_DIM:], cu_gen, cu_gen, 1101, W.N_Q_HEADS,
                                               W.N_K_HEADS, causal=False, out=att_c[:3303], workspace=ws_gen)
                s_gen = time_component(gen_step_attention, 3, stream)
                f_gen = 3 * 4.0 * W.N_Q_HEADS * 128 * 1024 * 1101
                per_op["attention_gen_step_3x1024_over_1101"] = round(s_gen * 1e6, 1)
                per_op["attention_gen_step_TFLOP/s"] = round(f_gen / s_gen / 1e12, 1)
            f_layer = 2.0 * real * (K * N + W.Q_DIM * K + K * 2 * W.FFN + W.FFN * K)
            components[f"layer_chain_{name}"] = {"us": round(s_layer * 1e6, 1),
                                                 "TFLOP/s": round(f_layer / s_layer / 1e12, 1),
                                                 "real_rows": real, "per_op_us": per_op}
            del act_c, att_c, ws_att_c

    def c_gen_step(components):
        """One decoder layer of a denoising step: the three CFG branches'
        latent rows only (3 x 1024 generation rows), the prompts' keys and
        values coming from a cache: norm -> QKV + QK norm/rotary -> attention
        of each branch's latents over its 77 cached prompt keys and its 1024
        latent keys (no mask) -> O -> norm -> gate/up + SwiGLU -> down.  The
        cache is a separate [3 x 1101, 4608] buffer (its latent rows stand
        for this step's keys and values; timing does not depend on values)."""
        gu_u, gu_g, dn_u, dn_g = mlp_dev()
        ou, og = (t.to(dev) for t in W.o_weights())
        Tg = 3 * 1024
        mg = torch.ones(Tg, dtype=torch.uint8, device=dev)
        xg, rg = (t.to(dev) for t in W.residual_inputs(Tg, K, base=9))
        y1 = torch.empty((Tg, K), dtype=torch.bfloat16, device=dev)
        qkv_g = torch.empty((Tg, N), dtype=torch.bfloat16, device=dev)
        kv = W.normal_bf16((3 * 1101, N), 10).to(dev)
        att = torch.empty((Tg, W.Q_DIM), dtype=torch.bfloat16, device=dev)
        o_g = torch.empty((Tg, K), dtype=torch.bfloat16, device=dev)
        act_g = torch.empty((Tg, W.FFN), dtype=torch.bfloat16, device=dev)
        out_g = torch.empty((Tg, K), dtype=torch.bfloat16, device=dev)
        wsg = mot.new_workspace(Tg, dev)
        cu_q = torch.from_numpy(W.cu_lengths([1024] * 3)).to(dev)
        cu_k = torch.from_numpy(W.cu_lengths([1101] * 3)).to(dev)
        ws_a = torch.empty(mot.attention_varlen_workspace_bytes(3 * 1101, 3, W.N_K_HEADS), dtype=torch.uint8,
                           device=dev)
        cos_g, sin_g, pos_g = (t.to(dev) for t in W.rope_inputs(Tg, 4096, base=9))
        ops = {
            "norm1": lambda: mot.fused_add_rmsnorm(xg, rg, nwu, nwg, mg, out=y1, rstd=None),
            "qkv_qk_norm_rope": lambda: mot.routed_gemm_qk_norm_rope(y1, wud, wgd, mg, W.N_Q_HEADS, W.N_K_HEADS, qn,
                                                                     kn, pos_g, cos_g, sin_g, out=qkv_g,
                                                                     workspace=wsg),
            "attention": lambda: mot.joint_attention_varlen(
                qkv_g[:, :W.Q_DIM], kv[:, W.Q_DIM:W.Q_DIM + W.KV_DIM], kv[:, W.Q_DIM + W.KV_DIM:], cu_q, cu_k, 1024,
                W.N_Q_HEADS, W.N_K_HEADS, causal=False, out=att, workspace=ws_a),
            "o": lambda: mot.routed_gemm(att, ou, og, mg, out=o_g, workspace=wsg),
            "norm2": lambda: mot.fused_add_rmsnorm(o_g, rg, nwu, nwg, mg, out=y1, rstd=None),
            "gate_up_swiglu": lambda: mot.routed_gemm_swiglu(y1, gu_u, gu_g, mg, out=act_g, workspace=wsg),
            "down": lambda: mot.routed_gemm(act_g, dn_u, dn_g, mg, out=out_g, workspace=wsg),
        }

        def layer():
            for f in ops.values():
                f()
        s_layer = time_component(layer, 2, stream)
        per_op = {k: round(time_component(f, 3, stream) * 1e6, 1) for k, f in ops.items()}
        f_lin = 2.0 * Tg * (K * N + W.Q_DIM * K + K * 2 * W.FFN + W.FFN * K)
        f_att = 4.0 * W.N_Q_HEADS * 128 * Tg * 1101
        components["layer_gen_step_3x1024_latents"] = {
            "us": round(s_layer * 1e6, 1), "TFLOP/s": round((f_lin + f_att) / s_layer / 1e12, 1),
            "rows": Tg, "per_op_us": per_op,
            "note": "flops: the routed linear steps and the attention (1101 keys per latent row)"}

    registry = {"norm": c_norm, "prologue": c_prologue, "small_packs": small_packs,
                "down_small_packs": down_small_packs, "backward": c_backward,
                "qk_norm_rope": c_qk_norm_rope, "qkv_qk_fused": c_qkv_qk_fused, "attention": c_attention,
                "context_blas": c_context_blas, "mlp": c_mlp, "tp4": c_tp4, "layer_chain": c_layer_chain,
                "gen_step": c_gen_step, "latent": latent_step}
    if args.no_components:
        chosen = []
    elif args.only:
        chosen = args.only.split(",")
        unknown = [c for c in chosen if c not in registry]
        if unknown:
            raise SystemExit(f"unknown component(s) {unknown}; known: {sorted(registry)}")
    else:
        chosen = list(registry)
    components = {}
    for cname in chosen:
        registry[cname](components)
        torch.cuda.synchronize()
        print(f"[bench] component {cname} done", file=sys.stderr, flush=True)
    mlp_w.clear()

    # ---- CPU oracle baseline on a bounded row sample -------------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rows = W.sample_rows(m, args.cpu_rows, seed=7) if args.cpu_rows < T else np.arange(T)
        xb, wub, wgb = W.bits(x)[rows], W.bits(wu), W.bits(wg)
        threads = oracle.max_threads()
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.routed_gemm(xb, wub, wgb, m[rows], want_ref=True, want_out=True)
            times.append(time.perf_counter() - t0)
        cs = sorted(times)[1]
        what = "all" if rows.size == T else f"{rows.size} of"
        cpu = {"value": round(2.0 * rows.size * K * N / cs / 1e12, 6), "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle",
               "sample": f"{what} {T} QKV rows (K={K}, N={N}), fp64 oracle, median of 3 runs "
                         f"of {cs:.2f} s each"}

    rev, dirty = git_rev()
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "soak_launches": soak_launches,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "BAGEL fused QKV routed GEMM: T=4096 packed rows (77 und + 1024 gen "
                               "cycled; 308 und, 3788 gen) after the routed RMSNorm, K=3584, N=4608, "
                               "two bf16 weight sets, fp32 accumulate, bf16 out",
                   "T": T, "K": K, "N": N, "n_und": n_und, "n_gen": n_gen,
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "components": components,
        "provenance": {"commit": rev, "dirty": dirty, "torch": torch.__version__,
                       "hip": torch.version.hip, "device": torch.cuda.get_device_name(dev)},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
