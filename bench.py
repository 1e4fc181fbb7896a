"""Benchmark of the selective-scan hot path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input.  The
default workload is the bidirectional Vim-Tiny block scan (fp32, batch 128,
L = 197 with the middle CLS token, d_inner 384, d_state 16): one
vm_bidir_scan_fwd call, which is a single kernel launch (B and C arrive
token-major, as the block's projection produces them).

Reported on one JSON line: whole-job throughput in algorithmic HBM GB/s (each
input read once, the output written once), tokens*channels/s, the roofline
record of the scan kernel (kernel time from HIP events on the launch stream:
around each replay of the graph of the K timed launches, over K, for the
graph-replayed steps, else around every launch; HBM traffic from the
committed rocprofv3 counter summary when it belongs to the current kernel
source), and the fp64 CPU oracle timed on the host's cores on the same
workload.

Inputs are resident in HBM before timing; the step cycles through several
independent input sets so that consecutive steps cannot be served from the
256 MB Infinity Cache.  Steps that allocate no temporary memory (the fp32
headline, the single direction, ES2D) are captured once in a HIP graph of all
K timed steps and replayed; the others launch eagerly (`launch` in config).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
# ALU ceiling of the state step, from the VALU issue-rate probe
# (csrc/valu_probe.hip, `bench.py --valu-probe`, summary in profiles/): one
# state update is dt*A, v_exp_f32, dt*u*B, the state fma and the readout fma.
# v_exp_f32 occupies a SIMD for 8 cycles per wave64 instruction and the other
# forms pair across waves at about 2.1 cycles only while no exponential is in
# flight; the best body measured (exponentials and the other operations in
# barrier-separated phases, 4 waves per SIMD) takes 20.1 SIMD cycles per wave
# of 64 state updates.  Ceiling: 1024 SIMDs x 64 lanes x 2.4 GHz / 20.1.
CYCLES_PER_WAVE_STATE_UPDATE = 20.1
UPDATES_PEAK_T = 256 * 4 * 64 * 2.4e9 / CYCLES_PER_WAVE_STATE_UPDATE / 1e12
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["selective_scan_fwd_amd/csrc/scan_kernel.hip",
                  "selective_scan_fwd_amd/csrc/scan_chunk.hip",
                  "selective_scan_fwd_amd/csrc/scan_bwd.hip",
                  "selective_scan_fwd_amd/csrc/scan_device.h",
                  "selective_scan_fwd_amd/csrc/layout_kernels.hip",
                  "selective_scan_fwd_amd/csrc/vm_internal.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1,
                    help="0 single, 1 Vim-T bidir (default), 2 bf16 L=4097, 3 ES2D 56x56, "
                         "4 FastVim pooled (axes alternate per step), 5 FastVim unpooled L=16384, "
                         "6 SS2D four-direction scan 56x56, 7 backward of the Vim-T bidirectional scan, "
                         "8 backward of the SS2D scan 56x56")
    ap.add_argument("--sets", type=int, default=0, help="input sets to cycle (0 = auto)")
    ap.add_argument("--size", type=int, default=56, choices=[56, 57],
                    help="config 3: the ES2D feature map (56x56, or 57x57 padded to 58x58)")
    ap.add_argument("--replays", type=int, default=0,
                    help="times the K timed steps are run (graph replays, or eager passes); the median is "
                         "reported (0 = at least 5, and at least 1000 steps in all: short passes of a few "
                         "milliseconds run on a GPU whose clock is still rising)")
    ap.add_argument("--conv", choices=["none", "fused", "unfused"], default="none",
                    help="configs 0-2: the scan input comes from the block's causal conv1d + SiLU, "
                         "computed inside the scan (fused) or by vm_causal_conv1d_silu first (unfused)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every timed step eagerly instead of replaying one HIP graph of them")
    ap.add_argument("--zoh", action="store_true",
                    help="zero-order-hold input coefficient instead of dt (the released model uses dt)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline (0 = skip)")
    ap.add_argument("--batch", type=int, default=0,
                    help="configs 0-2: another batch size at the same shape (0 = the config's); "
                         "the kernel time against batch shows how the launch fills the chip")
    ap.add_argument("--seed", type=int, default=1001)
    ap.add_argument("--valu-probe", action="store_true",
                    help="instead of the benchmark, run the VALU issue-rate probe (libvmprobe.so) and print "
                         "SIMD cycles per wave-instruction for each form the state step uses")
    ap.add_argument("--probe-kinds", default="", help="comma-separated probe bodies to run (default: all)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run --steps plain device copies of MIB MiB "
                         "(reference reading for the HBM byte counters)")
    return ap.parse_args()


def copy_calibration(mib, steps):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": steps}))


PROBE_KINDS = ["fma", "exp", "exp+3fma", "state-step-dpp", "state-step-dpp-no-exp", "permlane32-swap",
               "exp-latency", "fma-latency", "fma-3vgpr", "mul-2vgpr", "mul-sgpr", "fmac-sgpr", "mul-dpp",
               "state-step-sgpr", "state-step-sgpr-no-exp", "exp-waves+fma-waves", "state-step-vgpr",
               "state-step-vgpr-no-exp", "phased-2w-barrier", "phased-2w", "phased-4w-barrier", "phased-4w",
               "fetch-straight-4096", "fetch-loop-64x64", "state-step-vgpr-exp-groups-16",
               "state-step-vgpr-exp-groups-32", "state-step-vgpr-exp-groups-64"]
SIMDS = 256 * 4


def valu_probe(iters=4000, kinds=None):
    """Issue-rate probe (selective_scan_fwd_amd/csrc/valu_probe.hip).  For
    each body and W waves per SIMD (256 W workgroups of four waves), the SIMD
    cycles one wave-instruction takes, chip-wide: launch time x shader clock x
    1024 SIMDs / wave-instructions issued (the clock is the waves' median
    s_memtime rate against the 100 MHz real-time counter).  A 16-lane SIMD
    would take 4 per wave64 instruction.  The latency bodies are one
    dependent chain at one wave per SIMD: their per-wave figure (elapsed
    cycles / instructions) is the dependent-issue latency."""
    import ctypes

    import numpy as np
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "selective_scan_fwd_amd", "libvmprobe.so"))
    lib.vm_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.vm_probe_instr.argtypes = [ctypes.c_int]
    lib.vm_probe_threads.argtypes = [ctypes.c_int]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    inp = (torch.rand(64, device=dev) * 0.5 + 0.25).contiguous()
    rows = []
    for kind, name in enumerate(PROBE_KINDS):
        if kinds is not None and kind not in kinds:
            continue
        threads = lib.vm_probe_threads(kind)
        if "phased" in name:
            ws = (threads // 256,)          # one workgroup per CU
        else:
            ws = (1,) if "latency" in name else (1, 2, 4, 8)
        for w in ws:
            blocks = 256 * w * 256 // threads
            waves = blocks * threads // 64
            out = torch.empty(blocks * threads, device=dev)
            clk = torch.zeros(waves * 4, dtype=torch.int64, device=dev)
            it = iters // 4 if "latency" in name else iters
            if name.startswith("fetch"):
                it = 1 if "straight" in name else 64         # 4096 instructions either way
            for rep in range(2):                       # the first launch warms up
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                rc = lib.vm_probe_run(kind, blocks, it, inp.data_ptr(), out.data_ptr(), clk.data_ptr(),
                                      ctypes.c_void_p(stream.cuda_stream))
                e1.record(stream)
                if rc != 0:
                    raise RuntimeError(f"probe {name}: error {rc}")
                torch.cuda.synchronize()
            c = clk.cpu().numpy().reshape(-1, 4).astype(np.float64)
            cyc = c[:, 1] - c[:, 0]
            rt = (c[:, 3] - c[:, 2]) / 100e6                # 100 MHz real-time counter
            ninstr = lib.vm_probe_instr(kind)
            ghz = float(np.median(cyc / rt)) / 1e9
            ms = e0.elapsed_time(e1)
            per_chip = ms * 1e-3 * ghz * 1e9 * SIMDS / (waves * it * ninstr)
            per_wave = np.median(cyc) / (it * ninstr)
            rows.append({"body": name, "waves_per_simd": w, "instr_per_iter": ninstr, "iters": it,
                         "simd_cycles_per_wave_instr": round(float(per_chip), 3),
                         "wave_cycles_per_instr": round(float(per_wave), 3),
                         "wave_cycles_median": float(np.median(cyc)), "wave_cycles_max": float(cyc.max()),
                         "shader_clock_ghz": round(ghz, 3), "launch_ms": round(ms, 4)})
            print(json.dumps(rows[-1]), flush=True)
    return rows


# ---------------------------------------------------------------- workloads
def algorithmic_bytes_scan(batch, dim, L, N, es, dirs, gated):
    """Bytes a scan must move: u and delta per direction, z, out once; B and C
    once per (batch, token) and direction; A, D, bias once per direction."""
    tok = batch * dim * L
    per_dir = 2 * tok * es + 2 * batch * L * N * es + dim * N * 4 + 2 * dim * 4
    return dirs * per_dir + (tok * es if gated else 0) + tok * es


def build_step(cfg, seed, sets, dev, zoh=False, conv="none", es2d_size=56, batch=0):
    """Returns (step_fn(i), info dict, cpu_fn(budget_s) -> (seconds, bytes, tokens, threads, desc))."""
    import torch

    import selective_scan_fwd_amd as vm
    from selective_scan_fwd_amd import workloads as wl

    N = wl.DSTATE
    if cfg in (0, 1, 2):
        w = wl.WORKLOADS[cfg]
        if batch:
            w = dataclasses.replace(w, batch=batch, name=f"{w.name}@batch{batch}")
        dt = wl.torch_dtype(w.dtype)
        es = 2 if w.dtype == "bf16" else 4
        dirs = 2 if w.kind == "bidir" else 1
        inputs = []
        for k in range(sets):
            if dirs == 2:
                inputs.append(wl.bidir_inputs(seed + k, w.batch, w.dim, w.seqlen, device=dev, dtype=dt))
            else:
                p, z = wl.single_inputs(seed + k, w.batch, w.dim, w.seqlen, device=dev, dtype=dt)
                inputs.append((p, None, z))
        outs = [torch.empty_like(inputs[k][0]["u"]) for k in range(sets)]
        if conv != "none":
            # Vim: both directions read the same content x through their own convolutions
            gc = wl.generator(seed + 100, dev)
            for f, b, _ in inputs:
                if b is not None:
                    b["u"] = f["u"]
                for p in (f, b) if b is not None else (f,):
                    p["conv_w"], p["conv_b"] = wl.conv_params(gc, w.dim, dev)
        ubuf = [torch.empty_like(outs[0]) for _ in range(dirs)] if conv == "unfused" else None

        def strip(p, u):
            return {k: (u if k == "u" else v) for k, v in p.items() if not k.startswith("conv")}

        def step(i):
            f, b, z = inputs[i % sets]
            if conv == "unfused":
                f = strip(f, vm.vm_causal_conv1d_silu(f["u"], f["conv_w"], f["conv_b"], out=ubuf[0]))
                if b is not None:
                    b = strip(b, vm.vm_causal_conv1d_silu(b["u"], b["conv_w"], b["conv_b"], reverse=True,
                                                          out=ubuf[1]))
            if dirs == 2:
                vm.vm_bidir_scan_fwd(f, b, z=z, combine_scale=w.combine_scale, out=outs[i % sets], zoh=zoh)
            else:
                vm.vm_selective_scan_fwd(**f, z=z, out=outs[i % sets], zoh=zoh)

        nbytes = algorithmic_bytes_scan(w.batch, w.dim, w.seqlen, N, es, dirs, True)
        tokens = w.batch * w.dim * w.seqlen
        slots = dirs * tokens * N
        info = dict(workload=w.name, batch=w.batch, dim=w.dim, seqlen=w.seqlen, dstate=N,
                    directions=dirs, combine_scale=w.combine_scale, dtype=w.dtype,
                    bc_layout="token-major",
                    # no temporary memory: fp32, or an on-chip exchange
                    graphable=w.dtype == "f32" and (dirs == 1 or w.seqlen <= 520))
        if conv != "none":
            info["conv1d"] = conv

        def cpu(budget):
            import oracle
            f, b, z = inputs[0]
            sub = max(1, min(w.batch, w.batch))          # whole workload, repeated in time
            hf = {k: (v[:sub].double().cpu().numpy() if k in ("u", "delta", "B", "C") else
                      (v.double().cpu().numpy() if v is not None else None)) for k, v in f.items()}
            cvf = (hf.pop("conv_w", None), hf.pop("conv_b", None))
            hxf = hf["u"].copy()                         # the conv input, when there is a conv
            hz = z[:sub].double().cpu().numpy()
            if dirs == 2:
                hb = {k: (v[:sub].double().cpu().numpy() if k in ("u", "delta", "B", "C") else
                          (v.double().cpu().numpy() if v is not None else None)) for k, v in b.items()}
                cvb = (hb.pop("conv_w", None), hb.pop("conv_b", None))
                hxb = hb["u"].copy()

                def run():
                    if conv != "none":
                        hf["u"] = oracle.causal_conv1d_silu(hxf, *cvf)
                        hb["u"] = oracle.causal_conv1d_silu(hxb, *cvb, reverse=True)
                    return oracle.bidir_scan(hf, hb, z=hz, combine_scale=w.combine_scale, zoh=zoh)
            else:
                def run():
                    if conv != "none":
                        hf["u"] = oracle.causal_conv1d_silu(hxf, *cvf)
                    return oracle.selective_scan(**hf, z=hz, zoh=zoh)
            reps, t0 = 0, time.perf_counter()
            while True:
                run()
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget or reps >= 100:
                    break
            frac = sub / w.batch
            return el / reps, nbytes * frac, tokens * frac, oracle.num_threads(), \
                f"fp64 oracle on the whole workload ({sub} of {w.batch} batch rows), {reps} repetitions"

        return step, info, cpu, nbytes, tokens, slots

    if cfg == 3:
        w = wl.WORKLOADS[3]
        H = W = es2d_size
        inputs = [wl.es2d_inputs(seed + k, w.batch, w.dim, H, W, device=dev) for k in range(sets)]
        Lg = ((H + 1) // 2) * ((W + 1) // 2)
        streams = [torch.empty((w.batch, 4, w.dim, Lg), device=dev) for _ in range(sets)]
        ys = [torch.empty((4 * w.batch, w.dim, Lg), device=dev) for _ in range(sets)]
        outs = [torch.empty((w.batch, w.dim, H, W), device=dev) for _ in range(sets)]

        def gather(i):
            x, _ = inputs[i % sets]
            vm.vm_atrous_gather(x, out=streams[i % sets])

        def scan(i):
            _, p = inputs[i % sets]
            vm.vm_selective_scan_fwd(streams[i % sets].view(4 * w.batch, w.dim, Lg), **p, out=ys[i % sets], zoh=zoh)

        def scatter(i):
            vm.vm_atrous_scatter(ys[i % sets].view(w.batch, 4, w.dim, Lg), H, W, out=outs[i % sets])

        def step(i):
            gather(i)
            scan(i)
            scatter(i)

        # the three launches one by one (timed separately for the per-kernel rooflines)
        step.parts = (("gather", gather), ("scan", scan), ("scatter", scatter))

        # algorithmic bytes of the ES2D step: x read and y written once, plus
        # the scan's delta, B, C and parameters (the gathered u streams and the
        # scan's output streams are intermediates of the three launches)
        plane = w.batch * w.dim * H * W * 4
        streams_b = w.batch * 4 * w.dim * Lg * 4
        scan_b = algorithmic_bytes_scan(4 * w.batch, w.dim, Lg, N, 4, 1, False)
        nbytes = scan_b - 2 * streams_b + 2 * plane
        tokens = w.batch * w.dim * H * W
        slots = 4 * w.batch * w.dim * Lg * N
        # per kernel, each kernel's own inputs read once and outputs written
        # once (the gathered streams and the scan's output streams counted
        # by both kernels that touch them)
        step.part_bytes = {"gather": plane + streams_b, "scan": scan_b, "scatter": streams_b + plane}
        info = dict(workload=f"{w.name}@{H}x{W}", batch=w.batch, dim=w.dim, height=H, width=W,
                    group_len=Lg, dstate=N, kernels="gather+scan+scatter", graphable=True)

        def cpu(budget):
            import oracle
            x, p = inputs[0]
            sub = 8
            hx = x[:sub].double().cpu().numpy()
            rows = slice(0, 4 * sub)
            hp = {k: (v[rows].double().cpu().numpy() if k in ("delta", "B", "C") else
                      v.double().cpu().numpy()) for k, v in p.items()}

            def run():
                s = oracle.atrous_gather(hx)
                y = oracle.selective_scan(s.reshape(4 * sub, w.dim, Lg), **hp, zoh=zoh)
                oracle.atrous_scatter(y.reshape(sub, 4, w.dim, Lg), H, W)
            reps, t0 = 0, time.perf_counter()
            while True:
                run()
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget or reps >= 100:
                    break
            frac = sub / w.batch
            return el / reps, nbytes * frac, tokens * frac, oracle.num_threads(), \
                f"fp64 oracle gather+scan+scatter on {sub} of {w.batch} batch rows, {reps} repetitions"

        return step, info, cpu, nbytes, tokens, slots

    if cfg in (4, 5):
        w = wl.WORKLOADS[4]
        H, W = w.height, w.width
        L = H * W
        if cfg == 4:
            inputs = [wl.fastvim_inputs(seed, w.batch, w.dim, H, W, axis, device=dev) for axis in (0, 1)]
            out = torch.empty((w.batch, w.dim, H, W), device=dev)

            def step(i):
                f, b, z = inputs[i % 2]
                vm.vm_pool_scan_repeat(f, b, z=z, combine_scale=w.combine_scale, pool_axis=i % 2, out=out,
                                       zoh=zoh)

            tok_full = w.batch * w.dim * L
            Lp = H
            nbytes = (2 * tok_full + tok_full + tok_full) * 4 + \
                2 * (w.batch * w.dim * Lp * 4 + 2 * w.batch * Lp * N * 4 + w.dim * (N + 2) * 4)
            slots = 2 * w.batch * w.dim * Lp * N
            info = dict(workload=f"{w.name}-pooled", batch=w.batch, dim=w.dim, height=H, width=W,
                        pooled_len=Lp, dstate=N, pool_axis="alternating 0/1",
                        kernels="pool x2 + bidir scan + repeat-gate")
        else:
            f, b, z = wl.fastvim_inputs(seed, w.batch, w.dim, H, W, 0, device=dev, full_resolution=True)
            for p in (f, b):
                p["u"] = p["u"].view(w.batch, w.dim, L)
            zf = z.view(w.batch, w.dim, L)
            out = torch.empty_like(zf)

            def step(i):
                vm.vm_bidir_scan_fwd(f, b, z=zf, combine_scale=w.combine_scale, out=out, zoh=zoh)

            nbytes = algorithmic_bytes_scan(w.batch, w.dim, L, N, 4, 2, True)
            slots = 2 * w.batch * w.dim * L * N
            info = dict(workload=f"{w.name}-unpooled", batch=w.batch, dim=w.dim, seqlen=L, dstate=N)
        tokens = w.batch * w.dim * L
        return step, info, None, nbytes, tokens, slots

    if cfg == 6:
        w = wl.WORKLOADS[5]
        H, W = w.height, w.width
        L = H * W
        inputs = [wl.ss2d_inputs(seed + k, w.batch, w.dim, H, W, device=dev) for k in range(sets)]
        outs = [torch.empty((w.batch, w.dim, H, W), device=dev) for _ in range(sets)]

        def step(i):
            u, dirs, z = inputs[i % sets]
            vm.vm_ss2d_scan_fwd(u, dirs, z=z, combine_scale=w.combine_scale, out=outs[i % sets], zoh=zoh)

        tok = w.batch * w.dim * L
        # u, z and out once; delta, B, C and the parameters once per traversal
        nbytes = 3 * tok * 4 + 4 * (tok * 4 + 2 * w.batch * L * N * 4 + w.dim * (N + 2) * 4)
        tokens = tok
        slots = 4 * tok * N
        info = dict(workload=w.name, batch=w.batch, dim=w.dim, height=H, width=W, dstate=N,
                    directions=4, kernels="transpose + 2 bidir scans + merge")

        def cpu(budget):
            import oracle
            u, dirs, z = inputs[0]
            sub = 1
            hu = u[:sub].double().cpu().numpy()
            hz = z[:sub].double().cpu().numpy()
            hd = [{k: (v[:sub].double().cpu().numpy() if k in ("delta", "B", "C") else
                       v.double().cpu().numpy()) for k, v in p.items()} for p in dirs]
            run = lambda: oracle.ss2d_scan(hu, hd, z=hz, combine_scale=w.combine_scale, zoh=zoh)
            reps, t0 = 0, time.perf_counter()
            while True:
                run()
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget or reps >= 100:
                    break
            frac = sub / w.batch
            return el / reps, nbytes * frac, tokens * frac, oracle.num_threads(), \
                f"fp64 oracle SS2D on {sub} of {w.batch} batch rows, {reps} repetitions"

        return step, info, cpu, nbytes, tokens, slots

    if cfg == 7:
        w = wl.WORKLOADS[1]
        L = w.seqlen
        inputs = []
        for k in range(sets):
            f, b, z = wl.bidir_inputs(seed + k, w.batch, w.dim, L, device=dev)
            dout = torch.randn(f["u"].shape, generator=wl.generator(seed + 50 + k, dev), device=dev)
            inputs.append((f, b, z, dout))

        def step(i):
            f, b, z, dout = inputs[i % sets]
            vm.vm_bidir_scan_bwd(f, b, dout, z=z, combine_scale=w.combine_scale, zoh=zoh)

        tok = w.batch * w.dim * L
        bc = w.batch * L * N * 4
        # read u, delta per direction, z and dout once; B, C per direction;
        # write du, ddelta per direction, dz, and dB, dC per direction
        nbytes = 2 * (2 * tok * 4 + 2 * bc) + 2 * tok * 4 + 2 * (2 * tok * 4 + 2 * bc) + tok * 4
        tokens = tok
        # one state recompute (5 operations) and the adjoint (9) per state
        # step: 14 / 5 state-update equivalents
        slots = 2 * tok * N * 14 / 5
        info = dict(workload=w.name + "-backward", batch=w.batch, dim=w.dim, seqlen=L, dstate=N,
                    directions=2, combine_scale=w.combine_scale,
                    kernels="forward recompute + gate backward + 2 x (backward + reduce)")

        def cpu(budget):
            from oracle import grad as og
            f, b, z, dout = inputs[0]
            sub = 1
            hd = lambda p: {k: (v[:sub] if k in ("u", "delta", "B", "C") else v).double().cpu().numpy()
                            for k, v in p.items()}
            hf, hb = hd(f), hd(b)
            hz, hdo = z[:sub].double().cpu().numpy(), dout[:sub].double().cpu().numpy()
            reps, t0 = 0, time.perf_counter()
            while True:
                og.bidir_scan_grad(hf, hb, hdo, z=hz, combine_scale=w.combine_scale, zoh=zoh)
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget or reps >= 20:
                    break
            frac = sub / w.batch
            return el / reps, nbytes * frac, tokens * frac, torch.get_num_threads(), \
                f"fp64 autograd oracle on {sub} of {w.batch} batch rows, {reps} repetitions"

        return step, info, cpu, nbytes, tokens, slots

    if cfg == 8:
        w = wl.WORKLOADS[5]
        H, W = w.height, w.width
        L = H * W
        inputs = []
        for k in range(sets):
            u, dirs, z = wl.ss2d_inputs(seed + k, w.batch, w.dim, H, W, device=dev)
            dout = torch.randn(u.shape, generator=wl.generator(seed + 50 + k, dev), device=dev)
            inputs.append((u, dirs, z, dout))

        def step(i):
            u, dirs, z, dout = inputs[i % sets]
            vm.vm_ss2d_scan_bwd(u, dirs, dout, z=z, combine_scale=w.combine_scale, zoh=zoh)

        tok = w.batch * w.dim * L
        bc = w.batch * L * N * 4
        # read u, z and dout once, and delta, B, C per traversal; write du and
        # dz once, and ddelta, dB, dC per traversal
        nbytes = 3 * tok * 4 + 4 * (tok * 4 + 2 * bc) + 2 * tok * 4 + 4 * (tok * 4 + 2 * bc)
        tokens = tok
        # one state recompute (5 operations) and the adjoint (9) per state
        # step of each traversal: 14 / 5 state-update equivalents
        slots = 4 * tok * N * 14 / 5
        info = dict(workload=w.name + "-backward", batch=w.batch, dim=w.dim, height=H, width=W, dstate=N,
                    directions=4, combine_scale=w.combine_scale,
                    kernels="transposes + 2 bidir recomputes + gate backward + 4 x (backward + reduce) + sum")

        def cpu(budget):
            from oracle import grad as og
            u, dirs, z, dout = inputs[0]
            sub = 1
            h = lambda t: t[:sub].double().cpu().numpy()
            hd = [{k: (h(v) if k in ("delta", "B", "C") else v.double().cpu().numpy()) for k, v in p.items()}
                  for p in dirs]
            reps, t0 = 0, time.perf_counter()
            while True:
                og.ss2d_scan_grad(h(u), hd, h(dout), z=h(z), combine_scale=w.combine_scale, zoh=zoh)
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget or reps >= 20:
                    break
            frac = sub / w.batch
            return el / reps, nbytes * frac, tokens * frac, torch.get_num_threads(), \
                f"fp64 autograd oracle on {sub} of {w.batch} batch rows, {reps} repetitions"

        return step, info, cpu, nbytes, tokens, slots

    raise SystemExit(f"unknown --config {cfg}")


def load_traffic(source_hash, workload):
    """HBM bytes per step (the scan kernel; every kernel of the step for the
    multi-kernel workloads) from the committed counter summary, if it was
    taken on the current kernel sources and this workload (name plus any
    "+zoh" / "+conv-..." variant suffix)."""
    path = os.path.join(PROFILE_DIR, "scan_kernel_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_hash") != source_hash:
        return None
    return entry.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the scan shards by batch rows with no exchange)", file=sys.stderr)
        sys.exit(2)

    import torch

    import selective_scan_fwd_amd as vm

    if args.copy_calib:
        copy_calibration(args.copy_calib, args.steps)
        return
    if args.valu_probe:
        valu_probe(kinds=[int(k) for k in args.probe_kinds.split(",")] if args.probe_kinds else None)
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    vm.load_library()
    dev = torch.device("cuda:0")
    sets = args.sets or (3 if args.config in (0, 1, 2, 3, 6, 7) else 1)
    if args.conv != "none" and args.config not in (0, 1, 2):
        raise SystemExit("--conv applies to configs 0-2")
    if args.batch and args.config not in (0, 1, 2):
        raise SystemExit("--batch applies to configs 0-2")
    step, info, cpu_fn, nbytes, tokens, slots = build_step(args.config, args.seed, sets, dev, args.zoh,
                                                           args.conv, args.size, args.batch)
    if args.zoh:
        info = dict(info, discretization="zoh")
    torch.cuda.synchronize()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Kernel time (the roofline's): K eager steps with HIP events around every
    # launch, on the launch stream (mean, median and min per launch).
    # Whole-job time (value, ms_per_step): exactly K steps between
    # synchronisations, timed REPLAYS times; the median is reported, with
    # the min.  Workloads whose steps allocate no temporary memory are
    # captured once in a HIP graph of the K steps and replayed, which removes
    # the per-call host overhead between launches; the others repeat the K
    # eager steps.
    use_graph = info.pop("graphable", False) and not args.no_graph
    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    per_launch = sorted(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends))
    launch_ms = sum(per_launch) / args.steps
    launch_med = per_launch[len(per_launch) // 2]
    # multi-kernel steps with separately timed parts: each part over K
    # steps with HIP events around every launch
    kernels = None
    parts = getattr(step, "parts", None)
    if parts:
        kernels = {}
        for name, fn in parts:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            torch.cuda.synchronize()
            for i in range(args.steps):
                ev[i][0].record(stream)
                fn(i)
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
            nb = step.part_bytes[name]
            kernels[name] = {"ms": round(ms, 5), "algorithmic_bytes": nb,
                             "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                             "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(i)
        graph.replay()                                  # one untimed replay
        torch.cuda.synchronize()
    walls = []
    graph_ms = []      # HIP events on the launch stream around each replay of the K steps
    replays = args.replays or max(5, -(-1000 // args.steps))
    for r in range(replays):
        if graph is None and r == 0:
            walls.append(eager_wall)
            continue
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if graph is not None:
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            graph.replay()
            g1.record(stream)
        else:
            for i in range(args.steps):
                step(i)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        if graph is not None:
            graph_ms.append(g0.elapsed_time(g1) / args.steps)
    walls.sort()
    wall = walls[len(walls) // 2]
    graph_ms.sort()
    info["launch"] = "hip-graph" if use_graph else "eager"

    ms_per_step = 1e3 * wall / args.steps
    value = nbytes / (wall / args.steps) / 1e9
    # Kernel time of the roofline: in a replayed graph, the launches of the
    # timed region run back to back, and events around each replay over K
    # give their mean duration (median replay); eager steps take the mean of
    # the per-launch events.
    roof_ms = graph_ms[len(graph_ms) // 2] if graph_ms else launch_ms
    achieved_gbs = nbytes / (roof_ms * 1e-3) / 1e9
    achieved_updates = slots / (roof_ms * 1e-3) / 1e12
    src_hash = kernel_source_hash()
    variant = ("+zoh" if args.zoh else "") + (f"+conv-{args.conv}" if args.conv != "none" else "")
    traffic = load_traffic(src_hash, info["workload"] + variant)
    # The roofline is HBM bandwidth (algorithmic bytes of the step / mean
    # kernel time); the ALU ceiling of the state step is reported beside it.
    roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    other = {"bound": "alu", "achieved": round(achieved_updates, 3), "peak": round(UPDATES_PEAK_T, 3),
             "unit": "T state updates/s", "frac": round(achieved_updates / UPDATES_PEAK_T, 4),
             "cycles_per_wave_state_update": CYCLES_PER_WAVE_STATE_UPDATE}

    cpu = None
    if cpu_fn is not None and args.cpu_seconds > 0:
        sec, cbytes, ctok, threads, desc = cpu_fn(args.cpu_seconds)
        cpu = {"value": round(cbytes / sec / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": desc, "seconds_per_pass": round(sec, 4),
               "tokens_ch_per_s": round(ctok / sec, 1)}

    line = {
        "metric": "selective-scan HBM GB/s (% peak) + tokens*ch/s, bidir Vim-T B=128 L=197",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": dict(info, input_sets=sets),
        "tokens_ch_per_s": round(tokens / (wall / args.steps), 1),
        "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "kernel_ms": round(roof_ms, 5),
        "kernel_ms_from": "graph-replay events / K" if graph_ms else "per-launch events (eager)",
        "kernel_ms_events": round(launch_ms, 5),
        "kernel_ms_events_median": round(launch_med, 5),
        "kernel_ms_events_min": round(per_launch[0], 5),
        "ms_per_step_min": round(1e3 * walls[0] / args.steps, 5),
        "replays": len(walls),
        "roofline": roof,
        "roofline_other": other,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "kernel_source_hash": src_hash,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
