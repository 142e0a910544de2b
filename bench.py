"""Benchmark: one optimisation step of affine + deformable registration
(warp + MI + LNCC forward and backward + Adam) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c5]

A step is the whole hot path over one synthetic volume pair already resident
in device memory, as RegistrationStep runs it. The default workload is the
1280x1536x1280 gigavoxel layered-cortex pair (2.5 G voxels; F, M, u, m1, m2,
W, gW and the partial gradients resident, about 161 GB) with MI (32 bins)
and LNCC (9^3 window) and the moving image in 8 z-slabs: the largest
configuration, and the one that fits a single GPU only because nothing of
the step's intermediates is materialised. Its step is ngv_warp_zrange and
the forward slab sequence (ngv_warp_fwd_slab x 8), ngv_mi_loss_fwd_bwd (the
histogram, the loss and the log-ratio table; no gradient written),
ngv_lncc_loss_fwd_bwd (writing gW), then the backward slab sequence fused
with Adam, each slab call adding the MI gradient it forms from F and the
stored W (ngv_warp_bwd_adam_slab_mi x 8). On a workload with the moving
image in one piece (--config c4) the backward is one call that forms the MI
gradient from the W it recomputes (ngv_warp_bwd_adam_mi).

Prints one JSON line. `value` is voxels per second of whole steps.
`roofline` describes the dominant call (the longest): its algorithmic bytes
per launch of its kernel (the per-voxel figures below times the voxels of a
launch) over the mean launch time, timed with events on the stream the
kernels run on, against the 8 TB/s HBM peak. A slab sequence launches its
kernel once per slab and steps each voxel in one of them, so a launch there
is the call over the slab count; `kernel_name` is the kernel as the rocprofv3
summary in profiles/ names it. The LNCC call's fp64 issue rate is given
alongside. `traffic` is the
HBM bytes per launch that the committed counter passes in profiles/
measured, when they were taken on the current kernel source, else null.
`extra` holds, after the headline: the 640x768x640 step and the calls
outside the step on it, the iterated workloads (200 smoothed LNCC steps on
the 160x192x224 phantom, 100 MI steps on the 256^3 pair) as mean step times,
and the oracle's one-step time on the three smaller workloads at one thread
and at every thread. `cpu_baseline` is the oracle's whole step on a bounded
slab of the headline workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "voxels/s for warp+MI/LNCC fwd+bwd per step; % of MI355X HBM GB/s peak"
HBM_PEAK_GBS = 8000.0
# fp64 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2 flop (FMA) x 2.4 GHz
FP64_PEAK_TFLOPS = 78.6

# Algorithmic (compulsory) bytes per voxel of each call: each input read once
# per sweep its dependencies force, each output written once.
#   warp_fwd  u 12 + M 4 read, W 4 written                                 20
#   mi        F, W read twice (histogram, then gradient), gW written        20
#             (+4 when the gradient accumulates into gW)
#   lncc      F, W read once, gW written                                    12
#             (+4 when accumulating)
#   warp_bwd  u 12 + M 4 + gW 4 read, gu 12 written                         32
#   adam      u, gu, m1, m2 read (48), u, m1, m2 written (36)               84
#   warp_bwd_adam  u 12 + M 4 + gW 4 + m1, m2 24 read, u, m1, m2 written    80
#             (gu never reaches memory)
#   warp_fwd_mi  warp_fwd + F 4 read (the histogram is built in the sweep)  24
#   mi_grad   F, W read, gW written (+4 when accumulating)                  12
# With the MI gradient formed in the fused backward (the default with MI and
# one moving slab):
#   mi_fwd    F, W read once (histogram, loss and log-ratio table only)      8
#   warp_bwd_adam_mi  warp_bwd_adam + F 4 read, W recomputed from the      84
#             backward's own gathers; 80 when no other term's gW is read
#   warp_bwd_adam_slab_mi  the slab sequence's backward with Adam, F 4 and  88
#             the stored W 4 read (W cannot be recomputed from one slab);
#             84 when no other term's gW is read
# The two-sweep step (--fused-step; W and gW never stored):
#   mi_sweep  u 12 + M 4 + F 4 read (the samples feed the histogram)        20
#   warp_lncc_mi_bwd  u 12 + M 4 + F 4 read, gu 12 written                  32
#             (then adam, 84)
# Calls outside the step, timed on their own after it:
#   mse       F, W read, gW written                                         12
#   warp_compose  v 12 read, the composed field U 12 read once, w 12 written 36
#   mi_box_fixed  as mi (the box kernel on F, cubic on W)                     20
# The step's model without the optimiser (warp 20 + MI 20 + LNCC 16 +
# sampler backward 32) is 88 bytes per voxel; it is reported beside the
# timed step's own figure.
MODEL_STEP_BYTES_NO_ADAM = 88
# Algorithmic fp64 flops per output voxel of the LNCC call (FMA = 2), for the
# sliding-window algorithm without halo recomputation:
#   moments F^2, W^2, FW                                               3
#   w-box of 5 moment fields, 3 axes x (add entering, subtract leaving) 30
#   cross, v_F, v_W, D, 1/D, cc, alpha, beta, gamma, loss sum         24
#   w-box of 3 coefficient fields                                      18
#   gradient gamma + 2 W beta + F alpha, scaled                         5
LNCC_FLOPS_PER_VOXEL = 80

# Which source file holds each call's kernels (the counter summaries name it
# and its SHA-256; a summary taken on other source is stale).
CALL_SOURCE = {"warp_fwd": "warp.hip sampler_device.hpp", "mi": "mi.hip mi_device.hpp",
               "lncc": "lncc.hip lncc_maps.hpp sampler_device.hpp mi_device.hpp",
               "warp_bwd": "warp.hip sampler_device.hpp", "adam": "adam.hip",
               "warp_bwd_adam": "warp.hip sampler_device.hpp", "warp_fwd_mi": "warp.hip sampler_device.hpp mi_device.hpp",
               "mi_grad": "mi.hip mi_device.hpp", "mse": "mse.hip",
               "warp_compose": "warp.hip sampler_device.hpp", "mi_box_fixed": "mi.hip mi_device.hpp",
               "mi_fwd": "mi.hip mi_device.hpp", "warp_bwd_adam_mi": "warp.hip sampler_device.hpp mi_device.hpp",
               "mi_sweep": "warp.hip sampler_device.hpp mi_device.hpp",
               "warp_lncc_mi_bwd": "lncc.hip lncc_maps.hpp sampler_device.hpp mi_device.hpp",
               "warp_bwd_adam_slab_mi": "warp.hip sampler_device.hpp mi_device.hpp"}


def call_bytes(name, accumulate):
    """accumulate: the call adds to gW (mi, lncc, mi_grad), or reads another
    term's gW (warp_bwd_adam_mi)."""
    base = {"warp_fwd": 20, "mi": 20, "lncc": 12, "warp_bwd": 32, "adam": 84, "warp_bwd_adam": 80,
            "warp_fwd_mi": 24, "mi_grad": 12, "mse": 12, "warp_compose": 36, "mi_box_fixed": 20, "mi_fwd": 8,
            "warp_bwd_adam_mi": 80, "mi_sweep": 20, "warp_lncc_mi_bwd": 32, "warp_bwd_adam_slab_mi": 84}[name]
    if accumulate and name in ("mi", "lncc", "mi_grad", "warp_bwd_adam_mi", "warp_bwd_adam_slab_mi"):
        base += 4
    return base


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="c5", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip every oracle timing")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip everything after the headline steps (other workloads, calls outside the step, "
                         "loops, oracle timings of the small workloads)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step recorded once as a HIP graph (per-call times from the eager "
                         "warm-up steps)")
    ap.add_argument("--fused-mi", action="store_true",
                    help="the sampler sweep builds the MI histogram (ngv_warp_fwd_mi + ngv_mi_grad)")
    ap.add_argument("--no-mi-backward", action="store_true",
                    help="the MI call writes its gradient and the backward reads it (ngv_mi_loss_fwd_bwd + "
                         "ngv_warp_bwd_adam) instead of the backward forming it (ngv_warp_bwd_adam_mi)")
    ap.add_argument("--fused-step", action="store_true",
                    help="the two-sweep step: the MI forward on samples not stored (ngv_warp_fwd_mi, W = NULL), "
                         "then LNCC + MI gradients into the sampler backward (ngv_warp_lncc_mi_bwd), then "
                         "ngv_adam_step")
    ap.add_argument("--cpu-planes", type=int, default=0, help="planes of the oracle sample (0: auto)")
    ap.add_argument("--copy-gib", type=float, default=0.0,
                    help="after timing, copy a buffer of this many GiB once (a known-size kernel for scaling "
                         "FETCH_SIZE / WRITE_SIZE counter passes)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha256(call):
    """SHA-256 of the kernel source files of `call`, concatenated in order."""
    import hashlib
    h = hashlib.sha256()
    for name in CALL_SOURCE[call].split():
        with open(os.path.join(ROOT, "non_gemm_voxel_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(call, config):
    """HBM bytes per launch of `call` from the committed counter summary
    profiles/<call>_<config>_hbm_traffic.txt, if it was taken on the current
    kernel source (same SHA-256); else None."""
    path = os.path.join(ROOT, "profiles", f"{call}_{config}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != source_sha256(call) or "bytes_per_launch" not in fields:
        return None
    return float(fields["bytes_per_launch"])


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_step_seconds(F, M, A, t, lr, bins, win, smooth_sigma):
    """Wall time of the oracle's whole step from u = m1 = m2 = 0 on host
    volumes F, M (numpy float32)."""
    import numpy as np

    from oracle import oracle as orc
    shape = F.shape
    u0 = np.zeros((3,) + shape, np.float32)
    prm = orc.pack_prm(A, t)
    t0 = time.perf_counter()
    W = orc.warp_fwd(M, u0, prm)
    gW = np.zeros_like(W)
    if bins:
        _, g, _ = orc.mi_loss_grad(F, W, bins=bins)
        gW += g
    if win:
        _, g = orc.lncc_loss_grad(F, W, win)
        gW += g
    gu, _, _, _ = orc.warp_bwd(M, u0, prm, gW)
    if smooth_sigma > 0:
        gu = np.stack([orc.gauss_smooth(gu[k], smooth_sigma) for k in range(3)])
    z = np.zeros(gu.size)
    orc.adam(u0, gu, z, z, 1, lr)
    return time.perf_counter() - t0


def cpu_baseline(F, M, case, wl):
    """The oracle's whole step on host planes F, M of the workload, taken as a
    volume of its own (its z-faces zero padded like any volume's)."""
    from oracle import oracle as orc
    dt = oracle_step_seconds(F, M, case.A, case.t, case.lr, wl.bins, wl.win, wl.smooth_sigma)
    n = int(F.size)
    nz, ny, nx = F.shape
    return {"value": n / dt, "unit": "voxels/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"whole step (warp, MI, LNCC, sampler backward, Adam) on planes 0..{nz - 1} of the "
                      f"{wl.name} workload ({nx}x{ny}x{nz} = {n} voxels, as a volume of its own), {dt:.1f} s wall",
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def cpu_configs(dev):
    """The oracle's one-step time on the three smaller workloads at their full
    sizes, with every thread and with one (median of 3 runs for the 64^3
    case, one run otherwise)."""
    from non_gemm_voxel_amd import synth
    from oracle import oracle as orc
    out = {}
    threads = orc.num_threads()
    for name in ("c1", "c2", "c3"):
        wl = synth.WORKLOADS[name]
        c = synth.make_case(wl, device=dev)
        F, M = c.F.cpu().numpy(), c.M.cpu().numpy()
        del c.F, c.M
        n = int(F.size)
        row = {"voxels": n}
        for th in (threads, 1):
            orc.set_num_threads(th)
            reps = 3 if name == "c1" else 1
            ts = sorted(oracle_step_seconds(F, M, c.A, c.t, c.lr, wl.bins, wl.win, wl.smooth_sigma)
                        for _ in range(reps))
            row[f"threads_{th}"] = {"seconds": ts[len(ts) // 2], "voxels_per_s": n / ts[len(ts) // 2]}
        orc.set_num_threads(threads)
        out[name] = row
        log(f"oracle {name}: " + ", ".join(f"{k} {v['seconds']:.2f} s" for k, v in row.items() if k != "voxels"))
    return out


class StepTimer:
    """One RegistrationStep with each call bracketed by events on the current
    stream."""

    def __init__(self, st, wl):
        self.st, self.wl = st, wl
        if st.fused_step:
            self.active = (["mi_sweep"] if wl.bins else []) + ["warp_lncc_mi_bwd", "adam"]
            self.acc = {}
            return
        if st.mi_bwd:
            self.mi_call = None if st.fused_mi else "mi_fwd"
            self.bwd_calls = ["warp_bwd_adam_slab_mi" if st.zrange is not None else "warp_bwd_adam_mi"]
        else:
            self.mi_call = "mi_grad" if st.fused_mi else "mi"
            self.bwd_calls = ["warp_bwd_adam"] if st.fused else ["warp_bwd", "adam"]
        calls = (["warp_fwd_mi"] if st.fused_mi else ["warp_fwd"]) + [self.mi_call, "lncc"] + self.bwd_calls
        self.active = [c for c in calls if c is not None and not (c in ("mi", "mi_grad", "mi_fwd") and not wl.bins)
                       and not (c == "lncc" and not wl.win)]
        self.acc = {"mi": False, "mi_grad": False, "lncc": bool(wl.bins) and not st.mi_bwd,
                    "warp_bwd_adam_mi": bool(wl.win), "warp_bwd_adam_slab_mi": bool(wl.win)}

    def new_events(self):
        import torch
        return {c: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for c in self.active}

    def step(self, ev):
        import torch
        st, wl = self.st, self.wl
        s = torch.cuda.current_stream()
        if st.fused_step:
            for c, f in (("mi_sweep", st.mi_sweep), ("warp_lncc_mi_bwd", st.gradient_sweep), ("adam", st.update)):
                if c in self.active:
                    ev[c][0].record(s)
                    f()
                    ev[c][1].record(s)
            return
        first = self.active[0]
        ev[first][0].record(s)
        st.warp()
        ev[first][1].record(s)
        if self.mi_call in self.active:
            ev[self.mi_call][0].record(s)
            st.mi()
            ev[self.mi_call][1].record(s)
        if wl.win:
            ev["lncc"][0].record(s)
            st.lncc()
            ev["lncc"][1].record(s)
        if st.fused:
            ev[self.bwd_calls[0]][0].record(s)
            st.backward_update()
            ev[self.bwd_calls[0]][1].record(s)
            return
        ev["warp_bwd"][0].record(s)
        st.backward()
        ev["warp_bwd"][1].record(s)
        ev["adam"][0].record(s)
        st.update()
        ev["adam"][1].record(s)

    def run(self, steps, warmup, graph=False):
        """Returns (wall seconds of the timed steps, per-call mean ms)."""
        import torch
        if graph:
            if warmup < 1:
                sys.exit("--graph needs at least one warm-up step")
            evs = [self.new_events() for _ in range(warmup)]
            for k in range(warmup):
                self.step(evs[k])
            g = self.st.capture()
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                g.replay()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        else:
            for _ in range(warmup):
                self.step(self.new_events())
            torch.cuda.synchronize()
            evs = [self.new_events() for _ in range(steps)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for k in range(steps):
                self.step(evs[k])
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        per_call = {c: sum(e[c][0].elapsed_time(e[c][1]) for e in evs) / len(evs) for c in self.active}
        return wall, per_call


def main_kernel(call, st):
    """The kernel that does a call's work (as rocprofv3 names it, without its
    namespace) and how many times one call launches it: the slab sequences
    launch theirs once per slab. None for calls outside the default steps."""
    slabs = len(st.slabs) if st.zrange is not None else 1
    table = {"warp_fwd": ("warp_fwd_acc_kernel<true>", slabs) if slabs > 1 else ("warp_fwd_kernel", 1),
             "mi_fwd": ("mi_hist_kernel<3, false>", 1),
             "lncc": (f"lncc_kernel<{st.win // 2}, false>", 1) if st.win and st.win <= 11 else (None, 1),
             "warp_bwd_adam_slab_mi": ("warp_bwd_kernel<true, true, true>", slabs),
             "warp_bwd_adam_mi": ("warp_bwd_adam_pipe_kernel<true>", 1)}
    return table.get(call, (None, 1))


def summarise(timer, wall, per_call, steps, nvox, config_name):
    """Throughput, the step's bytes against the HBM peak, and the dominant
    call's roofline, per launch of its kernel: a slab sequence launches its
    kernel once per slab, and each voxel is stepped in one of those launches,
    so a launch takes the call's time and voxels over the slab count (the same
    rate as the whole call)."""
    ms_step = wall * 1e3 / steps
    step_bpv = sum(call_bytes(c, timer.acc.get(c, False)) for c in timer.active)
    step_gbs = step_bpv * nvox / (ms_step * 1e-3) / 1e9
    dom = max(timer.active, key=lambda c: per_call[c])
    dom_bpv = call_bytes(dom, timer.acc.get(dom, False))
    dom_gbs = dom_bpv * nvox / (per_call[dom] * 1e-3) / 1e9
    kname, launches = main_kernel(dom, timer.st)
    roofline = {"kernel": dom, "bound": "hbm", "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": dom_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(dom, config_name),
                "bytes_per_voxel": dom_bpv, "launches_per_call": launches, "voxels_per_launch": nvox / launches,
                "ms_per_launch": per_call[dom] / launches}
    if kname:
        roofline["kernel_name"] = kname
    if launches > 1 and roofline["traffic"] is not None:
        roofline["traffic"] /= launches
    if dom in ("lncc", "warp_lncc_mi_bwd"):
        tflops = LNCC_FLOPS_PER_VOXEL * nvox / (per_call[dom] * 1e-3) / 1e12
        roofline["fp64"] = {"achieved": tflops, "peak": FP64_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": tflops / FP64_PEAK_TFLOPS, "flops_per_voxel": LNCC_FLOPS_PER_VOXEL}
    # every call of the step against the same HBM roofline (the dominant one
    # above is the contract's; the rest show where each call stands)
    calls = {}
    for c in timer.active:
        bpv = call_bytes(c, timer.acc.get(c, False))
        gbs = bpv * nvox / (per_call[c] * 1e-3) / 1e9
        calls[c] = {"ms": per_call[c], "bytes_per_voxel": bpv, "achieved_gbs": gbs, "frac": gbs / HBM_PEAK_GBS,
                    "traffic": measured_traffic(c, config_name)}
    roofline["per_call"] = calls
    model_gbs = MODEL_STEP_BYTES_NO_ADAM * nvox / (ms_step * 1e-3) / 1e9
    hbm = {"step_bytes_per_voxel": step_bpv, "step_gbs": step_gbs, "frac_of_peak": step_gbs / HBM_PEAK_GBS,
           "model_bytes_per_voxel_without_adam": MODEL_STEP_BYTES_NO_ADAM,
           "model_frac_of_peak": model_gbs / HBM_PEAK_GBS}
    return {"value": nvox * steps / wall, "ms_per_step": ms_step, "per_call_ms": per_call, "hbm": hbm,
            "roofline": roofline, "step": "+".join(timer.active)}


def time_extra_calls(st, case, nvox, wl, reps=5):
    """The calls that are not part of the step, on the same workload and
    timed the same way (events on the stream they run on), after the step:
    the MSE similarity of F against the step's W, the composition of the
    updated displacement field with a second smooth field of that grid, and
    the MI with the box kernel on F (Mattes et al.'s original pair)."""
    import torch

    from non_gemm_voxel_amd import ngv, synth
    s = torch.cuda.current_stream()
    loss = torch.zeros(1, dtype=torch.float64, device=st.W.device)
    V = synth.random_field(wl.shape, wl.seed, 40, 0.02, device=st.W.device)
    w = torch.empty_like(V)
    xf = ngv.make_xform(case.A, case.t)
    runs = {"mse": lambda: ngv.ngv_mse_loss_fwd_bwd(st.F, st.W, loss, st.gW, ws=st.ws),
            "warp_compose": lambda: ngv.ngv_warp_compose(st.u, V, xf, w)}
    if wl.bins:
        runs["mi_box_fixed"] = lambda: ngv.ngv_mi_loss_fwd_bwd_order(st.F, st.W, loss, st.gW, bins=wl.bins,
                                                                     fixed_order=0, ws=st.ws)
    out = {}
    for name, fn in runs.items():
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(s)
            fn()
            b.record(s)
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / reps
        gbs = call_bytes(name, False) * nvox / (ms * 1e-3) / 1e9
        out[name] = {"ms_per_launch": ms, "bytes_per_voxel": call_bytes(name, False), "achieved_gbs": gbs,
                     "peak_gbs": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(name, wl.name)}
    log("extra calls ms: " + ", ".join(f"{k} {v['ms_per_launch']:.3f}" for k, v in out.items()))
    del V, w
    return out


def make_step(wl, case, args):
    from non_gemm_voxel_amd.step import RegistrationStep
    return RegistrationStep(case.F, case.M, case.A, case.t, bins=wl.bins, win=wl.win,
                            smooth_sigma=wl.smooth_sigma, lr=case.lr, slabs=wl.slabs, fused_mi=args.fused_mi,
                            mi_in_backward=not args.no_mi_backward, fused_step=args.fused_step)


def release():
    import gc

    import torch
    gc.collect()
    torch.cuda.empty_cache()


def extra_workload(name, args, dev):
    """Another workload's step at its full size, timed like the headline (10
    steps after 2 warm-up steps), with the calls outside the step on it."""
    import torch

    from non_gemm_voxel_amd import synth
    wl = synth.WORKLOADS[name]
    case = synth.make_case(wl, device=dev)
    torch.cuda.synchronize()
    st = make_step(wl, case, args)
    timer = StepTimer(st, wl)
    wall, per_call = timer.run(10, 2)
    nvox = int(case.F.numel())
    out = summarise(timer, wall, per_call, 10, nvox, wl.name)
    out["workload"] = f"{wl.name}: {wl.note}"
    log(f"{name}: {out['ms_per_step']:.3f} ms/step; per call " +
        ", ".join(f"{c} {v:.3f}" for c, v in per_call.items()))
    # the calls outside the step read the step's W, which the two-sweep step does not store
    out["extra_calls"] = None if st.fused_step else time_extra_calls(st, case, nvox, wl)
    del st, case, timer
    release()
    return out


def loops(args, dev):
    """The iterated workloads as their loops of RegistrationStep.step(): mean
    step time over all iterations (events around the whole loop, from the
    zero state, after a separate 3-step warm-up object), and the loss of the
    second and the last step."""
    import torch

    from non_gemm_voxel_amd import synth
    out = {}
    for name in ("c2", "c3"):
        wl = synth.WORKLOADS[name]
        case = synth.make_case(wl, device=dev)
        warm = make_step(wl, case, args)
        for _ in range(3):
            warm.step()
        del warm
        st = make_step(wl, case, args)
        s = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        losses = []
        a.record(s)
        for t in range(wl.iters):
            st.step()
            if t in (1, wl.iters - 1):
                losses.append(st.loss.clone())
        b.record(s)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / wl.iters
        ls = [float(l[0] if wl.bins else 0.0) + float(l[1] if wl.win else 0.0) for l in losses]
        nvox = int(case.F.numel())
        out[name] = {"workload": f"{wl.name}: {wl.note}", "iterations": wl.iters, "ms_per_step": ms,
                     "voxels_per_s": nvox / (ms * 1e-3), "loss_step_2": ls[0], "loss_last": ls[1]}
        log(f"loop {name}: {wl.iters} steps, {ms:.3f} ms/step, loss {ls[0]:.5f} -> {ls[1]:.5f}")
        del st, case
        release()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU path is not built.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from non_gemm_voxel_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS[args.config]
    log(f"generating {wl.name} {wl.shape} on {dev}")
    t0 = time.perf_counter()
    case = synth.make_case(wl, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    st = make_step(wl, case, args)
    if args.fused_step and not st.fused_step:
        sys.exit(f"--fused-step needs an LNCC term and the moving image in one piece ({wl.name} has "
                 f"win={wl.win}, slabs={wl.slabs})")
    nvox = int(case.F.numel())
    timer = StepTimer(st, wl)
    wall, per_call = timer.run(args.steps, args.warmup, graph=args.graph)
    head = summarise(timer, wall, per_call, args.steps, nvox, wl.name)
    loss = st.loss.cpu().tolist()
    log(f"{head['ms_per_step']:.3f} ms/step; per call " + ", ".join(f"{c} {v:.3f}" for c, v in per_call.items()))

    # host copy of the oracle's sample, then the headline workload's buffers go
    cpu_sample = None
    if not args.no_cpu_baseline:
        planes = args.cpu_planes or max(4, min(wl.shape[0], int(2.4e8 / (wl.shape[1] * wl.shape[2])) + 1))
        cpu_sample = (case.F[:planes].cpu().numpy(), case.M[:planes].cpu().numpy())
    headline_extra_calls = None
    if not args.no_extra and nvox <= 1_000_000_000 and not st.fused_step:
        headline_extra_calls = time_extra_calls(st, case, nvox, wl)
    del st, timer, case.F, case.M
    release()

    if args.copy_gib > 0:
        n = int(args.copy_gib * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n * 4} bytes for counter scaling")
        del src, dst
        release()

    extra = None
    if not args.no_extra:
        extra = {}
        if headline_extra_calls is not None:
            extra["extra_calls"] = headline_extra_calls
        if args.config != "c4":
            extra["c4"] = extra_workload("c4", args, dev)
        extra["loops"] = loops(args, dev)
        if not args.no_cpu_baseline:
            extra["oracle_configs"] = cpu_configs(dev)

    cpu = None
    if cpu_sample is not None:
        log(f"timing the oracle on {cpu_sample[0].shape[0]} planes")
        cpu = cpu_baseline(cpu_sample[0], cpu_sample[1], case, wl)
        log(f"oracle {cpu['value'] / 1e6:.1f} M voxels/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "voxels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.note}", "shape_zyx": list(wl.shape), "voxels": nvox,
                   "mi_bins": wl.bins, "lncc_win": wl.win, "smooth_sigma": wl.smooth_sigma,
                   "moving_slabs": wl.slabs, "step": head["step"], "graph": bool(args.graph)},
        "hbm": head["hbm"],
        "per_call_ms": head["per_call_ms"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "loss": {"mi": loss[0], "lncc": loss[1]},
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
