"""Benchmark: one optimisation step of affine + deformable registration
(warp + MI + LNCC forward and backward + Adam) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c4]

A step is the whole hot path over one synthetic volume pair already resident
in device memory: ngv_warp_fwd_mi (the sampler with the MI forward in its
sweep; ngv_warp_fwd for earlier z-slabs), ngv_mi_grad, ngv_lncc_loss_fwd_bwd
(accumulating into the same gradient), then ngv_warp_bwd_adam (the sampler
backward feeding the Adam update directly; ngv_warp_bwd + ngv_adam_step when
the workload smooths the gradient, and for all but the last z-slab). The
default workload is the 640x768x640 layered-cortex pair with MI (32 bins) and
LNCC (9^3 window), the largest configuration that carries both losses at a
size well beyond the 256 MB Infinity Cache.

Prints one JSON line. `value` is voxels per second of whole steps. `roofline`
describes the dominant call: the LNCC call is bound by fp64 arithmetic and LDS,
so it is given as algorithmic flops per second against the fp64 vector peak
(with its HBM rate alongside); a memory-bound call as algorithmic bytes per
second against 8 TB/s. Durations are timed with events on the stream the
kernels run on. `traffic` is the HBM bytes per launch measured by the counter
passes in profiles/ when they were taken on the current kernel source, else
null. `cpu_baseline` is the oracle on the host cores, timed on a bounded slab
of the same workload.
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
# Calls outside the step, timed on their own after it:
#   mse       F, W read, gW written                                         12
#   warp_compose  v 12 read, the composed field U 12 read once, w 12 written 36
#   mi_box_fixed  as mi (the box kernel on F, cubic on W)                     20
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
CALL_SOURCE = {"warp_fwd": "warp.hip", "mi": "mi.hip", "lncc": "lncc.hip lncc_maps.hpp", "warp_bwd": "warp.hip",
               "adam": "adam.hip", "warp_bwd_adam": "warp.hip", "warp_fwd_mi": "warp.hip", "mi_grad": "mi.hip",
               "mse": "mse.hip", "warp_compose": "warp.hip", "mi_box_fixed": "mi.hip", "mi_fwd": "mi.hip",
               "warp_bwd_adam_mi": "warp.hip"}


def call_bytes(name, accumulate):
    """accumulate: the call adds to gW (mi, lncc, mi_grad), or reads another
    term's gW (warp_bwd_adam_mi)."""
    base = {"warp_fwd": 20, "mi": 20, "lncc": 12, "warp_bwd": 32, "adam": 84, "warp_bwd_adam": 80,
            "warp_fwd_mi": 24, "mi_grad": 12, "mse": 12, "warp_compose": 36, "mi_box_fixed": 20, "mi_fwd": 8,
            "warp_bwd_adam_mi": 80}[name]
    if accumulate and name in ("mi", "lncc", "mi_grad", "warp_bwd_adam_mi"):
        base += 4
    return base


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step recorded once as a HIP graph (per-call times from the eager "
                         "warm-up steps)")
    ap.add_argument("--fused-mi", action="store_true",
                    help="the sampler sweep builds the MI histogram (ngv_warp_fwd_mi + ngv_mi_grad)")
    ap.add_argument("--no-mi-backward", action="store_true",
                    help="the MI call writes its gradient and the backward reads it (ngv_mi_loss_fwd_bwd + "
                         "ngv_warp_bwd_adam) instead of the backward forming it (ngv_warp_bwd_adam_mi)")
    ap.add_argument("--no-extra-calls", action="store_true",
                    help="skip the separate timing of the MSE and warp-composition calls")
    ap.add_argument("--cpu-planes", type=int, default=0, help="planes of the oracle sample (0: auto)")
    ap.add_argument("--copy-gib", type=float, default=0.0,
                    help="after timing, copy a buffer of this many GiB once (a known-size kernel for scaling "
                         "FETCH_SIZE / WRITE_SIZE counter passes)")
    return ap.parse_args()


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


def cpu_baseline(case, wl, planes):
    """The oracle's whole step on planes [0, planes) of the workload, taken as
    a volume of its own (its z-boundary is zero padded like any volume's)."""
    import numpy as np

    from oracle import oracle as orc
    F = np.ascontiguousarray(case.F[:planes].cpu().numpy())
    M = np.ascontiguousarray(case.M[:planes].cpu().numpy())
    shape = F.shape
    u0 = np.zeros((3,) + shape, np.float32)
    prm = orc.pack_prm(case.A, case.t)
    t0 = time.perf_counter()
    W = orc.warp_fwd(M, u0, prm)
    gW = np.zeros_like(W)
    if wl.bins:
        _, g, _ = orc.mi_loss_grad(F, W, bins=wl.bins)
        gW += g
    if wl.win:
        _, g = orc.lncc_loss_grad(F, W, wl.win)
        gW += g
    gu, _, _, _ = orc.warp_bwd(M, u0, prm, gW)
    if wl.smooth_sigma > 0:
        gu = np.stack([orc.gauss_smooth(gu[k], wl.smooth_sigma) for k in range(3)])
    z = np.zeros(gu.size)
    orc.adam(u0, gu, z, z, 1, case.lr)
    dt = time.perf_counter() - t0
    n = int(np.prod(shape))
    return {"value": n / dt, "unit": "voxels/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"whole step on planes 0..{planes - 1} of the workload ({shape[2]}x{shape[1]}x{planes} "
                      f"= {n} voxels, as its own volume), {dt:.1f} s wall"}


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
    print("[bench] extra calls ms: " + ", ".join(f"{k} {v['ms_per_launch']:.3f}" for k, v in out.items()),
          file=sys.stderr, flush=True)
    del V, w
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU path is not built.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from non_gemm_voxel_amd import ngv, synth
    from non_gemm_voxel_amd.step import RegistrationStep

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS[args.config]
    print(f"[bench] generating {wl.name} {wl.shape} on {dev}", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    case = synth.make_case(wl, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    st = RegistrationStep(case.F, case.M, case.A, case.t, bins=wl.bins, win=wl.win,
                          smooth_sigma=wl.smooth_sigma, lr=case.lr, slabs=wl.slabs, fused_mi=args.fused_mi,
                          mi_in_backward=not args.no_mi_backward)
    nvox = int(case.F.numel())

    # one step = the calls below, each bracketed by events on the current stream
    # with fused_mi the sampler sweep also does the MI forward, and the MI call
    # is the gradient sweep alone; with the MI gradient formed in the fused
    # backward the MI call is the forward alone (none after a fused_mi sweep)
    if st.mi_bwd:
        mi_call = None if st.fused_mi else "mi_fwd"
        bwd_calls = ["warp_bwd_adam_mi"]
    else:
        mi_call = "mi_grad" if st.fused_mi else "mi"
        bwd_calls = ["warp_bwd_adam"] if st.fused else ["warp_bwd", "adam"]
    calls = (["warp_fwd_mi"] if st.fused_mi else ["warp_fwd"]) + [mi_call, "lncc"] + bwd_calls
    active = [c for c in calls if c is not None and not (c in ("mi", "mi_grad", "mi_fwd") and not wl.bins) and
              not (c == "lncc" and not wl.win)]
    acc = {"mi": False, "mi_grad": False, "lncc": bool(wl.bins) and not st.mi_bwd,
           "warp_bwd_adam_mi": bool(wl.win)}

    def timed_step(ev):
        s = torch.cuda.current_stream()
        ev[calls[0]][0].record(s)
        st.warp()
        ev[calls[0]][1].record(s)
        if mi_call in active:
            ev[mi_call][0].record(s)
            st.mi()
            ev[mi_call][1].record(s)
        if wl.win:
            ev["lncc"][0].record(s)
            st.lncc()
            ev["lncc"][1].record(s)
        if st.fused:
            ev[bwd_calls[0]][0].record(s)
            st.backward_update()
            ev[bwd_calls[0]][1].record(s)
            return
        ev["warp_bwd"][0].record(s)
        st.backward()
        ev["warp_bwd"][1].record(s)
        ev["adam"][0].record(s)
        st.update()
        ev["adam"][1].record(s)

    def new_events():
        return {c: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for c in active}

    if args.graph:
        # eager warm-up steps give the per-call times; the timed steps are
        # replays of one recorded step (the same kernels, without launches)
        if args.warmup < 1:
            sys.exit("--graph needs at least one warm-up step")
        evs = [new_events() for _ in range(args.warmup)]
        for k in range(args.warmup):
            timed_step(evs[k])
        graph = st.capture()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        for _ in range(args.warmup):
            timed_step(new_events())
        torch.cuda.synchronize()
        evs = [new_events() for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            timed_step(evs[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    per_call = {c: sum(e[c][0].elapsed_time(e[c][1]) for e in evs) / len(evs) for c in active}  # ms
    ms_step = wall * 1e3 / args.steps
    value = nvox * args.steps / wall
    step_bpv = sum(call_bytes(c, acc.get(c, False)) for c in active)
    step_gbs = step_bpv * nvox / (ms_step * 1e-3) / 1e9
    dom = max(active, key=lambda c: per_call[c])
    dom_bytes = call_bytes(dom, acc.get(dom, False)) * nvox
    dom_gbs = dom_bytes / (per_call[dom] * 1e-3) / 1e9
    traffic = measured_traffic(dom, wl.name)
    if dom == "lncc":
        # bound by fp64 arithmetic and LDS, not HBM: flops against the fp64 vector peak
        tflops = LNCC_FLOPS_PER_VOXEL * nvox / (per_call[dom] * 1e-3) / 1e12
        roofline = {"kernel": dom, "bound": "alu", "achieved": tflops, "peak": FP64_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": tflops / FP64_PEAK_TFLOPS, "traffic": traffic,
                    "flops_per_voxel": LNCC_FLOPS_PER_VOXEL, "ms_per_launch": per_call[dom],
                    "hbm_gbs": dom_gbs, "hbm_frac": dom_gbs / HBM_PEAK_GBS}
    else:
        roofline = {"kernel": dom, "bound": "hbm", "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": dom_gbs / HBM_PEAK_GBS, "traffic": traffic,
                    "bytes_per_voxel": call_bytes(dom, acc.get(dom, False)), "ms_per_launch": per_call[dom]}
    loss = st.loss.cpu().tolist()
    print(f"[bench] per-call ms: " + ", ".join(f"{c} {per_call[c]:.3f}" for c in active), file=sys.stderr,
          flush=True)

    # (not at gigavoxel sizes, where the two extra fields would not fit beside the step's)
    extra = None if args.no_extra_calls or nvox > 1_000_000_000 else time_extra_calls(st, case, nvox, wl)

    if args.copy_gib > 0:
        n = int(args.copy_gib * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copied {n * 4} bytes for counter scaling", file=sys.stderr, flush=True)
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        planes = args.cpu_planes or max(4, min(wl.shape[0], int(2.4e8 / (wl.shape[1] * wl.shape[2])) + 1))
        print(f"[bench] timing the oracle on {planes} planes", file=sys.stderr, flush=True)
        cpu = cpu_baseline(case, wl, planes)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "voxels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.note}", "shape_zyx": list(wl.shape), "voxels": nvox,
                   "mi_bins": wl.bins, "lncc_win": wl.win, "smooth_sigma": wl.smooth_sigma,
                   "moving_slabs": wl.slabs, "step": "+".join(active), "graph": bool(args.graph)},
        "hbm": {"step_bytes_per_voxel": step_bpv, "step_gbs": step_gbs, "frac_of_peak": step_gbs / HBM_PEAK_GBS},
        "per_call_ms": per_call,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "loss": {"mi": loss[0], "lncc": loss[1]},
        "extra_calls": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
