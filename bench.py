"""Benchmark of the differentiable N:M mask path on one MI355X.

One step = one pass of the hot path over every linear weight of a 32-layer
LLaMA-2-7B-shaped model (224 tensors, 1.62e9 2:4 blocks, inputs resident in
HBM): the Gumbel soft-mask forward of every tensor (W (.) M~ in bf16, soft
index saved, regulariser reduced) with the hard mask of the same logits
(argmax, bit packing, 2:4 values and 2-bit indices) produced in the same pass,
then the logit backward of every tensor (from the saved soft index).  The
step's outputs equal those of forward, backward and a separate extraction
pass; that unfused order is timed too and reported beside the step.  Prior
seeding, an initialisation step, is timed once after the steps.  Then the
training step with the logit update fused into the backward
(maskgs_bwd_adamw) is timed with the soft index saved and recomputed, and
reported under `train_step` (--no-train-step skips it), and one pass of the
training diagnostics (maskgs_mask_stats) over every tensor under `diagnostics`,
and the step with the hard Gumbel-max sample (straight-through backward) under
`hard_sample_step`, and the step of the linear-space variant (M logits per
block, Gumbel-top-k draw, policy gradient) under `linear_space_step`.  Within
each phase the per-tensor launches alternate between two HIP streams
(--streams), so one tensor's kernel fills the GPU while the previous drains.

Prints ONE JSON line.  `value` = 2:4 weight blocks per second through the whole
step; `roofline` describes the kernel with the largest share of the step;
`cpu_baseline` times the CPU oracle (all host threads) on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(REPO, "profiles", "traffic_counters.json")
KERNEL_SOURCES = ["sparsity_masks_weights_amd/csrc/maskgs_k24.hip",
                  "sparsity_masks_weights_amd/csrc/maskgs_k48.hip",
                  "sparsity_masks_weights_amd/csrc/maskgs_device.hpp"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama7b_all_linear")
    ap.add_argument("--streams", type=int, default=2,
                    help="worker streams the launches of a phase alternate between (1: in order)")
    ap.add_argument("--layers", type=int, default=None,
                    help="use only the first L layers (profiling runs; default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-train-step", action="store_true",
                    help="skip the training step with the fused AdamW update")
    ap.add_argument("--step", choices=("recompute", "saved"), default="recompute",
                    help="recompute: the backward draws the soft index again from z; "
                         "saved: the forward writes it and the backward reads it")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.streams < 1:
        ap.error("--streams must be at least 1")
    return args


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(REPO, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the mask path shards by rows with no "
              "exchange, and this build measures one GPU's share (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparsity_masks_weights_amd as mg
    from workloads import WORKLOADS, tensor_inputs

    L = mg.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    wl = WORKLOADS[args.workload]
    specs = wl.tensors
    if args.layers is not None:
        specs = [t for t in specs if t.tensor_id < 7 * args.layers]
    stream = torch.cuda.current_stream()
    # The launches of one phase alternate between worker streams (two by
    # default, default priority), so that one tensor's kernel fills the CUs
    # while the previous one drains (7B 2:4 step 40.7 -> 39.3 ms, 4:8 layer set
    # 14.7 -> 14.0 ms; four streams gained less); every phase forks from and
    # joins back to the main stream, where the step and phase events are
    # recorded.  --streams 1 runs every launch in order on one stream.
    workers = [torch.cuda.Stream(device=dev) for _ in range(args.streams)]
    wptr = [ctypes.c_void_p(s.cuda_stream) for s in workers]

    def sp(i):
        return wptr[i % len(wptr)]

    def fork():
        e = torch.cuda.Event()
        e.record(stream)
        for s in workers:
            s.wait_event(e)

    def join():
        for s in workers:
            e = torch.cuda.Event()
            e.record(s)
            stream.wait_event(e)

    # ---- resident inputs and outputs --------------------------------------
    bufs = []
    compact = (wl.n, wl.m) == (2, 4)  # values + 2-bit indices exist for 2:4 only
    for spec in specs:
        w, z, G = tensor_inputs(wl, spec, dev)
        B = spec.rows * spec.cols // wl.m
        d = dict(spec=spec, w=w, z=z, G=G,
                 out=torch.empty_like(w), y=torch.empty_like(z), dz=torch.empty_like(z),
                 bits=torch.empty((B * wl.m + 7) // 8, dtype=torch.uint8, device=dev),
                 vals=torch.empty(B * wl.n, dtype=w.dtype, device=dev) if compact else None,
                 vidx=torch.empty((B + 1) // 2, dtype=torch.uint8, device=dev) if compact else None)
        d["desc"] = mg.TensorDesc(wl.n, wl.m, spec.rows, spec.cols, 0, spec.tensor_id)
        d["B"] = B
        bufs.append(d)
    reg = torch.zeros(1, dtype=torch.float64, device=dev)
    total_blocks = sum(d["B"] for d in bufs)
    torch.cuda.synchronize()

    bf = mg.MASKGS_BF16 if wl.w_dtype == "bf16" else mg.MASKGS_F32
    gdt = mg.MASKGS_BF16 if wl.g_dtype == "bf16" else mg.MASKGS_F32
    P = ctypes.c_void_p

    def ptr(t):
        return None if t is None else P(t.data_ptr())

    # pre-marshalled argument tuples: the timed loop only calls the C ABI
    calls = {"fwd": [], "bwd": [], "hard": [], "fwd_hard_noy": [], "bwd_rc": []}
    fused = []
    params = [mg.SampleParams(0, 0, wl.kappa, wl.tau, 0)]
    pref = ctypes.byref(params[0])
    for i, d in enumerate(bufs):
        dref = ctypes.byref(d["desc"])
        calls["fwd"].append((L.maskgs_fwd, (dref, pref, ptr(d["w"]), bf, ptr(d["z"]), ptr(d["out"]),
                                            bf, ptr(d["y"]), ptr(reg), sp(i))))
        calls["bwd"].append((L.maskgs_bwd, (dref, pref, ptr(d["w"]), bf, None, ptr(d["y"]),
                                            ptr(d["G"]), gdt, ctypes.c_float(wl.lam), ptr(d["dz"]), 0,
                                            sp(i))))
        calls["hard"].append((L.maskgs_hard_extract, (dref, ptr(d["z"]), ptr(d["w"]), bf, None,
                                                       ptr(d["bits"]), ptr(d["vals"]),
                                                       ptr(d["vidx"]), sp(i))))
        fused.append((L.maskgs_fwd_hard, (dref, pref, ptr(d["w"]), bf, ptr(d["z"]), ptr(d["out"]),
                                          bf, ptr(d["y"]), ptr(reg), None, ptr(d["bits"]),
                                          ptr(d["vals"]), ptr(d["vidx"]), sp(i))))
        calls["fwd_hard_noy"].append((L.maskgs_fwd_hard, (dref, pref, ptr(d["w"]), bf, ptr(d["z"]),
                                                          ptr(d["out"]), bf, None, ptr(reg), None,
                                                          ptr(d["bits"]), ptr(d["vals"]),
                                                          ptr(d["vidx"]), sp(i))))
        calls["bwd_rc"].append((L.maskgs_bwd, (dref, pref, ptr(d["w"]), bf, ptr(d["z"]), None,
                                               ptr(d["G"]), gdt, ctypes.c_float(wl.lam),
                                               ptr(d["dz"]), 0, sp(i))))

    # per-block algorithmic bytes of each kernel (bf16 weights, fp32 logits)
    K, M, N = wl.k, wl.m, wl.n
    wb = 2 if wl.w_dtype == "bf16" else 4
    hard_out = M / 8 + ((N * wb + 0.5) if compact else 0.0)   # bits (+ values, indices)
    per_block_bytes = {
        "fwd": M * wb + 4 * K + M * 2 + 4 * K,            # W, z in; W.M (bf16), y out
        "fwd_hard": M * wb + 4 * K + M * 2 + 4 * K + hard_out,
        "bwd": M * wb + M * 2 + 4 * K + 4 * K,            # W, G, y in; dz out
        "hard": 4 * K + (M * wb if compact else 0) + hard_out,
        # the soft index not saved: fwd (W, z in; W.M, hard outputs out) and the
        # backward drawing it again (W, G, z in; dz out)
        "fwd_hard_noy": M * wb + 4 * K + M * 2 + hard_out,
        "bwd_rc": M * wb + M * 2 + 4 * K + 4 * K,
    }
    calls["fwd_hard"] = fused
    big = [i for i, d in enumerate(bufs) if d["B"] == max(x["B"] for x in bufs)]
    # per-launch events bracket one launch on a largest tensor per timed step,
    # spread evenly over those tensors (step s times big[(s * stride) % len]):
    # a timed launch runs alone, which costs the step the overlap on both sides
    # of it
    big_stride = max(1, len(big) // max(1, args.steps))
    # The step: the forward of every tensor with the hard mask of the same
    # logits fused in (one read of z and W), then the backward of every tensor.
    # Outputs are bit-identical to forward, backward, then extraction (z is not
    # written by the step); that unfused order is timed after the timed steps.
    fused_kinds = ("fwd_hard_noy", "bwd_rc") if args.step == "recompute" else ("fwd_hard", "bwd")
    unfused_kinds = ("fwd", "bwd", "hard")
    phase = {k: [] for k in calls}
    launch_ev = {k: [] for k in calls}

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def step(kinds, timed_kind=None, step_no=0):
        """One step (number step_no).  Phase events bracket each kernel kind;
        per-launch events bracket one launch of `timed_kind` on a largest
        tensor (the launch shape the roofline reports).  That launch runs
        alone: it goes on the stream of the launch before it, which first
        waits for the other workers' queued work, and they wait for it; so
        its events time the kernel by itself and not its overlap with a
        neighbour, and its start event directly follows a kernel in order."""
        reg.zero_()
        nw = len(workers)
        for kind in kinds:
            p0, p1 = ev(), ev()
            p0.record(stream)
            fork()
            t = big[(step_no * big_stride) % len(big)] if kind == timed_kind else -1
            for i, (fn, a) in enumerate(calls[kind]):
                wi = (t - 1) % nw if i == t else i % nw
                own = workers[wi]
                others = [o for o in workers if o is not own]
                if t >= 0 and i == max(t - 1, 0):
                    for o in others:
                        x = torch.cuda.Event()
                        x.record(o)
                        own.wait_event(x)
                if i == t:
                    a = a[:-1] + (wptr[wi],)     # the stream is the last argument
                    e0, e1 = ev(), ev()
                    e0.record(own)
                rc = fn(*a)
                if rc != 0:
                    raise RuntimeError(f"{kind}: status {rc}")
                if i == t:
                    e1.record(own)
                    for o in others:
                        o.wait_event(e1)
                    launch_ev[kind].append((e0, e1))
            join()
            p1.record(stream)
            phase[kind].append((p0, p1))

    for _ in range(args.warmup):
        step(fused_kinds)
    torch.cuda.synchronize()
    # the dominant kernel (largest share of a step) is chosen from the warmup
    # phases; its launches on the largest tensors are timed in the timed steps
    warm = {k: sum(a.elapsed_time(b) for a, b in v) for k, v in phase.items() if v}
    dom = max(warm, key=warm.get) if args.warmup else fused_kinds[0]
    for v in phase.values():
        v.clear()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for s in range(args.steps):
        params[0].step = s
        step(fused_kinds, dom, s)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # ---- per-kernel statistics (phase events on the main stream) ----------
    def kernel_stats(kinds, nsteps):
        out = {}
        for kind in kinds:
            pairs = phase[kind]
            tot = sum(a.elapsed_time(b) for a, b in pairs) / nsteps
            bytes_per_step = per_block_bytes[kind] * total_blocks
            out[kind] = dict(ms_per_step=round(tot, 4), launches_per_step=len(calls[kind]),
                             algorithmic_bytes_per_block=per_block_bytes[kind],
                             achieved_gbs=round(bytes_per_step / (tot * 1e-3) / 1e9, 1))
        return out

    kstats = kernel_stats(fused_kinds, args.steps)
    big_times = [a.elapsed_time(b) for a, b in launch_ev[dom]]
    big_ms = sum(big_times) / len(big_times)
    big_blocks = bufs[big[0]]["B"]
    big_bytes = per_block_bytes[dom] * big_blocks
    achieved = big_bytes / (big_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        # HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, used
        # only while the kernel sources are the ones the counters were taken on
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f).get("workloads", {}).get(wl.key, {})
        k = tr.get("kernels", {}).get(dom)
        if (k and tr.get("source_hash") == source_hash()
                and tr.get("blocks_per_launch") == bufs[big[0]]["B"]):
            traffic = k.get("hbm_bytes_per_launch")
    spec = bufs[big[0]]["spec"]
    roofline = dict(bound="hbm", kernel=f"maskgs_{dom} ({wl.n}:{wl.m}, {spec.rows}x{spec.cols} "
                    f"{wl.w_dtype} tensor, {big_blocks} blocks)",
                    achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    avg_launch_us=round(big_ms * 1e3, 2), launches_timed=len(big_times),
                    algorithmic_bytes_per_launch=int(big_bytes))

    # ---- the unfused order (forward, backward, extraction), for reference --
    for v in phase.values():
        v.clear()
    u0, u1 = ev(), ev()
    torch.cuda.synchronize()
    u0.record(stream)
    for s in range(args.steps):
        params[0].step = s
        step(unfused_kinds)
    u1.record(stream)
    torch.cuda.synchronize()
    ms_unfused = u0.elapsed_time(u1) / args.steps
    ustats = kernel_stats(unfused_kinds, args.steps)

    # ---- prior seeding, timed once (initialisation row of the path) -------
    pe0 = torch.cuda.Event(enable_timing=True)
    pe1 = torch.cuda.Event(enable_timing=True)
    pe0.record(stream)
    fork()
    for i, d in enumerate(bufs):
        rc = L.maskgs_prior_init(ctypes.byref(d["desc"]), ptr(d["z"]), None, ptr(d["w"]), bf,
                                 ctypes.c_float(3.0), 0, sp(i))
        if rc != 0:
            raise RuntimeError(f"prior_init: status {rc}")
    join()
    pe1.record(stream)
    torch.cuda.synchronize()
    prior_ms = pe0.elapsed_time(pe1)

    # ---- training step with the logit update fused in (AdamW) -------------
    # maskgs_bwd_adamw keeps the logit gradient out of HBM, so the gradient
    # buffers hold the first moments; the second moments are allocated here.
    gb = 2 if wl.g_dtype == "bf16" else 4
    train = {}
    if not args.no_train_step:
        vbufs = [torch.zeros_like(d["z"]) for d in bufs]
        hp = mg.AdamWParams(5e-4, 0.9, 0.999, 1e-8, 0.1, 1)
        hpref = ctypes.byref(hp)
        modes = {
            # bytes per block: fwd_hard (W, z in; out, hard outputs, y out) and
            # bwd_adamw (W, G, y or z in; z, m, v in and out)
            "saved_y": (per_block_bytes["fwd_hard"], M * wb + M * gb + 4 * K + 24 * K),
            "recompute_y": (per_block_bytes["fwd_hard"] - 4 * K, M * wb + M * gb + 24 * K),
        }
        for mode, (fb, bb) in modes.items():
            seq = []
            for i, (d, v) in enumerate(zip(bufs, vbufs)):
                yp = ptr(d["y"]) if mode == "saved_y" else None
                dref = ctypes.byref(d["desc"])
                seq.append(("fwd_hard", L.maskgs_fwd_hard,
                            (dref, pref, ptr(d["w"]), bf, ptr(d["z"]), ptr(d["out"]), bf, yp,
                             ptr(reg), None, ptr(d["bits"]), ptr(d["vals"]), ptr(d["vidx"]),
                             sp(i))))
            for i, (d, v) in enumerate(zip(bufs, vbufs)):
                yp = ptr(d["y"]) if mode == "saved_y" else None
                dref = ctypes.byref(d["desc"])
                seq.append(("bwd_adamw", L.maskgs_bwd_adamw,
                            (dref, pref, ptr(d["w"]), bf, ptr(d["z"]), yp, ptr(d["G"]), gdt,
                             ctypes.c_float(wl.lam), ptr(d["dz"]), ptr(v), hpref, sp(i))))
            ph = {"fwd_hard": [], "bwd_adamw": []}
            t0, t1 = ev(), ev()
            torch.cuda.synchronize()
            t0.record(stream)
            for s_ in range(args.steps):
                params[0].step = s_
                hp.t = s_ + 1
                reg.zero_()
                for kind in ("fwd_hard", "bwd_adamw"):
                    p0, p1 = ev(), ev()
                    p0.record(stream)
                    fork()
                    for k_, fn, a in seq:
                        if k_ == kind:
                            rc = fn(*a)
                            if rc != 0:
                                raise RuntimeError(f"{kind}: status {rc}")
                    join()
                    p1.record(stream)
                    ph[kind].append((p0, p1))
            t1.record(stream)
            torch.cuda.synchronize()
            ms_t = t0.elapsed_time(t1) / args.steps
            ks = {}
            for kind, bpb in (("fwd_hard", fb), ("bwd_adamw", bb)):
                tot = sum(a.elapsed_time(b) for a, b in ph[kind]) / args.steps
                ks[kind] = dict(ms_per_step=round(tot, 4), algorithmic_bytes_per_block=bpb,
                                achieved_gbs=round(bpb * total_blocks / (tot * 1e-3) / 1e9, 1))
            train[mode] = dict(ms_per_step=round(ms_t, 3),
                               value=round(total_blocks / (ms_t * 1e-3), 1), kernels=ks)
        del vbufs

    # ---- training diagnostics, one pass over every tensor -----------------
    # (mask change against the step's hard masks, maximum probability, kept
    # weight norm against magnitude top-n, logit gradient norm)
    st = mg.new_stats(dev)
    stats_bpb = 4 * K + M / 8 + M * wb + 4 * K
    d0, d1 = ev(), ev()
    torch.cuda.synchronize()
    d0.record(stream)
    fork()
    for i, d in enumerate(bufs):
        rc = L.maskgs_mask_stats(ctypes.byref(d["desc"]), ptr(d["z"]), ctypes.c_float(wl.kappa),
                                 None, ptr(d["bits"]), ptr(d["w"]), bf, ptr(d["dz"]), ptr(st),
                                 sp(i))
        if rc != 0:
            raise RuntimeError(f"mask_stats: status {rc}")
    join()
    d1.record(stream)
    torch.cuda.synchronize()
    stats_ms = d0.elapsed_time(d1)
    sv = mg.read_stats(st)
    diagnostics = dict(ms_all_tensors=round(stats_ms, 3), algorithmic_bytes_per_block=stats_bpb,
                       achieved_gbs=round(stats_bpb * total_blocks / (stats_ms * 1e-3) / 1e9, 1),
                       changed_fraction=round(sv["changed"] / max(sv["blocks"], 1), 6),
                       mean_max_prob=round(sv["max_prob"] / max(sv["blocks"], 1), 6),
                       kept_over_magnitude_l1=round(sv["kept_l1"] / sv["magnitude_l1"], 6))

    # ---- hard Gumbel-max sample, straight-through backward ----------------
    # (forward with the hard mask of the same logits, soft index recomputed in
    # the backward, which needs the sample)
    hs_params = mg.SampleParams(0, 0, wl.kappa, wl.tau, mg.MASKGS_HARD_SAMPLE)
    hsref = ctypes.byref(hs_params)
    hs = {"fwd_hard": [], "bwd": []}
    h0, h1 = ev(), ev()
    torch.cuda.synchronize()
    h0.record(stream)
    for s_ in range(args.steps):
        hs_params.step = s_
        reg.zero_()
        for kind in ("fwd_hard", "bwd"):
            p0, p1 = ev(), ev()
            p0.record(stream)
            fork()
            for i, d in enumerate(bufs):
                dref = ctypes.byref(d["desc"])
                if kind == "fwd_hard":
                    rc = L.maskgs_fwd_hard(dref, hsref, ptr(d["w"]), bf, ptr(d["z"]), ptr(d["out"]),
                                           bf, None, ptr(reg), None, ptr(d["bits"]),
                                           ptr(d["vals"]), ptr(d["vidx"]), sp(i))
                else:
                    rc = L.maskgs_bwd(dref, hsref, ptr(d["w"]), bf, ptr(d["z"]), None, ptr(d["G"]),
                                      gdt, ctypes.c_float(wl.lam), ptr(d["dz"]), 0, sp(i))
                if rc != 0:
                    raise RuntimeError(f"hard sample {kind}: status {rc}")
            join()
            p1.record(stream)
            hs[kind].append((p0, p1))
    h1.record(stream)
    torch.cuda.synchronize()
    ms_hs = h0.elapsed_time(h1) / args.steps
    hs_bytes = {"fwd_hard": per_block_bytes["fwd_hard"] - 4 * K,
                "bwd": M * wb + M * gb + 4 * K + 4 * K}
    hard_sample_step = dict(
        what="MASKGS_HARD_SAMPLE: forward applying the Gumbel-max sample (hard mask of the "
             "same logits fused in, soft index not saved), straight-through backward "
             "recomputing the soft index",
        ms_per_step=round(ms_hs, 3), value=round(total_blocks / (ms_hs * 1e-3), 1),
        kernels={k: dict(ms_per_step=round(sum(a.elapsed_time(b) for a, b in v) / args.steps, 4),
                         algorithmic_bytes_per_block=hs_bytes[k],
                         achieved_gbs=round(hs_bytes[k] * total_blocks /
                                            (sum(a.elapsed_time(b) for a, b in v) / args.steps
                                             * 1e-3) / 1e9, 1))
                 for k, v in hs.items()})

    # ---- linear-space variant (maskpro_*): M logits per block ------------
    # A step draws N of M positions per block (masked weights, packed mask,
    # draw order), then forms the policy gradient of every tensor from a
    # scalar advantage (the loss and its baseline come from the model, which is
    # outside the path; a fixed advantage stands in).  The gradient reuses the
    # logit-gradient buffers (K >= M floats per block).
    from workloads import linear_logits
    torch.cuda.empty_cache()
    odt = torch.uint8 if M == 4 else torch.int16
    ob = 1 if M == 4 else 2
    mp_bufs = []
    for d in bufs:
        mp_bufs.append(dict(pi=linear_logits(wl, d["spec"], dev),
                            order=torch.empty(d["B"], dtype=odt, device=dev),
                            dpi=d["dz"].view(-1)[: d["B"] * M]))
    torch.cuda.synchronize()
    dp = mg.DrawParams(0, 0, 0)
    dpref = ctypes.byref(dp)
    adv = ctypes.c_float(0.1)
    mp_bytes = {
        "saved_order": {"fwd": M * wb + 4 * M + 2 * M + M / 8 + ob, "bwd": 4 * M + ob + 4 * M},
        "redrawn": {"fwd": M * wb + 4 * M + 2 * M + M / 8, "bwd": 8 * M},
    }
    linear = {}
    for mode, bpb in mp_bytes.items():
        keep_order = mode == "saved_order"
        ph = {"fwd": [], "bwd": []}
        l0, l1 = ev(), ev()
        for s_ in range(-args.warmup, args.steps):
            if s_ == 0:
                torch.cuda.synchronize()
                l0.record(stream)
            dp.step = s_ % (1 << 32)
            for kind in ("fwd", "bwd"):
                p0, p1 = ev(), ev()
                p0.record(stream)
                fork()
                for i, (d, e) in enumerate(zip(bufs, mp_bufs)):
                    dref = ctypes.byref(d["desc"])
                    op = ptr(e["order"]) if keep_order else None
                    if kind == "fwd":
                        rc = L.maskpro_fwd(dref, dpref, ptr(d["w"]), bf, ptr(e["pi"]),
                                           ptr(d["out"]), bf, ptr(d["bits"]), op, sp(i))
                    else:
                        rc = L.maskpro_bwd(dref, dpref, ptr(e["pi"]), op, adv, ptr(e["dpi"]), 0,
                                           sp(i))
                    if rc != 0:
                        raise RuntimeError(f"maskpro {kind}: status {rc}")
                join()
                p1.record(stream)
                if s_ >= 0:
                    ph[kind].append((p0, p1))
        l1.record(stream)
        torch.cuda.synchronize()
        ms_l = l0.elapsed_time(l1) / args.steps
        ks = {}
        for kind, v in ph.items():
            tot = sum(a.elapsed_time(b) for a, b in v) / args.steps
            ks[kind] = dict(ms_per_step=round(tot, 4), algorithmic_bytes_per_block=bpb[kind],
                            achieved_gbs=round(bpb[kind] * total_blocks / (tot * 1e-3) / 1e9, 1))
        linear[mode] = dict(ms_per_step=round(ms_l, 3),
                            value=round(total_blocks / (ms_l * 1e-3), 1), kernels=ks)
    linear_step = dict(
        what="maskpro_fwd (Gumbel-top-k draw of N of M positions on M fp32 logits per block; "
             "masked weights, packed mask, draw order) then maskpro_bwd (policy gradient "
             "A*dlogp of the ordered draw, A = 0.1), every tensor; saved_order reads the "
             "forward's draw order, redrawn draws again in the backward",
        logits=f"fp32 N(0,1), {M} per block", **linear)
    if not args.no_cpu_baseline:
        linear_step["cpu_baseline"] = cpu_baseline_linear(wl, bufs, mp_bufs)
    del mp_bufs

    if args.calibrate_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # the method's own bytes per block: what a forward (W, z in; W.M out) and a
    # backward (W, z, G in; dz out) must move, plus the hard-mask outputs,
    # whatever the kernels save in between (a saved soft index is not counted)
    method_bpb = (M * wb + 4 * K + M * 2) + (M * wb + 4 * K + M * gb + 4 * K) + hard_out
    fwd_bwd_ms = ustats["fwd"]["ms_per_step"] + ustats["bwd"]["ms_per_step"]
    fb_bytes = per_block_bytes["fwd"] + per_block_bytes["bwd"]
    step_bytes = sum(per_block_bytes[k] for k in fused_kinds) * total_blocks
    result = {
        "metric": (f"weight-blocks/s and HBM GB/s (% of peak), {wl.n}:{wl.m} mask fwd+bwd, "
                   f"{'LLaMA-2-7B' if wl.key.startswith('llama') else 'Nemotron-4-15B'} shapes"),
        "value": round(total_blocks / (ms_step * 1e-3), 1),
        "unit": "weight-blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.key, "tensors": len(bufs), "blocks": total_blocks,
                   "n_m": f"{wl.n}:{wl.m}", "weights": f"{wl.w_dtype} N(0,{wl.w_std})",
                   "logits": f"fp32 N(0,{wl.z_std})", "upstream_grad": f"{wl.g_dtype} N(0,{wl.g_std})",
                   "kappa": wl.kappa, "tau": wl.tau, "lambda": wl.lam,
                   "step": ("fwd (reg) with the hard mask of the same logits fused in (argmax, "
                            "bit-pack, 2:4 compaction) + bwd drawing the soft index again from z"
                            if args.step == "recompute" else
                            "fwd (y saved, reg) with the hard mask of the same logits fused in "
                            "(argmax, bit-pack, 2:4 compaction) + bwd (saved y)"),
                   "streams": args.streams, "parallelism": "single GPU"},
        # the whole timed step as one memory stream: its algorithmic bytes (every
        # kernel of the step, every tensor) over the step time
        "step_hbm_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        # the same step counted on the method's own bytes (method_bytes_per_block)
        "method_bytes_per_block": method_bpb,
        "method_hbm_gbs": round(method_bpb * total_blocks / (ms_step * 1e-3) / 1e9, 1),
        "method_hbm_frac": round(method_bpb * total_blocks / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                 4),
        "fwd_bwd_blocks_per_s": round(total_blocks / (fwd_bwd_ms * 1e-3), 1),  # unfused fwd + bwd
        "fwd_bwd_hbm_gbs": round(fb_bytes * total_blocks / (fwd_bwd_ms * 1e-3) / 1e9, 1),
        "kernels": kstats,
        "unfused_step": {"order": "fwd, bwd, then hard extract (separate pass over z and W)",
                         "ms_per_step": round(ms_unfused, 3),
                         "value": round(total_blocks / (ms_unfused * 1e-3), 1),
                         "kernels": ustats},
        "prior_init": {"ms_all_tensors": round(prior_ms, 3),
                       "achieved_gbs": round((M * wb + 8 * K) * total_blocks / (prior_ms * 1e-3) / 1e9,
                                             1)},
        "roofline": roofline,
    }
    result["diagnostics"] = diagnostics
    result["hard_sample_step"] = hard_sample_step
    result["linear_space_step"] = linear_step
    if train:
        result["train_step"] = {
            "what": "fwd with the hard mask fused in, then maskgs_bwd_adamw (backward fused with "
                    "the AdamW update of the logits: lr 5e-4, betas 0.9/0.999, eps 1e-8, "
                    "weight decay 0.1); the logit gradient never reaches HBM",
            **train}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, bufs, mg)
    print(json.dumps(result), flush=True)


def host_cpu():
    """The host the CPU baseline ran on: logical CPUs, the CPUs this process
    may use, and the CPU model from /proc/cpuinfo."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def oracle_threads():
    """OpenMP threads for the oracle: OMP_NUM_THREADS if set, else every CPU
    this process may use."""
    env = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return env or host_cpu()["usable_cpus"] or 1


def cpu_baseline(wl, bufs, mg, min_secs=10.0):
    """The CPU oracle (all host threads) on whole layers of the workload, in
    order, until at least `min_secs` of CPU work: fwd + bwd + hard extract."""
    import numpy as np
    import torch
    import oracle

    oracle.set_threads(oracle_threads())
    used = oracle.get_threads()
    blocks = 0
    secs = 0.0
    layers = 0
    tensors = 0
    nlayers = 1 + max(d["spec"].tensor_id for d in bufs) // 7
    while layers < nlayers and (layers == 0 or secs < min_secs):
        for d in bufs:
            spec = d["spec"]
            if spec.tensor_id // 7 != layers:
                continue
            wu = d["w"].view(torch.int16).cpu().numpy().view(np.uint16)
            wf = oracle.widen_bf16(wu).reshape(spec.rows, spec.cols)
            zf = d["z"].cpu().numpy()
            gf = oracle.widen_bf16(d["G"].view(torch.int16).cpu().numpy().view(np.uint16))
            gf = gf.reshape(spec.rows, spec.cols)
            kw = dict(kappa=wl.kappa, tau=wl.tau, seed=0, step=0, tensor_id=spec.tensor_id)
            t = time.perf_counter()
            oracle.fwd(wl.n, wl.m, wf, zf, **kw)
            oracle.bwd(wl.n, wl.m, wf, zf, gf, lam=wl.lam, **kw)
            oracle.hard_extract(wl.n, wl.m, zf, spec.rows, spec.cols,
                                w_raw=wu if (wl.n, wl.m) == (2, 4) else None)
            secs += time.perf_counter() - t
            blocks += d["B"]
            tensors += 1
            del wu, wf, zf, gf
        layers += 1
    return {"value": round(blocks / secs, 1), "unit": "weight-blocks/s", "cores": used,
            "kind": "oracle", "host": host_cpu(),
            "sample": f"first {layers} layer(s) of the same workload ({tensors} tensors, "
                      f"{blocks} blocks): fwd + bwd + hard extract, {secs:.1f} s of CPU time"}


def cpu_baseline_linear(wl, bufs, mp_bufs, min_secs=8.0):
    """The CPU oracle of the linear-space variant (all host threads) on whole
    tensors of the workload, in order, until at least `min_secs` of CPU work:
    draw + masked weights, then the policy gradient of the saved draw order."""
    import numpy as np
    import torch
    import oracle

    oracle.set_threads(oracle_threads())
    used = oracle.get_threads()

    blocks = 0
    secs = 0.0
    tensors = 0
    for d, e in zip(bufs, mp_bufs):
        if tensors and secs >= min_secs:
            break
        spec = d["spec"]
        if d["w"].dtype == torch.bfloat16:
            wf = oracle.widen_bf16(d["w"].view(torch.int16).cpu().numpy().view(np.uint16))
        else:
            wf = d["w"].cpu().numpy()
        wf = wf.reshape(spec.rows, spec.cols)
        pf = e["pi"].cpu().numpy()
        kw = dict(seed=0, step=0, tensor_id=spec.tensor_id)
        t = time.perf_counter()
        f = oracle.maskpro_fwd(wl.n, wl.m, wf, pf, **kw)
        oracle.maskpro_grad(wl.n, wl.m, pf, spec.rows, spec.cols, advantage=0.1,
                            order=f["order"])
        secs += time.perf_counter() - t
        blocks += d["B"]
        tensors += 1
        del wf, pf, f
    return {"value": round(blocks / secs, 1), "unit": "weight-blocks/s", "cores": used,
            "kind": "oracle", "host": host_cpu(),
            "sample": f"first {tensors} tensor(s) of the same workload ({blocks} blocks): draw + "
                      f"masked weights + policy gradient, {secs:.1f} s of CPU time"}


if __name__ == "__main__":
    main()
