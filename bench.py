"""Benchmark of the differentiable N:M mask path on one MI355X.

One step = one pass of the hot path over every linear weight of a 32-layer
LLaMA-2-7B-shaped model (224 tensors, 1.62e9 2:4 blocks, inputs resident in
HBM): the Gumbel soft-mask forward of every tensor (W (.) M~ in bf16,
regulariser reduced) with the hard mask of the same logits (argmax, bit
packing, 2:4 values and 2-bit indices) produced in the same pass, then the
logit backward of every tensor.  By default (--step recompute) the forward
saves nothing and the backward draws the soft index again from z, the faster
design for both patterns on this chip; --step saved has the forward write the
soft index and the backward read it.  The other design is timed too
(`other_step`), and so is the unfused order (forward, backward, separate
extraction).  Prior seeding, an initialisation step, is
timed once after the steps.  Then the training step with the logit update
fused into the backward (maskgs_bwd_adamw) is timed with the soft index saved
and recomputed (`train_step`, --no-train-step skips it), one pass of the
training diagnostics (`diagnostics`), the step with the hard Gumbel-max sample
(`hard_sample_step`) and the step of the linear-space variant
(`linear_space_step`).  Within each phase the per-tensor launches alternate
between two HIP streams (--streams), so one tensor's kernel fills the GPU
while the previous drains.

After the headline workload its buffers are freed and three more workloads
are measured the same way, under `sub_results` (--no-sub skips them): the
LLaMA-2-7B q_proj with logits seeded by the magnitude prior (its buffers held
in three copies that the steps rotate through, over 1 GB of step traffic, so
the last-level cache cannot serve repeats), the MLP trio over the 8-step
tau/kappa anneal, and the Nemotron-4-15B-shaped 4:8 layer set.

Prints ONE JSON line.  `value` = weight blocks per second through the whole
step; `roofline` describes the kernel with the largest share of the step;
`cpu_baseline` times the CPU oracle (all host threads) on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import gc
import hashlib
import json
import os
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

HBM_PEAK_GBS = 8000.0
# VALU issue peak of MI355X in wave64 instructions per microsecond: 256 CUs x
# 4 SIMDs at 2.4 GHz, one instruction per SIMD every 2 cycles when two issue
# together (fp32 arithmetic and simple integer instructions whose operands
# are VGPRs or constants), every 4 cycles otherwise (64-bit multiplies,
# conversions, fp64, instructions reading an SGPR).
VALU_PEAK_DUAL = 256 * 4 * 2400 / 2
VALU_PEAK_SINGLE = 256 * 4 * 2400 / 4
TRAFFIC_FILE = os.path.join(REPO, "profiles", "traffic_counters.json")
VALU_FILE = os.path.join(REPO, "profiles", "valu_counters.json")
KERNEL_SOURCES = ["sparsity_masks_weights_amd/csrc/maskgs_k24.hip",
                  "sparsity_masks_weights_amd/csrc/maskgs_k48.hip",
                  "sparsity_masks_weights_amd/csrc/maskgs_device.hpp",
                  "sparsity_masks_weights_amd/csrc/maskgs_gumbel_table.inc"]

# kernel kinds a --profile run can launch (the two hs_ kinds: the step's
# kernels under the hard Gumbel-max sample)
PROFILE_KINDS = ("fwd", "fwd_hard", "fwd_hard_noy", "bwd", "bwd_rc", "hard", "hs_fwd_hard_noy",
                 "hs_bwd_rc")

# what each kernel kind is, in entry-point terms
KIND_DESC = {
    "fwd": "maskgs_fwd (soft index saved)",
    "fwd_hard": "maskgs_fwd_hard (soft index saved)",
    "fwd_hard_noy": "maskgs_fwd_hard (soft index not saved)",
    "bwd": "maskgs_bwd (saved soft index)",
    "bwd_rc": "maskgs_bwd (soft index drawn again from z)",
    "hard": "maskgs_hard_extract",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama7b_all_linear")
    ap.add_argument("--step", choices=("recompute", "saved"), default="recompute",
                    help="recompute: the backward draws the soft index again from z; saved: the "
                         "forward writes it and the backward reads it")
    ap.add_argument("--streams", type=int, default=2,
                    help="worker streams the launches of a phase alternate between (1: in order)")
    ap.add_argument("--layers", type=int, default=None,
                    help="use only the first L layers (profiling runs; default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-train-step", action="store_true",
                    help="skip the training step with the fused AdamW update")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the step and the other step design only")
    ap.add_argument("--no-sub", action="store_true",
                    help="skip the q_proj, MLP-anneal and 4:8 sub-results")
    ap.add_argument("--profile", default=None, metavar="KINDS",
                    help="counter runs: launch each listed kernel kind (comma-separated: "
                         + ", ".join(PROFILE_KINDS) + ") 3 times on the workload's largest "
                         "tensor, in order, print their launch times and exit")
    args = ap.parse_args()
    if args.streams < 1:
        ap.error("--streams must be at least 1")
    if args.steps < 1:
        ap.error("--steps must be at least 1")
    return args


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(REPO, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def step_mode(args, wl) -> str:
    return args.step


def step_kinds(mode):
    return ("fwd_hard_noy", "bwd_rc") if mode == "recompute" else ("fwd_hard", "bwd")


def describe_step(mode):
    if mode == "recompute":
        return ("fwd (reg) with the hard mask of the same logits fused in (argmax, bit-pack, 2:4 "
                "compaction) + bwd drawing the soft index again from z")
    return ("fwd (y saved, reg) with the hard mask of the same logits fused in (argmax, bit-pack, "
            "2:4 compaction) + bwd (saved y)")


class Session:
    """Resident buffers of one workload (in `copies` copies that the steps
    rotate through) and the launch machinery: worker streams, phase events and
    per-launch events."""

    def __init__(self, mg, wl, specs, args, dev, copies=1, with_y=True):
        import torch
        from workloads import tensor_inputs
        self.torch, self.mg, self.wl, self.args, self.dev = torch, mg, wl, args, dev
        self.L = mg.load_library()
        self.stream = torch.cuda.current_stream()
        self.sptr = ctypes.c_void_p(self.stream.cuda_stream)
        # The launches of one phase alternate between worker streams (default
        # priority), so that one tensor's kernel fills the CUs while the
        # previous one drains; every phase forks from and joins back to the
        # main stream, where the step and phase events are recorded.
        self.workers = [torch.cuda.Stream(device=dev) for _ in range(args.streams)]
        self.wptr = [ctypes.c_void_p(s.cuda_stream) for s in self.workers]
        compact = (wl.n, wl.m) == (2, 4)  # values + 2-bit indices exist for 2:4 only
        self.bufs = []
        for c in range(copies):
            for spec in specs:
                w, z, G = tensor_inputs(wl, spec, dev)
                B = spec.rows * spec.cols // wl.m
                d = dict(spec=spec, w=w, z=z, G=G, B=B,
                         out=torch.empty_like(w), dz=torch.empty_like(z),
                         y=torch.empty_like(z) if with_y else None,
                         bits=torch.empty((B * wl.m + 7) // 8, dtype=torch.uint8, device=dev),
                         vals=torch.empty(B * wl.n, dtype=w.dtype, device=dev) if compact else None,
                         vidx=(torch.empty((B + 1) // 2, dtype=torch.uint8, device=dev)
                               if compact else None))
                d["desc"] = mg.TensorDesc(wl.n, wl.m, spec.rows, spec.cols, 0, spec.tensor_id)
                self.bufs.append(d)
        self.copies = copies
        self.per_copy = len(specs)
        self.reg = torch.zeros(1, dtype=torch.float64, device=dev)
        self.blocks = sum(d["B"] for d in self.bufs[:self.per_copy])
        torch.cuda.synchronize()
        self.params = mg.SampleParams(0, 0, wl.kappa, wl.tau, 0)
        self.pref = ctypes.byref(self.params)
        self.bf = mg.MASKGS_BF16 if wl.w_dtype == "bf16" else mg.MASKGS_F32
        self.gdt = mg.MASKGS_BF16 if wl.g_dtype == "bf16" else mg.MASKGS_F32
        K, M, N = wl.k, wl.m, wl.n
        self.wb = wb = 2 if wl.w_dtype == "bf16" else 4
        self.gb = gb = 2 if wl.g_dtype == "bf16" else 4
        ho = M / 8 + ((N * wb + 0.5) if compact else 0.0)   # bits (+ values, indices)
        self.hard_out = ho
        # algorithmic bytes per block of each kernel kind
        self.bpb = {
            "fwd": M * wb + 4 * K + M * 2 + 4 * K,               # W, z in; W.M (bf16), y out
            "fwd_hard": M * wb + 4 * K + M * 2 + 4 * K + ho,     # ... + hard-mask outputs
            "fwd_hard_noy": M * wb + 4 * K + M * 2 + ho,         # soft index not saved
            "bwd": M * wb + M * gb + 4 * K + 4 * K,              # W, G, y in; dz out
            "bwd_rc": M * wb + M * gb + 4 * K + 4 * K,           # W, G, z in; dz out
            "hard": 4 * K + (M * wb if compact else 0) + ho,     # z (, W) in; hard outputs
        }
        # the method's own bytes per block: what a forward (W, z in; W.M out)
        # and a backward (W, z, G in; dz out) must move, plus the hard-mask
        # outputs, whatever a design saves in between
        self.method_bpb = (M * wb + 4 * K + M * 2) + (M * wb + 4 * K + M * gb + 4 * K) + ho
        self.phase = {}
        self.launch_ev = {}
        big = max(d["B"] for d in self.bufs)
        self.big = [i for i, d in enumerate(self.bufs) if d["B"] == big]

    # -- launches -----------------------------------------------------------
    @staticmethod
    def ptr(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    def call(self, kind, d, stream, pref=None):
        L, p, bf, gdt = self.L, self.ptr, self.bf, self.gdt
        pref = self.pref if pref is None else pref
        dref = ctypes.byref(d["desc"])
        lam = ctypes.c_float(self.wl.lam)
        if kind == "fwd":
            rc = L.maskgs_fwd(dref, pref, p(d["w"]), bf, p(d["z"]), p(d["out"]), bf, p(d["y"]),
                              p(self.reg), stream)
        elif kind in ("fwd_hard", "fwd_hard_noy"):
            y = p(d["y"]) if kind == "fwd_hard" else None
            rc = L.maskgs_fwd_hard(dref, pref, p(d["w"]), bf, p(d["z"]), p(d["out"]), bf, y,
                                   p(self.reg), None, p(d["bits"]), p(d["vals"]), p(d["vidx"]),
                                   stream)
        elif kind == "bwd":
            rc = L.maskgs_bwd(dref, pref, p(d["w"]), bf, None, p(d["y"]), p(d["G"]), gdt, lam,
                              p(d["dz"]), 0, stream)
        elif kind == "bwd_rc":
            rc = L.maskgs_bwd(dref, pref, p(d["w"]), bf, p(d["z"]), None, p(d["G"]), gdt, lam,
                              p(d["dz"]), 0, stream)
        elif kind == "hard":
            rc = L.maskgs_hard_extract(dref, p(d["z"]), p(d["w"]), bf, None, p(d["bits"]),
                                       p(d["vals"]), p(d["vidx"]), stream)
        else:
            raise ValueError(kind)
        if rc != 0:
            raise RuntimeError(f"{kind}: status {rc}")

    def fork(self):
        e = self.torch.cuda.Event()
        e.record(self.stream)
        for s in self.workers:
            s.wait_event(e)

    def join(self):
        for s in self.workers:
            e = self.torch.cuda.Event()
            e.record(s)
            self.stream.wait_event(e)

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def run_phase(self, kind, tensors, timed=-1, pref=None, record=True, fn=None,
                  phase_events=True):
        """Launches `kind` (or fn(buffers, stream, index)) on every tensor
        index in `tensors`, alternating between the worker streams, between
        phase events on the main stream.  Launch number `timed` (on a largest
        tensor) runs alone: it goes on the stream of the launch before it,
        which first waits for the other workers' queued work, and they wait
        for it; so its events time the kernel by itself and not its overlap
        with a neighbour, and its start event directly follows a kernel in
        order.  Without phase_events (or record) the phase records no timing
        events of its own."""
        nw = len(self.workers)
        phase_events = phase_events and record
        p0, p1 = self.ev(), self.ev()
        if phase_events:
            p0.record(self.stream)
        if len(tensors) == 1:
            # one launch: nothing to overlap, so it runs on the main stream
            i = tensors[0]
            if timed == 0:
                e0, e1 = self.ev(), self.ev()
                e0.record(self.stream)
            if fn is None:
                self.call(kind, self.bufs[i], self.sptr, pref)
            else:
                fn(self.bufs[i], self.sptr, i)
            if timed == 0:
                e1.record(self.stream)
                self.launch_ev.setdefault(kind, []).append((e0, e1))
            if phase_events:
                p1.record(self.stream)
                self.phase.setdefault(kind, []).append((p0, p1))
            return
        self.fork()
        for n, i in enumerate(tensors):
            wi = (timed - 1) % nw if n == timed else n % nw
            own = self.workers[wi]
            others = [o for o in self.workers if o is not own]
            if timed >= 0 and n == max(timed - 1, 0):
                for o in others:
                    x = self.torch.cuda.Event()
                    x.record(o)
                    own.wait_event(x)
            if n == timed:
                e0, e1 = self.ev(), self.ev()
                e0.record(own)
            if fn is None:
                self.call(kind, self.bufs[i], self.wptr[wi], pref)
            else:
                fn(self.bufs[i], self.wptr[wi], i)
            if n == timed:
                e1.record(own)
                for o in others:
                    o.wait_event(e1)
                self.launch_ev.setdefault(kind, []).append((e0, e1))
        self.join()
        if phase_events:
            p1.record(self.stream)
            self.phase.setdefault(kind, []).append((p0, p1))

    def timed_steps(self, kinds, nsteps, warmup, timed_kind=None, schedule=None,
                    phase_events=True):
        """`warmup` untimed then `nsteps` timed steps of `kinds`; returns ms
        per timed step.  Copy c of the buffers serves steps c, c + copies, ...
        schedule(s) sets the sampling parameters of step s (default: the
        step number only).  Per-launch events bracket one launch of
        `timed_kind` on a largest tensor per timed step, spread evenly over
        those tensors; a timed launch runs alone, which costs the step the
        overlap on both sides of it.  phase_events: time every phase too
        (each timing event costs the stream a few microseconds)."""
        torch = self.torch

        def one(s, timed_launch):
            self.reg.zero_()
            if schedule is not None:
                schedule(s)
            else:
                self.params.step = s
            base = (s % self.copies) * self.per_copy
            tensors = list(range(base, base + self.per_copy))
            bigs = [n for n, i in enumerate(tensors) if i in self.big]
            for kind in kinds:
                t = -1
                if kind == timed_kind and timed_launch and bigs:
                    stride = max(1, len(bigs) // nsteps)
                    t = bigs[(s * stride) % len(bigs)]
                self.run_phase(kind, tensors, t, record=timed_launch,
                               phase_events=phase_events)

        for s in range(warmup):
            one(s, False)
        torch.cuda.synchronize()
        for v in self.phase.values():
            v.clear()
        self.launch_ev.clear()
        t0, t1 = self.ev(), self.ev()
        t0.record(self.stream)
        for s in range(nsteps):
            one(s, True)
        t1.record(self.stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / nsteps

    def measure(self, kinds, nsteps, timed_kind=None, schedule=None, warmup=0,
                breakdown_steps=3):
        """The timed steps without per-phase events (ms per step, and the
        roofline of `timed_kind` from its per-launch events), then
        `breakdown_steps` further steps with phase events for the per-kernel
        breakdown: each timing event costs the stream a few microseconds,
        a fifth of a single-tensor step's time."""
        ms = self.timed_steps(kinds, nsteps, warmup, timed_kind=timed_kind, schedule=schedule,
                              phase_events=False)
        roof = self.roofline(timed_kind) if timed_kind else None
        nb = max(1, min(nsteps, breakdown_steps))
        self.timed_steps(kinds, nb, 0, schedule=schedule)
        return ms, self.kernel_stats(kinds, nb), roof

    def phase_ms(self, kind, nsteps):
        return sum(a.elapsed_time(b) for a, b in self.phase.get(kind, [])) / nsteps

    def kernel_stats(self, kinds, nsteps):
        out = {}
        for kind in kinds:
            tot = self.phase_ms(kind, nsteps)
            out[kind] = dict(what=KIND_DESC[kind], ms_per_step=round(tot, 4),
                             launches_per_step=self.per_copy,
                             algorithmic_bytes_per_block=self.bpb[kind],
                             achieved_gbs=round(self.bpb[kind] * self.blocks / (tot * 1e-3) / 1e9,
                                                1))
        return out

    def dominant(self, kinds):
        """The kind with the largest share of a step, by its phase time."""
        return max(kinds, key=lambda k: self.phase_ms(k, 1))

    def roofline(self, kind):
        times = [a.elapsed_time(b) for a, b in self.launch_ev.get(kind, [])]
        ms = sum(times) / len(times)
        d = self.bufs[self.big[0]]
        nbytes = self.bpb[kind] * d["B"]
        achieved = nbytes / (ms * 1e-3) / 1e9
        spec, wl = d["spec"], self.wl
        roof = dict(bound="hbm", kernel=f"{KIND_DESC[kind]} ({wl.n}:{wl.m}, {spec.rows}x{spec.cols} "
                    f"{wl.w_dtype} tensor, {d['B']} blocks)",
                    achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=recorded(TRAFFIC_FILE, wl.key, kind, d["B"], "hbm_bytes_per_launch"),
                    avg_launch_us=round(ms * 1e3, 2), launches_timed=len(times),
                    algorithmic_bytes_per_launch=int(nbytes))
        insts = recorded(VALU_FILE, wl.key, kind, d["B"], "valu_insts_per_launch")
        if insts:
            # the VALU side of the same launch: its wave-level VALU instruction
            # count (rocprofv3 SQ_INSTS_VALU) over the launch time measured here
            pairs = recorded(VALU_FILE, wl.key, kind, d["B"], "valu_dual_issued_per_launch") or 0
            trans = recorded(VALU_FILE, wl.key, kind, d["B"], "valu_trans_per_launch") or 0
            rate = insts / (ms * 1e3)
            # SIMD issue time the instructions need: 2 cycles per dual-issued
            # instruction, 8 per fp32 transcendental, 4 per other one, over the
            # launch's SIMD cycles
            need = (2 * pairs + 8 * trans + 4 * (insts - pairs - trans)) / (256 * 4 * 2.4e9)
            roof["valu"] = dict(achieved=round(rate, 1), peak=VALU_PEAK_DUAL,
                                single_issue_peak=VALU_PEAK_SINGLE,
                                unit="wave instructions/us", frac=round(rate / VALU_PEAK_DUAL, 4),
                                dual_issued_frac=round(pairs / insts, 4),
                                issue_time_frac=round(need / (ms * 1e-3), 4),
                                insts_per_launch=int(insts), trans_insts_per_launch=int(trans))
        return roof


def recorded(path, workload, kind, blocks, field):
    """A per-launch counter value recorded (rocprofv3) for `kind` on a tensor
    of `blocks` blocks: the workload's own record, else another workload's
    record of the same N:M pattern and tensor size (the same kernel over the
    same bytes); used only while the kernel sources hash to the value it was
    recorded on."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        recs = json.load(f).get("workloads", {})
    from workloads import WORKLOADS
    nm = f"{WORKLOADS[workload].n}:{WORKLOADS[workload].m}"
    order = [workload] + [w for w in recs if w != workload]
    for w in order:
        tr = recs.get(w, {})
        if w != workload and tr.get("n_m") != nm:
            continue
        k = tr.get("kernels", {}).get(kind)
        if k and tr.get("source_hash") == source_hash() and tr.get("blocks_per_launch") == blocks:
            return k.get(field)
    return None


def metric_for(wl):
    return (f"weight-blocks/s and HBM GB/s (% of peak), {wl.n}:{wl.m} mask fwd+bwd, "
            f"{'LLaMA-2-7B' if wl.key.startswith('llama') else 'Nemotron-4-15B'} shapes")


def line(sess, ms_step, kinds, nsteps, args, mode, extra_config=None):
    """The fields of a bench line for `sess`'s workload."""
    wl = sess.wl
    step_bytes = sum(sess.bpb[k] for k in kinds) * sess.blocks
    cfg = {"workload": wl.key, "tensors": sess.per_copy, "blocks": sess.blocks,
           "n_m": f"{wl.n}:{wl.m}", "weights": f"{wl.w_dtype} N(0,{wl.w_std})",
           "logits": f"fp32 N(0,{wl.z_std})", "upstream_grad": f"{wl.g_dtype} N(0,{wl.g_std})",
           "kappa": wl.kappa, "tau": wl.tau, "lambda": wl.lam,
           "step": describe_step(mode), "step_mode": mode,
           "streams": args.streams, "parallelism": "single GPU"}
    cfg.update(extra_config or {})
    gbs = lambda nbytes: nbytes / (ms_step * 1e-3) / 1e9  # noqa: E731
    return {
        "metric": metric_for(wl),
        "value": round(sess.blocks / (ms_step * 1e-3), 1),
        "unit": "weight-blocks/s",
        "n_gpus": 1,
        "steps": nsteps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": cfg,
        # the whole timed step as one memory stream: the algorithmic bytes of
        # every kernel of the step over the step time
        "step_hbm_gbs": round(gbs(step_bytes), 1),
        "step_hbm_frac": round(gbs(step_bytes) / HBM_PEAK_GBS, 4),
        # the same step counted on the method's own bytes per block
        "method_bytes_per_block": sess.method_bpb,
        "method_hbm_gbs": round(gbs(sess.method_bpb * sess.blocks), 1),
        "method_hbm_frac": round(gbs(sess.method_bpb * sess.blocks) / HBM_PEAK_GBS, 4),
    }


# ---------------------------------------------------------------------------
# One workload's step (the headline; the 4:8 layer set as a sub-result).
# ---------------------------------------------------------------------------
def run_main(mg, wl, specs, args, dev, extras=True, cpu_secs=10.0):
    mode = step_mode(args, wl)
    kinds = step_kinds(mode)
    sess = Session(mg, wl, specs, args, dev, with_y=True)
    # the dominant kernel is chosen from one step after the warm-up steps (the
    # first launches of a kernel run slower), then one of its launches on a
    # largest tensor is timed alone in each timed step
    sess.timed_steps(kinds, 1, max(1, args.warmup))
    dom = sess.dominant(kinds)
    ms_step, kern, roof = sess.measure(kinds, args.steps, timed_kind=dom)
    result = line(sess, ms_step, kinds, args.steps, args, mode)
    result["kernels"] = kern
    result["roofline"] = roof
    # the other design of the step, for comparison
    other = "saved" if mode == "recompute" else "recompute"
    okinds = step_kinds(other)
    ms_o, kern_o, _ = sess.measure(okinds, args.steps, warmup=1)
    result["other_step"] = dict(step_mode=other, what=describe_step(other),
                                ms_per_step=round(ms_o, 3),
                                value=round(sess.blocks / (ms_o * 1e-3), 1),
                                kernels=kern_o)
    if extras:
        ukinds = ("fwd", "bwd", "hard")
        ms_u, kern_u, _ = sess.measure(ukinds, args.steps)
        result["unfused_step"] = dict(
            order="fwd, bwd, then hard extract (separate pass over z and W)",
            ms_per_step=round(ms_u, 3), value=round(sess.blocks / (ms_u * 1e-3), 1),
            kernels=kern_u)
        result.update(extra_sections(mg, sess, args))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, sess.bufs[:sess.per_copy], min_secs=cpu_secs)
    return result, sess


def extra_sections(mg, sess, args):
    """Prior seeding, the training step with the fused AdamW update, the
    diagnostics pass, the hard-sample step and the linear-space variant."""
    import torch
    wl, L, p, bf, gdt = sess.wl, sess.L, sess.ptr, sess.bf, sess.gdt
    K, M = wl.k, wl.m
    wb, gb = sess.wb, sess.gb
    dev = sess.dev
    tensors = list(range(sess.per_copy))
    out = {}

    def timed(fn_step, nsteps, warm=0):
        for s in range(warm):
            fn_step(s)
        torch.cuda.synchronize()
        e0, e1 = sess.ev(), sess.ev()
        e0.record(sess.stream)
        for s in range(nsteps):
            fn_step(s)
        e1.record(sess.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / nsteps

    def phases(seq, ph):
        """Runs (name, fn) phases in order, bracketing each with events."""
        for name, fn, pref in seq:
            a, b = sess.ev(), sess.ev()
            a.record(sess.stream)
            sess.run_phase(name, tensors, fn=fn, pref=pref, record=False)
            b.record(sess.stream)
            ph.setdefault(name, []).append((a, b))

    def ph_stats(ph, bpb, nsteps):
        res = {}
        for name, v in ph.items():
            tot = sum(a.elapsed_time(b) for a, b in v[-nsteps:]) / nsteps
            res[name] = dict(ms_per_step=round(tot, 4), algorithmic_bytes_per_block=bpb[name],
                             achieved_gbs=round(bpb[name] * sess.blocks / (tot * 1e-3) / 1e9, 1))
        return res

    # ---- prior seeding, once (initialisation of the logits) ---------------
    def prior(d, st, i):
        rc = L.maskgs_prior_init(ctypes.byref(d["desc"]), p(d["z"]), None, p(d["w"]), bf,
                                 ctypes.c_float(3.0), 0, st)
        if rc != 0:
            raise RuntimeError(f"prior_init: status {rc}")
    ms = timed(lambda s: sess.run_phase("prior", tensors, fn=prior, record=False), 1)
    out["prior_init"] = {"ms_all_tensors": round(ms, 3),
                         "achieved_gbs": round((M * wb + 8 * K) * sess.blocks / (ms * 1e-3) / 1e9,
                                               1)}

    # ---- training step with the logit update fused in (AdamW) -------------
    # maskgs_bwd_adamw keeps the logit gradient out of HBM, so the gradient
    # buffers hold the first moments; the second moments are allocated here.
    if not args.no_train_step:
        vbufs = [torch.zeros_like(d["z"]) for d in sess.bufs]
        hp = mg.AdamWParams(5e-4, 0.9, 0.999, 1e-8, 0.1, 1)
        hpref = ctypes.byref(hp)
        train = {}
        for mode, fwd_kind, bwd_bytes in (
                ("saved_y", "fwd_hard", M * wb + M * gb + 4 * K + 24 * K),
                ("recompute_y", "fwd_hard_noy", M * wb + M * gb + 24 * K)):

            def adam(d, st, i, saved=(mode == "saved_y")):
                rc = L.maskgs_bwd_adamw(ctypes.byref(d["desc"]), sess.pref, p(d["w"]), bf,
                                        p(d["z"]), p(d["y"]) if saved else None, p(d["G"]), gdt,
                                        ctypes.c_float(wl.lam), p(d["dz"]), p(vbufs[i]), hpref,
                                        st)
                if rc != 0:
                    raise RuntimeError(f"bwd_adamw: status {rc}")

            ph = {}

            def tstep(s, fwd_kind=fwd_kind, adam=adam, ph=ph):
                sess.params.step = s
                hp.t = s + 1
                sess.reg.zero_()
                phases(((fwd_kind, lambda d, st, i, k=fwd_kind: sess.call(k, d, st), None),
                        ("bwd_adamw", adam, None)), ph)
            ms = timed(tstep, args.steps)
            train[mode] = dict(ms_per_step=round(ms, 3),
                               value=round(sess.blocks / (ms * 1e-3), 1),
                               kernels=ph_stats(ph, {fwd_kind: sess.bpb[fwd_kind],
                                                     "bwd_adamw": bwd_bytes}, args.steps))
        out["train_step"] = {
            "what": "fwd with the hard mask fused in, then maskgs_bwd_adamw (backward fused with "
                    "the AdamW update of the logits: lr 5e-4, betas 0.9/0.999, eps 1e-8, weight "
                    "decay 0.1); the logit gradient never reaches HBM", **train}
        del vbufs

    # ---- training diagnostics, one pass over every tensor -----------------
    st_buf = mg.new_stats(dev)
    stats_bpb = 4 * K + M / 8 + M * wb + 4 * K

    def stats(d, st, i):
        rc = L.maskgs_mask_stats(ctypes.byref(d["desc"]), p(d["z"]), ctypes.c_float(wl.kappa),
                                 None, p(d["bits"]), p(d["w"]), bf, p(d["dz"]), p(st_buf), st)
        if rc != 0:
            raise RuntimeError(f"mask_stats: status {rc}")
    ms = timed(lambda s: sess.run_phase("stats", tensors, fn=stats, record=False), 1)
    sv = mg.read_stats(st_buf)
    out["diagnostics"] = dict(
        ms_all_tensors=round(ms, 3), algorithmic_bytes_per_block=stats_bpb,
        achieved_gbs=round(stats_bpb * sess.blocks / (ms * 1e-3) / 1e9, 1),
        changed_fraction=round(sv["changed"] / max(sv["blocks"], 1), 6),
        mean_max_prob=round(sv["max_prob"] / max(sv["blocks"], 1), 6),
        kept_over_magnitude_l1=round(sv["kept_l1"] / sv["magnitude_l1"], 6))

    # ---- hard Gumbel-max sample, straight-through backward ----------------
    hs_params = mg.SampleParams(0, 0, wl.kappa, wl.tau, mg.MASKGS_HARD_SAMPLE)
    hsref = ctypes.byref(hs_params)
    ph = {}

    def hs_step(s):
        hs_params.step = s
        sess.reg.zero_()
        phases((("fwd_hard_noy", lambda d, st, i: sess.call("fwd_hard_noy", d, st, hsref), None),
                ("bwd_rc", lambda d, st, i: sess.call("bwd_rc", d, st, hsref), None)), ph)
    ms = timed(hs_step, args.steps)
    out["hard_sample_step"] = dict(
        what="MASKGS_HARD_SAMPLE: forward applying the Gumbel-max sample (hard mask of the same "
             "logits fused in, soft index not saved), straight-through backward drawing the soft "
             "index again",
        ms_per_step=round(ms, 3), value=round(sess.blocks / (ms * 1e-3), 1),
        kernels=ph_stats(ph, sess.bpb, args.steps))

    # ---- linear-space variant (maskpro_*): M logits per block ------------
    # A step draws N of M positions per block (masked weights, packed mask,
    # draw order), then forms the policy gradient of every tensor from a
    # scalar advantage (the loss and its baseline come from the model, which
    # is outside the path; a fixed advantage stands in).  The gradient reuses
    # the logit-gradient buffers (K >= M floats per block).
    from workloads import linear_logits
    odt = torch.uint8 if M == 4 else torch.int16
    ob = 1 if M == 4 else 2
    mp = [dict(pi=linear_logits(wl, d["spec"], dev),
               order=torch.empty(d["B"], dtype=odt, device=dev),
               dpi=d["dz"].view(-1)[: d["B"] * M]) for d in sess.bufs[:sess.per_copy]]
    torch.cuda.synchronize()
    dp = mg.DrawParams(0, 0, 0)
    dpref = ctypes.byref(dp)
    adv = ctypes.c_float(0.1)
    linear = {}
    for mode, bpb in (("saved_order", {"mp_fwd": M * wb + 4 * M + 2 * M + M / 8 + ob,
                                       "mp_bwd": 4 * M + ob + 4 * M}),
                      ("redrawn", {"mp_fwd": M * wb + 4 * M + 2 * M + M / 8, "mp_bwd": 8 * M})):

        def mfwd(d, st, i, keep=(mode == "saved_order")):
            e = mp[i]
            rc = L.maskpro_fwd(ctypes.byref(d["desc"]), dpref, p(d["w"]), bf, p(e["pi"]),
                               p(d["out"]), bf, p(d["bits"]), p(e["order"]) if keep else None, st)
            if rc != 0:
                raise RuntimeError(f"maskpro_fwd: status {rc}")

        def mbwd(d, st, i, keep=(mode == "saved_order")):
            e = mp[i]
            rc = L.maskpro_bwd(ctypes.byref(d["desc"]), dpref, p(e["pi"]),
                               p(e["order"]) if keep else None, adv, p(e["dpi"]), 0, st)
            if rc != 0:
                raise RuntimeError(f"maskpro_bwd: status {rc}")
        ph = {}

        def lstep(s, mfwd=mfwd, mbwd=mbwd, ph=ph):
            dp.step = s % (1 << 32)
            phases((("mp_fwd", mfwd, None), ("mp_bwd", mbwd, None)), ph)
        ms = timed(lstep, args.steps, warm=args.warmup)
        linear[mode] = dict(ms_per_step=round(ms, 3), value=round(sess.blocks / (ms * 1e-3), 1),
                            kernels=ph_stats(ph, bpb, args.steps))
    out["linear_space_step"] = dict(
        what="maskpro_fwd (Gumbel-top-k draw of N of M positions on M fp32 logits per block; "
             "masked weights, packed mask, draw order) then maskpro_bwd (policy gradient A*dlogp "
             "of the ordered draw, A = 0.1), every tensor; saved_order reads the forward's draw "
             "order, redrawn draws again in the backward",
        logits=f"fp32 N(0,1), {M} per block", **linear)
    if not args.no_cpu_baseline:
        out["linear_space_step"]["cpu_baseline"] = cpu_baseline_linear(
            wl, sess.bufs[:sess.per_copy], mp)
    del mp
    return out


# ---------------------------------------------------------------------------
# Sub-results
# ---------------------------------------------------------------------------
def run_qproj_prior(mg, args, dev):
    """LLaMA-2-7B q_proj (4096x4096 bf16), N(0, 0.01) base logits seeded by
    the magnitude top-2 prior (alpha 3), then the step.  The tensor's buffers
    exist in three copies and step s uses copy s mod 3, so the step traffic
    between two uses of a copy exceeds the 256 MB last-level cache."""
    import torch
    from workloads import WORKLOADS
    wl = WORKLOADS["llama7b_qproj_prior"]
    mode = step_mode(args, wl)
    kinds = step_kinds(mode)
    copies = 3
    sess = Session(mg, wl, wl.tensors, args, dev, copies=copies, with_y=(mode == "saved"))
    e0, e1 = sess.ev(), sess.ev()
    e0.record(sess.stream)
    for d in sess.bufs:
        rc = sess.L.maskgs_prior_init(ctypes.byref(d["desc"]), sess.ptr(d["z"]), None,
                                      sess.ptr(d["w"]), sess.bf, ctypes.c_float(wl.prior_alpha),
                                      0, sess.sptr)
        if rc != 0:
            raise RuntimeError(f"prior_init: status {rc}")
    e1.record(sess.stream)
    torch.cuda.synchronize()
    copy_traffic = sum(sess.bpb[k] for k in kinds) * sess.blocks
    sess.timed_steps(kinds, 1, max(1, args.warmup))
    dom = sess.dominant(kinds)
    nsteps = copies * max(1, args.steps // copies)
    ms, kern, roof = sess.measure(kinds, nsteps, timed_kind=dom)
    res = line(sess, ms, kinds, nsteps, args, mode, {
        "logits": f"fp32 N(0,{wl.z_std}) seeded by the magnitude top-2 prior, alpha "
                  f"{wl.prior_alpha}",
        "buffer_rotation": f"{copies} copies, step s uses copy s mod {copies}; "
                           f"{copy_traffic / 1e6:.0f} MB of step traffic per copy"})
    res["kernels"] = kern
    res["roofline"] = roof
    res["prior_init"] = {"ms_per_tensor": round(e0.elapsed_time(e1) / copies, 4)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, sess.bufs[:1], min_secs=5.0)
    return res


def run_mlp_anneal(mg, args, dev):
    """LLaMA-2-7B MLP trio over the 8-step anneal: tau 4 -> 0.05 and kappa
    100 -> 500 (linear, both ends included); step s of the anneal is the
    step number of the noise stream."""
    from workloads import WORKLOADS
    wl = WORKLOADS["llama7b_mlp_anneal"]
    mode = step_mode(args, wl)
    kinds = step_kinds(mode)
    sess = Session(mg, wl, wl.tensors, args, dev, with_y=(mode == "saved"))

    def sched(s):
        k, t = wl.schedule(s % wl.steps)
        sess.params.step = s % wl.steps
        sess.params.kappa = k
        sess.params.tau = t
    sess.timed_steps(kinds, 1, max(1, args.warmup), schedule=sched)
    dom = sess.dominant(kinds)
    nsteps = wl.steps * max(1, args.steps // wl.steps)
    ms, kern, roof = sess.measure(kinds, nsteps, timed_kind=dom, schedule=sched)
    res = line(sess, ms, kinds, nsteps, args, mode, {
        "kappa": f"{wl.kappa} -> {wl.kappa_end}", "tau": f"{wl.tau} -> {wl.tau_end}",
        "schedule": f"linear over {wl.steps} steps (both ends included), the anneal repeated "
                    f"{nsteps // wl.steps}x"})
    res["kernels"] = kern
    res["roofline"] = roof
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, sess.bufs, min_secs=5.0)
    return res


def run_layer_48(mg, args, dev):
    """Nemotron-4-15B-shaped 4:8 layer set, measured as the headline workload
    is (its extra sections included)."""
    from workloads import WORKLOADS
    wl = WORKLOADS["nemotron15b_layer_48"]
    res, sess = run_main(mg, wl, wl.tensors, args, dev, extras=not args.no_extras, cpu_secs=5.0)
    del sess
    return res


# ---------------------------------------------------------------------------
# CPU baselines (the oracle, all usable host threads)
# ---------------------------------------------------------------------------
def host_cpu():
    """The host the CPU baseline ran on: logical CPUs, the CPUs this process
    may use, and the CPU model from /proc/cpuinfo."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
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


def host_array(t, shape=None):
    """A device tensor as an fp64-exact numpy array (bf16 widened)."""
    import numpy as np
    import torch
    import oracle
    if t.dtype == torch.bfloat16:
        a = oracle.widen_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))
    else:
        a = t.cpu().numpy()
    return a if shape is None else a.reshape(shape)


def cpu_baseline(wl, bufs, min_secs=10.0):
    """The CPU oracle (all host threads) on whole tensors of the workload, in
    order (starting over after the last one), until the oracle has run for at
    least `min_secs` of wall time: fwd + bwd + hard extract."""
    import itertools
    import numpy as np
    import torch
    import oracle

    oracle.set_threads(oracle_threads())
    used = oracle.get_threads()
    blocks, secs, tensors = 0, 0.0, 0
    for d in itertools.cycle(bufs):
        if tensors and secs >= min_secs:
            break
        spec = d["spec"]
        shape = (spec.rows, spec.cols)
        wf = host_array(d["w"], shape)
        w_raw = (d["w"].view(torch.int16).cpu().numpy().view(np.uint16)
                 if d["w"].dtype == torch.bfloat16 else d["w"].cpu().numpy())
        zf = d["z"].cpu().numpy()
        gf = host_array(d["G"], shape)
        kw = dict(kappa=wl.kappa, tau=wl.tau, seed=0, step=0, tensor_id=spec.tensor_id)
        t = time.perf_counter()
        oracle.fwd(wl.n, wl.m, wf, zf, **kw)
        oracle.bwd(wl.n, wl.m, wf, zf, gf, lam=wl.lam, **kw)
        oracle.hard_extract(wl.n, wl.m, zf, spec.rows, spec.cols,
                            w_raw=w_raw if (wl.n, wl.m) == (2, 4) else None)
        secs += time.perf_counter() - t
        blocks += d["B"]
        tensors += 1
        del wf, w_raw, zf, gf
    what = (f"first {tensors} tensor(s) of the same workload" if tensors <= len(bufs) else
            f"{tensors} tensor passes over the first {len(bufs)} tensor(s) of the workload")
    return {"value": round(blocks / secs, 1), "unit": "weight-blocks/s", "cores": used,
            "kind": "oracle", "host": host_cpu(),
            "sample": f"{what} ({blocks} blocks): fwd + bwd + hard extract, {secs:.1f} s of "
                      f"oracle wall time on {used} threads"}


def cpu_baseline_linear(wl, bufs, mp_bufs, min_secs=8.0):
    """The CPU oracle of the linear-space variant (all host threads) on whole
    tensors of the workload, in order, until the oracle has run for at least
    `min_secs` of wall time:
    draw + masked weights, then the policy gradient of the saved draw order."""
    import oracle

    oracle.set_threads(oracle_threads())
    used = oracle.get_threads()
    blocks, secs, tensors = 0, 0.0, 0
    for d, e in zip(bufs, mp_bufs):
        if tensors and secs >= min_secs:
            break
        spec = d["spec"]
        wf = host_array(d["w"], (spec.rows, spec.cols))
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
                      f"masked weights + policy gradient, {secs:.1f} s of oracle wall time on "
                      f"{used} threads"}


def run_profile(mg, wl, args, dev):
    """Each listed kind launched 3 times on the workload's largest tensor, on
    the main stream, one after another (the dispatch order a counter run
    sees); prints the launch times as one JSON line."""
    kinds = [k for k in args.profile.split(",") if k]
    bad = [k for k in kinds if k not in PROFILE_KINDS]
    if bad:
        raise SystemExit(f"--profile: unknown kind(s) {bad}; known: {', '.join(PROFILE_KINDS)}")
    big = max(wl.tensors, key=lambda t: t.rows * t.cols)
    sess = Session(mg, wl, [big], args, dev, with_y=True)
    hs = mg.SampleParams(0, 0, wl.kappa, wl.tau, mg.MASKGS_HARD_SAMPLE)
    d = sess.bufs[0]
    times = {}
    for kind in kinds:
        base, pref = kind, None
        if kind.startswith("hs_"):
            base, pref = kind[3:], ctypes.byref(hs)
        for _ in range(3):
            e0, e1 = sess.ev(), sess.ev()
            e0.record(sess.stream)
            sess.call(base, d, sess.sptr, pref)
            e1.record(sess.stream)
            sess.torch.cuda.synchronize()
            times.setdefault(kind, []).append(round(e0.elapsed_time(e1) * 1e3, 2))
    print(json.dumps({"profile": times, "unit": "us per launch", "workload": wl.key,
                      "tensor": f"{big.name} {big.rows}x{big.cols}", "blocks": d["B"],
                      "source_hash": source_hash()}), flush=True)


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
    from workloads import WORKLOADS

    mg.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    wl = WORKLOADS[args.workload]
    if args.profile:
        run_profile(mg, wl, args, dev)
        return
    specs = wl.tensors
    if args.layers is not None:
        specs = [t for t in specs if t.tensor_id < 7 * args.layers]
    result, sess = run_main(mg, wl, specs, args, dev, extras=not args.no_extras)
    del sess
    gc.collect()
    torch.cuda.empty_cache()
    if not args.no_sub and args.workload == "llama7b_all_linear" and args.layers is None:
        sub = {}
        for name, fn in (("llama7b_qproj_prior", run_qproj_prior),
                         ("llama7b_mlp_anneal", run_mlp_anneal),
                         ("nemotron15b_layer_48", run_layer_48)):
            print(f"# sub-result {name}", file=sys.stderr, flush=True)
            sub[name] = fn(mg, args, dev)
            gc.collect()
            torch.cuda.empty_cache()
        result["sub_results"] = sub
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
