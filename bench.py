#!/usr/bin/env python3
"""Throughput of rank-major MoE expert-parallel dispatch + combine on one GPU.

    python bench.py [--steps K] [--warmup W] [--workload dsv3]

A step is one round of the hot path over one batch of synthetic input: one
dispatch (routing, placement, invalid-row fill: one kernel) and one combine
(gather-reduce: one kernel) through the C ABI of libmoe_ep.so.  Inputs are
resident in HBM before the timed region.  The expert computation between
the two (a torch stand-in writing the combine input buffers) runs once per
instance before timing, so the timed steps are exactly the two launches.

To keep the 256 MB MALL (Infinity Cache) from serving repeated steps, the
bench rotates over --instances independent copies (workspace, inputs,
outputs); each DeepSeek-V3-shaped instance touches ~265 MB, 8 of them ~2 GB.

Printed: one JSON line with the whole-job throughput (algorithmic bytes per
round / wall time per round over the K timed steps), each kernel's share of
the HBM peak and the slower (dominant) kernel's roofline figures from HIP
events on the launch stream (a separate pass of K steps whose launches queue
behind a spin kernel, so the events time the kernels alone), and the CPU
oracle's throughput on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import dataclasses
import functools
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine µs/round and effective HBM GB/s (% peak), DSv3 shape"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
# The kernels and the host code that picks their launch shapes.
KERNEL_SOURCES = [os.path.join(ROOT, "combine_token_dest_amd", "csrc", f)
                  for f in ("moe_ep_kernels.hip", "moe_ep_plan.cpp", "moe_ep_internal.h")]
# PMC summaries are named <workload>_<dispatch kernel>_combine_kernel_traffic.txt
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "{workload}_{dispatch}_combine_kernel_traffic.txt")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic bytes
# ---------------------------------------------------------------------------
BYTES_FORMULA = ("dispatch N*(4K(1+w)+H+S) + P*(H+S+4K*w) + R*4K; combine N*4K + P*O + N*O "
                 "(N tokens, P routed (token, rank) pairs, R = ep*ep*tpr receive rows, w = weights present)")


def algorithmic_bytes(w, n, masks, tpr, has_w):
    """Bytes the method must move in one round (BYTES_FORMULA):
    dispatch reads every real token's ids, weights, hidden and scale row once,
    writes every routed (token, rank) pair's hidden row, scale row and
    weights, and the ids slot of every receive row of every rank (the
    invalid id where the token did not go); combine reads what says where
    each token went (its K ids' worth), every routed pair's expert row, and
    writes every real token's output row.  The zero weights of invalid rows
    and the route masks are not counted."""
    K, H, S = w.top_k, w.hidden_row_bytes, w.scale_row_bytes
    O = w.hidden_size * w.combine_elem_bytes
    N = sum(n)
    P = int(sum(bin(m).count("1") for m in masks))
    R = w.ep_size * w.ep_size * tpr
    wb = 1 if has_w else 0
    b_dispatch = N * (4 * K * (1 + wb) + H + S) + P * (H + S + 4 * K * wb) + R * 4 * K
    b_combine = N * 4 * K + P * O + N * O
    return b_dispatch, b_combine, N, P, R


def destination_masks(w, inp):
    """Per-token destination masks from the inputs (contiguous ownership, the
    active-rank mask applied); only used to count bytes."""
    epr = w.num_experts // w.ep_size
    active = inp.active_rank_mask if inp.active_rank_mask is not None else (1 << w.ep_size) - 1
    masks = []
    for s in range(w.ep_size):
        ids = inp.topk_ids[s]
        owners = ids // epr
        for t in range(ids.shape[0]):
            m = 0
            for e, o in zip(ids[t], owners[t]):
                if 0 <= e < w.num_experts:
                    m |= 1 << int(o)
            masks.append(m & active)
    return masks


# ---------------------------------------------------------------------------
# one instance: workspace + inputs + outputs at their own addresses
# ---------------------------------------------------------------------------
class Instance:
    def __init__(self, w, inp, dev_inputs, device, order="auto"):
        import torch
        from combine_token_dest_amd import MoEEp, _lib
        self.w = w
        self.moe = MoEEp(w.ep_size, w.num_experts, w.top_k, w.max_tokens_per_rank, w.hidden_size,
                         hidden_row_bytes=w.hidden_row_bytes, scale_row_bytes=w.scale_row_bytes,
                         combine_max_elem_bytes=w.combine_elem_bytes,
                         enable_rank_mask=inp.active_rank_mask is not None, dispatch_order=order,
                         device=device)
        # The group's per-rank inputs and outputs each live in one allocation
        # per instance ([ep, capacity, ...], rank s's rows at the start of
        # slice s), as one process holding every rank would lay them out.
        # (Per-rank tensors from torch's caching allocator landed wherever
        # freed blocks were: the same dispatch then took 15.8-17.3 us from one
        # instance to the next; in one allocation it takes 15.6-15.9.)
        hid, ids, wts, scl = [grouped_copy(lst, w.ep_size, w.max_tokens_per_rank, device)
                              if lst is not None else None for lst in dev_inputs[:4]]
        self.inputs = (hid, ids, wts, scl)
        self.cdtype = torch.float32 if w.combine_dtype == "f32" else torch.bfloat16
        out_all = torch.empty((w.ep_size, w.max_tokens_per_rank, w.hidden_size), dtype=self.cdtype, device=device)
        self.outputs = [out_all[s, :n] for s, n in enumerate(inp.local_num_tokens)]
        rtpr = inp.runtime_max_tokens_per_rank
        mask = inp.active_rank_mask
        # First round through the Python API, with the expert stand-in in between.
        res = self.moe.dispatch(hid, ids, wts, hidden_states_scale=scl, runtime_max_tokens_per_rank=rtpr,
                                active_rank_mask=mask)
        self.tpr = res[0].tokens_per_rank
        self.order = self.moe.last_dispatch_order
        values = dev_inputs[4]
        for d in range(w.ep_size):
            buf = self.moe.get_combine_input_buffer(d, self.cdtype)
            expert_standin_torch(w, d, res[d], values, self.tpr, buf)
        self.moe.combine([self.moe.get_combine_input_buffer(d, self.cdtype) for d in range(w.ep_size)],
                         output=self.outputs, active_rank_mask=mask)
        # Prebuilt C-ABI arguments for the timed steps (same values as above).
        a = _lib.moe_ep_dispatch_args()
        for s in range(w.ep_size):
            n = inp.local_num_tokens[s]
            a.local_num_tokens[s] = n
            a.hidden[s] = hid[s].data_ptr() if n else None
            a.topk_ids[s] = ids[s].data_ptr() if n else None
            a.topk_weights[s] = wts[s].data_ptr() if n else None
            if scl is not None:
                a.hidden_scale[s] = scl[s].data_ptr() if n else None
        a.weights_present = (1 << w.ep_size) - 1
        a.scales_present = (1 << w.ep_size) - 1 if scl is not None else 0
        a.runtime_max_tokens_per_rank = -1 if rtpr is None else rtpr
        a.active_rank_mask = _lib.MOE_EP_ALL_RANKS if mask is None else mask
        self.dargs = a
        c = _lib.moe_ep_combine_args()
        for s in range(w.ep_size):
            c.expert_output[s] = None                 # the rank's combine input buffer
            c.output[s] = self.outputs[s].data_ptr() if inp.local_num_tokens[s] else None
        c.dtype = _lib.MOE_EP_F32 if w.combine_dtype == "f32" else _lib.MOE_EP_BF16
        c.active_rank_mask = a.active_rank_mask
        self.cargs = c
        self.results = (_lib.moe_ep_dispatch_result * w.ep_size)()
        self.handle = ctypes.c_void_p(self.moe._handle)
        self.lib = _lib.load()
        # The call arguments are built once: the timed steps pay only for
        # the two foreign calls, as a C caller would.
        self._dispatch_call = functools.partial(self.lib.moe_ep_dispatch, self.handle, ctypes.byref(self.dargs),
                                                self.results)
        self._combine_call = functools.partial(self.lib.moe_ep_combine, self.handle, ctypes.byref(self.cargs))

    def dispatch(self, stream):
        st = self._dispatch_call(stream)
        if st:
            raise RuntimeError(f"moe_ep_dispatch: {st} {self.lib.moe_ep_last_error().decode()}")

    def combine(self, stream):
        st = self._combine_call(stream)
        if st:
            raise RuntimeError(f"moe_ep_combine: {st} {self.lib.moe_ep_last_error().decode()}")


def grouped_copy(per_rank, ep, cap, device):
    """Copies of per-rank [n_s, ...] tensors as slices [s, :n_s] of one
    [ep, cap, ...] allocation."""
    import torch
    t0 = per_rank[0]
    alls = torch.empty((ep, cap) + tuple(t0.shape[1:]), dtype=t0.dtype, device=device)
    views = []
    for s, t in enumerate(per_rank):
        v = alls[s, :t.shape[0]]
        v.copy_(t)
        views.append(v)
    return views


def expert_standin_torch(w, d, res, values, tpr, out):
    """The caller's expert computation, stood in for: on rank d, row r of a
    routed token (s, t) = value(s, t) x (weights of its experts that rank d
    owns); rows holding no token are NaN.  Untimed."""
    import torch
    epr = w.num_experts // w.ep_size
    ids = res.topk_ids.long()
    wts = res.topk_weights
    local = (ids >= d * epr) & (ids < (d + 1) * epr)
    wsum = (wts * local.float()).sum(dim=1)
    rows = w.ep_size * tpr
    full = torch.zeros((rows, w.hidden_size), dtype=torch.float32, device=out.device)
    for s in range(w.ep_size):
        n = values[s].shape[0]
        if n:
            full[s * tpr:s * tpr + n] = values[s]
    full = full * wsum[:, None]
    valid = ids[:, 0] != -1
    full[~valid] = float("nan")
    out.copy_(full.to(out.dtype))


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------
def cpu_baseline(w, inp, bytes_per_round, seconds):
    import oracle
    p = oracle.Params(w.ep_size, w.num_experts, w.top_k, w.max_tokens_per_rank, w.hidden_size,
                      w.hidden_row_bytes, w.scale_row_bytes, -1, inp.active_rank_mask is not None)
    spent = 0.0
    rounds = 0
    while spent < seconds:
        om = oracle.OracleMoEEp(p)
        t0 = time.perf_counter()
        res = om.dispatch(inp.hidden, inp.topk_ids, inp.topk_weights, hidden_states_scale=inp.scale,
                          runtime_max_tokens_per_rank=inp.runtime_max_tokens_per_rank,
                          active_rank_mask=inp.active_rank_mask)
        t1 = time.perf_counter()
        if rounds == 0:
            eo = oracle.expert_standin(p, res, inp.values, w.combine_dtype)
        t2 = time.perf_counter()
        om.combine(eo, w.combine_dtype, active_rank_mask=inp.active_rank_mask)
        t3 = time.perf_counter()
        spent += (t1 - t0) + (t3 - t2)
        rounds += 1
    gbs = bytes_per_round * rounds / spent / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{rounds} full {w.name} rounds (dispatch+combine, stand-in excluded), "
                      f"{spent:.1f} s, single-threaded NumPy",
            "us_per_round": round(spent / rounds * 1e6, 1),
            "host_cpus": os.cpu_count(), "host_affinity": len(os.sched_getaffinity(0))}


class HipEvents:
    """HIP events created with hipEventDisableSystemFence: recording one adds
    no system-scope release (no L2 writeback between the kernels it
    brackets), so launch-to-launch event pairs time the kernels themselves."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")      # the runtime torch already loaded
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        st = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if st:
            raise RuntimeError(f"hipEventCreateWithFlags: {st}")
        return ev

    def record(self, ev, stream):
        st = self.hip.hipEventRecord(ev, ctypes.c_void_p(stream))
        if st:
            raise RuntimeError(f"hipEventRecord: {st}")

    def elapsed_ms(self, a, b):
        st = self.hip.hipEventSynchronize(b)
        if st:
            raise RuntimeError(f"hipEventSynchronize: {st}")
        ms = ctypes.c_float()
        st = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if st:
            raise RuntimeError(f"hipEventElapsedTime: {st}")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def solve_kernel_times(td, tc, n, round_ms):
    """Per-launch dispatch and combine times of each group from the grouped
    pass: td[g] = n[g] * D + m and tc[g] = n[g] * C + m, where m is the
    stream time one event costs, and D + C = round_ms (the alternating pass).
    Summing over the G groups, sum(td) + sum(tc) = K * round_ms + 2 * G * m
    with K = sum(n).  Returns (per-group D, per-group C, m), m clamped at 0."""
    td, tc, n = (np.asarray(x, dtype=float) for x in (td, tc, n))
    G, K = len(n), float(n.sum())
    m = max(0.0, float(td.sum() + tc.sum() - K * round_ms) / (2 * G))
    return (td - m) / n, (tc - m) / n, m


def spin_cycles_for_us(us, stream):
    """Argument of torch.cuda._sleep (a spin kernel that touches no memory)
    for about `us` microseconds, from one timed spin on this device."""
    import torch
    probe = 1 << 20
    torch.cuda._sleep(probe)                        # first launch: load the kernel
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    torch.cuda._sleep(probe)
    e1.record(stream)
    torch.cuda.synchronize()
    per_us = probe / max(e0.elapsed_time(e1) * 1e3, 1e-3)
    return int(per_us * us)


def kernel_source_hash():
    """sha256[:16] of the kernel sources with comments and whitespace removed,
    so the PMC traffic figures stay tied to the code they were taken on."""
    import re
    src = ""
    for path in KERNEL_SOURCES:
        with open(path) as f:
            src += f.read() + "\n"
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def read_traffic(workload, dispatch_kernel, kernel):
    """HBM bytes per launch of `kernel` from the committed PMC summary of the
    workload's round (`dispatch_kernel` + combine_kernel), if it was taken on
    the current kernel source; else None."""
    path = TRAFFIC_FILE.format(workload=workload, dispatch=dispatch_kernel)
    if not os.path.exists(path):
        return None
    src_hash = None
    val = None
    for line in open(path):
        parts = line.split()
        if len(parts) >= 2 and parts[0] == "kernel_code_sha256:":
            src_hash = parts[1]
        if len(parts) >= 3 and parts[0] == "traffic_bytes_per_launch:" and parts[1] == kernel:
            val = float(parts[2])
    if src_hash != kernel_source_hash():
        return None
    return val


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3", choices=["tiny", "dsv3", "fp8", "ragged", "large"])
    ap.add_argument("--tokens-per-rank", type=int, default=None,
                    help="the workload at another capacity (tokens per rank), e.g. decode batch sizes")
    ap.add_argument("--instances", type=int, default=8)
    ap.add_argument("--kernel-steps", type=int, default=160,
                    help="steps of each per-kernel timing pass (at least --steps)")
    ap.add_argument("--dispatch-order", default="auto", choices=["auto", "source", "destination"],
                    help="copy order of the dispatch kernel (the library picks by shape under auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="(default) time a plain 1 GiB device-to-device copy: the PMC byte scale, and the "
                         "measured copy bandwidth the round is compared with")
    ap.add_argument("--no-copy-calibration", action="store_true", help="skip the 1 GiB copy")
    ap.add_argument("--two-streams", action="store_true",
                    help="also time the rounds as two overlapping streams of work (off by default: their "
                         "overlapped launches would enter a kernel trace's per-kernel averages)")
    ap.add_argument("--no-two-streams", action="store_true", help="(default) skip the two-stream pass")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP graph replays after the timed passes (profiled runs: the kernel "
                         "trace then holds only the set-up, warm-up and timed launches)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0 or args.instances < 1 or args.kernel_steps < 1:
        ap.error("--steps, --instances and --kernel-steps must be at least 1, --warmup at least 0")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (the EP group's ranks are partitions of one GPU's HBM); "
              f"--gpus {args.gpus} / WORLD_SIZE {world} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from synth import workloads as wl
    from combine_token_dest_amd import _lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    _lib.load()
    if not _lib.moe_ep_is_platform_supported():
        print("not a gfx950 device", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)

    w = wl.BY_NAME[args.workload]
    if args.tokens_per_rank is not None:
        if args.tokens_per_rank < 1:
            print("--tokens-per-rank must be at least 1", file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, max_tokens_per_rank=args.tokens_per_rank)
    log(f"[bench] workload {w.name} seed {w.seed}: generating inputs")
    inp = wl.make_inputs(w)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    dev_hidden = [to(h) for h in inp.hidden]
    dev_ids = [to(i) for i in inp.topk_ids]
    dev_w = [to(x) for x in inp.topk_weights]
    dev_s = [to(x) for x in inp.scale] if inp.scale is not None else None
    dev_vals = [to(v) for v in inp.values]
    dev_inputs = (dev_hidden, dev_ids, dev_w, dev_s, dev_vals)

    log(f"[bench] building {args.instances} instances")
    insts = []
    for i in range(args.instances):
        insts.append(Instance(w, inp, dev_inputs, device, args.dispatch_order))
        log(f"[bench] instance {i + 1}/{args.instances} ready")
    del dev_vals
    torch.cuda.synchronize()
    tpr = insts[0].tpr
    masks = destination_masks(w, inp)
    b_d, b_c, N, P, R = algorithmic_bytes(w, inp.local_num_tokens, masks, tpr, True)
    bytes_round = b_d + b_c

    stream = torch.cuda.current_stream(device)
    sp = stream.cuda_stream
    I = len(insts)

    # First launches of every instance (module load, first-touch of the
    # workspaces), untimed; the W warm-up steps run right before the timed
    # region below.
    log("[bench] one round on each instance")
    for inst in insts:
        inst.dispatch(sp)
        inst.combine(sp)
    torch.cuda.synchronize()

    # Per-kernel passes (untimed for `value`), of KP = max(K, --kernel-steps)
    # steps each so that the split between the kernels does not rest on a
    # few groups.  Each queues its launches behind a spin kernel (no memory
    # traffic) that runs long enough for the host to enqueue all of them, so
    # no kernel waits for its launch call.
    #  1. KP steps in groups of I (one per instance): the group's I
    #     dispatches back to back, then its I combines (every instance still
    #     runs dispatch -> combine), with a HIP event before each run of
    #     dispatches and of combines and after the last: t_d(g) and t_c(g).
    #  2. KP steps alternating as a caller would, one event at each end: R,
    #     the time per round (dispatch + combine).
    # An event costs the stream some idle time of its own (m per event,
    # unknown), so t_d(g) = n_g * D + m and t_c(g) = n_g * C + m; with
    # D + C = R this gives m and the per-launch kernel times D and C.
    K = args.steps
    KP = max(K, args.kernel_steps)
    sizes = [I] * (KP // I) + ([KP % I] if KP % I else [])
    G = len(sizes)
    hev = HipEvents()
    ev = [[hev.create() for _ in range(3)] for _ in range(G)]
    ea, eb = hev.create(), hev.create()
    spin_cycles = spin_cycles_for_us(max(1000.0, 12.0 * (2 * KP + 3 * G)), stream)
    log(f"[bench] per-kernel passes: {KP} steps ({G} groups of up to {I}), then {KP} alternating")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(spin_cycles)
    for g in range(G):
        e = ev[g]
        group = insts[:sizes[g]]
        hev.record(e[0], sp)
        for inst in group:
            inst.dispatch(sp)
        hev.record(e[1], sp)
        for inst in group:
            inst.combine(sp)
        hev.record(e[2], sp)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_s = t1 - t0
    torch.cuda._sleep(spin_cycles)
    hev.record(ea, sp)
    for i in range(KP):
        insts[i % I].dispatch(sp)
        insts[i % I].combine(sp)
    hev.record(eb, sp)
    torch.cuda.synchronize()
    round_ms = hev.elapsed_ms(ea, eb) / KP
    td = np.array([hev.elapsed_ms(ev[g][0], ev[g][1]) for g in range(G)])
    tc = np.array([hev.elapsed_ms(ev[g][1], ev[g][2]) for g in range(G)])
    w_g = np.array(sizes, dtype=float)
    d_ms, c_ms, marker_ms = solve_kernel_times(td, tc, w_g, round_ms)
    # The events go before the timed steps: while timing events are alive
    # (even just two), launches cost more: decode-size rounds measured
    # 9.2-9.5 instead of 7.6-7.8 us and a 20-step DSv3 region 0.7-0.8 us per
    # step slower.
    for e in ev + [[ea, eb]]:
        for x in e:
            hev.destroy(x)

    # W untimed warm-up steps, then the timed region: K steps without
    # events, alternating dispatch and combine per instance as a caller
    # would, bracketed by synchronizations: this pass gives the step time and
    # `value` (the passes above attribute time to each kernel).  The warm-up
    # sits right before the timed steps: after 1-100 ms of idle GPU (host
    # work such as the solve above) a 20-step region measured 0.2-0.5 us per
    # step slower than one started on a part that had just been busy.
    log(f"[bench] warmup {args.warmup}, then timing {K} steps")
    for i in range(args.warmup):
        insts[i % I].dispatch(sp)
        insts[i % I].combine(sp)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(K):
        insts[i % I].dispatch(sp)
        insts[i % I].combine(sp)
    torch.cuda.synchronize()
    wall_plain = time.perf_counter() - t2

    # The same rounds replayed from HIP graphs (one captured dispatch +
    # combine per instance): what a caller that captures the round sees.
    graph_us = None
    graph_all_us = None
    if not args.no_graph:
        try:
            graphs = []
            for inst in insts:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    cs = torch.cuda.current_stream(device).cuda_stream
                    inst.dispatch(cs)
                    inst.combine(cs)
                graphs.append(g)
            for g in graphs:
                g.replay()
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            for i in range(K):
                graphs[i % I].replay()
            torch.cuda.synchronize()
            graph_us = round((time.perf_counter() - t3) / K * 1e6, 2)
            del graphs
            # All I rounds in one graph (2*I kernel nodes): the per-launch cost
            # of a graph is then spread over I rounds.
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = torch.cuda.current_stream(device).cuda_stream
                for inst in insts:
                    inst.dispatch(cs)
                    inst.combine(cs)
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, K // I)
            t4 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            graph_all_us = round((time.perf_counter() - t4) / (reps * I) * 1e6, 2)
            del g
        except Exception as e:          # reported, never fatal: this is an extra
            log(f"[bench] graph replay skipped: {e}")

    # The same rounds as two independent streams of work, as a caller that
    # overlaps two micro-batches would run them: instance j always runs on
    # stream j % 2 (so each handle's dispatch -> combine order holds), and
    # one stream's kernel ramps and tails overlap the other's.  Reported
    # beside `value`, which stays the one-stream round.
    two_stream_us = None
    if args.two_streams and not args.no_two_streams and I >= 2:
        streams = [torch.cuda.Stream(device), torch.cuda.Stream(device)]     # default priority
        def two_stream_rounds(n):
            for i in range(n):
                j = i % I
                cs = streams[j % 2].cuda_stream
                insts[j].dispatch(cs)
                insts[j].combine(cs)
        two_stream_rounds(max(2 * I, args.warmup))       # first launches on new queues are slow
        torch.cuda.synchronize()
        t5 = time.perf_counter()
        two_stream_rounds(K)
        torch.cuda.synchronize()
        two_stream_us = round((time.perf_counter() - t5) / K * 1e6, 2)

    ms_step = wall_plain / K * 1e3
    value = bytes_round / (wall_plain / K) / 1e9
    d_us = float((d_ms * w_g).sum() / w_g.sum() * 1e3)
    c_us = float((c_ms * w_g).sum() / w_g.sum() * 1e3)
    d_gbs, c_gbs = b_d / (d_us * 1e-6) / 1e9, b_c / (c_us * 1e-6) / 1e9
    # kernel names as rocprofv3 lists them (template arguments aside)
    dname = "dispatch_dst_kernel" if insts[0].order == "destination" else "dispatch_kernel"
    # The dominant kernel is the slower one (the larger share of the round).
    dominant = dname if d_us >= c_us else "combine_kernel"
    dom_bytes, dom_us, dom_gbs = (b_d, d_us, d_gbs) if dominant == dname else (b_c, c_us, c_gbs)
    # The counters were taken on the workloads as defined, not at other capacities.
    traffic = {k: read_traffic(w.name, dname, k) if args.tokens_per_rank is None else None
               for k in (dname, "combine_kernel")}

    copy_info = None
    if not args.no_copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        copy_info = {"bytes": 2 * (1 << 30), "ms": round(ms, 4), "GB/s": round(2 * (1 << 30) / ms / 1e6, 1)}
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline, ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(w, inp, bytes_round, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "payload_dtype": w.row_format,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: ep_size={w.ep_size} logical ranks on 1 GPU, "
                               f"tokens_per_rank={tpr}, hidden={w.hidden_size} {w.row_format}, "
                               f"num_experts={w.num_experts}, top_k={w.top_k}",
                   "ep_size": w.ep_size, "tokens_per_rank": tpr, "hidden": w.hidden_size,
                   "num_experts": w.num_experts, "top_k": w.top_k, "row_format": w.row_format,
                   "instances_rotated": I, "seed": w.seed, "dispatch_order": insts[0].order},
        "us_per_round": round(ms_step * 1e3, 2),
        "us_per_round_kernels": round(d_us + c_us, 2),
        "us_per_round_kernels_p10_p50_p90": [round(float(np.percentile(d_ms + c_ms, q)) * 1e3, 2)
                                             for q in (10, 50, 90)],
        "timing": "kernel times from fence-free HIP events around runs of I back-to-back launches and "
                  "around K alternating rounds, queued behind a spin kernel; each event's own stream time "
                  "(marker_us) solved out",
        "marker_us": round(marker_ms * 1e3, 3),
        "us_per_round_events": round(round_ms * 1e3, 3),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "pct_hbm_peak_kernels": round(100 * bytes_round / ((d_us + c_us) * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
        "bytes_per_round": bytes_round,
        "routed_pairs": P, "tokens": N, "receive_rows": R,
        "kernels": {
            dname: {"us_mean": round(d_us, 3), "us_p10": round(float(np.percentile(d_ms, 10)) * 1e3, 3),
                                "us_p50": round(float(np.median(d_ms)) * 1e3, 3),
                                "us_p90": round(float(np.percentile(d_ms, 90)) * 1e3, 3),
                                "bytes": b_d, "GB/s": round(d_gbs, 1),
                                "frac": round(d_gbs / HBM_PEAK_GBS, 4), "traffic": traffic[dname]},
            "combine_kernel": {"us_mean": round(c_us, 3), "us_p10": round(float(np.percentile(c_ms, 10)) * 1e3, 3),
                               "us_p50": round(float(np.median(c_ms)) * 1e3, 3),
                               "us_p90": round(float(np.percentile(c_ms, 90)) * 1e3, 3),
                               "bytes": b_c, "GB/s": round(c_gbs, 1),
                               "frac": round(c_gbs / HBM_PEAK_GBS, 4), "traffic": traffic["combine_kernel"]},
        },
        "us_per_round_grouped_with_events": round(wall_s / KP * 1e6, 2),
        "kernel_steps": KP,
        "us_per_round_graph_replay": graph_us,
        "us_per_round_graph_replay_all_instances": graph_all_us,
        "us_per_round_two_streams": two_stream_us,
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic[dominant], "algorithmic_bytes_per_launch": dom_bytes,
                     "us_per_launch": round(dom_us, 3), "bytes_formula": BYTES_FORMULA,
                     "timing": "HIP events around runs of back-to-back launches queued behind a spin kernel, event overhead solved out"},
        "cpu_baseline": cpu,
        "kernel_code_sha256": kernel_source_hash(),
    }
    if copy_info:
        out["copy_1GiB"] = copy_info
        out["pct_of_copy_bw"] = round(100 * value / copy_info["GB/s"], 2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
