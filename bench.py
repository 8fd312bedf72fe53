"""Benchmark: MoE layout + dispatch + combine on one MI355X.

One step is one pass of the whole hot path over one batch: the layout
(counts, token-to-rank map, offsets, slots) and the dispatch (row scatter into
the [R*S, H] receive buffer) through the one-call ep_layout_dispatch, or as
ep_get_layout + ep_dispatch with --two-calls, then ep_combine (top-k weighted
gather-reduce back to token order, reading the dispatched buffer as the expert
outputs).  Inputs are synthetic and seeded (ep_inputs), resident in HBM
before timing starts.

The default workload is the largest one that fits one GPU: 16384 tokens,
hidden 7168, top-8 of 256 experts over 16 ranks in two groups of eight.

Prints ONE JSON line: tokens/s for the whole step, effective HBM bandwidth,
per-phase times warm and after a cache flush, the decode-sized batch's
per-call microseconds, the practical ceilings measured by the probe kernels,
the roofline of the dominant kernel (timed live with HIP events on the stream
the kernels run on) and the CPU oracle's throughput on a bounded sample.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload large16k]
  python bench.py --write-traffic FETCH.csv WRITE.csv   # rocprofv3 --pmc runs -> profiles/traffic.json
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ep_inputs  # noqa: E402

PEAK_HBM_GBPS = 8000.0   # MI355X HBM3E peak, GB/s (1e9 bytes)
METRIC = "dispatch+combine tokens/s and effective HBM GB/s (% of peak), 1 MI355X"
HEADLINE_WORKLOAD = "large16k"
DECODE_WORKLOAD = "decode128"
PROBE_BYTES = 1 << 30
# the sources each kernel family is built from (its code and its launch); a
# counter record is valid only while these files are unchanged
_CSRC = "combine_ep_get_amd/csrc/"
_COMMON = [_CSRC + "device_common.h", _CSRC + "ep_internal.h"]
KERNEL_SOURCES = {
    "layout": [_CSRC + "layout.hip"] + _COMMON,
    "dispatch": [_CSRC + "rows.hip"] + _COMMON,
    "combine": [_CSRC + "rows.hip"] + _COMMON,
    # the one-call form: the count pass and the dispatching kernel in
    # layout.hip, launched with the copy grid of rows.hip
    "layout_dispatch": [_CSRC + "layout.hip", _CSRC + "rows.hip"] + _COMMON,
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
PROBE_LIB = os.path.join(ROOT, "combine_ep_get_amd", "libepprobe.so")


def algorithmic_bytes(wl, fp8=False):
    """Bytes each kernel must move per launch (what the method itself needs).

    layout:   read topk_idx (4TK), write token_slot (4TK) and is_token_in_rank (TR)
    dispatch: read x (2TH), write K rows per token (2TKH); read slot and weight
              (8TK), write source index and weight per row (8TK).  FP8: rows
              of H bytes plus H/128 fp32 scales per row (TH + 4T*H/128 read,
              K times that written)
    combine:  read K rows per token (2TKH), write out (2TH); read slot and
              weight (8TK)
    """
    T, H, K, R = wl.T, wl.H, wl.K, wl.R
    lay = 8 * T * K + T * R
    if fp8:
        row = H + 4 * (H // 128)
        dis = T * row + T * K * row + 16 * T * K
    else:
        dis = 2 * T * H + 2 * T * K * H + 16 * T * K
    com = 2 * T * K * H + 2 * T * H + 8 * T * K
    return {"layout": lay, "dispatch": dis, "combine": com}


def _code_only(text):
    """Source text without comments and with whitespace collapsed, so that a
    comment edit does not count as a kernel change."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernels changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload, {}).get(kernel)
    if entry is None or entry.get("source_hash") != kernel_source_hash(kernel):
        return None
    return entry.get("bytes_per_launch")


def _kernel_family(name, one_call):
    """Family of a kernel in a rocprofv3 CSV row, by its function name."""
    found = re.findall(r"(\w+_kernel)\b", name)
    base = found[-1] if found else ""
    if base == "combine_kernel":
        return "combine"
    if base in ("dispatch_chunks_kernel", "layout_dispatch_kernel"):
        return "layout_dispatch"
    if base.startswith("layout_"):
        return "layout_dispatch" if one_call else "layout"
    if base == "dispatch_kernel":
        return "dispatch"
    if base in ("read_kernel", "write_kernel", "copy_kernel"):
        return "probe_" + base[:-len("_kernel")]
    return None


def _counter_kib(path):
    """Counter value (KiB) per dispatch, grouped by kernel family, from a
    rocprofv3 --pmc CSV (the per-instance rows of a dispatch are summed)."""
    import csv

    with open(path) as f:
        rows = list(csv.DictReader(f))
    one_call = any(re.search(r"(dispatch_chunks|layout_dispatch)_kernel", r["Kernel_Name"]) for r in rows)
    fam = {}
    for r in rows:
        key = _kernel_family(r["Kernel_Name"], one_call)
        if key is None:
            continue
        fam.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
        fam[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return fam, one_call


def write_traffic(workload, fetch_csv, write_csv, probe_bytes=PROBE_BYTES):
    """Turn two rocprofv3 --pmc runs of this bench (FETCH_SIZE, then
    WRITE_SIZE) into HBM bytes per launch.  FETCH_SIZE is scaled so that the
    read probe of `probe_bytes` reads exactly that many bytes, WRITE_SIZE so
    that the write probe writes them.  Adds the workload (and mode) to
    profiles/traffic.json."""
    (fetch, one_call), (write, _) = _counter_kib(fetch_csv), _counter_kib(write_csv)

    def probe_kib(fam, key):
        # every launch of a probe moves probe_bytes: the median launch
        v = sorted(fam[key].values())
        return v[len(v) // 2]

    f_fetch = probe_bytes / (probe_kib(fetch, "probe_read") * 1024)
    f_write = probe_bytes / (probe_kib(write, "probe_write") * 1024)
    kernels = ("layout_dispatch", "combine") if one_call else ("layout", "dispatch", "combine")
    steps = len(fetch["combine"])
    per_kernel = {}
    for k in kernels:
        fv, wv = list(fetch[k].values()), list(write[k].values())
        fk, wk = sum(fv) / steps, sum(wv) / steps
        per_kernel[k] = {"fetch_kib": fk, "write_kib": wk, "launches_per_step": len(fv) // steps,
                         "bytes_per_launch": (fk * f_fetch + wk * f_write) * 1024,
                         "source_hash": kernel_source_hash(k)}
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    key = workload + ("" if one_call else "+two-calls")
    rec.setdefault("workloads", {})[key] = {
        "factor_fetch": f_fetch, "factor_write": f_write, "calibration": "probe read/write kernels",
        "probe_bytes": probe_bytes, "steps": steps, **per_kernel}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    return rec["workloads"][key]


def _oracle_step_seconds(wl, inp, S, recv):
    import oracle

    t0 = time.perf_counter()
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S, wl.G, wl.A)
    oracle.dispatch(inp.x, lay.token_slot, wl.R * S, inp.topk_weights, recv_x=recv)
    oracle.combine(recv, lay.token_slot, inp.topk_weights)
    return time.perf_counter() - t0


def cpu_baseline(wl, inp, S, budget_s=15.0, samples=3):
    """Time the CPU oracle (single-threaded C) on whole steps of the
    workload: `samples` samples of whole steps, each running until about
    budget_s / samples seconds have passed (at least one step), and report
    the median sample's tokens/s."""
    recv = np.zeros((wl.R * S, wl.H), np.uint16)   # only the slots' rows are touched
    rates, steps_total, t_total = [], 0, 0.0
    for _ in range(samples):
        steps, t = 0, 0.0
        while steps == 0 or t < budget_s / samples:
            t += _oracle_step_seconds(wl, inp, S, recv)
            steps += 1
        rates.append(wl.T * steps / t)
        steps_total += steps
        t_total += t
    return {
        "value": float(np.median(rates)),
        "unit": "tokens/s",
        "cores": 1,
        "host_cpus": os.cpu_count(),
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "samples_tokens_per_s": rates,
        "sample": f"median of {samples} samples, {steps_total} whole step(s) in all of the {wl.name} "
                  f"workload (layout+dispatch+combine, T={wl.T}), single-threaded C oracle, "
                  f"{t_total:.1f} s",
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _time_ms(torch, stream, fn, iters):
    """Mean milliseconds of fn() over iters calls, between two HIP events on
    `stream`, after three untimed calls."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def probe_lib():
    """The bandwidth probes (libepprobe.so), with their argument types."""
    lib = ctypes.CDLL(PROBE_LIB)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.ep_probe_read.argtypes = [vp, i64, ctypes.c_int, vp, vp]
    lib.ep_probe_write.argtypes = [vp, i64, ctypes.c_int, vp]
    lib.ep_probe_copy.argtypes = [vp, vp, i64, vp]
    ip = ctypes.POINTER(ctypes.c_int)
    lib.ep_probe_mix_shapes.argtypes = [ctypes.c_int]
    lib.ep_probe_mix_shape.argtypes = [ctypes.c_int, ctypes.c_int, ip, ip, ip]
    lib.ep_probe_mix.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, i64, vp]
    lib.ep_probe_empty.argtypes = [vp]
    return lib


def ceilings(torch, nbytes=PROBE_BYTES, iters=20):
    """Practical HBM ceilings on this part: the probe kernels (streaming read
    with and without the non-temporal hint, streaming write plain and
    non-temporal, copy with non-temporal loads, the combine's 8 : 1 and the
    dispatch's 1 : 8 mixes) and HIP's own device copy, each over
    nbytes-sized buffers.  GB/s of bytes moved (a copy counts its reads and
    its writes)."""
    lib = probe_lib()
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    # the row kernels' mixes: 8 planes of nbytes/8 folded into one, and one
    # plane stored to 8 (nbytes + nbytes/8 moved either way)
    plane = nbytes // 8
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream

    def call(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed ({rc})")

    probes = {
        "read_nt": (lambda: call(lib.ep_probe_read(src.data_ptr(), nbytes, 1, sink.data_ptr(), st)), 1),
        "read": (lambda: call(lib.ep_probe_read(src.data_ptr(), nbytes, 0, sink.data_ptr(), st)), 1),
        "write": (lambda: call(lib.ep_probe_write(dst.data_ptr(), nbytes, 0, st)), 1),
        "write_nt": (lambda: call(lib.ep_probe_write(dst.data_ptr(), nbytes, 1, st)), 1),
        "copy": (lambda: call(lib.ep_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, st)), 2),
        "device_copy": (lambda: dst.copy_(src), 2),
    }
    for scatter, name in ((0, "gather8"), (1, "scatter8")):
        for i in range(lib.ep_probe_mix_shapes(scatter)):
            v, nt, w = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
            lib.ep_probe_mix_shape(scatter, i, ctypes.byref(v), ctypes.byref(nt), ctypes.byref(w))
            tag = f"{name}_v{v.value}x{nt.value}" + ("_wait" if w.value else "")
            probes[tag] = ((lambda s=scatter, i=i: call(lib.ep_probe_mix(s, i, src.data_ptr(), dst.data_ptr(),
                                                                         plane, st))), 9 / 8)
    out = {}
    for name, (fn, ways) in probes.items():
        ms = _time_ms(torch, stream, fn, iters)
        out[name + "_gbps"] = ways * nbytes / (ms * 1e-3) / 1e9
    for name in ("gather8", "scatter8"):
        out[name + "_gbps"] = max(v for k, v in out.items() if k.startswith(name + "_v"))
    # launch-to-launch floor of the stream: an empty one-workgroup kernel
    # back to back (what a latency-bound step of n kernels cannot go below n
    # times)
    out["empty_kernel_us"] = 1e3 * _time_ms(torch, stream, lambda: call(lib.ep_probe_empty(st)), 200)
    out["gather8_scatter8_note"] = ("gather8: 8 planes of 128 MiB folded into one (the combine's "
                                   "8 : 1 reads to writes); scatter8: one plane stored to 8 (the "
                                   "dispatch's 1 : 8); each the best of the workgroup shapes listed "
                                   "(vectors per thread x threads, with or without a wait per plane)")
    out["bytes"] = nbytes
    del src, dst
    return out


class Bench:
    """One workload's buffers and bound calls on one stream."""

    def __init__(self, ep, torch, wl, args, fused):
        self.ep, self.torch, self.wl, self.args, self.fused = ep, torch, wl, args, fused
        inp = ep_inputs.make_inputs(wl)
        self.inp = inp
        p = ep.Problem.make(wl.T, wl.H, wl.E, wl.K, wl.R, wl.G, wl.A, 1)
        S = ep.ep_rank_stride_hint(p)      # worst-case symmetric slice, as a real buffer is sized
        p.rank_stride_rows = S
        self.S = S
        dev = torch.device("cuda:0")
        self.dev = dev
        self.d_idx = torch.from_numpy(inp.topk_idx).to(dev)
        self.d_w = torch.from_numpy(inp.topk_weights).to(dev)
        self.d_x = torch.from_numpy(inp.x.view(np.int16)).to(dev)
        self.recv = torch.empty((wl.R * S, wl.H), dtype=torch.int16, device=dev)
        self.recv_src = torch.empty(wl.R * S, dtype=torch.int32, device=dev)
        self.recv_w = torch.empty(wl.R * S, dtype=torch.float32, device=dev)
        self.out = torch.empty((wl.T, wl.H), dtype=torch.int16, device=dev)
        self.stream = torch.cuda.current_stream()
        self.quant_us = None
        if args.fp8:
            nsf = wl.H // 128
            self.nsf = nsf
            # received scale rows token-major, padded to whole 128-byte
            # lines, which the dispatch then writes whole
            self.sf_stride = -(-nsf // 32) * 32
            self.d_q = torch.empty((wl.T, wl.H), dtype=torch.uint8, device=dev)
            self.d_sf = torch.empty((wl.T, nsf), dtype=torch.float32, device=dev)
            self.recv_q = torch.empty((wl.R * S, wl.H), dtype=torch.uint8, device=dev)
            self.recv_sf = torch.empty(wl.R * S * self.sf_stride, dtype=torch.float32, device=dev)
            # quantisation happens upstream of dispatch (in the producing
            # layer); it is timed on its own and not part of the step
            self.quant_us = 1e3 * _time_ms(
                torch, self.stream, lambda: ep.ep_quantize_fp8(p, self.d_x, self.d_q, self.d_sf,
                                                              stream=self.stream), 20)
        if args.hier:
            G = max(wl.G, 2)
            if wl.R % G:
                raise SystemExit(f"--hier needs R divisible by the group count ({wl.R} % {G})")
            p.num_groups = G
            self.G, self.SG = G, wl.T
            self.gslot = torch.empty((wl.T, G), dtype=torch.int32, device=dev)
            self.gbuf = torch.empty((G * self.SG, wl.H), dtype=torch.int16, device=dev)
        self.p = p
        self.bufs = ep.alloc_layout(p, dev)
        self.phases = self.make_calls(self.stream, fused)

    def make_calls(self, st, fused):
        """The step's calls on stream st, marshalled once (bound calls), as
        (layout, dispatch, combine) lists; when fused the layout list is
        empty and the dispatch list holds the one-call layout-and-dispatch."""
        ep, p, a, bufs = self.ep, self.p, self.args, self.bufs
        b = dict(stream=st, bind=True)
        layout = [] if fused else [ep.ep_get_layout(p, self.d_idx, *bufs.args(), **b)]
        if fused and a.fp8:
            dispatch = [ep.ep_layout_dispatch_fp8(p, self.d_idx, *bufs.args(), None, self.d_q, self.d_sf,
                                                  self.d_w, self.recv_q, self.recv_sf, self.sf_stride, 1,
                                                  self.recv_src, self.recv_w, **b)]
        elif fused:
            dispatch = [ep.ep_layout_dispatch(p, self.d_idx, *bufs.args(), None, self.d_x, self.d_w,
                                              self.recv, self.recv_src, self.recv_w, **b)]
        elif a.hier:
            dispatch = [ep.ep_get_group_layout(p, bufs.is_token_in_rank, self.SG, self.gslot,
                                               bufs.workspace, **b),
                        ep.ep_dispatch_hier(p, self.d_x, self.d_w, bufs.token_slot, self.gslot, self.SG,
                                            self.gbuf, self.recv, self.recv_src, self.recv_w, **b)]
        elif a.fp8:
            dispatch = [ep.ep_dispatch_fp8(p, self.d_q, self.d_sf, self.d_w, bufs.token_slot, self.recv_q,
                                           self.recv_sf, self.sf_stride, 1, self.recv_src, self.recv_w, **b)]
        else:
            dispatch = [ep.ep_dispatch(p, self.d_x, self.d_w, bufs.token_slot, self.recv, self.recv_src,
                                       self.recv_w, **b)]
        if a.hier:
            combine = [ep.ep_combine_hier(p, self.recv, bufs.token_slot, self.d_w, self.gslot, self.SG,
                                          self.gbuf, self.out, **b)]
        else:
            combine = [ep.ep_combine(p, self.recv, bufs.token_slot, self.d_w, self.out, **b)]
        return layout, dispatch, combine

    @staticmethod
    def run(calls):
        for f in calls:
            f()

    def step(self, ev=None, calls=None):
        calls = self.phases if calls is None else calls
        for k, part in enumerate(calls):
            if ev is not None:
                ev[k].record(self.stream)
            self.run(part)
        if ev is not None:
            ev[3].record(self.stream)

    def check_status(self):
        self.torch.cuda.synchronize()
        status = self.ep.ep_read_status(self.bufs.workspace, self.stream)
        if status != self.ep.EP_OK:
            raise RuntimeError(f"layout status {self.ep.error_string(status)}")

    def timed_steps(self, steps, warmup, run_step=None):
        """Mean ms per step: exactly `steps` steps between two HIP events on
        the stream the kernels run on (no events inside: each extra event
        record leaves the GPU idle for a few microseconds)."""
        torch = self.torch
        run_step = run_step or self.step
        for _ in range(warmup):
            run_step()
        self.check_status()
        e_start = torch.cuda.Event(enable_timing=True)
        e_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e_start.record(self.stream)
        for _ in range(steps):
            run_step()
        e_end.record(self.stream)
        torch.cuda.synchronize()
        self.wall_s = time.perf_counter() - t0
        return e_start.elapsed_time(e_end) / steps

    def phase_us(self, steps, calls=None):
        """Mean µs per phase: the same steps again, each phase bracketed by
        HIP events on the same stream."""
        torch = self.torch
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for _ in range(3):
            self.step(calls=calls)
        torch.cuda.synchronize()
        for i in range(steps):
            self.step(events[i], calls=calls)
        torch.cuda.synchronize()
        return {k: float(np.mean([e[n].elapsed_time(e[n + 1]) for e in events])) * 1e3
                for n, k in enumerate(("layout", "dispatch", "combine"))}

    def cold_phase_us(self, steps):
        """Mean µs per phase with the last-level cache flushed before each
        phase, outside the timed event pair, as expert compute between the
        phases would: a plain read of 512 MiB (larger than the 256 MB MALL)
        evicts what the cache held and writes back the previous phase's dirty
        lines, and leaves no dirty lines of its own whose write-back would
        land in the timed phase (a fill would)."""
        torch = self.torch
        lib = probe_lib()
        flush_bytes = 512 << 20
        scratch = torch.ones(flush_bytes, dtype=torch.uint8, device=self.dev)
        sink = torch.zeros(4, dtype=torch.uint8, device=self.dev)
        st = self.stream.cuda_stream

        def flush():
            if lib.ep_probe_read(scratch.data_ptr(), flush_bytes, 0, sink.data_ptr(), st) != 0:
                raise RuntimeError("flush read failed")

        cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            ev = cold_ev[i]
            for k, part in enumerate(self.phases):
                flush()
                ev[2 * k].record(self.stream)
                self.run(part)
                ev[2 * k + 1].record(self.stream)
        torch.cuda.synchronize()
        del scratch
        return {k: float(np.mean([e[2 * n].elapsed_time(e[2 * n + 1]) for e in cold_ev])) * 1e3
                for n, k in enumerate(("layout", "dispatch", "combine"))}

    def fuse(self, d):
        """Layout and dispatch as one phase when they are one call."""
        if d is None or not self.fused:
            return d
        d = dict(d)
        return {"layout_dispatch": d.pop("layout") + d.pop("dispatch"), **d}


def decode_figures(ep, torch, args, steps=200):
    """µs per call of the decode-sized batch (128 tokens, hidden 7168, top-8
    of 256 experts, 8 ranks): the whole step in a timed region, and each
    call with an event pair, warm and after a cache flush."""
    wl = ep_inputs.WORKLOADS[DECODE_WORKLOAD]
    b = Bench(ep, torch, wl, args, fused=True)
    ms = b.timed_steps(steps, 20)
    return b, {
        "workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "K": wl.K, "R": wl.R,
        "us_per_step": ms * 1e3,
        "us_per_phase": b.fuse(b.phase_us(steps)),
        "us_per_phase_cold": b.fuse(b.cold_phase_us(50)),
        "steps": steps,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE_WORKLOAD, choices=sorted(ep_inputs.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the per-phase times after a 512 MiB cache flush")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-sized batch's per-call figures")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the bandwidth probes")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 --pmc: only the timed steps, the per-phase pass and "
                         "the probes that calibrate the counters (no two-call, cold, decode or CPU legs)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time graph replays (no host launch cost)")
    ap.add_argument("--hier", action="store_true",
                    help="two-level path: group layout, dispatch via the group buffer, per-group partial combine")
    ap.add_argument("--two-calls", action="store_true",
                    help="layout and dispatch as two calls (ep_get_layout + ep_dispatch) instead of the "
                         "one-call ep_layout_dispatch")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 dispatch (e4m3 rows + per-128-channel scales); combine stays bf16")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="build profiles/traffic.json from rocprofv3 --pmc counter CSVs (no GPU needed)")
    args = ap.parse_args()
    if args.counters:
        args.no_cold = args.no_decode = args.no_cpu_baseline = True
    # the two-level path needs the layout's slots before its group stage
    fused = not (args.two_calls or args.hier)

    # counter records are kept per workload and mode
    traffic_key = (args.workload + ("+fp8" if args.fp8 else "") + ("+two-level" if args.hier else "")
                   + ("" if fused else "+two-calls"))
    if args.write_traffic:
        wkey = args.workload + ("+fp8" if args.fp8 else "") + ("+two-level" if args.hier else "")
        print(json.dumps(write_traffic(wkey, *args.write_traffic), indent=1))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the hot path; --gpus {args.gpus} is not "
              "supported (multi-GPU dispatch/combine is not built: one GPU only).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import combine_ep_get_amd as ep

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    ep.load()

    wl = ep_inputs.WORKLOADS[args.workload]
    # the decode-sized batch first, on a fresh device: measured after the
    # 16384-token workload's 30 GB buffers, its step read about 1 µs slower
    decode = None
    if not args.no_decode and wl.name != DECODE_WORKLOAD and not (args.fp8 or args.hier or args.graph):
        db, decode = decode_figures(ep, torch, args)
        del db
        torch.cuda.empty_cache()
    b = Bench(ep, torch, wl, args, fused)

    run_step = b.step
    if args.graph:
        # one step captured once (on a side stream, as capture requires) and
        # replayed on the bench stream
        side = torch.cuda.Stream()
        side.wait_stream(b.stream)
        torch.cuda.synchronize()
        side_calls = b.make_calls(side, fused)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            b.step(calls=side_calls)
        torch.cuda.synchronize()
        run_step = graph.replay

    ms_step = b.timed_steps(args.steps, args.warmup, run_step)
    t_wall = b.wall_s
    phase = b.phase_us(args.steps)
    # the same steps as two calls, so that the layout and the dispatch are
    # also timed apart
    two_call_us = (b.phase_us(args.steps, calls=b.make_calls(b.stream, False))
                   if fused and not args.counters else None)
    cold = None if args.no_cold else b.cold_phase_us(args.steps)

    nbytes = algorithmic_bytes(wl, fp8=args.fp8)
    if args.hier:
        # the two-level path also writes each (token, group) row into the
        # group buffer and reads it back, once in dispatch and once in
        # combine; its dispatch phase also derives the group slots (reads the
        # rank map, writes [T,G] slots)
        group_rows = int(b.bufs.group_token_count.sum().item())
        nbytes["dispatch"] += wl.T * wl.R + 4 * wl.T * b.G + 2 * group_rows * wl.H * 2
        nbytes["combine"] += 2 * group_rows * wl.H * 2
    total_bytes = sum(nbytes.values())
    eff_gbps = total_bytes / (ms_step * 1e-3) / 1e9
    phase, cold = b.fuse(phase), b.fuse(cold)
    if fused:
        nbytes = {"layout_dispatch": nbytes["layout"] + nbytes["dispatch"], "combine": nbytes["combine"]}
    cold_step_us = sum(cold.values()) if cold else None

    dominant = max((k for k in ("dispatch", "layout_dispatch", "combine") if k in phase),
                   key=lambda k: phase[k])
    achieved = nbytes[dominant] / (phase[dominant] * 1e-6) / 1e9
    # the FP8 mode runs the very same combine launch as the bf16 mode (bf16
    # expert outputs), so the bf16 counter record applies to it
    traffic = measured_traffic(args.workload if args.fp8 and dominant == "combine" else traffic_key,
                               dominant)
    roofline = {
        "kernel": dominant,
        "kernel_note": ("the one-call layout and dispatch: the count pass and the dispatching kernel"
                        if dominant == "layout_dispatch" else dominant),
        "bound": "hbm",
        "achieved": achieved,
        "peak": PEAK_HBM_GBPS,
        "unit": "GB/s",
        "frac": achieved / PEAK_HBM_GBPS,
        "traffic": traffic,
        "algorithmic_bytes": nbytes[dominant],
        "achieved_cold": nbytes[dominant] / (cold[dominant] * 1e-6) / 1e9 if cold else None,
    }
    if cold:
        roofline["frac_cold"] = roofline["achieved_cold"] / PEAK_HBM_GBPS

    result = {
        "metric": METRIC,
        "value": wl.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 dispatch, bf16 combine" if args.fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "K": wl.K, "R": wl.R,
                   "G": b.p.num_groups, "A": wl.A, "S": b.S, "routing": wl.routing, "seed": wl.seed,
                   "dispatch": "fp8" if args.fp8 else "bf16",
                   **({"recv_sf": f"token-major, rows of {b.sf_stride} floats (H/128 padded to 128-byte lines)"}
                      if args.fp8 else {}),
                   "path": "two-level (group buffer)" if args.hier else "flat",
                   "layout_dispatch": ("one call (ep_layout_dispatch_fp8)" if args.fp8 else
                                       "one call (ep_layout_dispatch)") if fused else "two calls",
                   "launch": "hip_graph" if args.graph else "eager"},
        "effective_hbm_gbps": eff_gbps,
        "frac_of_peak_hbm": eff_gbps / PEAK_HBM_GBPS,
        "us_per_step": ms_step * 1e3,
        "us_per_phase": phase,
        "us_per_phase_note": "separate pass of the same steps with an event pair around each call",
        "us_per_phase_cold": cold,
        "us_per_step_cold": cold_step_us,
        "effective_hbm_gbps_cold": total_bytes / (cold_step_us * 1e-6) / 1e9 if cold_step_us else None,
        "cold_note": "each phase after a plain 512 MiB read (larger than the 256 MB last-level cache); "
                     "the cold step is the sum of the cold phases",
        "us_per_phase_two_calls": two_call_us,
        "us_quantize_fp8": b.quant_us,
        "wall_s_timed": t_wall,
        "roofline": roofline,
    }
    b.check_status()
    inp, S = b.inp, b.S
    del b

    if decode is not None:
        result["us_per_step_decode128"] = decode["us_per_step"]
        result["decode128"] = decode
    if not args.no_ceilings:
        torch.cuda.empty_cache()
        c = ceilings(torch)
        result["ceilings"] = c
        result["copy_ceiling_gbps"] = c["device_copy_gbps"]
    if not args.no_cpu_baseline and not args.fp8 and not args.hier:
        result["cpu_baseline"] = cpu_baseline(wl, inp, S)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
