#!/usr/bin/env python3
"""Throughput of the 1-bit Adam step on one MI355X.

Default workload: a Llama-2-7B-sized flat buffer (6,738,415,616 elements, bf16 gradients, fp32 state,
scale chunks of 2^24) with the tutorial's variant of the step (clip at 5, EMA error feedback, int8
signs) and a variance refresh every 16th step.  The schedule's dense steps -- the warmup steps before
freeze_step (BERT-base) or refresh steps (Llama-2-7B) -- run first and are timed on their own; then
`--warmup` untimed compressed steps; then `--steps` timed compressed steps, the compressed phase whose
step time the pages' acceptance table names.  One JSON line is printed.

Inputs are synthetic and resident in HBM before timing starts: a ring of up to 4 pre-drawn gradients
(seeded) is cycled, so no random generation runs inside the timed region.  Before any timing, every
kernel runs once on a small scratch plan, so no timed launch pays for loading the device code.

Other workloads: --workload NAME (see adam_ob_compress_amd/synth.py: GPT-2-1.5B, Llama-2-7B, LAMB and
16-bit error variants); --workload 'server-2^28-W8' times a server round (ob_server_reduce + ob_unpack)
instead of an optimizer step; --split times the worker step split at the exchange.

Other modes:
  --rocprof-summary DIR   summarise rocprofv3 CSV output found under DIR (kernel trace per kernel and
                          grid size, and FETCH_SIZE / WRITE_SIZE counters per dispatch) as markdown.
  --traffic-profile DIR   from the FETCH_SIZE and WRITE_SIZE runs under DIR (made with
                          --copy-probe-mib 1024), write the calibrated HBM traffic of --kernel on
                          --workload as markdown on stdout (the profiles/traffic_*.md format).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "elements/s and achieved HBM GB/s (% of peak) of fused 1-bit Adam step, 1 GPU"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
DEFAULT_WORKLOAD = "llama2-7B-bf16-ema"
# the kernels and the host code that sizes their launches (block tables): a change to any of them makes
# the committed counter summaries stale
KERNEL_SOURCES = ("adam_ob_compress_amd/csrc/ob_compress.hip", "adam_ob_compress_amd/csrc/ob_kernels.hip",
                  "adam_ob_compress_amd/csrc/ob_device.h", "adam_ob_compress_amd/csrc/ob_internal.h",
                  "adam_ob_compress_amd/csrc/ob_tables.h", "adam_ob_compress_amd/csrc/ob_api.cpp")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def bytes_per_elem(w, kernel: str) -> float:
    """Algorithmic (compulsory) HBM bytes per element of one launch of `kernel` on workload w."""
    gb = 2.0 if w.grad_dtype == "bf16" else 4.0
    eb = 4.0 if w.err_dtype == "f32" else 2.0
    sb = 1.0 if w.int8_signs else 0.0
    lamb = w.optimizer == "lamb"
    if kernel == "compress":          # read g err m v p, write err m p + 1 bit (+ int8 sign)
        if lamb:                      # LAMB pass 2: no p; read g err m v, write err m + bits
            return gb + eb + 8.0 + eb + 4.0 + 0.125 + sb
        return gb + eb + 12.0 + eb + 8.0 + 0.125 + sb
    if kernel == "worker_compress":   # read g err, write err + 1 bit (+ int8 sign)
        return gb + eb + eb + 0.125 + sb
    if kernel == "worker_update":     # read 1 bit m v p, write m p (LAMB: m only)
        return 0.125 + 12.0 + (4.0 if lamb else 8.0)
    if kernel == "chunk_sumsq":       # read g err (LAMB: and p)
        return gb + eb + (4.0 if lamb else 0.0)
    if kernel == "dense":             # read g m v p, write m v p (LAMB: m v only)
        return gb + 12.0 + (8.0 if lamb else 12.0)
    if kernel == "lamb_apply":        # read m v p, write p
        return 16.0
    if kernel in ("trust_ratio", "diag", "scale"):   # one block per chunk over the per-block partial sums
        return 0.0
    if kernel == "server_sumsq":      # read W sign bits and the server error
        return w.workers / 8.0 + 4.0
    if kernel == "server_apply":      # read W bits + error, write error + 1 bit
        return w.workers / 8.0 + 4.0 + 4.0 + 0.125
    if kernel == "unpack":            # read 1 bit, write fp32
        return 0.125 + 4.0
    raise KeyError(kernel)


def step_compulsory_bytes(w, kind: str) -> float:
    """Bytes per element the method must move once per step: every array read and written once (the
    re-reads that the per-chunk scale and LAMB's per-layer ratio force are not counted)."""
    import dataclasses
    adam = dataclasses.replace(w, optimizer="adam")   # LAMB touches the same arrays once each
    if kind == "dense":
        return bytes_per_elem(adam, "dense")
    if w.workers:
        return w.workers / 8.0 + 4.0 + 4.0 + 0.125 + bytes_per_elem(w, "unpack")
    return bytes_per_elem(adam, "compress")


def load_traffic(kernel: str, workload: str):
    """Counter-derived HBM bytes per launch from profiles/, or None if absent or stale."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic-json:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("kernel_src_sha") != kernel_source_sha():
                return None
            return rec.get("bytes_per_launch")
    return None


# ------------------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, single thread, on a bounded sample
# ------------------------------------------------------------------------------------------------

def host_info() -> dict:
    """The host the CPU baseline ran on: logical CPUs, the CPUs this process may use, the CPU model."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


# threads of the all-cores oracle line: the CPUs this process may use, at most 16 (one GPU's share of
# the host's cores)
MAX_CPU_THREADS = 16


def _sample(w, limit: int):
    """Whole chunks of w from the start until `limit` elements: (K, n_s, workload of those chunks)."""
    import dataclasses

    from adam_ob_compress_amd import synth

    off = w.chunk_offsets()
    K = 1
    while K < w.n_chunks and off[K] < limit:
        K += 1
    n_s = int(off[K])
    if w.offsets is None:
        return K, n_s, synth.scaled(w, n_s, w.chunk)
    return K, n_s, dataclasses.replace(w, n=n_s, offsets=tuple(int(o) for o in off[:K + 1]))


def cpu_baseline(w, seconds: float):
    """The oracle as it stands on a bounded sample of the workload: single thread (the reported value),
    and the same oracle run chunk-parallel on up to MAX_CPU_THREADS threads (one chunk per task; the
    oracle releases the GIL) as a second line."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    from adam_ob_compress_amd import synth

    # whole chunks from the start until ~2^27 elements (all of BERT-base); 2^25 for the server round,
    # whose oracle runs ~8x slower per element (W workers' bits per element)
    K, n_s, sub = _sample(w, (1 << 25) if w.workers else (1 << 27))
    host = host_info()
    if w.workers:
        res = _cpu_baseline_server(w, sub, K, sub.chunk_offsets(), seconds)
        res["host"] = host
        return res
    step = oracle.lamb_compress_step if w.optimizer == "lamb" else oracle.compress_step
    hp = dict(lr=w.lr, beta1=w.beta1, eps=w.eps, clip=w.clip, ef_mode=w.ef_mode, ef_beta=w.ef_beta,
              want_signs=w.int8_signs)

    def sr(s, index0=0):
        return (dict(stochastic=True, sr_seed=synth.SR_SEED, sr_step=s, sr_index0=index0)
                if w.err_rounding == "stochastic" else {})

    offs = sub.chunk_offsets()
    err, m, v, p = (synth.host(t) for t in synth.draw_state(sub, "cpu"))
    g = synth.host(synth.draw_grad(sub, 0, "cpu"))
    times = []
    t_end = time.perf_counter() + seconds
    while len(times) < 2 or (time.perf_counter() < t_end and len(times) < 20):
        t0 = time.perf_counter()
        step(g, err, m, v, p, offs, **hp, **sr(len(times)))
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    res = {"value": n_s / t, "unit": "elements/s", "cores": 1, "kind": "oracle",
           "sample": f"{len(times)} compressed steps of the oracle on the first {K} chunks "
                     f"({n_s} elements) of {w.name}, single thread, median step {t:.3f} s",
           "host": host}
    del err, m, v, p, g

    # the same oracle, one chunk per task on all usable CPUs (at most MAX_CPU_THREADS), over as many
    # chunks as threads when the workload has them
    threads = max(1, min(MAX_CPU_THREADS, host["usable_cpus"] or 1))
    if w.n_chunks < 2 or threads < 2:
        return res
    Kp, n_p, subp = _sample(w, threads * int(w.chunk_offsets()[1]))
    Kp = min(Kp, w.n_chunks)
    offp = subp.chunk_offsets()
    state = [synth.host(t) for t in synth.draw_state(subp, "cpu")]
    gp = synth.host(synth.draw_grad(subp, 0, "cpu"))
    slices = [(int(offp[c]), int(offp[c + 1])) for c in range(Kp)]
    views = [[a[lo:hi] for a in (gp, *state)] for lo, hi in slices]

    def chunk(c, s):
        lo, hi = slices[c]
        gg, ee, mm, vv, pp = views[c]
        step(gg, ee, mm, vv, pp, np.asarray([0, hi - lo], np.int64), **hp, **sr(s, lo))

    times = []
    t_end = time.perf_counter() + seconds
    with cf.ThreadPoolExecutor(max_workers=threads) as pool:
        while len(times) < 2 or (time.perf_counter() < t_end and len(times) < 20):
            t0 = time.perf_counter()
            for f in [pool.submit(chunk, c, len(times)) for c in range(Kp)]:
                f.result()
            times.append(time.perf_counter() - t0)
    tp = float(np.median(times))
    res["all_cores"] = {"value": n_p / tp, "unit": "elements/s", "cores": min(threads, Kp), "kind": "oracle",
                        "sample": f"{len(times)} compressed steps of the oracle on the first {Kp} chunks "
                                  f"({n_p} elements) of {w.name}, one chunk per task on "
                                  f"{min(threads, Kp)} threads, median step {tp:.3f} s"}
    return res


def _cpu_baseline_server(w, sub, K, offs, seconds):
    import numpy as np

    import oracle
    from adam_ob_compress_amd import synth

    ww = synth.host(synth.draw_worker_words(sub, 0, "cpu"))
    ws = synth.host(synth.draw_worker_scales(sub, 0, "cpu"))
    err = np.zeros(sub.n, np.float32)
    times = []
    t_end = time.perf_counter() + seconds
    while len(times) < 2 or (time.perf_counter() < t_end and len(times) < 20):
        t0 = time.perf_counter()
        rw, rs = oracle.server_reduce(ww, ws, err, offs)
        oracle.unpack(rw, sub.n, offs, rs)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": sub.n / t, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(times)} server rounds (reduce + unpack) of the oracle on the first {K} chunks "
                      f"({sub.n} elements) of {w.name}, single thread, median round {t:.3f} s"}


# ------------------------------------------------------------------------------------------------
# GPU run
# ------------------------------------------------------------------------------------------------

def run(args):
    import torch

    import adam_ob_compress_amd as ob
    from adam_ob_compress_amd import schedule, synth

    w = synth.WORKLOADS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if w.workers:
        return w, run_server(args, w)
    plan = ob.ob_plan_create(w.n, chunk_size=w.chunk if w.offsets is None else 0, chunk_offsets=w.offsets)
    ring = 1 if w.n > (1 << 31) else min(4, max(1, args.steps))
    if args.slab:
        err, m, v, p, grads = slab_buffers(w, ring, dev, args.slab_stagger)
        synth.draw_state(w, dev, out=(err, m, v, p))
        grads = [synth.draw_grad(w, s, dev, out=grads[s]) for s in range(ring)]
    else:
        err, m, v, p = synth.draw_state(w, dev)
        grads = [synth.draw_grad(w, s, dev) for s in range(ring)]
    cls = schedule.OneBitLamb if w.optimizer == "lamb" else schedule.OneBitAdam
    opt = cls(plan, err, m, v, p, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                              clip=w.clip, ef_mode=w.ef_mode, ef_beta=w.ef_beta, int8_signs=w.int8_signs,
                              freeze_step=w.freeze_step, refresh_period=w.refresh_period,
                              diagnostics=args.diagnostics, err_rounding=w.err_rounding,
                              sr_seed=synth.SR_SEED)
    stream = torch.cuda.current_stream()
    print(f"# {w.name}: n={w.n} chunks={plan.num_chunks} blocks={plan.num_blocks} "
          f"block_elems={plan.block_elems}", file=sys.stderr, flush=True)

    warm_kernels(w, opt, dev)
    # the schedule's dense steps, timed on their own with events: the warmup steps before freeze_step,
    # or (a refresh schedule) two of its refresh steps
    dense_ms, dense_kind, dense_n = None, None, 0
    if w.freeze_step or w.refresh_period:
        ob.ob_plan_set_timing(plan, True)
        if w.freeze_step:
            dense_kind = "warmup"
            for s in range(w.freeze_step):
                assert opt.step(grads[s % ring]) == "dense"
        else:
            dense_kind = f"refresh (every {w.refresh_period}th step)"
            for r in range(2):
                opt.step_index = (r + 1) * w.refresh_period - 1
                assert opt.step(grads[r % ring]) == "dense"
            opt.step_index = 0
        torch.cuda.synchronize()
        ms, dense_n = ob.ob_plan_read_timing(plan, ob.OB_KERNEL_DENSE)
        dense_ms = ms / max(dense_n, 1)
        ob.ob_plan_set_timing(plan, False)
    # the timed steps are the compressed phase; the refresh steps its schedule inserts are timed above
    opt.refresh_period = 0

    step = opt.step
    if args.split:
        def step(g, s=None):
            # the worker's step split at the exchange, with one worker: its own words are the exchange's
            ob.ob_adam_worker_compress(plan, g, err, opt.words, opt.scales, opt.hp, opt.signs, None, s)
            if w.optimizer == "lamb":
                ob.ob_lamb_worker_update(plan, opt.words, opt.scales, m, v, p, opt.ratios, opt.hp, s)
            else:
                ob.ob_adam_worker_update(plan, opt.words, opt.scales, m, v, p, opt.hp, s)
            return "compressed"

    for k in range(args.warmup):
        step(grads[k % ring])
    torch.cuda.synchronize()

    ob.ob_plan_set_timing(plan, True)
    kinds = {"dense": 0, "compressed": 0}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        kinds[step(grads[k % ring], stream)] += 1
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    kern = kernel_times(plan, w.n, args.steps, w)
    ob.ob_plan_set_timing(plan, False)

    if args.copy_probe_mib:
        kern["copy_probes"] = copy_probe(args.copy_probe_mib, dev)

    # the dominant kernel of the timed steps: the most time per step (the fused pass 2 for 1-bit Adam)
    dom = max((k for k in ("compress", "lamb_apply", "worker_compress", "worker_update") if k in kern),
              key=lambda k: kern[k]["ms_per_step"])
    traffic = load_traffic(dom, w.name)
    value = w.n / (ms_per_step * 1e-3)
    step_gbps = step_compulsory_bytes(w, "compressed") * w.n / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic: compensation and the stored state in fp32, each formula line evaluated in
        # fp64 and rounded once (the storage types are in config)
        "dtype": "f32",
        "data": f"synthetic (seeded; {ring} pre-drawn gradient{'s' if ring > 1 else ''} cycled)",
        "config": {"workload": w.name, "elements": w.n, "chunks": plan.num_chunks,
                   "optimizer": "1-bit " + ("LAMB" if w.optimizer == "lamb" else "Adam"),
                   "grad_dtype": w.grad_dtype, "err_dtype": w.err_dtype, "err_rounding": w.err_rounding,
                   "state_dtype": "f32", "formula_dtype": "f64",
                   "clip": w.clip,
                   "error_feedback": "ema" if w.ef_mode else "plain", "int8_signs": w.int8_signs,
                   "freeze_step": w.freeze_step, "refresh_period": w.refresh_period,
                   "block_elems": plan.block_elems, "work_blocks": plan.num_blocks,
                   "diagnostics": bool(args.diagnostics), "split": bool(args.split),
                   "slab": bool(args.slab), "slab_stagger": args.slab_stagger if args.slab else None},
        "roofline": roofline_of(kern, dom, w, traffic),
        "step_compulsory_GBps": step_gbps,
        "step_hbm_frac": step_gbps / PEAK_HBM_GBPS,
        "timed_step_kinds": kinds,
        "dense_step_ms": dense_ms,
        "dense_step": None if dense_ms is None else {
            "kind": dense_kind, "steps_timed": dense_n, "avg_ms": dense_ms,
            "elements_per_s": w.n / (dense_ms * 1e-3),
            "GBps": bytes_per_elem(w, "dense") * w.n / (dense_ms * 1e-3) / 1e9,
            "bytes_per_elem": bytes_per_elem(w, "dense")},
        "kernels": kern,
        "kernel_src_sha": kernel_source_sha(),
        "cpu_baseline": None,
    }
    return w, res


def kernel_times(plan, n: int, steps: int, w) -> dict:
    """Per kernel kind, from the plan's event timing over `steps` timed steps: launches, average launch
    duration, and the kernel's time per step.  A kernel launched once per chunk group runs several times a
    step; its rate is the step's algorithmic bytes over its time per step, which is the same as the
    average elements per launch over the average launch duration."""
    from adam_ob_compress_amd import _native as ob

    kern = {}
    for kid, name in ob.KERNEL_NAMES.items():
        ms, cnt = ob.ob_plan_read_timing(plan, kid)
        if cnt:
            per_step = ms / steps
            kern[name] = {"avg_ms": ms / cnt, "launches": cnt, "launches_per_step": cnt / steps,
                          "ms_per_step": per_step,
                          "GBps": bytes_per_elem(w, name) * n / (per_step * 1e-3) / 1e9}
    return kern


def roofline_of(kern: dict, dom: str, w, traffic) -> dict:
    """The roofline record of the dominant kernel (see kernel_times for the per-launch reading)."""
    k = kern[dom]
    bpe = bytes_per_elem(w, dom)
    elems = w.n / k["launches_per_step"]
    achieved = bpe * elems / (k["avg_ms"] * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS, "bytes_per_elem": bpe, "launches_per_step": k["launches_per_step"],
            "elements_per_launch": elems, "avg_launch_ms": k["avg_ms"], "traffic": traffic}


SLAB_ALIGN = 2 << 20


def slab_buffers(w, ring: int, dev: str, stagger: int = 0):
    """err, m, v, p and `ring` gradients carved from one device allocation, each at a 2 MiB-aligned
    offset plus j * stagger bytes for array j (an allocation-strategy experiment: all arrays then come
    from one allocation, at chosen distances from each other)."""
    import torch

    from adam_ob_compress_amd import synth

    kinds = [synth.ERR_TORCH_DTYPES[w.err_dtype]] + [torch.float32] * 3
    kinds += [torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32] * ring
    sizes = [w.n * torch.empty(0, dtype=k).element_size() for k in kinds]
    assert stagger % 256 == 0
    offs, total = [], 0
    for j, b in enumerate(sizes):
        offs.append(total + j * stagger)
        total += (b + SLAB_ALIGN - 1) // SLAB_ALIGN * SLAB_ALIGN
    total += len(sizes) * stagger
    slab = torch.empty(total + SLAB_ALIGN, dtype=torch.uint8, device=dev)
    shift = (-slab.data_ptr()) % SLAB_ALIGN
    views = [slab[shift + o:shift + o + b].view(k) for o, b, k in zip(offs, sizes, kinds)]
    return views[0], views[1], views[2], views[3], views[4:]


def warm_kernels(w, opt, dev: str):
    """One dense and one compressed step of the same kernels on a small scratch buffer, untimed, so
    that no timed launch pays for the first-use loading of the library's device code.  The workload's
    own state is not touched."""
    import torch

    import adam_ob_compress_amd as ob
    from adam_ob_compress_amd import schedule

    n = WARM_N
    plan = ob.ob_plan_create(n, chunk_size=1 << 14)
    gdt = torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32
    edt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.err_dtype]
    err = torch.zeros(n, dtype=edt, device=dev)
    m, v, p = (torch.zeros(n, device=dev) for _ in range(3))
    cls = schedule.OneBitLamb if w.optimizer == "lamb" else schedule.OneBitAdam
    scratch = cls(plan, err, m, v, p, lr=w.lr, clip=w.clip, ef_mode=w.ef_mode, ef_beta=w.ef_beta,
                  int8_signs=w.int8_signs, freeze_step=1, err_rounding=w.err_rounding,
                  sr_seed=opt.hp.sr_seed)
    g = torch.ones(n, dtype=gdt, device=dev)
    scratch.step(g)      # dense
    scratch.step(g)      # compressed
    ob.ob_adam_worker_compress(plan, g, err, scratch.words, scratch.scales, scratch.hp)
    if w.optimizer == "lamb":
        ob.ob_lamb_worker_update(plan, scratch.words, scratch.scales, m, v, p, scratch.ratios, scratch.hp)
    else:
        ob.ob_adam_worker_update(plan, scratch.words, scratch.scales, m, v, p, scratch.hp)
    torch.cuda.synchronize()
    plan.destroy()


def copy_probe(mib: int, dev: str) -> dict:
    """Copies of `mib` MiB, each 3 untimed + 5 timed: a plain torch copy (ordinary loads and stores)
    and the probe library's copy with nontemporal loads and stores (the library's streaming kernels'
    access kind).  They are the counters' calibration runs and practical bandwidth references."""
    import ctypes

    import torch

    from adam_ob_compress_amd import build

    nb = mib << 20
    src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    probe = ctypes.CDLL(build.PROBE_LIB)
    probe.ob_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    probe.ob_probe_copy.restype = ctypes.c_int
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def nt_copy():
        rc = probe.ob_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nb, 1, stream)
        if rc != 0:
            raise RuntimeError(f"ob_probe_copy failed ({rc})")

    out = {}
    for name, copy in (("torch_copy", lambda: dst.copy_(src)), ("nontemporal_copy", nt_copy)):
        for _ in range(3):
            copy()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(5):
            copy()
        ev1.record()
        torch.cuda.synchronize()
        out[name] = {"bytes_per_launch": 2 * nb, "GBps": 2 * nb / (ev0.elapsed_time(ev1) / 5 * 1e-3) / 1e9}
    assert torch.equal(src, dst)
    return out


def run_server(args, w):
    """One "step" is a server round on one GPU's share: ob_server_reduce over W workers' packed signs
    and scales (pass 1 + pass 2), then ob_unpack of the re-packed result.  W rows of words and scales
    are pre-drawn for two rounds and alternated; the server error carries across rounds."""
    import torch

    import adam_ob_compress_amd as ob
    from adam_ob_compress_amd import synth

    dev = "cuda:0"
    plan = ob.ob_plan_create(w.n, chunk_size=w.chunk)
    K = plan.num_chunks
    ww = [synth.draw_worker_words(w, r, dev) for r in range(2)]
    ws = [synth.draw_worker_scales(w, r, dev) for r in range(2)]
    err = torch.zeros(w.n, dtype=torch.float32, device=dev)
    words = torch.empty((w.n + 31) // 32, dtype=torch.int32, device=dev)
    scales = torch.empty(K, dtype=torch.float32, device=dev)
    out = torch.empty(w.n, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    print(f"# {w.name}: n={w.n} W={w.workers} chunks={K}", file=sys.stderr, flush=True)

    def rnd(r):
        ob.ob_server_reduce(plan, ww[r % 2], ws[r % 2], err, words, scales, stream)
        ob.ob_unpack(plan, words, w.n, out, scales, stream)

    for r in range(args.warmup):
        rnd(r)
    torch.cuda.synchronize()
    ob.ob_plan_set_timing(plan, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(args.steps):
        rnd(r)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern = kernel_times(plan, w.n, args.steps, w)
    ob.ob_plan_set_timing(plan, False)
    if args.copy_probe_mib:
        kern["copy_probes"] = copy_probe(args.copy_probe_mib, dev)
    dom = max((k for k in ("server_sumsq", "server_apply", "unpack") if k in kern),
              key=lambda k: kern[k]["ms_per_step"])
    step_gbps = step_compulsory_bytes(w, "server") * w.n / (ms_per_step * 1e-3) / 1e9
    return {
        "metric": METRIC,
        "value": w.n / (ms_per_step * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32 sign words + f32 scales and error",
        "data": "synthetic (seeded; two pre-drawn rounds of worker words and scales)",
        "config": {"workload": w.name, "elements": w.n, "chunks": K, "workers": w.workers,
                   "step": "server round: ob_server_reduce (2 passes) + ob_unpack"},
        "roofline": roofline_of(kern, dom, w, load_traffic(dom, w.name)),
        "step_compulsory_GBps": step_gbps,
        "step_hbm_frac": step_gbps / PEAK_HBM_GBPS,
        "timed_step_kinds": {"server_round": args.steps},
        "dense_step_ms": None,
        "kernels": kern,
        "kernel_src_sha": kernel_source_sha(),
        "cpu_baseline": None,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also copy this many MiB with torch and with the probe's nontemporal "
                         "copy (counter calibration)")
    ap.add_argument("--split", action="store_true",
                    help="time the worker step split at the exchange (worker compress + worker update, "
                         "one worker) instead of the fused compressed step")
    ap.add_argument("--slab", action="store_true",
                    help="place the state arrays and gradients in one allocation at 2 MiB-aligned offsets")
    ap.add_argument("--slab-stagger", type=int, default=0,
                    help="with --slab: array j starts j times this many bytes (a multiple of 256) later")
    ap.add_argument("--diagnostics", action="store_true",
                    help="also compute the per-chunk error norm and +1 count in every compressed step")
    ap.add_argument("--rocprof-summary", metavar="DIR")
    ap.add_argument("--traffic-profile", metavar="DIR")
    ap.add_argument("--kernel", default="compress")
    args = ap.parse_args()

    if args.rocprof_summary:
        print(rocprof_summary(args.rocprof_summary))
        return 0
    if args.traffic_profile:
        print(traffic_profile(args.traffic_profile, args.kernel, args.workload))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): the "
              "compressed step is one GPU's share; the multi-GPU exchange is not implemented here.",
              file=sys.stderr)
        return 2
    w, res = run(args)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


# ------------------------------------------------------------------------------------------------
# rocprofv3 CSV summaries
# ------------------------------------------------------------------------------------------------

def _short(name: str) -> str:
    for key in ("k_chunk_sumsq", "k_compress", "k_dense", "k_server_sumsq_lines", "k_server", "k_unpack", "k_pack",
                "k_lamb_apply",
                "k_trust_ratio", "k_diag_reduce", "k_scale_finalize", "k_worker_compress", "k_worker_update"):
        if key in name:
            tmpl = name.split(key, 1)[1]
            return key + (tmpl[:60] if tmpl else "")
    return name[:80]


# the kernel names each timing kind covers (server pass 1: the whole-line kernel where the layout allows
# it, the per-lane one elsewhere)
KERNEL_SYMBOL = {"compress": "k_compress<", "chunk_sumsq": "k_chunk_sumsq<", "dense": "k_dense<",
                 "server_sumsq": ("k_server_sumsq_lines", "k_server<false>"), "server_apply": "k_server<true>",
                 "unpack": "k_unpack",
                 "lamb_apply": "k_lamb_apply<", "trust_ratio": "k_trust_ratio", "diag": "k_diag_reduce",
                 "scale": "k_scale_finalize", "worker_compress": "k_worker_compress<",
                 "worker_update": "k_worker_update"}


def _counter_rows(d: str, counter: str):
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                yield r


# Kernels whose streaming loads are nontemporal (their counters are calibrated on the probe's
# nontemporal copy); the others (server pass 2) use ordinary loads (calibrated on the torch copy).
NONTEMPORAL_KERNELS = {"compress", "chunk_sumsq", "dense", "worker_compress", "worker_update", "lamb_apply",
                       "server_sumsq", "unpack"}
# the probes of --copy-probe-mib 1024: (name, kernel-name fragment, grid in threads)
COPY_PROBES = (("torch copy", "copyBuffer", 131072), ("nontemporal copy", "k_probe_copy<true>", 16777216))


# the counter runs' timed steps (their commands pass --steps 5)
PMC_STEPS = 5
# kernels launched once per chunk group of the compressed step
GROUPED_KERNELS = {"chunk_sumsq", "compress", "worker_compress"}


# the library's default pass-1 bytes per chunk group (OB_GROUP_BYTES overrides it, as in the library)
GROUP_BYTES = 320 << 20


def chunk_groups(w, lamb: bool = False) -> list:
    """The chunk groups [(c0, c1), ...] the library's compressed step runs its two kernels over for
    workload w (host arithmetic, no GPU): consecutive chunks while their pass-1 bytes (g and err) stay
    within the budget, a larger chunk alone; one group for 1-bit LAMB, when grouping is off, or when a
    chunk has more than 4096 pass-1 blocks (then the library forms per-chunk sums first).
    tests/test_gpu_groups.py checks it against ob_plan_num_groups for every workload."""
    off = [int(o) for o in w.chunk_offsets()]
    K = len(off) - 1
    if lamb:                       # 1-bit LAMB runs one group
        return [(0, K)]
    budget = int(os.environ.get("OB_GROUP_BYTES", GROUP_BYTES))
    width = (2 if w.grad_dtype == "bf16" else 4) + (4 if w.err_dtype == "f32" else 2)
    be1 = int(os.environ.get("OB_BLOCK_ELEMS", 0))
    if not (be1 >= 1024 and be1 <= (1 << 20) and be1 % 1024 == 0):
        be1 = min(max(-(-(-(-w.n // 8192)) // 1024) * 1024, 4096), 24576)
    p1_max = max(-(-(off[c + 1] - off[c]) // be1) for c in range(K))
    max_elems = max(1, budget // width) if budget > 0 and p1_max <= 4096 else 0
    out, c0 = [], 0
    while c0 < K:
        c1 = c0 + 1 if max_elems > 0 else K
        while c1 < K and off[c1 + 1] - off[c0] <= max_elems:
            c1 += 1
        out.append((c0, c1))
        c0 = c1
    return out


def launches_per_step(w, kernel: str) -> int:
    """Launches of `kernel` in one step of workload w: the chunk groups for the compressed step's two
    kernels, else 1."""
    if kernel not in GROUPED_KERNELS:
        return 1
    return len(chunk_groups(w, lamb=w.optimizer == "lamb" and kernel != "worker_compress"))


def traffic_profile(d: str, kernel: str, workload: str) -> str:
    """Calibrated HBM bytes per launch of `kernel` from FETCH_SIZE / WRITE_SIZE runs under d."""
    from adam_ob_compress_amd import synth

    w = synth.WORKLOADS[workload]
    groups = launches_per_step(w, kernel)
    probe_kib = 1 << 20  # the --copy-probe-mib 1024 copies read and write 1 GiB each
    res, factors = {}, {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = list(_counter_rows(d, counter))
        # each probe's dispatches are the run's last 8 of its kernel and grid (3 warm-up + 5 timed)
        for pname, frag, grid in COPY_PROBES:
            copies = sorted((r for r in rows if frag in r["Kernel_Name"] and int(r["Grid_Size"]) == grid),
                            key=lambda r: int(r["Dispatch_Id"]))
            vals = [float(r["Counter_Value"]) for r in copies[-8:]]
            if vals:
                factors.setdefault(pname, {})[counter] = sum(vals) / len(vals) / probe_kib
        syms = KERNEL_SYMBOL[kernel] if isinstance(KERNEL_SYMBOL[kernel], tuple) else (KERNEL_SYMBOL[kernel],)
        mine = sorted((r for r in rows if any(sym in r["Kernel_Name"] for sym in syms)),
                      key=lambda r: int(r["Dispatch_Id"]))
        if groups > 1:
            # launched once per chunk group: the timed steps' launches are the kernel's last
            # PMC_STEPS * groups dispatches
            kern = [float(r["Counter_Value"]) for r in mine[-PMC_STEPS * groups:]]
            ok = len(kern) == PMC_STEPS * groups
        else:
            # the workload's own launches: the kernel's largest grid (the warm-up on a small scratch
            # plan launches the same kernels on small grids)
            top = max((int(r["Grid_Size"]) for r in mine), default=0)
            kern = [float(r["Counter_Value"]) for r in mine if int(r["Grid_Size"]) == top]
            ok = bool(kern)
        if not ok or "torch copy" not in factors or counter not in factors["torch copy"]:
            raise SystemExit(f"no {counter} rows for the copy probe or {kernel} under {d}")
        # KiB per step of the workload, and the dispatches that gave it
        res[counter] = (sum(kern) / len(kern) * groups, len(kern))
    nt = "nontemporal copy" in factors and len(factors["nontemporal copy"]) == 2
    used = "nontemporal copy" if nt and kernel in NONTEMPORAL_KERNELS else "torch copy"
    ff, wf = factors[used]["FETCH_SIZE"], factors[used]["WRITE_SIZE"]
    (fk, fn), (wk, wn) = res["FETCH_SIZE"], res["WRITE_SIZE"]
    traffic = (fk / ff + wk / wf) * 1024            # HBM bytes per step
    alg = bytes_per_elem(w, kernel) * w.n
    if traffic < 0.5 * alg:
        raise SystemExit(f"{kernel}: no launch of the workload's size under {d} (only the warm-up's?)")
    fk, wk = fk / groups, wk / groups                # per launch from here on
    run_flags = " --split" if kernel.startswith("worker_") else ""   # the split step's kernels
    rec = {"kernel": kernel, "workload": w.name, "kernel_src_sha": kernel_source_sha(),
           "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
           "calibration": used, "fetch_factor": round(ff, 5), "write_factor": round(wf, 5),
           "factors": {k: {c: round(v, 5) for c, v in f.items()} for k, f in factors.items()},
           "launches_per_step": groups, "bytes_per_step": round(traffic),
           "bytes_per_launch": round(traffic / groups),
           "algorithmic_bytes_per_launch": round(alg / groups), "traffic_over_algorithmic": round(traffic / alg, 4)}
    group_note = "" if groups == 1 else (
        f"`{kernel}` runs once per chunk group, {groups} launches per step: the figures below are the\n"
        f"last {PMC_STEPS} steps' {PMC_STEPS * groups} dispatches (the timed ones), summed per step and divided by {groups}.\n\n")
    cal = "\n".join(f"| {k} | {f.get('FETCH_SIZE', float('nan')) * probe_kib:,.1f} | "
                     f"{f.get('WRITE_SIZE', float('nan')) * probe_kib:,.1f} | {f.get('FETCH_SIZE', float('nan')):.5f} | "
                     f"{f.get('WRITE_SIZE', float('nan')):.5f} |" for k, f in factors.items())
    return f"""# HBM traffic of `{kernel}` on {w.name}

Kernel source sha (ob_compress.hip, ob_kernels.hip, ob_device.h, ob_internal.h, ob_tables.h, ob_api.cpp): {rec['kernel_src_sha']}.

Commands (each its own run on one MI355X, from the repository root, `export TMPDIR=/tmp`):

    rocprofv3 --pmc FETCH_SIZE -d rocprof_out/fetch -o run --output-format csv -- python bench.py --workload {w.name}{run_flags} --steps 5 --warmup 2 --no-cpu --copy-probe-mib 1024
    rocprofv3 --pmc WRITE_SIZE -d rocprof_out/write -o run --output-format csv -- python bench.py --workload {w.name}{run_flags} --steps 5 --warmup 2 --no-cpu --copy-probe-mib 1024
    python bench.py --traffic-profile rocprof_out --kernel {kernel} --workload {w.name}

Calibration: the run also copies 1 GiB twice over -- with torch (`__amd_rocclr_copyBuffer`, grid
131072, ordinary loads and stores) and with the probe library's copy (`k_probe_copy<true>`, grid
16777216, 16-byte lanes with nontemporal loads and stores) -- each reading and writing 1,048,576 KiB
per dispatch.  Counter readings per such dispatch and the factors they give:

| copy | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch factor | write factor |
|---|---|---|---|---|
{cal}

`{kernel}` is calibrated with the {used} (its streaming accesses are {"nontemporal" if used == "nontemporal copy" else "ordinary"}).

{group_note}| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | HBM bytes/launch (calibrated) | algorithmic bytes/launch | ratio |
|---|---|---|---|---|---|---|
| {kernel} | {fn} / {wn} | {fk:,.1f} | {wk:,.1f} | {traffic / groups:,.0f} | {alg / groups:,.0f} ({bytes_per_elem(w, kernel)} B x n{" / " + str(groups) if groups > 1 else ""}) | {traffic / alg:.4f} |

traffic-json: {json.dumps(rec)}
"""


def _grid(r) -> int:
    if r.get("Grid_Size"):
        return int(r["Grid_Size"])
    return int(r.get("Grid_Size_X", 0)) * int(r.get("Grid_Size_Y", 1) or 1) * int(r.get("Grid_Size_Z", 1) or 1)


# the largest grid (threads) of a library kernel in warm_kernels' scratch plan of WARM_N elements: the
# dense table's blocks of 2 tiles (2048 elements), 256 threads each
WARM_N = 1 << 16
WARM_GRID = WARM_N // 2048 * 256


def rocprof_summary(d: str) -> str:
    out = []
    # per kernel and grid size from the dispatch trace, so that the warm-up's small launches of the
    # same kernels are reported apart from the workload's
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        groups = {}
        for r in csv.DictReader(open(f)):
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups.setdefault((_short(r["Kernel_Name"]), _grid(r)), []).append(us)
        total = sum(sum(v) for v in groups.values()) or 1.0
        out.append(f"### kernel trace by kernel and grid size: {os.path.relpath(f, d)}\n")
        out.append("| kernel | grid (threads) | calls | avg us | min us | max us | total % |")
        out.append("|---|---|---|---|---|---|---|")
        for (k, g), v in sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:14]:
            out.append(f"| {k} | {g} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                       f"{100.0 * sum(v) / total:.1f} |")
        out.append("")
        # the library's kernels over all their launches on the workload (the compressed step's two
        # kernels run once per chunk group, with grids that differ between groups); the bench's warm-up
        # on a scratch plan launches them with grids of at most WARM_GRID threads
        lib_k = {}
        for (k, g), v in groups.items():
            if k.startswith("k_") and g > WARM_GRID:
                lib_k.setdefault(k, []).extend(v)
        if lib_k:
            out.append(f"### library kernels over all launches with grids above {WARM_GRID} threads (the workload's)\n")
            out.append("| kernel | calls | avg us | total us |")
            out.append("|---|---|---|---|")
            for k, v in sorted(lib_k.items(), key=lambda kv: -sum(kv[1])):
                out.append(f"| {k} | {len(v)} | {sum(v) / len(v):.2f} | {sum(v):.1f} |")
            out.append("")
    ctr = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    for f in ctr:
        agg = {}
        for r in csv.DictReader(open(f)):
            key = (_short(r["Kernel_Name"]), r["Counter_Name"])
            a = agg.setdefault(key, [0.0, set()])
            a[0] += float(r["Counter_Value"])
            a[1].add(r.get("Dispatch_Id") or r.get("Correlation_Id"))
        out.append(f"### counters: {os.path.relpath(f, d)}\n")
        out.append("| kernel | counter | dispatches | per dispatch (KiB) |")
        out.append("|---|---|---|---|")
        for (k, c), (tot, ids) in sorted(agg.items()):
            out.append(f"| {k} | {c} | {len(ids)} | {tot / max(len(ids), 1):.1f} |")
        out.append("")
    return "\n".join(out) if out else f"no rocprofv3 CSV output under {d}"


if __name__ == "__main__":
    sys.exit(main())
