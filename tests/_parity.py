"""Parity harness: the HIP path against the CPU oracle, per step, from identical input state.

Each step: the oracle's own state for the checked chunks is written into the GPU buffers, the GPU
step runs over the whole buffer (the launch configuration the bench times), the oracle runs the same
step on host copies of the checked chunks, and the outputs of those chunks are compared.  The oracle
never receives anything the HIP path computed: its inputs come from the seeded generators
(adam_ob_compress_amd.synth) and from its own previous steps.

Every chunk's outputs depend only on that chunk (pinned on the CPU by
tests/test_oracle.py::test_chunks_are_independent), so checking a subset of chunks is exact for them,
and the oracle may run on different chunks in parallel threads (ctypes releases the GIL).

Tolerances:
  * packed words and int8 signs: bit-exact;
  * a 16-bit error buffer (nearest or stochastic rounding): the stored words bit-equal on every chunk
    whose scale matched (see assert_err_close); on a chunk whose scale differed by an ulp, the fp32
    bound below plus one unit in the last place of the storage format;
  * scales: equal, or 1 ulp apart (the double sum of squares is reduced in a different order);
    mismatches are counted and returned;
  * fp32 state: |gpu - ref| <= 2e-6*|ref| + 1e-9 (+ the exact propagation of a scale difference:
    err moves by |dscale| (EMA: (1-ef_beta)|dscale|), m by (1-beta1)|dscale|, p by
    lr*(1-beta1)|dscale|/(sqrt(v)+eps)); NaN must match NaN and +-Inf must match exactly;
  * 1-bit LAMB: the layer's trust ratio equal or 1 ulp apart (2 after a scale difference: the sums of
    squares are reduced in a different order); p then also moves by lr*|dr|*|u|.
"""
from __future__ import annotations

import collections
import concurrent.futures as cf
import os

import numpy as np
import torch

import oracle
from adam_ob_compress_amd import schedule, synth
import adam_ob_compress_amd as ob

REL, ABS = 2e-6, 1e-9
_POOL = cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))


def ulp_diff(a, b):
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    # map sign-magnitude to a monotone integer line
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def assert_f32_close(gpu, ref, what, slack=0.0):
    gpu = np.asarray(gpu, np.float32)
    ref = np.asarray(ref, np.float32)
    assert gpu.shape == ref.shape, what
    gn, rn = np.isnan(gpu), np.isnan(ref)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ ({int(np.sum(gn != rn))})"
    gi, ri = np.isinf(gpu), np.isinf(ref)
    assert np.array_equal(gi, ri) and np.array_equal(gpu[gi], ref[ri]), f"{what}: Inf differ"
    fin = ~(rn | ri)
    g64 = gpu[fin].astype(np.float64)
    r64 = ref[fin].astype(np.float64)
    tol = REL * np.abs(r64) + ABS
    if not np.isscalar(slack):
        slack = np.asarray(slack, np.float64)[fin]
    tol = tol + slack
    bad = np.abs(g64 - r64) > tol
    if np.any(bad):
        k = int(np.argmax(np.abs(g64 - r64) - tol))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst gpu="
                             f"{g64[k]!r} ref={r64[k]!r} tol={tol[k]!r}")


# significand bits (implicit bit included) and the smallest subnormal of the 16-bit error formats
_FMT = {"bf16": (8, 2.0 ** -133), "f16": (11, 2.0 ** -24)}


def err_format(a: np.ndarray) -> str:
    return {np.dtype(np.float32): "f32", np.dtype(np.uint16): "bf16", np.dtype(np.float16): "f16"}[a.dtype]


def widen_err(a: np.ndarray) -> np.ndarray:
    """A host error buffer as fp32: float16 by numpy, bf16 bits by shifting into the high half."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def assert_err_close(gpu, ref, what, slack=0.0, exact=True):
    """Error buffers of any storage format.

    fp32: assert_f32_close(gpu, ref, what, slack).

    bf16 / fp16: wherever `exact` holds (a bool, or one per element: True where the element's chunk
    had the same scale on both sides) the stored 16-bit words must be equal; only NaN payloads are not
    compared (NaN must meet NaN).  With the same scale both sides store the same fp32 value: plain
    error feedback is one fp32 subtraction, and in the EMA line both products (fp32 x fp32, and
    1 - ef_beta times fp32) are exact in double, so the line is rounded once in double whether or not
    the products are fused, then once to fp32.  Rounding that value to nearest-even, or stochastically
    with the same random bits, has one result, so any other rounding (truncation, ties away from zero,
    round-half-down, a wrong random stream) is rejected.
    Elsewhere (the chunk's scale differed by one ulp, moving the fp32 error by up to `slack`): the
    fp32 bound plus `slack` plus one unit in the last place of the storage format."""
    fmt = err_format(np.asarray(ref))
    assert err_format(np.asarray(gpu)) == fmt, what
    g32, r32 = widen_err(np.asarray(gpu)), widen_err(np.asarray(ref))
    if fmt == "f32":
        return assert_f32_close(g32, r32, what, slack)
    assert g32.shape == r32.shape, what
    ex = np.broadcast_to(np.asarray(exact, dtype=bool), r32.shape)
    if ex.any():
        gb = np.asarray(gpu).view(np.uint16)[ex]
        rb = np.asarray(ref).view(np.uint16)[ex]
        gn, rn = np.isnan(g32[ex]), np.isnan(r32[ex])
        bad = (gn != rn) | (~rn & (gb != rb))
        if np.any(bad):
            k = int(np.argmax(bad))
            raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} stored {fmt} words differ where the "
                                 f"scale matched; first: gpu=0x{int(gb[k]):04x} ({g32[ex][k]!r}) "
                                 f"ref=0x{int(rb[k]):04x} ({r32[ex][k]!r})")
    rest = ~ex
    if not rest.any():
        return
    prec, tiny = _FMT[fmt]
    ulp = np.abs(r32[rest].astype(np.float64)) * 2.0 ** (1 - prec) + tiny
    if not np.isscalar(slack):
        slack = np.broadcast_to(np.asarray(slack, np.float64), r32.shape)[rest]
    assert_f32_close(g32[rest], r32[rest], what + " (chunks whose scale differed)",
                     np.where(np.isfinite(ulp), ulp, 0.0) + slack)


class ChunkRef:
    """The oracle's state for one chunk [a, b)."""

    def __init__(self, c, a, b, err, m, v, p):
        self.c, self.a, self.b = c, a, b
        self.err, self.m, self.v, self.p = err, m, v, p
        self.out = None


def host_chunks(w, chunks, err, m, v, p):
    off = w.chunk_offsets()
    refs = []
    for c in chunks:
        a, b = int(off[c]), int(off[c + 1])
        refs.append(ChunkRef(c, a, b, *(synth.host(t[a:b]) for t in (err, m, v, p))))
    return refs


def upload(refs, err, m, v, p):
    """Write the oracle's chunk state into the GPU buffers (identical input state, bit for bit)."""
    for r in refs:
        for dst, src in ((err, r.err), (m, r.m), (v, r.v), (p, r.p)):
            d = dst[r.a:r.b]
            if src.dtype == np.uint16:          # bf16 bits
                d.view(torch.int16).copy_(torch.from_numpy(src.view(np.int16)), non_blocking=False)
            else:
                d.copy_(torch.from_numpy(src), non_blocking=False)


def _oracle_compress(r, g, w, s):
    off = np.asarray([0, r.b - r.a], np.int64)
    hp = dict(lr=w.lr, beta1=w.beta1, eps=w.eps, clip=w.clip, ef_mode=w.ef_mode, ef_beta=w.ef_beta,
              want_signs=w.int8_signs, count_nonfinite=True)
    if w.err_rounding == "stochastic":
        hp.update(stochastic=True, sr_seed=synth.SR_SEED, sr_step=s, sr_index0=r.a)
    if w.optimizer == "lamb":
        words, scales, ratios, signs, nf = oracle.lamb_compress_step(g, r.err, r.m, r.v, r.p, off, **hp)
        r.out = dict(words=words, scale=scales[0], signs=signs, nf=nf, ratio=ratios[0])
    else:
        words, scales, signs, nf = oracle.compress_step(g, r.err, r.m, r.v, r.p, off, **hp)
        r.out = dict(words=words, scale=scales[0], signs=signs, nf=nf)


def _oracle_dense(r, g, w, bias_correction, t):
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, bias_correction=bias_correction, step=t)
    if w.optimizer == "lamb":
        ratios = oracle.lamb_warmup_step(g, r.m, r.v, r.p, np.asarray([0, r.b - r.a], np.int64), **hp)
        r.out = dict(ratio=ratios[0])
    else:
        oracle.warmup_step(g, r.m, r.v, r.p, **hp)
        r.out = {}


def oracle_step(refs, g_dev, w, kind, bias_correction=False, t=0, s=0):
    def one(r):
        g = synth.host(g_dev[r.a:r.b])
        r.err_before = r.err.copy()
        if kind == "compressed":
            _oracle_compress(r, g, w, s)
        else:
            _oracle_dense(r, g, w, bias_correction, t)
    for f in [_POOL.submit(one, r) for r in refs]:
        f.result()


def compare_chunks(refs, w, kind, err, m, v, p, words=None, scales=None, signs=None, ratios=None,
                   diag=None):
    """Compare the GPU buffers on the checked chunks with the oracle; returns scale-ulp mismatches.
    diag: (err_sumsq, plus_count) device arrays of a compressed step's diagnostics, or None.
    Chunks are compared in parallel threads (numpy and the device-to-host copies release the GIL)."""
    futs = [_POOL.submit(_compare_one, r, w, kind, err, m, v, p, words, scales, signs, ratios, diag)
            for r in refs]
    return sum(f.result() for f in futs)


def _compare_one(r, w, kind, err, m, v, p, words, scales, signs, ratios, diag):
    mism = 0
    b1 = np.float64(np.float32(w.beta1))
    eb = np.float64(np.float32(w.ef_beta))
    lr = np.float64(np.float32(w.lr))
    eps = np.float64(np.float32(w.eps))
    tag = f"{w.name} chunk {r.c} [{r.a},{r.b}) {kind}"
    ge, gm, gv, gp = (synth.host(t[r.a:r.b]) for t in (err, m, v, p))
    ds = 0.0
    if kind == "compressed":
        ws = synth.host(words[r.a // 32:(r.b + 31) // 32])
        assert np.array_equal(ws, r.out["words"]), f"{tag}: packed words differ"
        sc = np.float32(scales[r.c].item())
        d = int(ulp_diff(sc, r.out["scale"]))
        assert d <= 1 or (np.isnan(sc) and np.isnan(r.out["scale"])), \
            f"{tag}: scale {sc!r} vs {r.out['scale']!r} ({d} ulp)"
        if d == 1:
            mism += 1
            ds = abs(float(sc) - float(r.out["scale"]))
        if signs is not None:
            assert np.array_equal(synth.host(signs[r.a:r.b]), r.out["signs"]), f"{tag}: int8 signs differ"
        if diag is not None:
            rss, rpc = oracle.diagnostics(r.err_before, r.out["words"], np.asarray([0, r.b - r.a], np.int64))
            gss = float(diag[0][r.c].item())
            assert abs(gss - rss[0]) <= 1e-10 * rss[0], f"{tag}: error norm^2 {gss} vs {rss[0]}"
            assert int(diag[1][r.c].item()) == int(rpc[0]), f"{tag}: +1 count"
        assert np.array_equal(gv, r.v), f"{tag}: v changed in the compressed step"
    else:
        assert_f32_close(gv, r.v, f"{tag}: v")
    err_slack = ds * ((1 - eb) if w.ef_mode == 1 else 1.0)
    m_slack = ds * (1 - b1)
    den = np.sqrt(r.v.astype(np.float64)) + eps
    p_slack = lr * m_slack / den if ds else 0.0
    if w.optimizer == "lamb":
        rg, rr = np.float32(ratios[r.c].item()), np.float32(r.out["ratio"])
        dr_ulp = int(ulp_diff(rg, rr))
        assert dr_ulp <= (2 if ds else 1) or (np.isnan(rg) and np.isnan(rr)), \
            f"{tag}: trust ratio {rg!r} vs {rr!r} ({dr_ulp} ulp)"
        dr = abs(float(rg) - float(rr)) if np.isfinite(rr) else 0.0
        u = np.abs(r.m.astype(np.float64)) / den     # run_workload's steps have no bias correction
        p_slack = float(abs(rr)) * p_slack + lr * dr * u
    assert_err_close(ge, r.err, f"{tag}: err", err_slack, exact=ds == 0.0)
    assert_f32_close(gm, r.m, f"{tag}: m", m_slack)
    assert_f32_close(gp, r.p, f"{tag}: p", p_slack)
    return mism


def run_workload(w, chunks=None, steps=None, device="cuda:0", log=print, diagnostics=False):
    """Run w's schedule on the GPU and check the given chunks (all if None) every step.

    Returns a dict of counts (steps by kind, scale mismatches)."""
    K = w.n_chunks
    chunks = list(range(K)) if chunks is None else sorted(set(chunks))
    steps = w.steps if steps is None else steps
    plan = ob.ob_plan_create(w.n, chunk_size=w.chunk if w.offsets is None else 0,
                             chunk_offsets=w.offsets)
    err, m, v, p = synth.draw_state(w, device)
    cls = schedule.OneBitLamb if w.optimizer == "lamb" else schedule.OneBitAdam
    opt = cls(plan, err, m, v, p, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                              clip=w.clip, ef_mode=w.ef_mode, ef_beta=w.ef_beta,
                              int8_signs=w.int8_signs, count_nonfinite=True,
                              freeze_step=w.freeze_step, refresh_period=w.refresh_period,
                              diagnostics=diagnostics, err_rounding=w.err_rounding, sr_seed=synth.SR_SEED)
    refs = host_chunks(w, chunks, err, m, v, p)
    g = None
    counts = {"dense": 0, "compressed": 0, "scale_ulp_mismatch": 0}
    nf_ref = 0
    for s in range(steps):
        g = synth.draw_grad(w, s, device, out=g)
        upload(refs, err, m, v, p)
        torch.cuda.synchronize()
        kind = opt.step(g)
        torch.cuda.synchronize()
        oracle_step(refs, g, w, kind, t=opt.dense_steps, s=s)
        counts[kind] += 1
        counts["scale_ulp_mismatch"] += compare_chunks(refs, w, kind, err, m, v, p, opt.words,
                                                       opt.scales, opt.signs,
                                                       getattr(opt, "ratios", None),
                                                       (opt.err_sumsq, opt.plus_count)
                                                       if diagnostics and kind == "compressed" else None)
        if kind == "compressed":
            nf_ref += sum(r.out["nf"] for r in refs)
        log(f"{w.name} step {s} {kind}: {len(refs)} chunks match")
    if len(chunks) == K:
        assert int(opt.nonfinite.item()) == nf_ref
    del plan
    return counts


def tracked_chunks(K: int, fixed, n_random: int = 6, seed: int = 0) -> list[int]:
    """The fixed chunks plus n_random others drawn by a seeded generator (the same ones every run), so
    that a run's checks also reach chunks nobody picked by hand."""
    rng = np.random.default_rng([synth.SEED, K, seed])
    rest = np.setdiff1d(np.arange(K), np.asarray(sorted(fixed), dtype=np.int64))
    pick = rng.choice(rest, size=min(n_random, rest.size), replace=False) if rest.size else []
    return sorted({int(c) for c in fixed} | {int(c) for c in pick})


def _make_optimizer(w, plan, err, m, v, p, diagnostics=False):
    cls = schedule.OneBitLamb if w.optimizer == "lamb" else schedule.OneBitAdam
    return cls(plan, err, m, v, p, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
               clip=w.clip, ef_mode=w.ef_mode, ef_beta=w.ef_beta,
               int8_signs=w.int8_signs, count_nonfinite=True,
               freeze_step=w.freeze_step, refresh_period=w.refresh_period,
               diagnostics=diagnostics, err_rounding=w.err_rounding, sr_seed=synth.SR_SEED)


def _check_one_chunk(r, g, w, kind, s, opt):
    r.err_before = r.err.copy()
    if kind == "compressed":
        _oracle_compress(r, g, w, s)
    else:
        _oracle_dense(r, g, w, False, 0)
    mism = _compare_one(r, w, kind, opt.err, opt.m, opt.v, opt.p, opt.words, opt.scales, opt.signs,
                        getattr(opt, "ratios", None), None)
    return mism, int(r.out.get("nf", 0))


def _every_chunk_one_step(w, plan, kind, s, device, err_sigma, m_sigma, log):
    err, m, v, p = synth.draw_state(w, device, err_sigma, m_sigma)
    opt = _make_optimizer(w, plan, err, m, v, p)
    opt.step_index = s
    g = synth.draw_grad(w, s, device)
    torch.cuda.synchronize()
    got = opt.step(g)
    assert got == kind, f"{w.name}: step index {s} is a {got} step, not {kind}"
    torch.cuda.synchronize()
    del g
    off = w.chunk_offsets()
    pending = collections.deque()
    mism = nf = 0
    inflight = 0      # elements of the chunks queued or being checked (host memory ~100 B each)

    def drain(max_tasks, max_elems):
        nonlocal mism, nf, inflight
        while pending and (len(pending) > max_tasks or inflight > max_elems):
            fut, size = pending.popleft()
            a, b = fut.result()
            mism += a
            nf += b
            inflight -= size

    for c in range(w.n_chunks):
        a, b = int(off[c]), int(off[c + 1])
        # bound the host memory: at most 2 chunks per thread and 2^29 elements in flight
        drain(2 * _POOL._max_workers - 1, (1 << 29) - (b - a))
        # this chunk's inputs, drawn again on their own: nothing the step wrote reaches the oracle
        gh = synth.host(synth.draw_grad_window(w, s, a, b, device))
        st = [synth.host(t) for t in synth.draw_state_window(w, a, b, device, err_sigma, m_sigma)]
        pending.append((_POOL.submit(_check_one_chunk, ChunkRef(c, a, b, *st), gh, w, kind, s, opt), b - a))
        inflight += b - a
    drain(0, 0)
    if kind == "compressed":
        assert int(opt.nonfinite.item()) == nf, f"{w.name}: non-finite count"
    log(f"{w.name} {kind} step {s}: all {w.n_chunks} chunks match ({mism} scale ulp mismatches)")
    return mism


def check_every_chunk(w, device="cuda:0", dense_step=None, err_sigma=1e-4, m_sigma=1e-4, log=print):
    """Every chunk of w against the oracle after one compressed step, and (dense_step: its step index)
    after one dense step, each over the whole buffer in the bench's launch configuration and from a
    seeded state with every term non-zero (err ~ N(0, err_sigma) in w's error format, m ~ N(0, m_sigma)).
    The oracle's inputs for chunk c are drawn again for that chunk alone by synth's window draws, and
    the chunks are checked in parallel threads, a bounded number at a time, so the host never holds
    more than a few chunks of state.  Returns the number of chunks whose scale differed by an ulp."""
    plan = ob.ob_plan_create(w.n, chunk_size=w.chunk if w.offsets is None else 0, chunk_offsets=w.offsets)
    first = next(t for t in range(w.steps) if schedule.step_kind(t, w.freeze_step, w.refresh_period)
                 == "compressed")
    runs = [("compressed", first)]
    if dense_step is not None:
        assert schedule.step_kind(dense_step, w.freeze_step, w.refresh_period) == "dense"
        runs.append(("dense", dense_step))
    mism = 0
    for kind, s in runs:
        mism += _every_chunk_one_step(w, plan, kind, s, device, err_sigma, m_sigma, log)
        torch.cuda.empty_cache()
    del plan
    return mism
