"""GPU parity: every entry point of libobadam.so against the CPU oracle (marked gpu).

Sizes: brute force over n = 1..130; several tiles and work blocks with ragged tails; and the five
workloads at full size in the launch configuration the bench uses (checked chunks listed per test).
Inputs come only from adam_ob_compress_amd.synth; nothing the HIP path computes is fed to the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import adam_ob_compress_amd as ob
from adam_ob_compress_amd import synth

import _parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    ob.lib()  # raises if the HIP library was not built


@pytest.fixture(autouse=True)
def _gpu():
    _require_gpu()
    yield
    torch.cuda.synchronize()


def _t(a, dtype=None):
    """Host numpy -> device tensor (bf16 from uint16 bits, uint32 into int32 storage)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32).copy()).to(DEV)
    return torch.from_numpy(a.copy()).to(DEV)


def _bf16_bits(x):
    """Round fp32 to bf16 (nearest even) and return the uint16 bit patterns (NaN kept quiet)."""
    return synth.host(torch.from_numpy(x).to(torch.bfloat16))


# ------------------------------------------------------------------------------------------------
# pack / unpack
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("pattern", ["normal", "signed_zeros", "denormals", "special", "alternating"])
def test_pack_bruteforce(pattern):
    for n in list(range(1, 131)) + [1023, 1024, 1025, 16384 + 4, 100003]:
        x = synth.draw_values(n, 17, pattern)
        for arr in (x, _bf16_bits(x)):
            words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
            ob.ob_pack(_t(arr), words)
            assert np.array_equal(synth.host(words), oracle.pack(arr)), (pattern, n, arr.dtype)


def test_unpack_with_and_without_scales():
    for n, chunk in ((1, 64), (33, 64), (130, 64), (5000, 1024), (100003, 4096)):
        x = synth.draw_values(n, 23, "special")
        words_np = oracle.pack(x)
        off = oracle.uniform_offsets(n, chunk)
        sc = synth.draw_values(off.size - 1, 29, "normal") * np.float32(7)
        plan = ob.ob_plan_create(n, chunk_size=chunk)
        out = torch.empty(n, dtype=torch.float32, device=DEV)
        ob.ob_unpack(plan, _t(words_np), n, out, scales=_t(sc))
        assert np.array_equal(synth.host(out), oracle.unpack(words_np, n, off, sc))
        ob.ob_unpack(None, _t(words_np), n, out)
        assert np.array_equal(synth.host(out), oracle.unpack(words_np, n))


# ------------------------------------------------------------------------------------------------
# compressed / dense step: brute force on tiny and multi-tile inputs
# ------------------------------------------------------------------------------------------------

VARIANTS = {
    "fp32_plain": dict(gdt="f32", clip=0.0, ef_mode=0, signs=False),
    "bf16_ema_clip_int8": dict(gdt="bf16", clip=5.0, ef_mode=1, signs=True),
    "fp32_ema": dict(gdt="f32", clip=0.0, ef_mode=1, signs=True),
    "bf16_plain": dict(gdt="bf16", clip=0.0, ef_mode=0, signs=False),
    # 16-bit error buffers
    "fp32_plain_f16err": dict(gdt="f32", clip=0.0, ef_mode=0, signs=False, edt="f16"),
    "fp32_ema_bf16err": dict(gdt="f32", clip=0.0, ef_mode=1, signs=True, edt="bf16"),
    "bf16_ema_clip_int8_f16err": dict(gdt="bf16", clip=5.0, ef_mode=1, signs=True, edt="f16"),
    "bf16_plain_bf16err": dict(gdt="bf16", clip=0.0, ef_mode=0, signs=False, edt="bf16"),
    # ... stored with stochastic rounding
    "fp32_ema_bf16err_sr": dict(gdt="f32", clip=0.0, ef_mode=1, signs=True, edt="bf16", sr=True),
    "bf16_plain_f16err_sr": dict(gdt="bf16", clip=0.0, ef_mode=0, signs=False, edt="f16", sr=True),
}
SR_SEED = 0x5EED0B17


def _sr_hp(var, step):
    """hparams fields and oracle keywords of a variant's error rounding at one step."""
    if not var.get("sr"):
        return {}, {}
    return (dict(err_rounding=ob.OB_ROUND_STOCHASTIC, sr_seed=SR_SEED, step=step),
            dict(stochastic=True, sr_seed=SR_SEED, sr_step=step))


def _as_err_format(err32, edt):
    """An fp32 error array rounded (nearest even, by numpy / torch) to the variant's storage format."""
    if edt == "f16":
        with np.errstate(over="ignore"):
            return err32.astype(np.float16)
    if edt == "bf16":
        return _bf16_bits(err32)
    return err32


def _small_state(n, seed, wide=False):
    rng = np.random.default_rng([seed, n])
    s = 20.0 if wide else 1e-3
    g = (rng.standard_normal(n) * s).astype(np.float32)
    err = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (np.abs(rng.standard_normal(n)) * 1e-6 + 1e-8).astype(np.float32)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    return g, err, m, v, p


def _gpu_vs_oracle_compress(n, chunk, var, seed, g=None, state=None, steps=1, lr=1e-4):
    gnp, err, m, v, p = _small_state(n, seed, wide=var["clip"] > 0)
    if g is not None:
        gnp = g
    if state is not None:
        err, m, v, p = state
    err = _as_err_format(err, var.get("edt", "f32"))
    if var["gdt"] == "bf16":
        gnp = _bf16_bits(gnp)
    off = oracle.uniform_offsets(n, chunk)
    plan = ob.ob_plan_create(n, chunk_size=chunk)
    for _ in range(steps):
        sr_h, sr_o = _sr_hp(var, 7 + _)
        hp = ob.hparams(lr=lr, beta1=0.9, eps=1e-8, clip=var["clip"], ef_mode=var["ef_mode"], ef_beta=0.9,
                        **sr_h)
        d = [_t(a) for a in (gnp, err, m, v, p)]
        words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
        scales = torch.zeros(off.size - 1, dtype=torch.float32, device=DEV)
        signs = torch.zeros(n, dtype=torch.int8, device=DEV) if var["signs"] else None
        nf = torch.zeros(1, dtype=torch.int64, device=DEV)
        ob.ob_adam_compress_step(plan, d[0], d[1], d[2], d[3], d[4], words, scales, hp, signs, nf)
        rw, rs, rsg, rnf = oracle.compress_step(gnp, err, m, v, p, off, lr=lr, beta1=0.9, eps=1e-8,
                                                clip=var["clip"], ef_mode=var["ef_mode"], ef_beta=0.9,
                                                want_signs=var["signs"], count_nonfinite=True, **sr_o)
        tag = f"n={n} chunk={chunk} {var}"
        assert np.array_equal(synth.host(words), rw), f"{tag}: words"
        if signs is not None:
            assert np.array_equal(synth.host(signs), rsg), f"{tag}: signs"
        gs = synth.host(scales)
        d_ulp = P.ulp_diff(gs, rs)
        assert np.all(d_ulp <= 1), f"{tag}: scales {gs} vs {rs}"
        cidx = np.repeat(np.arange(off.size - 1), np.diff(off))
        ds = np.abs(gs.astype(np.float64) - rs.astype(np.float64))[cidx]
        ds = np.where(np.isfinite(ds), ds, 0.0)
        eslack = ds * (0.1 if var["ef_mode"] else 1.0)
        # 16-bit stores (nearest or stochastic) bit-equal on every chunk whose scale matched
        P.assert_err_close(synth.host(d[1]), err, f"{tag}: err", eslack, exact=d_ulp[cidx] == 0)
        P.assert_f32_close(synth.host(d[2]), m, f"{tag}: m", 0.1 * ds)
        P.assert_f32_close(synth.host(d[4]), p, f"{tag}: p",
                           lr * 0.1 * ds / (np.sqrt(v.astype(np.float64)) + 1e-8))
        assert np.array_equal(synth.host(d[3]), v), f"{tag}: v changed"
        assert int(nf.item()) == rnf, f"{tag}: non-finite count"
        gnp = _small_state(n, seed + 1000 + _, wide=var["clip"] > 0)[0]
        if var["gdt"] == "bf16":
            gnp = _bf16_bits(gnp)
    return rnf


@pytest.mark.parametrize("vname", sorted(VARIANTS))
def test_compress_bruteforce_small(vname):
    var = VARIANTS[vname]
    for n in range(1, 131):
        for chunk in sorted({64, 128, n}):
            _gpu_vs_oracle_compress(n, chunk, var, seed=n * 7 + chunk)


@pytest.mark.parametrize("vname", sorted(VARIANTS))
@pytest.mark.parametrize("n,chunk", [(1 << 20, 1 << 20), (1_000_003, 1 << 16), (300_037, 4096),
                                     (70_000, 64 * 1000), (5_000_000, 5_000_000 - 64 * 7)])
def test_compress_multi_tile(vname, n, chunk):
    """Several tiles and work blocks per chunk, ragged chunk and buffer tails, 3 steps each from the
    oracle's state."""
    _gpu_vs_oracle_compress(n, chunk, VARIANTS[vname], seed=n, steps=3)


@pytest.mark.parametrize("vname", ["fp32_plain", "bf16_ema_clip_int8_f16err"])
def test_compress_single_huge_chunk(vname):
    """One chunk of 17,000,003 elements: more than 4096 pass-1 blocks, so the scale is formed by its own
    kernel before pass 2 (the other tests take the in-block reduction)."""
    n = 17_000_003
    plan = ob.ob_plan_create(n, chunk_size=n)
    assert plan.num_chunks == 1
    _gpu_vs_oracle_compress(n, n, VARIANTS[vname], seed=5, steps=2)
    _gpu_vs_oracle_lamb(n, n, VARIANTS[vname], seed=6)


def test_compress_edge_values():
    """Negative denormals, both zeros, NaN and Inf in g and in the error buffer."""
    n = 4096 + 17
    rng = np.random.default_rng(5)
    for pattern in ("denormals", "signed_zeros", "special"):
        g = synth.draw_values(n, 31, pattern)
        err = np.where(rng.random(n) < 0.5, np.float32(0.0), synth.draw_values(n, 37, pattern))
        state = (err.astype(np.float32), np.zeros(n, np.float32),
                 np.ones(n, np.float32), np.zeros(n, np.float32))
        for vname in ("fp32_plain", "fp32_ema", "fp32_plain_f16err", "fp32_ema_bf16err"):
            _gpu_vs_oracle_compress(n, 1024, VARIANTS[vname], seed=1, g=g,
                                    state=tuple(a.copy() for a in state))


def test_compress_and_dense_divide_by_zero():
    """v = 0 with eps = 0: the update divides by zero (m/0 = +-Inf, 0/0 = NaN) on both sides, per IEEE;
    a few v are also negative denormals and +Inf."""
    n = 4096 + 5
    rng = np.random.default_rng(21)
    for vname in ("fp32_plain", "bf16_ema_clip_int8"):
        var = VARIANTS[vname]
        gnp = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        gnp[::7] = 0.0
        v = np.zeros(n, np.float32)
        v[1::11] = np.float32(-1e-45)
        v[2::13] = np.inf
        m = np.where(rng.random(n) < 0.5, np.float32(0.0), (rng.standard_normal(n) * 1e-4).astype(np.float32))
        state = (np.zeros(n, np.float32), m.astype(np.float32), v, (rng.standard_normal(n) * 0.02).astype(np.float32))
        _gpu_vs_oracle_compress_eps0(n, var, gnp, state)


def _gpu_vs_oracle_compress_eps0(n, var, gnp, state):
    err, m, v, p = (a.copy() for a in state)
    err = _as_err_format(err, var.get("edt", "f32"))
    gin = _bf16_bits(gnp) if var["gdt"] == "bf16" else gnp
    off = oracle.uniform_offsets(n, 1024)
    plan = ob.ob_plan_create(n, chunk_size=1024)
    hp = ob.hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=0.0, clip=var["clip"], ef_mode=var["ef_mode"],
                    ef_beta=0.9)
    d = [_t(a) for a in (gin, err, m, v, p)]
    words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
    scales = torch.zeros(off.size - 1, dtype=torch.float32, device=DEV)
    ob.ob_adam_compress_step(plan, d[0], d[1], d[2], d[3], d[4], words, scales, hp)
    rw, rs, _, _ = oracle.compress_step(gin, err, m, v, p, off, lr=1e-3, beta1=0.9, eps=0.0, clip=var["clip"],
                                        ef_mode=var["ef_mode"], ef_beta=0.9)
    tag = f"eps=0 v=0 {var}"
    assert np.array_equal(synth.host(words), rw), tag
    assert np.all(P.ulp_diff(synth.host(scales), rs) <= 1), tag
    P.assert_f32_close(synth.host(d[4]), p, tag + ": p")
    assert np.isinf(p).any() and np.isnan(p).any(), "the case must reach +-Inf and NaN"
    # the dense step from the same state: v grows from 0, and where g = 0 too, 0/0
    m2, v2, p2 = (a.copy() for a in state[1:])
    dd = [_t(a) for a in (gin, m2, v2, p2)]
    ob.ob_adam_warmup_step(plan, dd[0], dd[1], dd[2], dd[3], hp)
    oracle.warmup_step(gin, m2, v2, p2, lr=1e-3, beta1=0.9, beta2=0.999, eps=0.0)
    for name, t, ref in (("m", dd[1], m2), ("v", dd[2], v2), ("p", dd[3], p2)):
        P.assert_f32_close(synth.host(t), ref, tag + ": dense " + name)


def test_compress_f16_error_overflow_is_counted():
    """New errors beyond fp16's range are stored as +-Inf and counted as non-finite."""
    n = 10_000 + 3
    rng = np.random.default_rng(9)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    hit = rng.random(n) < 0.01
    # |g| = 1e6 on 1% of elements: scale ~ 1e5, so |x - g_hat| ~ 9e5 and the EMA's (1-0.9) share
    # ~ 9e4, both past fp16's largest finite value 65504
    g[hit] = np.where(rng.random(int(hit.sum())) < 0.5, -1e6, 1e6).astype(np.float32)
    for vname in ("fp32_plain_f16err", "bf16_ema_clip_int8_f16err"):
        var = dict(VARIANTS[vname], clip=0.0)
        nf = _gpu_vs_oracle_compress(n, 1024, var, seed=2, g=g)
        assert nf > 0, vname


@pytest.mark.parametrize("gdt", ["f32", "bf16"])
@pytest.mark.parametrize("bias_correction", [False, True])
def test_dense_step(gdt, bias_correction):
    for n in (1, 7, 130, 5000, 1_000_003):
        g, _, m, v, p = _small_state(n, 3)
        if gdt == "bf16":
            g = _bf16_bits(g)
        plan = ob.ob_plan_create(n, chunk_size=1 << 16)
        d = [_t(a) for a in (g, m, v, p)]
        hp = ob.hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, bias_correction=bias_correction,
                        step=3)
        ob.ob_adam_warmup_step(plan, d[0], d[1], d[2], d[3], hp)
        oracle.warmup_step(g, m, v, p, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                           bias_correction=bias_correction, step=3)
        for name, dev_t, ref in (("m", d[1], m), ("v", d[2], v), ("p", d[3], p)):
            P.assert_f32_close(synth.host(dev_t), ref, f"dense n={n} {gdt} bc={bias_correction}: {name}")


@pytest.mark.parametrize("W", [2, 8, 9])
def test_server_single_huge_chunk(W):
    """One 17,000,003-element chunk (scale formed by its own kernel before pass 2), one round."""
    n = 17_000_003
    off = oracle.uniform_offsets(n, n)
    rng = np.random.default_rng([W, 17])
    ww = rng.integers(0, 1 << 32, size=(W, (n + 31) // 32), dtype=np.uint64).astype(np.uint32)
    ws = rng.uniform(1e-4, 1e-2, size=(W, 1)).astype(np.float32)
    e = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    plan = ob.ob_plan_create(n, chunk_size=n)
    de = _t(e)
    words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
    scales = torch.zeros(1, dtype=torch.float32, device=DEV)
    ob.ob_server_reduce(plan, _t(ww).view(W, -1), _t(ws), de, words, scales)
    rw, rs = oracle.server_reduce(ww, ws, e, off)
    assert np.array_equal(synth.host(words), rw)
    gs = synth.host(scales)
    assert np.all(P.ulp_diff(gs, rs) <= 1)
    P.assert_f32_close(synth.host(de), e, f"server W={W} huge chunk: err", abs(float(gs[0]) - float(rs[0])))


def test_server_bruteforce_small():
    """W <= 8 takes the kernels' per-chunk table of averages, W > 8 the per-element sums.  Pass 1 takes
    its whole-line variant where chunk offsets are multiples of 128 and the word rows 16-byte aligned
    (n = 1000, 70001 and 1052772 here: whole wave tiles, partial ones and both), the per-lane one
    elsewhere."""
    for W in (1, 2, 3, 5, 8, 9, 16):
        for n, chunk in ((1, 64), (31, 64), (130, 64), (1000, 128), (5000, 1024), (70001, 1 << 14),
                         (1_052_772, 1 << 16)):
            off = oracle.uniform_offsets(n, chunk)
            K = off.size - 1
            rng = np.random.default_rng([W, n])
            ww = rng.integers(0, 1 << 32, size=(W, (n + 31) // 32), dtype=np.uint64).astype(np.uint32)
            ws = rng.uniform(1e-4, 1e-2, size=(W, K)).astype(np.float32)
            e = (rng.standard_normal(n) * 1e-3).astype(np.float32)
            plan = ob.ob_plan_create(n, chunk_size=chunk)
            de = _t(e)
            words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
            scales = torch.zeros(K, dtype=torch.float32, device=DEV)
            ob.ob_server_reduce(plan, _t(ww).view(W, -1), _t(ws), de, words, scales)
            rw, rs = oracle.server_reduce(ww, ws, e, off)
            tag = f"server W={W} n={n}"
            assert np.array_equal(synth.host(words), rw), tag
            gs = synth.host(scales)
            assert np.all(P.ulp_diff(gs, rs) <= 1), tag
            ds = np.abs(gs.astype(np.float64) - rs)[np.repeat(np.arange(K), np.diff(off))]
            P.assert_f32_close(synth.host(de), e, tag + ": server err", ds)


# ------------------------------------------------------------------------------------------------
# 1-bit LAMB: compressed and dense steps with the layer-wise trust ratio
# ------------------------------------------------------------------------------------------------

def _gpu_vs_oracle_lamb(n, chunk, var, seed, kind="compressed", steps=1, lr=1e-4, bias_correction=False,
                        mutate=None):
    gnp, err, m, v, p = _small_state(n, seed, wide=var["clip"] > 0)
    if mutate is not None:
        mutate(gnp, err, m, v, p)
    err = _as_err_format(err, var.get("edt", "f32"))
    if var["gdt"] == "bf16":
        gnp = _bf16_bits(gnp)
    off = oracle.uniform_offsets(n, chunk)
    K = off.size - 1
    plan = ob.ob_plan_create(n, chunk_size=chunk)
    hp = ob.hparams(lr=lr, beta1=0.9, beta2=0.999, eps=1e-8, clip=var["clip"], ef_mode=var["ef_mode"],
                    ef_beta=0.9, bias_correction=bias_correction, step=3)
    for st in range(steps):
        d = [_t(a) for a in (gnp, err, m, v, p)]
        ratios = torch.full((K,), -7.0, dtype=torch.float32, device=DEV)
        tag = f"lamb {kind} n={n} chunk={chunk} {var} step {st}"
        if kind == "compressed":
            words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
            scales = torch.zeros(K, dtype=torch.float32, device=DEV)
            signs = torch.zeros(n, dtype=torch.int8, device=DEV) if var["signs"] else None
            nf = torch.zeros(1, dtype=torch.int64, device=DEV)
            sr_h, sr_o = _sr_hp(var, 3 + st)
            for k, val in sr_h.items():
                setattr(hp, k, val)
            ob.ob_lamb_compress_step(plan, d[0], d[1], d[2], d[3], d[4], words, scales, ratios, hp, signs, nf)
            rw, rs, rr, rsg, rnf = oracle.lamb_compress_step(
                gnp, err, m, v, p, off, lr=lr, beta1=0.9, eps=1e-8, clip=var["clip"], ef_mode=var["ef_mode"],
                ef_beta=0.9, want_signs=var["signs"], count_nonfinite=True, **sr_o)
            assert np.array_equal(synth.host(words), rw), f"{tag}: words"
            if signs is not None:
                assert np.array_equal(synth.host(signs), rsg), f"{tag}: signs"
            gs = synth.host(scales)
            assert np.all(P.ulp_diff(gs, rs) <= 1), f"{tag}: scales"
            assert int(nf.item()) == rnf, f"{tag}: non-finite count"
            assert np.array_equal(synth.host(d[3]), v), f"{tag}: v changed"
            ds = np.abs(gs.astype(np.float64) - rs.astype(np.float64))
        else:
            ob.ob_lamb_warmup_step(plan, d[0], d[2], d[3], d[4], ratios, hp)
            rr = oracle.lamb_warmup_step(gnp, m, v, p, off, lr=lr, beta1=0.9, beta2=0.999, eps=1e-8,
                                         bias_correction=bias_correction, step=3)
            P.assert_f32_close(synth.host(d[3]), v, f"{tag}: v")
            ds = np.zeros(K)
        gr = synth.host(ratios)
        both_nan = np.isnan(gr) & np.isnan(rr)
        dr_ulp = np.where(both_nan, 0, P.ulp_diff(gr, rr))
        assert np.all(dr_ulp <= np.where(ds > 0, 2, 1)), f"{tag}: ratios {gr} vs {rr}"
        cidx = np.repeat(np.arange(K), np.diff(off))
        ds_e = np.where(np.isfinite(ds), ds, 0.0)[cidx]
        dr = np.where(both_nan, 0.0, np.abs(gr.astype(np.float64) - rr.astype(np.float64)))[cidx]
        dr = np.where(np.isfinite(dr), dr, 0.0)
        den = np.sqrt(v.astype(np.float64)) + 1e-8
        if bias_correction and kind == "dense":
            den = np.sqrt(v.astype(np.float64) / (1 - 0.999 ** 3)) + 1e-8
        u = np.abs(m.astype(np.float64)) / den
        rabs = np.where(np.isfinite(rr), np.abs(rr.astype(np.float64)), 0.0)[cidx]
        if kind == "compressed":
            P.assert_err_close(synth.host(d[1]), err, f"{tag}: err", ds_e * (0.1 if var["ef_mode"] else 1.0),
                               exact=ds_e == 0.0)
        P.assert_f32_close(synth.host(d[2]), m, f"{tag}: m", 0.1 * ds_e)
        P.assert_f32_close(synth.host(d[4]), p, f"{tag}: p", lr * (rabs * 0.1 * ds_e / den + dr * u))
        gnp = _small_state(n, seed + 1000 + st, wide=var["clip"] > 0)[0]
        if var["gdt"] == "bf16":
            gnp = _bf16_bits(gnp)
    return rr


LAMB_VARIANTS = ("fp32_plain", "bf16_ema_clip_int8_f16err", "fp32_ema_bf16err_sr")


@pytest.mark.parametrize("vname", LAMB_VARIANTS)
def test_lamb_compress_bruteforce_small(vname):
    for n in range(1, 131):
        for chunk in sorted({64, 128, n}):
            _gpu_vs_oracle_lamb(n, chunk, VARIANTS[vname], seed=n * 5 + chunk)


@pytest.mark.parametrize("bias_correction", [False, True])
def test_lamb_dense_bruteforce_small(bias_correction):
    for n in range(1, 131, 3):
        for chunk in sorted({64, n}):
            _gpu_vs_oracle_lamb(n, chunk, VARIANTS["fp32_plain"], seed=n, kind="dense",
                                bias_correction=bias_correction)


@pytest.mark.parametrize("vname", LAMB_VARIANTS + ("bf16_plain_bf16err",))
@pytest.mark.parametrize("n,chunk", [(1 << 20, 1 << 20), (1_000_003, 1 << 16), (5_000_000, 5_000_000 - 64 * 7)])
def test_lamb_compress_multi_tile(vname, n, chunk):
    _gpu_vs_oracle_lamb(n, chunk, VARIANTS[vname], seed=n, steps=3)


@pytest.mark.parametrize("n,chunk", [(1_000_003, 1 << 16), (3_000_017, 1 << 20)])
def test_lamb_dense_multi_tile(n, chunk):
    for bc in (False, True):
        _gpu_vs_oracle_lamb(n, chunk, VARIANTS["bf16_plain"], seed=n, kind="dense", steps=2, bias_correction=bc)


def test_lamb_degenerate_layers():
    """A zero layer (r = 1), a zero direction (r = 1, p unchanged) and a NaN parameter (its layer's
    ratio and update are NaN, the other layers are not touched by it)."""
    n, chunk = 4 * 4096 + 100, 4096

    def mutate(g, err, m, v, p):
        p[4096:8192] = 0.0
        g[8192:12288] = 0.0
        err[8192:12288] = 0.0
        m[8192:12288] = 0.0
        p[5] = np.nan

    for kind in ("compressed", "dense"):
        rr = _gpu_vs_oracle_lamb(n, chunk, VARIANTS["fp32_plain"], seed=4, kind=kind, mutate=mutate)
        assert np.isnan(rr[0]) and rr[1] == 1.0
        if kind == "compressed":
            assert rr[2] == 1.0


def bert_sample_chunks(K: int) -> list[int]:
    """A spread of BERT-base's tensors for the variant workloads: the embeddings and embedding
    LayerNorm (chunks 0-4, the word embedding being the largest chunk), every 7th tensor after them
    (which walks through every kind of tensor of the 16-tensor layers), and the last."""
    return sorted(set(range(5)) | set(range(5, K, 7)) | {K - 1})


def test_workload_bert_base_lamb():
    """1-bit LAMB on BERT-base's 197 tensors (one layer each): 5 dense LAMB steps, then 20 compressed;
    34 layers (every kind of tensor, the embedding included) checked every step, ratios included."""
    w = synth.BERT_BASE_LAMB
    counts = P.run_workload(w, chunks=bert_sample_chunks(w.n_chunks), log=lambda *_: None)
    assert counts["dense"] == 5 and counts["compressed"] == 20


# ------------------------------------------------------------------------------------------------
# diagnostics: per-chunk error-buffer norm and +1 count
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("vname", ["fp32_plain", "bf16_ema_clip_int8_f16err", "fp32_ema_bf16err"])
@pytest.mark.parametrize("lamb", [False, True])
def test_diagnostics(vname, lamb):
    var = VARIANTS[vname]
    for n, chunk in ((1, 64), (130, 64), (5000, 1024), (1_000_003, 1 << 16), (3_000_017, 3_000_017)):
        gnp, err, m, v, p = _small_state(n, n + 3, wide=var["clip"] > 0)
        err = _as_err_format(err, var.get("edt", "f32"))
        if var["gdt"] == "bf16":
            gnp = _bf16_bits(gnp)
        off = oracle.uniform_offsets(n, chunk)
        K = off.size - 1
        plan = ob.ob_plan_create(n, chunk_size=chunk)
        ss = torch.full((K,), -1.0, dtype=torch.float64, device=DEV)
        pc = torch.full((K,), -1, dtype=torch.int64, device=DEV)
        ob.ob_plan_set_diagnostics(plan, ss, pc)
        d = [_t(a) for a in (gnp, err, m, v, p)]
        words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
        scales = torch.zeros(K, dtype=torch.float32, device=DEV)
        hp = ob.hparams(lr=1e-4, clip=var["clip"], ef_mode=var["ef_mode"], ef_beta=0.9)
        if lamb:
            ob.ob_lamb_compress_step(plan, *d, words, scales, torch.zeros(K, device=DEV), hp)
        else:
            ob.ob_adam_compress_step(plan, *d, words, scales, hp)
        rss, rpc = oracle.diagnostics(err, synth.host(words), off)
        tag = f"diagnostics n={n} chunk={chunk} {vname} lamb={lamb}"
        gss = synth.host(ss)
        assert np.all(np.abs(gss - rss) <= 1e-10 * rss), f"{tag}: {gss} vs {rss}"
        assert np.array_equal(synth.host(pc), rpc), tag
        # switched off: the next step leaves the arrays alone
        ob.ob_plan_set_diagnostics(plan, None, None)
        ss.fill_(-1.0)
        ob.ob_adam_compress_step(plan, *d, words, scales, hp)
        torch.cuda.synchronize()
        assert bool((ss == -1.0).all()), tag


# ------------------------------------------------------------------------------------------------
# edge cases of the boundary
# ------------------------------------------------------------------------------------------------

def test_zero_size_is_noop():
    plan = ob.ob_plan_create(0, chunk_size=64)
    z = torch.zeros(0, dtype=torch.float32, device=DEV)
    zi = torch.zeros(0, dtype=torch.int32, device=DEV)
    hp = ob.hparams()
    ob.ob_adam_compress_step(plan, z, z, z, z, z, zi, torch.zeros(0, device=DEV), hp)
    ob.ob_adam_warmup_step(plan, z, z, z, z, hp)
    ob.ob_pack(z, zi)
    ob.ob_unpack(None, zi, 0, z)


def test_misaligned_and_invalid_arguments():
    n = 1024
    plan = ob.ob_plan_create(n, chunk_size=256)
    big = torch.zeros(n + 4, dtype=torch.float32, device=DEV)
    ok = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(5)]
    words = torch.zeros(n // 32, dtype=torch.int32, device=DEV)
    scales = torch.zeros(4, dtype=torch.float32, device=DEV)
    hp = ob.hparams()
    with pytest.raises(ob.ObError) as e:
        ob.ob_adam_compress_step(plan, big[1:n + 1], *ok[1:], words, scales, hp)   # g + 4 bytes
    assert e.value.status == 2
    with pytest.raises(ob.ObError) as e:
        ob.ob_adam_compress_step(plan, ok[0], big[2:n + 2], *ok[2:], words, scales, hp)
    assert e.value.status == 2
    with pytest.raises(ob.ObError) as e:       # interior chunk boundary not a multiple of 64
        ob.ob_plan_create(200, chunk_offsets=[0, 100, 200])
    assert e.value.status == 2
    with pytest.raises(ob.ObError) as e:       # offsets do not end at n
        ob.ob_plan_create(200, chunk_offsets=[0, 64, 199])
    assert e.value.status == 1
    with pytest.raises(ob.ObError) as e:
        ob.ob_plan_create(-1, chunk_size=64)
    assert e.value.status == 1
    with pytest.raises(ob.ObError) as e:       # W = 0 workers
        ob.ob_server_reduce(plan, torch.zeros((0, n // 32), dtype=torch.int32, device=DEV),
                            torch.zeros((0, 4), device=DEV), ok[0], words, scales)
    assert e.value.status == 1
    with pytest.raises(ob.ObError) as e:       # unpack n differs from the plan
        ob.ob_unpack(plan, torch.zeros(n // 64, dtype=torch.int32, device=DEV), n // 2,
                     torch.zeros(n // 2, device=DEV), scales=scales)
    assert e.value.status == 1
    with pytest.raises(ValueError):            # host tensors are refused: no CPU path
        ob.ob_pack(torch.zeros(64), words[:2])
    e16 = torch.zeros(n + 4, dtype=torch.float16, device=DEV)
    with pytest.raises(ob.ObError) as e:       # 16-bit error buffer 2 bytes off an 8-byte boundary
        ob.ob_adam_compress_step(plan, ok[0], e16[1:n + 1], *ok[2:], words, scales, hp)
    assert e.value.status == 2
    with pytest.raises(TypeError):
        ob.ob_adam_compress_step(plan, ok[0], torch.zeros(n, dtype=torch.int16, device=DEV), *ok[2:],
                                 words, scales, hp)
    # through the C ABI: an unknown error dtype, and fp16 gradients (not supported), are OB_ERR_DTYPE
    import ctypes
    L = ob.lib()
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in ok]
    for gdt, edt in ((0, 3), (2, 0), (0, -1)):
        st = L.ob_adam_compress_step(plan.handle, ptrs[0], gdt, ptrs[1], edt, ptrs[2], ptrs[3], ptrs[4],
                                     ctypes.c_void_p(words.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                                     None, None, ctypes.byref(hp), None)
        assert st == 3, (gdt, edt, st)
    # stochastic rounding of an fp32 error buffer, or an unknown rounding mode, is OB_ERR_ARG
    for edt, rounding in ((0, ob.OB_ROUND_STOCHASTIC), (1, 2), (2, -1)):
        bad = ob.hparams(err_rounding=rounding)
        st = L.ob_adam_compress_step(plan.handle, ptrs[0], 0, ptrs[1], edt, ptrs[2], ptrs[3], ptrs[4],
                                     ctypes.c_void_p(words.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                                     None, None, ctypes.byref(bad), None)
        assert st == 1, (edt, rounding, st)


def test_deterministic():
    n = 3_000_017
    var = VARIANTS["bf16_ema_clip_int8"]
    g, err, m, v, p = _small_state(n, 77, wide=True)
    gb = _bf16_bits(g)
    plan = ob.ob_plan_create(n, chunk_size=1 << 18)
    hp = ob.hparams(lr=1e-4, clip=5.0, ef_mode=1, ef_beta=0.9)
    outs = []
    for _ in range(2):
        d = [_t(a) for a in (gb, err, m, v, p)]
        words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
        scales = torch.zeros(plan.num_chunks, dtype=torch.float32, device=DEV)
        signs = torch.zeros(n, dtype=torch.int8, device=DEV)
        ob.ob_adam_compress_step(plan, d[0], d[1], d[2], d[3], d[4], words, scales, hp, signs)
        outs.append([synth.host(t) for t in (d[1], d[2], d[4], words, scales, signs)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert var["signs"]


@pytest.mark.parametrize("optimizer", ["adam", "lamb"])
def test_resume_is_bit_identical(optimizer):
    """Checkpoint / resume: the whole optimizer state is the caller's buffers (err, m, v, p, the
    non-finite counter) plus the schedule's step counters; the plan holds none of it.  Run 4 steps and
    save that state to the host, run 4 more; then restore it into fresh buffers with a fresh plan and
    optimizer and run the same 4 steps: every output of every step is bit-identical.  The schedule
    crosses the freeze step and a refresh step, and the error buffer is bf16 with stochastic
    rounding, whose random stream follows the step index."""
    from adam_ob_compress_amd import schedule

    n, chunk = 1_000_003, 1 << 16
    cls = schedule.OneBitLamb if optimizer == "lamb" else schedule.OneBitAdam
    kw = dict(lr=1e-4, clip=5.0, ef_mode=ob.OB_EF_EMA, ef_beta=0.9, int8_signs=True, count_nonfinite=True,
              freeze_step=2, refresh_period=5, err_rounding="stochastic", sr_seed=0x5EED)
    gen = torch.Generator(device=DEV)
    grads = []
    for s in range(8):
        gen.manual_seed(1000 + s)
        grads.append(torch.randn(n, generator=gen, device=DEV) * 1e-3)
    gen.manual_seed(7)
    err0 = (torch.randn(n, generator=gen, device=DEV) * 1e-4).to(torch.bfloat16)
    m0 = torch.zeros(n, device=DEV)
    v0 = torch.zeros(n, device=DEV)
    p0 = torch.randn(n, generator=gen, device=DEV) * 0.02

    def outputs(opt, kind):
        """What a step of this kind writes (a dense step leaves the sign outputs alone)."""
        out = [opt.err, opt.m, opt.v, opt.p, opt.nonfinite]
        if kind == "compressed":
            out += [opt.words, opt.scales, opt.signs]
        if optimizer == "lamb":
            out.append(opt.ratios)
        return [synth.host(t) for t in out]

    def make(state, counters):
        plan = ob.ob_plan_create(n, chunk_size=chunk)
        bufs = [torch.from_numpy(a.copy()).to(DEV) for a in state[:4]]
        bufs[0] = bufs[0].view(torch.bfloat16)          # saved as the bf16 bits (int16)
        opt = cls(plan, *bufs, **kw)
        opt.nonfinite.copy_(torch.from_numpy(state[4].astype(np.int64)))
        opt.step_index, opt.dense_steps = counters
        return plan, opt

    def save(opt):
        st = [synth.host(t) for t in (opt.err, opt.m, opt.v, opt.p, opt.nonfinite)]
        st[0] = st[0].view(np.int16)
        return st, (opt.step_index, opt.dense_steps)

    plan = ob.ob_plan_create(n, chunk_size=chunk)
    opt = cls(plan, err0.clone(), m0.clone(), v0.clone(), p0.clone(), **kw)
    kinds = [opt.step(g) for g in grads[:4]]
    torch.cuda.synchronize()
    state, counters = save(opt)
    ref = []
    for g in grads[4:]:
        kinds.append(opt.step(g))
        torch.cuda.synchronize()
        ref.append(outputs(opt, kinds[-1]))
    assert kinds == ["dense", "dense", "compressed", "compressed", "dense", "compressed", "compressed",
                     "compressed"]

    plan2, opt2 = make(state, counters)
    for k, g in enumerate(grads[4:]):
        kind = opt2.step(g)
        assert kind == kinds[4 + k]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref[k], outputs(opt2, kind))):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"step {4 + k}, output {i}"


def test_kernel_timing_api():
    n = 1 << 20
    plan = ob.ob_plan_create(n, chunk_size=1 << 18)
    d = [torch.ones(n, dtype=torch.float32, device=DEV) for _ in range(5)]
    words = torch.zeros(n // 32, dtype=torch.int32, device=DEV)
    scales = torch.zeros(4, dtype=torch.float32, device=DEV)
    ob.ob_plan_set_timing(plan, True)
    for _ in range(3):
        ob.ob_adam_compress_step(plan, *d, words, scales, ob.hparams())
    ob.ob_adam_warmup_step(plan, d[0], d[2], d[3], d[4], ob.hparams())
    groups = plan.num_groups(ob.OB_F32, ob.OB_F32)   # launches of each pass per step (1 by default)
    ms, cnt = ob.ob_plan_read_timing(plan, ob.OB_KERNEL_COMPRESS)
    assert cnt == 3 * groups and ms > 0
    assert ob.ob_plan_read_timing(plan, ob.OB_KERNEL_CHUNK_SUMSQ)[1] == 3 * groups
    assert ob.ob_plan_read_timing(plan, ob.OB_KERNEL_DENSE)[1] == 1


# ------------------------------------------------------------------------------------------------
# the workloads at full size
# ------------------------------------------------------------------------------------------------

def test_workload_single_1m():
    """2^20 fp32 elements, one chunk, 10 compressed steps, every output checked every step."""
    counts = P.run_workload(synth.SINGLE_1M, log=lambda *_: None)
    assert counts["compressed"] == 10 and counts["dense"] == 0


def test_workload_bert_base():
    """197 per-tensor chunks (108,891,648 fp32 elements): 5 dense steps, then 20 compressed; every
    chunk checked every step, diagnostics (error norm, +1 count) included."""
    counts = P.run_workload(synth.BERT_BASE, log=lambda *_: None, diagnostics=True)
    assert counts["dense"] == 5 and counts["compressed"] == 20


@pytest.mark.parametrize("edt", ["bf16", "f16", "bf16-sr"])
def test_workload_bert_base_16bit_error(edt):
    """The BERT-base workload with its error buffer stored in bf16 / fp16 (bf16-sr: stochastically
    rounded, a new random stream every step); the sampled chunks (every kind of tensor) checked every
    step.
    The word embedding (23.4M elements, the largest chunk) is checked in the bf16 case only: the
    oracle runs one chunk per thread, so that chunk alone sets the test's time."""
    w = synth.WORKLOADS[f"{synth.BERT_BASE.name}-err-{edt}"]
    chunks = bert_sample_chunks(w.n_chunks)
    if edt != "bf16":
        chunks = chunks[1:]
    counts = P.run_workload(w, chunks=chunks, log=lambda *_: None)
    assert counts["dense"] == 5 and counts["compressed"] == 20


@pytest.mark.parametrize("name", ["bert-base-110M-fp32-err-bf16", "bert-base-110M-fp32-err-f16",
                                  "bert-base-110M-fp32-err-bf16-sr", "bert-base-110M-fp32-lamb"])
def test_workload_bert_base_variants_every_chunk(name):
    """BERT-base's variants, every one of the 197 chunks (layers, for LAMB): after the first compressed
    step (step index 5) and after a dense step (index 0), each over the whole buffer from a seeded state
    with a non-zero error buffer and momentum; LAMB's ratios included."""
    P.check_every_chunk(synth.WORKLOADS[name], dense_step=0, log=lambda *_: None)


def test_workload_server_2p28_w8():
    """n = 2^28, W = 8, chunks of 2^20: 10 rounds of server reduce + unpack; the server error carries
    across rounds.  Round 0 (server error 0, seeded worker words and scales) checks all 256 chunks;
    later rounds check 39 (every 8th, the last and 6 seeded random ones), whose server error the
    oracle carries from round 0."""
    w = synth.SERVER_W8
    off = w.chunk_offsets()
    K = w.n_chunks
    plan = ob.ob_plan_create(w.n, chunk_size=w.chunk)
    e = torch.zeros(w.n, dtype=torch.float32, device=DEV)
    words = torch.zeros((w.n + 31) // 32, dtype=torch.int32, device=DEV)
    scales = torch.zeros(K, dtype=torch.float32, device=DEV)
    out = torch.empty(w.n, dtype=torch.float32, device=DEV)
    tracked = P.tracked_chunks(K, set(range(0, K, 8)) | {K - 1})
    ref_e = {c: np.zeros(int(off[c + 1] - off[c]), np.float32) for c in range(K)}
    for r in range(w.steps):
        chunks = range(K) if r == 0 else tracked
        if r == 1:
            ref_e = {c: ref_e[c] for c in tracked}
        ww = synth.draw_worker_words(w, r, DEV)
        ws = synth.draw_worker_scales(w, r, DEV)
        for c in chunks:
            e[int(off[c]):int(off[c + 1])].copy_(torch.from_numpy(ref_e[c]))
        ob.ob_server_reduce(plan, ww, ws, e, words, scales)
        ob.ob_unpack(plan, words, w.n, out, scales=scales)
        torch.cuda.synchronize()
        wwh, wsh, gsc = synth.host(ww), synth.host(ws), synth.host(scales)

        def check(c, r=r, wwh=wwh, wsh=wsh, gsc=gsc):
            a, b = int(off[c]), int(off[c + 1])
            rw, rs = oracle.server_reduce(np.ascontiguousarray(wwh[:, a // 32:b // 32]),
                                          np.ascontiguousarray(wsh[:, c:c + 1]), ref_e[c],
                                          np.asarray([0, b - a], np.int64))
            tag = f"server round {r} chunk {c}"
            assert np.array_equal(synth.host(words[a // 32:b // 32]), rw), tag
            gs = gsc[c]
            assert P.ulp_diff(gs, rs[0]) <= 1, tag
            ds = abs(float(gs) - float(rs[0]))
            P.assert_f32_close(synth.host(e[a:b]), ref_e[c], tag + ": server err", ds)
            ro = oracle.unpack(rw, b - a, np.asarray([0, b - a], np.int64), rs)
            P.assert_f32_close(synth.host(out[a:b]), ro, tag + ": unpack", ds)
            if ds == 0.0:
                assert np.array_equal(synth.host(out[a:b]), ro), tag + ": unpack"

        for f in [P._POOL.submit(check, c) for c in chunks]:
            f.result()


@pytest.mark.slow
def test_one_chunk_beyond_2_32_elements():
    """One chunk of 2^32 + 4099 elements (bf16 g, fp32 state; ~78 GB resident), in the launch
    configuration the bench uses for large buffers (the per-chunk sums before pass 2 run here: the
    chunk has ~175,000 pass-1 blocks).  The oracle cannot take the chunk whole in test time, so:
      * the scale against the oracle's sum of squares over host copies of x = g + err, taken in
        2^28-element pieces (the same double sum in a different grouping; 1 ulp allowed, as for the
        GPU's own order);
      * at 8,192 random elements plus the first and last 96: the sign bit against x >= 0, and err, m
        and p against the oracle's pack / unpack / worker update of those elements given that scale;
      * the tail word's bits beyond n are 0."""
    w = dataclasses.replace(synth.GPT2_XL, name="one-chunk-2^32+4099", n=(1 << 32) + 4099, chunk=(1 << 32) + 4099)
    n = w.n
    err, m, v, p = synth.draw_state(w, DEV)
    synth._fill_normal(err, 1e-4, 77, 1, 0)                 # a non-zero error buffer (seeded input)
    synth._fill_normal(m, 1e-4, 77, 2, 0)
    g = synth.draw_grad(w, 0, DEV)
    rng = np.random.default_rng(2024)
    idx = np.unique(np.concatenate([rng.integers(0, n, 8192), np.arange(96), np.arange(n - 96, n)]))
    it = torch.from_numpy(idx).to(DEV)
    g_s = synth.host(g[it]).astype(np.uint32) << 16
    x_s = (g_s.view(np.float32) + synth.host(err[it])).astype(np.float32)
    m_s, v_s, p_s = (synth.host(t[it]) for t in (m, v, p))
    # the oracle's sum of squares of x, piece by piece (ascending within each piece)
    S = 0.0
    piece = 1 << 28
    for a in range(0, n, piece):
        b = min(n, a + piece)
        gp = synth.host(g[a:b]).astype(np.uint32) << 16
        xp = gp.view(np.float32) + synth.host(err[a:b])
        S += oracle.chunk_sumsq(xp, 0, b - a)
        del gp, xp
    scale_ref = np.float32(np.sqrt(S / n))

    plan = ob.ob_plan_create(n, chunk_size=n)
    words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
    scales = torch.zeros(1, dtype=torch.float32, device=DEV)
    hp = ob.hparams(lr=w.lr, beta1=w.beta1, eps=w.eps)
    ob.ob_adam_compress_step(plan, g, err, m, v, p, words, scales, hp)
    torch.cuda.synchronize()

    sc = np.float32(scales[0].item())
    assert P.ulp_diff(sc, scale_ref) <= 1, (sc, scale_ref)
    ds = abs(float(sc) - float(scale_ref))
    wd = synth.host(words[torch.from_numpy(idx // 32).to(DEV)])
    bits = (wd >> (idx % 32).astype(np.uint32)) & 1
    assert np.array_equal(bits.astype(bool), x_s >= np.float32(0.0)), "sign bits"
    last = int(synth.host(words[-1:])[0])
    assert last >> (n % 32) == 0, "bits beyond n"
    k = idx.size
    off = np.asarray([0, k], np.int64)
    w_ref = oracle.pack(x_s)
    ghat = oracle.unpack(w_ref, k, off, np.asarray([scale_ref], np.float32))
    err_ref = (x_s - ghat).astype(np.float32)               # plain error feedback: x - g_hat, one rounding
    oracle.worker_update(w_ref, np.asarray([scale_ref], np.float32), m_s, v_s, p_s, off,
                         lr=w.lr, beta1=w.beta1, eps=w.eps)
    b1, lr, eps = (np.float64(np.float32(t)) for t in (w.beta1, w.lr, w.eps))
    P.assert_f32_close(synth.host(err[it]), err_ref, "err", ds)
    P.assert_f32_close(synth.host(m[it]), m_s, "m", ds * (1 - b1))
    P.assert_f32_close(synth.host(p[it]), p_s, "p", lr * ds * (1 - b1) / (np.sqrt(v_s.astype(np.float64)) + eps))
    del plan


@pytest.mark.slow
def test_workload_gpt2_1p5b():
    """1,557,611,200 bf16-gradient elements, chunks of 2^24 (93 chunks, ragged tail): 10 compressed
    steps; chunks 0, 1, 46, the tail chunk 92 and 6 seeded random chunks checked every step."""
    w = synth.GPT2_XL
    chunks = P.tracked_chunks(w.n_chunks, [0, 1, 46, w.n_chunks - 1])
    assert len(chunks) == 10
    counts = P.run_workload(w, chunks=chunks, log=lambda *_: None)
    assert counts["compressed"] == 10


@pytest.mark.slow
def test_workload_gpt2_1p5b_every_chunk():
    """GPT-2-1.5B: all 93 chunks against the oracle after a compressed step over the whole buffer, from
    a seeded state with a non-zero error buffer and momentum."""
    P.check_every_chunk(synth.GPT2_XL, log=lambda *_: None)


@pytest.mark.slow
def test_workload_llama2_7b():
    """6,738,415,616 bf16-gradient elements (~129 GB resident), chunks of 2^24 (402 chunks), clip 5,
    EMA error, int8 signs, dense refresh at t = 16, 32, 48: chunks 0, 200, the tail 401 and 6 seeded
    random chunks checked on all 48 steps."""
    w = synth.LLAMA2_7B
    chunks = P.tracked_chunks(w.n_chunks, [0, 200, w.n_chunks - 1])
    assert len(chunks) == 9
    counts = P.run_workload(w, chunks=chunks, log=lambda *_: None)
    assert counts["dense"] == 3 and counts["compressed"] == 45


@pytest.mark.slow
def test_workload_llama2_7b_every_chunk():
    """Llama-2-7B: all 402 chunks against the oracle after a compressed step (step index 0) and after a
    variance refresh (step index 15, t = 16), each over the whole buffer from a seeded state with a
    non-zero error buffer and momentum."""
    P.check_every_chunk(synth.LLAMA2_7B, dense_step=15, log=lambda *_: None)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["llama2-7B-bf16-lamb", "gpt2-1.5B-bf16-err-bf16"])
def test_workload_large_variants_every_chunk(name):
    """Every chunk of 1-bit LAMB on Llama-2-7B's 291 layers (ratios included; the two 131M-element
    layers take the per-chunk sums kernel) and of GPT-2-1.5B with a bf16 error buffer, after the first
    compressed step over the whole buffer from a seeded state.  (LAMB's dense step on these layers is
    checked every step on the tracked layers of test_workload_llama2_7b_lamb; checking it on every
    layer too would double this test's ~75 s of host copies.)"""
    P.check_every_chunk(synth.WORKLOADS[name], log=lambda *_: None)


@pytest.mark.slow
def test_workload_llama2_7b_bf16_error():
    """The Llama-2-7B workload with a bf16 error buffer, 20 steps (one dense refresh at t = 16):
    chunks 0, 200, the tail 401 and 6 seeded random chunks checked every step."""
    w = dataclasses.replace(synth.WORKLOADS[f"{synth.LLAMA2_7B.name}-err-bf16"], steps=20)
    counts = P.run_workload(w, chunks=P.tracked_chunks(w.n_chunks, [0, 200, w.n_chunks - 1]),
                            log=lambda *_: None)
    assert counts["dense"] == 1 and counts["compressed"] == 19


@pytest.mark.slow
def test_workload_llama2_7b_lamb():
    """1-bit LAMB on Llama-2-7B's 291 tensors (6,738,415,616 bf16-gradient elements), clip, EMA error,
    int8 signs, 2 dense steps then 4 compressed: the embedding (layer 0), a mid-network projection
    (145), the output head (290) and 6 seeded random layers checked every step."""
    w = dataclasses.replace(synth.LLAMA2_7B_LAMB, steps=6)
    counts = P.run_workload(w, chunks=P.tracked_chunks(w.n_chunks, [0, 145, w.n_chunks - 1]),
                            log=lambda *_: None)
    assert counts["dense"] == 2 and counts["compressed"] == 4
