"""GPU parity of the worker's step split at the exchange (reading R19), marked gpu.

* worker compress and worker update against the oracle's, brute force over n = 1..130 and on
  multi-tile inputs (the update takes the oracle's words and scales, so no GPU output feeds the oracle);
* at one worker, worker compress then worker update against the fused compressed step on the GPU,
  bit for bit;
* a data-parallel round on one GPU: W workers' compress, the server reduce of their words and scales,
  and the shared update from the server's words, against the same pipeline in the oracle, over
  several steps (worker errors and the server error carried).
"""
import numpy as np
import pytest
import torch

import oracle
import adam_ob_compress_amd as ob
from adam_ob_compress_amd import synth

import _parity as P
from test_gpu_parity import DEV, VARIANTS, _as_err_format, _bf16_bits, _small_state, _t

pytestmark = pytest.mark.gpu

SPLIT_VARIANTS = ("fp32_plain", "bf16_ema_clip_int8", "fp32_plain_f16err", "fp32_ema_bf16err_sr")
HP = dict(lr=1e-4, beta1=0.9, eps=1e-8)


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    ob.lib()
    yield
    torch.cuda.synchronize()


def _sr(var, step):
    if not var.get("sr"):
        return {}, {}
    return (dict(err_rounding=ob.OB_ROUND_STOCHASTIC, sr_seed=77, step=step),
            dict(stochastic=True, sr_seed=77, sr_step=step))


def _compress_vs_oracle(n, chunk, var, seed, steps=1):
    gnp, err, m, v, p = _small_state(n, seed, wide=var["clip"] > 0)
    err = _as_err_format(err, var.get("edt", "f32"))
    if var["gdt"] == "bf16":
        gnp = _bf16_bits(gnp)
    off = oracle.uniform_offsets(n, chunk)
    plan = ob.ob_plan_create(n, chunk_size=chunk)
    for st in range(steps):
        sr_h, sr_o = _sr(var, 3 + st)
        hp = ob.hparams(**HP, clip=var["clip"], ef_mode=var["ef_mode"], ef_beta=0.9, **sr_h)
        d_g, d_err = _t(gnp), _t(err)
        words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
        scales = torch.zeros(off.size - 1, dtype=torch.float32, device=DEV)
        signs = torch.zeros(n, dtype=torch.int8, device=DEV) if var["signs"] else None
        nf = torch.zeros(1, dtype=torch.int64, device=DEV)
        ob.ob_adam_worker_compress(plan, d_g, d_err, words, scales, hp, signs, nf)
        rw, rs, rsg, rnf = oracle.worker_compress(gnp, err, off, clip=var["clip"], ef_mode=var["ef_mode"],
                                                  ef_beta=0.9, want_signs=var["signs"], count_nonfinite=True,
                                                  **sr_o)
        tag = f"worker compress n={n} chunk={chunk} {var} step {st}"
        assert np.array_equal(synth.host(words), rw), f"{tag}: words"
        if signs is not None:
            assert np.array_equal(synth.host(signs), rsg), f"{tag}: signs"
        gs = synth.host(scales)
        assert np.all(P.ulp_diff(gs, rs) <= 1), f"{tag}: scales"
        assert int(nf.item()) == rnf, f"{tag}: non-finite count"
        cidx = np.repeat(np.arange(off.size - 1), np.diff(off))
        ds = np.abs(gs.astype(np.float64) - rs.astype(np.float64))[cidx]
        ds = np.where(np.isfinite(ds), ds, 0.0)
        P.assert_err_close(synth.host(d_err), err, f"{tag}: err", ds * (0.1 if var["ef_mode"] else 1.0),
                           exact=ds == 0.0)

        # the update from the oracle's words and scales
        d_m, d_v, d_p = _t(m), _t(v), _t(p)
        ob.ob_adam_worker_update(plan, _t(rw), _t(rs), d_m, d_v, d_p, hp)
        oracle.worker_update(rw, rs, m, v, p, off, **HP)
        tag = f"worker update n={n} chunk={chunk} step {st}"
        assert np.array_equal(synth.host(d_m), m), f"{tag}: m"
        assert np.array_equal(synth.host(d_p), p), f"{tag}: p"
        assert np.array_equal(synth.host(d_v), v), f"{tag}: v changed"
        gnp = _small_state(n, seed + 1000 + st, wide=var["clip"] > 0)[0]
        if var["gdt"] == "bf16":
            gnp = _bf16_bits(gnp)


@pytest.mark.parametrize("vname", SPLIT_VARIANTS)
def test_worker_split_bruteforce_small(vname):
    for n in range(1, 131):
        for chunk in sorted({64, 128, n}):
            _compress_vs_oracle(n, chunk, VARIANTS[vname], seed=n * 3 + chunk)


@pytest.mark.parametrize("vname", SPLIT_VARIANTS)
@pytest.mark.parametrize("n,chunk", [(1_000_003, 1 << 16), (5_000_000, 5_000_000 - 64 * 7), (17_000_003, 17_000_003)])
def test_worker_split_multi_tile(vname, n, chunk):
    """Several tiles and blocks, ragged tails, 2 steps; the last case is one chunk of more than 4096
    pass-1 blocks (its scale formed by the per-chunk sums kernel)."""
    _compress_vs_oracle(n, chunk, VARIANTS[vname], seed=n, steps=2)


@pytest.mark.parametrize("vname", SPLIT_VARIANTS)
def test_one_worker_split_equals_fused_step(vname):
    """At one worker the exchange returns the worker's own words and scales: compress then update is
    the fused step, bit for bit, on the GPU (BERT-base's chunk layout)."""
    var = VARIANTS[vname]
    w = synth.BERT_BASE
    n, offs = w.n, w.offsets
    plan = ob.ob_plan_create(n, chunk_offsets=offs)
    err, m, v, p = synth.draw_state(w, DEV)
    if var.get("edt", "f32") != "f32":
        err = err.to(torch.bfloat16 if var["edt"] == "bf16" else torch.float16)
    g = synth.draw_grad(w, 0, DEV)
    if var["gdt"] == "bf16":
        g = g.to(torch.bfloat16)
    sr_h, _ = _sr(var, 11)
    hp = ob.hparams(**HP, clip=var["clip"], ef_mode=var["ef_mode"], ef_beta=0.9, **sr_h)
    K = plan.num_chunks
    outs = []
    for split in (False, True):
        e, mm, pp = err.clone(), m.clone(), p.clone()
        words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
        scales = torch.zeros(K, dtype=torch.float32, device=DEV)
        signs = torch.zeros(n, dtype=torch.int8, device=DEV) if var["signs"] else None
        nf = torch.zeros(1, dtype=torch.int64, device=DEV)
        if split:
            ob.ob_adam_worker_compress(plan, g, e, words, scales, hp, signs, nf)
            ob.ob_adam_worker_update(plan, words, scales, mm, v, pp, hp)
        else:
            ob.ob_adam_compress_step(plan, g, e, mm, v, pp, words, scales, hp, signs, nf)
        torch.cuda.synchronize()
        outs.append([t.view(torch.uint8).cpu() if t is not None else None
                     for t in (words, scales, e.view(torch.int16) if e.dtype != torch.float32 else e, mm, pp,
                               signs, nf)])
    for name, a, b in zip(("words", "scales", "err", "m", "p", "signs", "nonfinite"), *outs):
        if a is not None:
            assert torch.equal(a, b), f"{vname}: {name} differs between split and fused"


@pytest.mark.parametrize("W", [2, 4, 8])
def test_data_parallel_round(W):
    """W workers (own gradients and error buffers, replicated m, v, p) exchange packed signs and scales
    through the server reduce on one GPU; the shared update uses the server's words.  Three steps
    against the same pipeline in the oracle (worker errors and the server error carried)."""
    n, chunk = 1_000_003, 1 << 16
    off = oracle.uniform_offsets(n, chunk)
    K = off.size - 1
    plan = ob.ob_plan_create(n, chunk_size=chunk)
    rng = np.random.default_rng(W)
    errs = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(W)]
    _, _, m, v, p = _small_state(n, 91)
    e_srv = np.zeros(n, np.float32)
    hp = ob.hparams(**HP)
    compared = 0
    for st in range(3):
        grads = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(W)]
        # GPU: state copied in from the oracle's, so each step starts from identical inputs
        d_words = torch.zeros((W, (n + 31) // 32), dtype=torch.int32, device=DEV)
        d_scales = torch.zeros((W, K), dtype=torch.float32, device=DEV)
        d_errs = [_t(e) for e in errs]
        for w_ in range(W):
            ob.ob_adam_worker_compress(plan, _t(grads[w_]), d_errs[w_], d_words[w_], d_scales[w_], hp)
        d_esrv = _t(e_srv)
        g_words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
        g_scales = torch.zeros(K, dtype=torch.float32, device=DEV)
        ob.ob_server_reduce(plan, d_words, d_scales, d_esrv, g_words, g_scales)
        d_m, d_v, d_p = _t(m), _t(v), _t(p)
        ob.ob_adam_worker_update(plan, g_words, g_scales, d_m, d_v, d_p, hp)
        torch.cuda.synchronize()
        # oracle
        ww = np.zeros((W, (n + 31) // 32), np.uint32)
        ws = np.zeros((W, K), np.float32)
        for w_ in range(W):
            ww[w_], ws[w_], _, _ = oracle.worker_compress(grads[w_], errs[w_], off)
        gw, gs = oracle.server_reduce(ww, ws, e_srv, off)
        oracle.worker_update(gw, gs, m, v, p, off, **HP)
        tag = f"W={W} step {st}"
        for w_ in range(W):
            assert np.array_equal(synth.host(d_words[w_]), ww[w_]), f"{tag}: worker {w_} words"
            assert np.all(P.ulp_diff(synth.host(d_scales[w_]), ws[w_]) <= 1), f"{tag}: worker {w_} scales"
            P.assert_f32_close(synth.host(d_errs[w_]), errs[w_], f"{tag}: worker {w_} err",
                               np.repeat(np.abs(synth.host(d_scales[w_]).astype(np.float64) - ws[w_]), np.diff(off)))
        if np.array_equal(synth.host(d_scales), ws):
            # identical worker scales: the server sees identical inputs
            compared += 1
            assert np.array_equal(synth.host(g_words), gw), f"{tag}: server words"
            assert np.all(P.ulp_diff(synth.host(g_scales), gs) <= 1), f"{tag}: server scales"
            P.assert_f32_close(synth.host(d_esrv), e_srv, f"{tag}: server error",
                               np.repeat(np.abs(synth.host(g_scales).astype(np.float64) - gs), np.diff(off)))
            ds = np.repeat(np.abs(synth.host(g_scales).astype(np.float64) - gs), np.diff(off))
            P.assert_f32_close(synth.host(d_m), m, f"{tag}: m", 0.1 * ds)
            P.assert_f32_close(synth.host(d_p), p, f"{tag}: p", 1e-4 * 0.1 * ds / (np.sqrt(v.astype(np.float64)) + 1e-8))
    assert compared >= 1, "every step had a worker scale an ulp apart; nothing past the workers was compared"


# ------------------------------------------------------------------------------------------------
# 1-bit LAMB: the update half after the exchange (trust ratios on the exchanged direction)
# ------------------------------------------------------------------------------------------------

def _check_lamb_update(d_m, d_p, d_r, m, p, v, rr, off, lr, tag):
    """m exact; ratios within 2 ulp (sums grouped by other blocks); p within lr * |dr| * |u|."""
    assert np.array_equal(synth.host(d_m), m), f"{tag}: m"
    gr = synth.host(d_r)
    assert np.all(P.ulp_diff(gr, rr) <= 2), f"{tag}: ratios {gr} vs {rr}"
    dr = np.repeat(np.abs(gr.astype(np.float64) - rr.astype(np.float64)), np.diff(off))
    u = np.abs(m.astype(np.float64)) / (np.sqrt(v.astype(np.float64)) + np.float64(np.float32(1e-8)))
    P.assert_f32_close(synth.host(d_p), p, f"{tag}: p", lr * dr * u)


@pytest.mark.parametrize("n,chunk", [(130, 64), (4096 + 17, 1024), (1_000_003, 1 << 16), (5_000_000, 5_000_000 - 448)])
def test_lamb_worker_update(n, chunk):
    """The LAMB update from the oracle's exchanged words and scales, with a zero layer (r = 1)."""
    gnp, err, m, v, p = _small_state(n, n + 5)
    off = oracle.uniform_offsets(n, chunk)
    p[int(off[0]):int(off[1])] = 0.0
    plan = ob.ob_plan_create(n, chunk_size=chunk)
    rw, rs, _, _ = oracle.worker_compress(gnp, err, off)
    d_m, d_v, d_p = _t(m), _t(v), _t(p)
    d_r = torch.full((off.size - 1,), -7.0, dtype=torch.float32, device=DEV)
    ob.ob_lamb_worker_update(plan, _t(rw), _t(rs), d_m, d_v, d_p, d_r, ob.hparams(**HP))
    rr = oracle.lamb_worker_update(rw, rs, m, v, p, off, **HP)
    assert rr[0] == 1.0
    _check_lamb_update(d_m, d_p, d_r, m, p, v, rr, off, HP["lr"], f"lamb worker update n={n}")


def test_lamb_worker_update_with_block_knobs(monkeypatch):
    """The LAMB worker update writes one p^2 partial per compressed-pass-2 block.  With the dense step's
    blocks set to 8 tiles (a tuning knob read at plan creation) the compressed-pass-2 table is the
    plan's largest, about twice the dense table; the plan sizes that workspace for it and the update
    still matches the oracle (the workspace size is fixed by reading ob_plan_create; this is the
    regression test of that fix)."""
    monkeypatch.setenv("OB_BLOCK_ELEMS_DENSE", str(8 * 1024))
    n, chunk = 1_000_003, 1 << 16
    gnp, err, m, v, p = _small_state(n, 44)
    off = oracle.uniform_offsets(n, chunk)
    plan = ob.ob_plan_create(n, chunk_size=chunk)
    assert plan.block_elems == 4 * 1024
    rw, rs, _, _ = oracle.worker_compress(gnp, err, off)
    d_m, d_v, d_p = _t(m), _t(v), _t(p)
    d_r = torch.full((off.size - 1,), -7.0, dtype=torch.float32, device=DEV)
    ob.ob_lamb_worker_update(plan, _t(rw), _t(rs), d_m, d_v, d_p, d_r, ob.hparams(**HP))
    rr = oracle.lamb_worker_update(rw, rs, m, v, p, off, **HP)
    _check_lamb_update(d_m, d_p, d_r, m, p, v, rr, off, HP["lr"], "lamb worker update, dense blocks of 8 tiles")


@pytest.mark.parametrize("W", [1, 4])
def test_lamb_data_parallel_round(W):
    """1-bit LAMB with W workers through the server reduce on one GPU, two steps against the oracle."""
    n, chunk = 1_000_003, 1 << 16
    off = oracle.uniform_offsets(n, chunk)
    K = off.size - 1
    plan = ob.ob_plan_create(n, chunk_size=chunk)
    rng = np.random.default_rng(100 + W)
    errs = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(W)]
    _, _, m, v, p = _small_state(n, 92)
    e_srv = np.zeros(n, np.float32)
    hp = ob.hparams(**HP)
    for st in range(2):
        grads = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(W)]
        ww = np.zeros((W, (n + 31) // 32), np.uint32)
        ws = np.zeros((W, K), np.float32)
        for w_ in range(W):
            ww[w_], ws[w_], _, _ = oracle.worker_compress(grads[w_], errs[w_], off)
        gw, gs = oracle.server_reduce(ww, ws, e_srv, off)
        # the GPU update from the oracle's server words (the worker and server kernels are covered above)
        d_m, d_v, d_p = _t(m), _t(v), _t(p)
        d_r = torch.zeros(K, dtype=torch.float32, device=DEV)
        ob.ob_lamb_worker_update(plan, _t(gw), _t(gs), d_m, d_v, d_p, d_r, hp)
        rr = oracle.lamb_worker_update(gw, gs, m, v, p, off, **HP)
        _check_lamb_update(d_m, d_p, d_r, m, p, v, rr, off, HP["lr"], f"LAMB W={W} step {st}")
        # the next step starts from the oracle's state (p within the bound above)


def test_one_worker_lamb_split_matches_fused_step():
    """At one worker the LAMB split gives the fused LAMB step's words, scales, errors and m bit for bit;
    ratios within 2 ulp and p within the resulting bound (the norms' sums are grouped differently)."""
    w = synth.BERT_BASE
    n = w.n
    plan = ob.ob_plan_create(n, chunk_offsets=w.offsets)
    off = w.chunk_offsets()
    err, m, v, p = synth.draw_state(w, DEV)
    g = synth.draw_grad(w, 0, DEV)
    hp = ob.hparams(**HP)
    K = plan.num_chunks
    res = []
    for split in (False, True):
        e, mm, pp = err.clone(), m.clone(), p.clone()
        words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
        scales = torch.zeros(K, dtype=torch.float32, device=DEV)
        ratios = torch.zeros(K, dtype=torch.float32, device=DEV)
        if split:
            ob.ob_adam_worker_compress(plan, g, e, words, scales, hp)
            ob.ob_lamb_worker_update(plan, words, scales, mm, v, pp, ratios, hp)
        else:
            ob.ob_lamb_compress_step(plan, g, e, mm, v, pp, words, scales, ratios, hp)
        torch.cuda.synchronize()
        res.append([synth.host(t) for t in (words, scales, e, mm, pp, ratios)])
    (w0, s0, e0, m0, p0, r0), (w1, s1, e1, m1, p1, r1) = res
    for name, a, b in (("words", w0, w1), ("scales", s0, s1), ("err", e0, e1), ("m", m0, m1)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{name} differs between split and fused"
    assert np.all(P.ulp_diff(r1, r0) <= 2), "ratios"
    dr = np.repeat(np.abs(r1.astype(np.float64) - r0.astype(np.float64)), np.diff(off))
    u = np.abs(m0.astype(np.float64)) / (np.sqrt(synth.host(v).astype(np.float64)) + np.float64(np.float32(1e-8)))
    P.assert_f32_close(p1, p0, "p", HP["lr"] * dr * u)
