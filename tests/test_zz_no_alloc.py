"""The compressed step without any allocation (ob_adam_compress_step_noalloc), marked gpu.

Called through the C ABI (the ctypes binding), it must give bit for bit the outputs of
ob_adam_compress_step with a plan of the same n and chunk size -- the same kernels over the same
block tables, the tables and partial sums living in the library's static device buffer instead of the
plan's allocations.  Each case makes calls in a row on one stream, later ones smaller than the first
(the buffer then still holds the first call's larger tables), and then the first size again.  The
same with small chunk-group budgets (both steps then run their passes group by group, the plan's
greedy groups against the no-allocation step's equal groups), and the step captured into a HIP graph
and replayed.
"""
import numpy as np
import pytest
import torch

import adam_ob_compress_amd as ob

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    ob.lib()
    yield
    torch.cuda.synchronize()


def _state(n, gdt, edt, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    g = torch.randn(n, generator=gen, device=DEV) * (20.0 if gdt == "bf16" else 1e-3)
    err = torch.randn(n, generator=gen, device=DEV) * 1e-3
    m = torch.randn(n, generator=gen, device=DEV) * 1e-4
    v = torch.randn(n, generator=gen, device=DEV).abs() * 1e-6 + 1e-8
    p = torch.randn(n, generator=gen, device=DEV) * 0.02
    g = g.to(torch.bfloat16) if gdt == "bf16" else g
    err = err.to({"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[edt])
    return g, err, m, v, p


def _bits(t):
    t = t.contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint8)


def _one(n, chunk, gdt, edt, ema, clip, signs, sr, seed):
    g, err, m, v, p = _state(n, gdt, edt, seed)
    hp = ob.hparams(lr=1e-4, clip=clip, ef_mode=ob.OB_EF_EMA if ema else ob.OB_EF_PLAIN, ef_beta=0.9,
                    err_rounding=ob.OB_ROUND_STOCHASTIC if sr else ob.OB_ROUND_NEAREST, sr_seed=0x5EED,
                    step=3)
    K = (n + chunk - 1) // chunk
    outs = []
    for noalloc in (False, True):
        e, mm, pp = err.clone(), m.clone(), p.clone()
        words = torch.full(((n + 31) // 32,), -1, dtype=torch.int32, device=DEV)
        scales = torch.full((K,), -1.0, dtype=torch.float32, device=DEV)
        sg = torch.zeros(n, dtype=torch.int8, device=DEV) if signs else None
        nf = torch.zeros(1, dtype=torch.int64, device=DEV)
        if noalloc:
            ob.ob_adam_compress_step_noalloc(n, chunk, g, e, mm, v, pp, words, scales, hp, sg, nf)
        else:
            plan = ob.ob_plan_create(n, chunk_size=chunk)
            ob.ob_adam_compress_step(plan, g, e, mm, v, pp, words, scales, hp, sg, nf)
        torch.cuda.synchronize()
        outs.append([_bits(t) for t in (e, mm, pp, words, scales, nf) + ((sg,) if signs else ())])
        if not noalloc:
            plan.destroy()
    names = ("err", "m", "p", "words", "scales", "nonfinite", "signs")
    for name, a, b in zip(names, *outs):
        assert np.array_equal(a, b), f"n={n} chunk={chunk} {gdt}/{edt}: {name} differs from the plan's step"
    return outs[1]


# (n, chunk, g dtype, error dtype, EMA, clip, int8 signs, stochastic rounding)
SEQUENCES = {
    # one chunk of more than 4096 first-pass blocks (its sum formed by the per-chunk kernel), then
    # smaller buffers in several chunks with ragged tails, then the first again
    "huge-chunk-then-smaller": [
        (17_000_003, 17_000_003, "bf16", "f16", True, 5.0, True, False),
        (1_000_003, 1 << 16, "f32", "f32", False, 0.0, False, False),
        (130, 64, "f32", "bf16", True, 0.0, True, True),
        (17_000_003, 17_000_003, "bf16", "f16", True, 5.0, True, False),
    ],
    # many chunks, then one chunk, then a tiny buffer
    "many-chunks-then-smaller": [
        (5_000_000, 1 << 14, "f32", "bf16", False, 0.0, True, True),
        (300_037, 300_037, "bf16", "f32", True, 5.0, False, False),
        (33, 64, "f32", "f32", False, 0.0, True, False),
    ],
}


@pytest.mark.parametrize("name", sorted(SEQUENCES))
def test_noalloc_step_equals_the_plan_step(name):
    for k, case in enumerate(SEQUENCES[name]):
        _one(*case, seed=100 + k)


def test_noalloc_step_by_groups_equals_the_plan_step(monkeypatch):
    """OB_GROUP_BYTES of a few chunks: many groups on both sides.  The last case's plan puts its three
    chunks (the last one short) in one group where the no-allocation step makes two."""
    monkeypatch.setenv("OB_GROUP_BYTES", "200000")
    _one(5_000_000, 1 << 14, "f32", "bf16", False, 0.0, True, True, seed=7)
    _one(1_000_003, 1 << 16, "f32", "f32", True, 5.0, True, False, seed=8)
    monkeypatch.setenv("OB_GROUP_BYTES", str(8 * (2 * 16384 + 1000)))
    _one(2 * 16384 + 1000, 16384, "f32", "f32", True, 0.0, False, False, seed=9)


def test_noalloc_step_under_graph_capture():
    """The reason the entry point exists: captured once into a HIP graph (its table kernel and both passes,
    nothing allocated while capturing) and replayed with new gradients copied in between, every replay
    gives bit for bit what the same step gives eagerly."""
    n, chunk = 3 * (1 << 20) + 4096, 1 << 20
    K = (n + chunk - 1) // chunk
    hp = ob.hparams(lr=1e-4, clip=5.0, ef_mode=ob.OB_EF_EMA, ef_beta=0.9)
    gen = torch.Generator(device=DEV)
    grads = []
    for s in range(4):
        gen.manual_seed(500 + s)
        grads.append((torch.randn(n, generator=gen, device=DEV) * 20.0).to(torch.bfloat16))

    def buffers(seed):
        _, err, m, v, p = _state(n, "bf16", "f16", seed)
        return dict(err=err, m=m, v=v, p=p,
                    words=torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV),
                    scales=torch.zeros(K, dtype=torch.float32, device=DEV),
                    signs=torch.zeros(n, dtype=torch.int8, device=DEV),
                    nf=torch.zeros(1, dtype=torch.int64, device=DEV))

    def step(b, g):
        ob.ob_adam_compress_step_noalloc(n, chunk, g, b["err"], b["m"], b["v"], b["p"], b["words"], b["scales"],
                                         hp, b["signs"], b["nf"])

    def snapshot(b):
        return [_bits(b[k]) for k in ("err", "m", "p", "words", "scales", "signs", "nf")]

    a = buffers(9)
    eager = []
    for s in range(4):
        step(a, grads[s])
        torch.cuda.synchronize()
        eager.append(snapshot(a))

    b = buffers(9)
    g_in = torch.empty_like(grads[0])
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        g_in.copy_(grads[0])
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            step(b, g_in)
    torch.cuda.synchronize()
    for s in range(4):
        g_in.copy_(grads[s])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("err", "m", "p", "words", "scales", "signs", "nonfinite"), snapshot(b), eager[s]):
            assert np.array_equal(x, y), f"replay {s}: {name} differs from the eager step"
