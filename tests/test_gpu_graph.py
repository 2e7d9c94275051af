"""The C ABI under a captured HIP graph and under concurrency (marked gpu).

A step enqueues kernels only (no allocation, no memset, no host synchronisation), so it can be captured
into a graph: every replay must give bit-identical results to the same steps run eagerly, with the
program's own eager work and synchronisations between replays.  Two plans on two streams running at once
must give the results each gives alone.  Inputs come from adam_ob_compress_amd.synth.
"""
import dataclasses

import numpy as np
import pytest
import torch

import adam_ob_compress_amd as ob
from adam_ob_compress_amd import schedule, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    ob.lib()
    yield
    torch.cuda.synchronize()


def _state(w):
    err, m, v, p = synth.draw_state(w, DEV)
    return [err, m, v, p]


def _bits(t):
    return synth.host(t).view(np.uint8)


@pytest.mark.parametrize("lamb", [False, True])
def test_graph_replay_matches_eager(lamb):
    """Compressed steps (bf16 g, bf16 error buffer, EMA + clip, int8 signs, non-finite counter and
    diagnostics on) captured once and replayed 4 times == 4 eager steps."""
    w = synth.scaled(synth.LLAMA2_7B, 3 * (1 << 20) + 4096, 1 << 20)
    w = dataclasses.replace(w, err_dtype="bf16")
    cls = schedule.OneBitLamb if lamb else schedule.OneBitAdam
    kw = dict(lr=w.lr, clip=w.clip, ef_mode=w.ef_mode, ef_beta=w.ef_beta, int8_signs=True,
              count_nonfinite=True, diagnostics=True)
    grads = [synth.draw_grad(w, s, DEV) for s in range(4)]
    g_in = torch.empty_like(grads[0])

    plan_a = ob.ob_plan_create(w.n, chunk_size=w.chunk)
    a = cls(plan_a, *_state(w), **kw)
    eager = []
    for s in range(4):
        a.nonfinite.zero_()
        a.step(grads[s])
        torch.cuda.synchronize()
        eager.append([_bits(t) for t in (a.err, a.m, a.p, a.words, a.scales, a.signs, a.nonfinite,
                                         a.err_sumsq, a.plus_count) + ((a.ratios,) if lamb else ())])

    plan_b = ob.ob_plan_create(w.n, chunk_size=w.chunk)
    b = cls(plan_b, *_state(w), **kw)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        g_in.copy_(grads[0])            # warm the allocator outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            b.nonfinite.zero_()         # a fill kernel, not a memset node
            b.step(g_in)
    torch.cuda.synchronize()
    for s in range(4):
        g_in.copy_(grads[s])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [_bits(t) for t in (b.err, b.m, b.p, b.words, b.scales, b.signs, b.nonfinite,
                                  b.err_sumsq, b.plus_count) + ((b.ratios,) if lamb else ())]
        for name, x, y in zip("err m p words scales signs nonfinite err_sumsq plus_count ratios".split(),
                              got, eager[s]):
            assert np.array_equal(x, y), f"replay {s}: {name} differs from the eager step"


def test_two_plans_on_two_streams():
    """Two independent optimizers stepping concurrently on two streams == each run alone."""
    wa = synth.scaled(synth.GPT2_XL, 5 * (1 << 20) + 64, 1 << 20)
    wb = synth.scaled(synth.BERT_BASE, 3 * (1 << 20) + 1000, 1 << 18)
    ga = [synth.draw_grad(wa, s, DEV) for s in range(3)]
    gb = [synth.draw_grad(wb, s, DEV) for s in range(3)]

    def make(w):
        return schedule.OneBitAdam(ob.ob_plan_create(w.n, chunk_size=w.chunk), *_state(w), lr=w.lr,
                                   freeze_step=1)

    ref = {}
    for name, w, gs in (("a", wa, ga), ("b", wb, gb)):
        o = make(w)
        for g in gs:
            o.step(g)
        torch.cuda.synchronize()
        ref[name] = [_bits(t) for t in (o.err, o.m, o.v, o.p, o.words, o.scales)]

    oa, ob_ = make(wa), make(wb)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for s in range(3):
        with torch.cuda.stream(sa):
            oa.step(ga[s], stream=sa)
        with torch.cuda.stream(sb):
            ob_.step(gb[s], stream=sb)
    torch.cuda.synchronize()
    for name, o in (("a", oa), ("b", ob_)):
        got = [_bits(t) for t in (o.err, o.m, o.v, o.p, o.words, o.scales)]
        for x, y in zip(got, ref[name]):
            assert np.array_equal(x, y), name
