"""GPU parity of the compressed step run by chunk groups (marked gpu).

The compressed step runs its two kernels group by group: consecutive chunks whose pass-1 bytes fit a
budget (320 MB; OB_GROUP_BYTES, read when a plan is created, overrides it), pass 1 then pass 2 per
group (1-bit LAMB runs one group).  The default gives one group for the small cases of
test_gpu_parity.py, so here budgets of a few chunks force many groups on the same cases, against the
oracle: every variant of the step, the diagnostics and the worker split, and BERT-base at full size
with every chunk checked; 1-bit LAMB stays one group under any budget.  The number of groups a plan
reports matches bench.py's host rule for every workload.
"""
import dataclasses
import os
import sys

import pytest
import torch

import adam_ob_compress_amd as ob
from adam_ob_compress_amd import synth

import _parity as P
import test_gpu_parity as T
import test_gpu_worker as TW

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

pytestmark = pytest.mark.gpu
EDT = {"f32": ob.OB_F32, "bf16": ob.OB_BF16, "f16": ob.OB_F16}


@pytest.fixture(autouse=True)
def _gpu():
    T._require_gpu()
    yield
    torch.cuda.synchronize()


def _groups(n, chunk, var, lamb=False):
    plan = ob.ob_plan_create(n, chunk_size=chunk)
    g = plan.num_groups(ob.OB_BF16 if var["gdt"] == "bf16" else ob.OB_F32, EDT[var.get("edt", "f32")], lamb)
    plan.destroy()
    return g


def test_group_counts_match_the_host_rule(monkeypatch):
    for budget in (None, 0, 1, 3 << 20, 64 << 20):
        if budget is None:
            monkeypatch.delenv("OB_GROUP_BYTES", raising=False)
        else:
            monkeypatch.setenv("OB_GROUP_BYTES", str(budget))
        for w in synth.WORKLOADS.values():
            plan = ob.ob_plan_create(w.n, chunk_size=w.chunk if w.offsets is None else 0, chunk_offsets=w.offsets)
            gdt = ob.OB_BF16 if w.grad_dtype == "bf16" else ob.OB_F32
            for lamb in (False, True):
                got = plan.num_groups(gdt, EDT[w.err_dtype], lamb)
                assert got == len(bench.chunk_groups(w, lamb)), (w.name, budget, lamb, got)
            plan.destroy()


# budgets (bytes): one chunk per group, and a few chunks per group (how many depends on the variant's
# bytes per element)
CASES = [(1_000_003, 1 << 16, 1), (1_000_003, 1 << 16, 3 * (1 << 16) * 6), (300_037, 4096, 20_000 * 8)]


@pytest.mark.parametrize("vname", sorted(T.VARIANTS))
@pytest.mark.parametrize("n,chunk,budget", CASES)
def test_compress_by_groups(vname, n, chunk, budget, monkeypatch):
    monkeypatch.setenv("OB_GROUP_BYTES", str(budget))
    var = T.VARIANTS[vname]
    assert _groups(n, chunk, var) > 1
    T._gpu_vs_oracle_compress(n, chunk, var, seed=n + 11, steps=2)


@pytest.mark.parametrize("vname", T.LAMB_VARIANTS)
def test_lamb_runs_one_group(vname, monkeypatch):
    """1-bit LAMB runs its passes as one group whatever the budget (its pass 1 also reads p, and groups
    measured no faster), and matches the oracle there."""
    monkeypatch.setenv("OB_GROUP_BYTES", "1")
    var = T.VARIANTS[vname]
    assert _groups(1_000_003, 1 << 16, var, lamb=True) == 1
    assert _groups(1_000_003, 1 << 16, var) == 16
    T._gpu_vs_oracle_lamb(1_000_003, 1 << 16, var, seed=12, steps=2)


@pytest.mark.parametrize("vname", ["fp32_plain", "bf16_ema_clip_int8_f16err"])
@pytest.mark.parametrize("lamb", [False, True])
def test_diagnostics_by_groups(vname, lamb, monkeypatch):
    monkeypatch.setenv("OB_GROUP_BYTES", "1")
    T.test_diagnostics(vname, lamb)


@pytest.mark.parametrize("vname", TW.SPLIT_VARIANTS)
def test_worker_compress_by_groups(vname, monkeypatch):
    monkeypatch.setenv("OB_GROUP_BYTES", "1")
    var = T.VARIANTS[vname]
    assert _groups(1_000_003, 1 << 16, var) == 16
    TW._compress_vs_oracle(1_000_003, 1 << 16, var, seed=13, steps=2)


def test_bert_base_by_small_groups_every_chunk(monkeypatch):
    """BERT-base's 197 tensors in 16 MB groups (every tensor kind and size, groups of one large or many
    small tensors): one dense step, then three compressed steps, every chunk checked every step."""
    monkeypatch.setenv("OB_GROUP_BYTES", str(16 << 20))
    w = dataclasses.replace(synth.BERT_BASE, freeze_step=1, steps=4)
    plan = ob.ob_plan_create(w.n, chunk_offsets=w.offsets)
    assert plan.num_groups(ob.OB_F32, ob.OB_F32) == len(bench.chunk_groups(w)) > 20
    plan.destroy()
    counts = P.run_workload(w, log=lambda *_: None)
    assert counts["dense"] == 1 and counts["compressed"] == 3


def test_timing_of_grouped_launches(monkeypatch):
    """With timing on, a grouped step's launches are counted one by one (the groups' launches share
    their events): G launches of each pass per step, and the passes' summed times never exceed the
    span of the steps (no launch is counted twice)."""
    monkeypatch.setenv("OB_GROUP_BYTES", "1")
    n, chunk = 1 << 22, 1 << 18
    plan = ob.ob_plan_create(n, chunk_size=chunk)
    G = plan.num_groups(ob.OB_F32, ob.OB_F32)
    assert G == 16
    d = [torch.ones(n, dtype=torch.float32, device=T.DEV) for _ in range(5)]
    words = torch.zeros(n // 32, dtype=torch.int32, device=T.DEV)
    scales = torch.zeros(n // chunk, dtype=torch.float32, device=T.DEV)
    ob.ob_plan_set_timing(plan, True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        ob.ob_adam_compress_step(plan, *d, words, scales, ob.hparams())
    b.record()
    torch.cuda.synchronize()
    ms_c, cnt_c = ob.ob_plan_read_timing(plan, ob.OB_KERNEL_COMPRESS)
    ms_s, cnt_s = ob.ob_plan_read_timing(plan, ob.OB_KERNEL_CHUNK_SUMSQ)
    assert cnt_c == cnt_s == 3 * G
    assert ms_c > 0 and ms_s > 0
    span = a.elapsed_time(b)
    assert ms_c + ms_s <= span * 1.001 + 0.005, (ms_c, ms_s, span)
    plan.destroy()


def test_destroy_with_undrained_grouped_timing(monkeypatch):
    """A plan destroyed with grouped launches' timing records still pending (never read): each shared
    event is destroyed once, and a new plan's timing works after it."""
    monkeypatch.setenv("OB_GROUP_BYTES", "1")
    n, chunk = 1 << 20, 1 << 18
    d = [torch.ones(n, dtype=torch.float32, device=T.DEV) for _ in range(5)]
    words = torch.zeros(n // 32, dtype=torch.int32, device=T.DEV)
    scales = torch.zeros(n // chunk, dtype=torch.float32, device=T.DEV)
    for _ in range(3):
        plan = ob.ob_plan_create(n, chunk_size=chunk)
        assert plan.num_groups(ob.OB_F32, ob.OB_F32) == 4
        ob.ob_plan_set_timing(plan, True)
        ob.ob_adam_compress_step(plan, *d, words, scales, ob.hparams())
        torch.cuda.synchronize()
        plan.destroy()
    plan = ob.ob_plan_create(n, chunk_size=chunk)
    ob.ob_plan_set_timing(plan, True)
    ob.ob_adam_compress_step(plan, *d, words, scales, ob.hparams())
    ms, cnt = ob.ob_plan_read_timing(plan, ob.OB_KERNEL_COMPRESS)
    assert cnt == 4 and ms > 0
    plan.destroy()
