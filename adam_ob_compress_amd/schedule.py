"""Host-side step schedules and a small driver over the C ABI (no arithmetic here).

[P2] "DeepSpeed Communication Compression and Hiding":
  * section "1-bit Adam: warmup, frozen variance, error feedback": dense Adam while
    step < freeze_step (step counted from 0), the compressed step afterwards;
  * section "0/1 Adam": a full-precision variance refresh on chosen steps, 1-bit steps otherwise; the
    refresh here is every period-th step with steps counted from 1;
  * section "1-bit LAMB": the same warmup / compressed schedule with LAMB's layer-wise trust ratio
    (OneBitLamb; the plan's chunks are the layers).
"""
from __future__ import annotations

import torch

from . import _native as nat


def step_kind(step_index: int, freeze_step: int = 0, refresh_period: int = 0) -> str:
    """'dense' or 'compressed' for step_index (from 0) of a run."""
    if step_index < freeze_step:
        return "dense"
    if refresh_period and (step_index + 1) % refresh_period == 0:
        return "dense"
    return "compressed"


class OneBitAdam:
    """Optimizer state (err, m, v, p; fp32, flat, caller-visible) plus the schedule.

    ``step(g)`` enqueues one dense or compressed step on the current stream and returns its kind.
    The compressed step's outputs (packed words, per-chunk scales, optional int8 signs and the
    non-finite counter) stay in ``self.words`` etc. for the caller to send or inspect.

    ``err_rounding="stochastic"`` (16-bit error buffers) rounds each new error stochastically, with
    random bits from (``sr_seed``, the step index).

    With ``diagnostics=True`` every compressed step also leaves, per chunk, the squared L2 norm of the
    error buffer it read (``err_sumsq``) and its number of +1 signs (``plus_count``) ([P1] sec. 6.2
    and 8); ``small_error_chunks`` applies the tutorial's warning threshold to them.
    """

    def __init__(self, plan: nat.Plan, err, m, v, p, *, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                 clip=0.0, ef_mode=nat.OB_EF_PLAIN, ef_beta=0.9, int8_signs=False,
                 count_nonfinite=False, freeze_step=0, refresh_period=0, bias_correction=False,
                 diagnostics=False, err_rounding="nearest", sr_seed=0):
        self.plan = plan
        self.err, self.m, self.v, self.p = err, m, v, p
        self.freeze_step, self.refresh_period = freeze_step, refresh_period
        self.bias_correction = bias_correction
        self.hp = nat.hparams(lr=lr, beta1=beta1, beta2=beta2, eps=eps, clip=clip, ef_mode=ef_mode,
                              ef_beta=ef_beta, sr_seed=sr_seed,
                              err_rounding={"nearest": nat.OB_ROUND_NEAREST,
                                            "stochastic": nat.OB_ROUND_STOCHASTIC}[err_rounding])
        dev = p.device
        n = plan.n
        self.words = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
        self.scales = torch.zeros(plan.num_chunks, dtype=torch.float32, device=dev)
        self.signs = torch.zeros(n, dtype=torch.int8, device=dev) if int8_signs else None
        self.nonfinite = torch.zeros(1, dtype=torch.int64, device=dev) if count_nonfinite else None
        self.step_index = 0
        self.dense_steps = 0
        self.err_sumsq = self.plus_count = None
        if diagnostics:
            self.err_sumsq = torch.zeros(plan.num_chunks, dtype=torch.float64, device=dev)
            self.plus_count = torch.zeros(plan.num_chunks, dtype=torch.int64, device=dev)
            nat.ob_plan_set_diagnostics(plan, self.err_sumsq, self.plus_count)

    def kind(self) -> str:
        return step_kind(self.step_index, self.freeze_step, self.refresh_period)

    def step(self, g, stream=None) -> str:
        kind = self.kind()
        if kind == "dense":
            self.dense_steps += 1
            self.hp.bias_correction = 1 if self.bias_correction else 0
            self.hp.step = self.dense_steps
            self._dense(g, stream)
        else:
            self.hp.step = self.step_index      # the stochastic-rounding stream of this step
            self._compressed(g, stream)
        self.step_index += 1
        return kind

    def small_error_chunks(self, threshold: float = 1e-6) -> list[int]:
        """Chunks whose error buffer, as the last compressed step read it, had an L2 norm below
        `threshold` ([P1] sec. 6.2's warning).  Host policy over the library's per-chunk sums of
        squares (``self.err_sumsq``): a norm below t is a sum of squares below t*t, so no arithmetic is
        done here; the library's outputs (``err_sumsq``, ``plus_count``) are the diagnostics."""
        return torch.nonzero(self.err_sumsq < threshold * threshold).flatten().tolist()

    def _dense(self, g, stream):
        nat.ob_adam_warmup_step(self.plan, g, self.m, self.v, self.p, self.hp, stream)

    def _compressed(self, g, stream):
        nat.ob_adam_compress_step(self.plan, g, self.err, self.m, self.v, self.p, self.words, self.scales,
                                  self.hp, self.signs, self.nonfinite, stream)


class OneBitLamb(OneBitAdam):
    """1-bit LAMB: OneBitAdam's state and schedule, with the layer-wise trust ratio in both step kinds.
    ``self.ratios`` holds each layer's (chunk's) ratio from the last step."""

    def __init__(self, plan: nat.Plan, err, m, v, p, **kw):
        super().__init__(plan, err, m, v, p, **kw)
        self.ratios = torch.zeros(plan.num_chunks, dtype=torch.float32, device=p.device)

    def _dense(self, g, stream):
        nat.ob_lamb_warmup_step(self.plan, g, self.m, self.v, self.p, self.ratios, self.hp, stream)

    def _compressed(self, g, stream):
        nat.ob_lamb_compress_step(self.plan, g, self.err, self.m, self.v, self.p, self.words, self.scales,
                                  self.ratios, self.hp, self.signs, self.nonfinite, stream)
