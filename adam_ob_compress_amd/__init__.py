"""1-bit Adam (and 1-bit LAMB) optimizer step on AMD MI355X (gfx950): HIP kernels behind a C ABI
(libobadam.so).

Python side = argument marshalling (``_native``), host schedules (``schedule``) and the seeded
synthetic workloads (``synth``).  Importing the package does not load the library; the first call does,
and raises if it has not been built (there is no CPU fallback).
"""
from ._native import (  # noqa: F401
    KERNEL_NAMES, OB_BF16, OB_EF_EMA, OB_EF_PLAIN, OB_F16, OB_F32, OB_ROUND_NEAREST, OB_ROUND_STOCHASTIC,
    OB_KERNEL_CHUNK_SUMSQ,
    OB_KERNEL_COMPRESS, OB_KERNEL_DENSE, OB_KERNEL_DIAG, OB_KERNEL_LAMB_APPLY, OB_KERNEL_SERVER_APPLY,
    OB_KERNEL_SERVER_SUMSQ, OB_KERNEL_TRUST_RATIO, OB_KERNEL_UNPACK, LIB_PATH, ObError, Plan, hparams,
    OB_ERR_OOM, OB_ERR_SIZE, OB_NOALLOC_SCRATCH_BYTES,
    lib, ob_adam_compress_step, ob_adam_compress_step_noalloc, ob_adam_warmup_step, ob_adam_worker_compress,
    ob_adam_worker_update,
    ob_hparams, ob_lamb_compress_step, ob_lamb_worker_update,
    ob_lamb_warmup_step, ob_pack, ob_plan_create, ob_plan_read_timing, ob_plan_set_diagnostics,
    ob_plan_set_timing,
    ob_server_reduce, ob_status_str, ob_unpack,
)
from .schedule import OneBitAdam, OneBitLamb, step_kind  # noqa: F401
