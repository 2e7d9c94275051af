"""ctypes binding of libobadam.so: the C-ABI entry points under the same names.

Argument marshalling only: torch tensors are turned into device pointers (``data_ptr()``) and torch's
current HIP stream; every step of the optimizer runs in the library's HIP kernels.  There is no
fallback: if the library is not built, or a tensor is not on the GPU, a call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libobadam.so")

OB_OK, OB_ERR_ARG, OB_ERR_ALIGN, OB_ERR_DTYPE, OB_ERR_HIP, OB_ERR_OOM, OB_ERR_SIZE = range(7)
OB_NOALLOC_SCRATCH_BYTES = 64 << 20
OB_F32, OB_BF16, OB_F16 = 0, 1, 2
OB_EF_PLAIN, OB_EF_EMA = 0, 1
OB_ROUND_NEAREST, OB_ROUND_STOCHASTIC = 0, 1
(OB_KERNEL_CHUNK_SUMSQ, OB_KERNEL_COMPRESS, OB_KERNEL_DENSE, OB_KERNEL_SERVER_SUMSQ,
 OB_KERNEL_SERVER_APPLY, OB_KERNEL_UNPACK, OB_KERNEL_TRUST_RATIO, OB_KERNEL_LAMB_APPLY,
 OB_KERNEL_DIAG, OB_KERNEL_SCALE, OB_KERNEL_WORKER_COMPRESS, OB_KERNEL_WORKER_UPDATE) = range(12)
KERNEL_NAMES = {
    OB_KERNEL_CHUNK_SUMSQ: "chunk_sumsq", OB_KERNEL_COMPRESS: "compress", OB_KERNEL_DENSE: "dense",
    OB_KERNEL_SERVER_SUMSQ: "server_sumsq", OB_KERNEL_SERVER_APPLY: "server_apply",
    OB_KERNEL_UNPACK: "unpack", OB_KERNEL_TRUST_RATIO: "trust_ratio", OB_KERNEL_LAMB_APPLY: "lamb_apply",
    OB_KERNEL_DIAG: "diag", OB_KERNEL_SCALE: "scale", OB_KERNEL_WORKER_COMPRESS: "worker_compress",
    OB_KERNEL_WORKER_UPDATE: "worker_update",
}


class ObError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {ob_status_str(status)} (status {status})")


class ob_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("clip", ctypes.c_float), ("ef_mode", ctypes.c_int32),
                ("ef_beta", ctypes.c_float), ("bias_correction", ctypes.c_int32),
                ("step", ctypes.c_int64), ("err_rounding", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("sr_seed", ctypes.c_uint64)]


def hparams(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, clip=0.0, ef_mode=OB_EF_PLAIN, ef_beta=0.9,
            bias_correction=False, step=0, err_rounding=OB_ROUND_NEAREST, sr_seed=0) -> ob_hparams:
    return ob_hparams(lr, beta1, beta2, eps, clip, ef_mode, ef_beta, 1 if bias_correction else 0, step,
                      err_rounding, 0, sr_seed)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libobadam.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(there is no non-HIP fallback)")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    HP = ctypes.POINTER(ob_hparams)
    sig = {
        "ob_plan_create": (I32, [I64, I64, P, I64, ctypes.POINTER(P)]),
        "ob_plan_destroy": (I32, [P]),
        "ob_plan_num_elements": (I64, [P]),
        "ob_plan_num_chunks": (I64, [P]),
        "ob_plan_num_blocks": (I64, [P]),
        "ob_plan_block_elems": (I64, [P]),
        "ob_plan_num_groups": (I64, [P, I32, I32, I32]),
        "ob_adam_warmup_step": (I32, [P, P, I32, P, P, P, HP, P]),
        "ob_adam_compress_step": (I32, [P, P, I32, P, I32, P, P, P, P, P, P, P, HP, P]),
        "ob_adam_compress_step_noalloc": (I32, [I64, I64, P, I32, P, I32, P, P, P, P, P, P, P, HP, P]),
        "ob_lamb_compress_step": (I32, [P, P, I32, P, I32, P, P, P, P, P, P, P, P, HP, P]),
        "ob_lamb_warmup_step": (I32, [P, P, I32, P, P, P, P, HP, P]),
        "ob_adam_worker_compress": (I32, [P, P, I32, P, I32, P, P, P, P, HP, P]),
        "ob_adam_worker_update": (I32, [P, P, P, P, P, P, HP, P]),
        "ob_lamb_worker_update": (I32, [P, P, P, P, P, P, P, HP, P]),
        "ob_server_reduce": (I32, [P, I32, P, P, P, P, P, P]),
        "ob_pack": (I32, [P, I32, I64, P, P]),
        "ob_unpack": (I32, [P, P, I64, P, P, P]),
        "ob_status_str": (ctypes.c_char_p, [I32]),
        "ob_plan_set_timing": (I32, [P, I32]),
        "ob_plan_set_diagnostics": (I32, [P, P, P]),
        "ob_plan_read_timing": (I32, [P, I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def ob_status_str(status: int) -> str:
    return lib().ob_status_str(status).decode()


def _check(status: int, what: str):
    if status != OB_OK:
        raise ObError(status, what)


def _dev(t: torch.Tensor | None, name: str):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device}); there is no CPU path")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _want(t, name, dtype, numel=None):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def _gdtype(g: torch.Tensor) -> int:
    if g.dtype == torch.float32:
        return OB_F32
    if g.dtype == torch.bfloat16:
        return OB_BF16
    raise TypeError(f"gradient dtype must be float32 or bfloat16, got {g.dtype}")


_ERR_DTYPES = {torch.float32: OB_F32, torch.bfloat16: OB_BF16, torch.float16: OB_F16}


def _errdtype(err: torch.Tensor) -> int:
    if err.dtype not in _ERR_DTYPES:
        raise TypeError(f"error buffer dtype must be float32, bfloat16 or float16, got {err.dtype}")
    return _ERR_DTYPES[err.dtype]


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


class Plan:
    """Owner of an ob_plan handle (destroyed with the object)."""

    def __init__(self, handle: ctypes.c_void_p, n: int):
        self.handle = handle
        self.n = n

    @property
    def num_chunks(self) -> int:
        return int(lib().ob_plan_num_chunks(self.handle))

    @property
    def num_blocks(self) -> int:
        return int(lib().ob_plan_num_blocks(self.handle))

    @property
    def block_elems(self) -> int:
        return int(lib().ob_plan_block_elems(self.handle))

    def num_groups(self, g_dtype: int, err_dtype: int = OB_F32, lamb: bool = False) -> int:
        """Launches of each of the compressed step's two kernels per step (its chunk groups)."""
        return int(lib().ob_plan_num_groups(self.handle, g_dtype, err_dtype, 1 if lamb else 0))

    def destroy(self):
        if self.handle:
            _check(lib().ob_plan_destroy(self.handle), "ob_plan_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def ob_plan_create(n: int, chunk_size: int = 0, chunk_offsets=None) -> Plan:
    """Plan over n elements: uniform chunks of chunk_size, or per-tensor chunk_offsets (K+1 ints)."""
    h = ctypes.c_void_p()
    if chunk_offsets is not None:
        offs = (ctypes.c_int64 * len(chunk_offsets))(*[int(o) for o in chunk_offsets])
        st = lib().ob_plan_create(n, 0, offs, len(chunk_offsets) - 1, ctypes.byref(h))
    else:
        st = lib().ob_plan_create(n, chunk_size, None, 0, ctypes.byref(h))
    _check(st, "ob_plan_create")
    return Plan(h, n)


def ob_adam_warmup_step(plan: Plan, g, m, v, p, hp: ob_hparams, stream=None):
    n = plan.n
    _want(g, "g", g.dtype, n)
    for name, t in (("m", m), ("v", v), ("p", p)):
        _want(t, name, torch.float32, n)
    _check(lib().ob_adam_warmup_step(plan.handle, _dev(g, "g"), _gdtype(g), _dev(m, "m"), _dev(v, "v"),
                                     _dev(p, "p"), ctypes.byref(hp), _stream(stream)),
           "ob_adam_warmup_step")


def ob_adam_compress_step(plan: Plan, g, err, m, v, p, words_out, scales_out, hp: ob_hparams,
                          signs_out=None, nonfinite_out=None, stream=None):
    n = plan.n
    _want(g, "g", g.dtype, n)
    _want(err, "err", err.dtype, n)
    for name, t in (("m", m), ("v", v), ("p", p)):
        _want(t, name, torch.float32, n)
    _want(words_out, "words_out", torch.int32, (n + 31) // 32)
    _want(scales_out, "scales_out", torch.float32, plan.num_chunks)
    _want(signs_out, "signs_out", torch.int8, n)
    _want(nonfinite_out, "nonfinite_out", torch.int64, 1)
    _check(lib().ob_adam_compress_step(
        plan.handle, _dev(g, "g"), _gdtype(g), _dev(err, "err"), _errdtype(err), _dev(m, "m"), _dev(v, "v"),
        _dev(p, "p"),
        _dev(words_out, "words_out"), _dev(scales_out, "scales_out"), _dev(signs_out, "signs_out"),
        _dev(nonfinite_out, "nonfinite_out"), ctypes.byref(hp), _stream(stream)), "ob_adam_compress_step")


def ob_adam_compress_step_noalloc(n: int, chunk_size: int, g, err, m, v, p, words_out, scales_out,
                                  hp: ob_hparams, signs_out=None, nonfinite_out=None, stream=None):
    """ob_adam_compress_step for uniform chunks of chunk_size, without a plan and without any device
    allocation (the library's static buffer holds the tables and partial sums)."""
    K = (n + chunk_size - 1) // chunk_size if n > 0 and chunk_size > 0 else 0
    _want(g, "g", g.dtype, n)
    _want(err, "err", err.dtype, n)
    for name, t in (("m", m), ("v", v), ("p", p)):
        _want(t, name, torch.float32, n)
    _want(words_out, "words_out", torch.int32, (n + 31) // 32)
    _want(scales_out, "scales_out", torch.float32, K)
    _want(signs_out, "signs_out", torch.int8, n)
    _want(nonfinite_out, "nonfinite_out", torch.int64, 1)
    _check(lib().ob_adam_compress_step_noalloc(
        n, chunk_size, _dev(g, "g"), _gdtype(g), _dev(err, "err"), _errdtype(err), _dev(m, "m"), _dev(v, "v"),
        _dev(p, "p"), _dev(words_out, "words_out"), _dev(scales_out, "scales_out"), _dev(signs_out, "signs_out"),
        _dev(nonfinite_out, "nonfinite_out"), ctypes.byref(hp), _stream(stream)), "ob_adam_compress_step_noalloc")


def ob_adam_worker_compress(plan: Plan, g, err, words_out, scales_out, hp: ob_hparams, signs_out=None,
                            nonfinite_out=None, stream=None):
    """The worker's half before the exchange: signs, scales and the error from its own g_hat."""
    n = plan.n
    _want(g, "g", g.dtype, n)
    _want(err, "err", err.dtype, n)
    _want(words_out, "words_out", torch.int32, (n + 31) // 32)
    _want(scales_out, "scales_out", torch.float32, plan.num_chunks)
    _want(signs_out, "signs_out", torch.int8, n)
    _want(nonfinite_out, "nonfinite_out", torch.int64, 1)
    _check(lib().ob_adam_worker_compress(
        plan.handle, _dev(g, "g"), _gdtype(g), _dev(err, "err"), _errdtype(err), _dev(words_out, "words_out"),
        _dev(scales_out, "scales_out"), _dev(signs_out, "signs_out"), _dev(nonfinite_out, "nonfinite_out"),
        ctypes.byref(hp), _stream(stream)), "ob_adam_worker_compress")


def ob_adam_worker_update(plan: Plan, words, scales, m, v, p, hp: ob_hparams, stream=None):
    """The worker's half after the exchange: g_hat from the exchanged words and scales, then m and p."""
    n = plan.n
    _want(words, "words", torch.int32, (n + 31) // 32)
    _want(scales, "scales", torch.float32, plan.num_chunks)
    for name, t in (("m", m), ("v", v), ("p", p)):
        _want(t, name, torch.float32, n)
    _check(lib().ob_adam_worker_update(
        plan.handle, _dev(words, "words"), _dev(scales, "scales"), _dev(m, "m"), _dev(v, "v"), _dev(p, "p"),
        ctypes.byref(hp), _stream(stream)), "ob_adam_worker_update")


def ob_lamb_worker_update(plan: Plan, words, scales, m, v, p, ratios_out, hp: ob_hparams, stream=None):
    """1-bit LAMB's half after the exchange: m on the exchanged g_hat, then trust ratios and the update."""
    n = plan.n
    _want(words, "words", torch.int32, (n + 31) // 32)
    _want(scales, "scales", torch.float32, plan.num_chunks)
    _want(ratios_out, "ratios_out", torch.float32, plan.num_chunks)
    for name, t in (("m", m), ("v", v), ("p", p)):
        _want(t, name, torch.float32, n)
    _check(lib().ob_lamb_worker_update(
        plan.handle, _dev(words, "words"), _dev(scales, "scales"), _dev(m, "m"), _dev(v, "v"), _dev(p, "p"),
        _dev(ratios_out, "ratios_out"), ctypes.byref(hp), _stream(stream)), "ob_lamb_worker_update")


def ob_lamb_compress_step(plan: Plan, g, err, m, v, p, words_out, scales_out, ratios_out, hp: ob_hparams,
                          signs_out=None, nonfinite_out=None, stream=None):
    n = plan.n
    _want(g, "g", g.dtype, n)
    _want(err, "err", err.dtype, n)
    for name, t in (("m", m), ("v", v), ("p", p)):
        _want(t, name, torch.float32, n)
    _want(words_out, "words_out", torch.int32, (n + 31) // 32)
    _want(scales_out, "scales_out", torch.float32, plan.num_chunks)
    _want(ratios_out, "ratios_out", torch.float32, plan.num_chunks)
    _want(signs_out, "signs_out", torch.int8, n)
    _want(nonfinite_out, "nonfinite_out", torch.int64, 1)
    _check(lib().ob_lamb_compress_step(
        plan.handle, _dev(g, "g"), _gdtype(g), _dev(err, "err"), _errdtype(err), _dev(m, "m"), _dev(v, "v"),
        _dev(p, "p"), _dev(words_out, "words_out"), _dev(scales_out, "scales_out"),
        _dev(ratios_out, "ratios_out"), _dev(signs_out, "signs_out"), _dev(nonfinite_out, "nonfinite_out"),
        ctypes.byref(hp), _stream(stream)), "ob_lamb_compress_step")


def ob_lamb_warmup_step(plan: Plan, g, m, v, p, ratios_out, hp: ob_hparams, stream=None):
    n = plan.n
    _want(g, "g", g.dtype, n)
    for name, t in (("m", m), ("v", v), ("p", p)):
        _want(t, name, torch.float32, n)
    _want(ratios_out, "ratios_out", torch.float32, plan.num_chunks)
    _check(lib().ob_lamb_warmup_step(plan.handle, _dev(g, "g"), _gdtype(g), _dev(m, "m"), _dev(v, "v"),
                                     _dev(p, "p"), _dev(ratios_out, "ratios_out"), ctypes.byref(hp),
                                     _stream(stream)), "ob_lamb_warmup_step")


def ob_server_reduce(plan: Plan, worker_words, worker_scales, server_err, words_out, scales_out,
                     stream=None):
    n = plan.n
    W = worker_words.shape[0]
    _want(worker_words, "worker_words", torch.int32, W * ((n + 31) // 32))
    _want(worker_scales, "worker_scales", torch.float32, W * plan.num_chunks)
    _want(server_err, "server_err", torch.float32, n)
    _want(words_out, "words_out", torch.int32, (n + 31) // 32)
    _want(scales_out, "scales_out", torch.float32, plan.num_chunks)
    _check(lib().ob_server_reduce(plan.handle, W, _dev(worker_words, "worker_words"),
                                  _dev(worker_scales, "worker_scales"), _dev(server_err, "server_err"),
                                  _dev(words_out, "words_out"), _dev(scales_out, "scales_out"),
                                  _stream(stream)), "ob_server_reduce")


def ob_pack(x, words_out, stream=None):
    n = x.numel()
    _want(words_out, "words_out", torch.int32, (n + 31) // 32)
    _check(lib().ob_pack(_dev(x, "x"), _gdtype(x), n, _dev(words_out, "words_out"), _stream(stream)),
           "ob_pack")


def ob_unpack(plan: Plan | None, words, n: int, out, scales=None, stream=None):
    _want(words, "words", torch.int32, (n + 31) // 32)
    _want(out, "out", torch.float32, n)
    if scales is not None:
        if plan is None:
            raise ValueError("ob_unpack with scales needs the plan that defines the chunks")
        _want(scales, "scales", torch.float32, plan.num_chunks)
    _check(lib().ob_unpack(plan.handle if plan is not None else None, _dev(words, "words"), n,
                           _dev(scales, "scales"), _dev(out, "out"), _stream(stream)), "ob_unpack")


def ob_plan_set_diagnostics(plan: Plan, err_sumsq=None, plus_count=None):
    """Per-chunk diagnostics of later compressed steps into err_sumsq (float64[K]) and plus_count
    (int64[K]); both None switches them off."""
    _want(err_sumsq, "err_sumsq", torch.float64, plan.num_chunks)
    _want(plus_count, "plus_count", torch.int64, plan.num_chunks)
    _check(lib().ob_plan_set_diagnostics(plan.handle, _dev(err_sumsq, "err_sumsq"),
                                         _dev(plus_count, "plus_count")), "ob_plan_set_diagnostics")


def ob_plan_set_timing(plan: Plan, enable: bool):
    _check(lib().ob_plan_set_timing(plan.handle, 1 if enable else 0), "ob_plan_set_timing")


def ob_plan_read_timing(plan: Plan, kernel: int) -> tuple[float, int]:
    ms = ctypes.c_double()
    cnt = ctypes.c_int64()
    _check(lib().ob_plan_read_timing(plan.handle, kernel, ctypes.byref(ms), ctypes.byref(cnt)),
           "ob_plan_read_timing")
    return ms.value, cnt.value
