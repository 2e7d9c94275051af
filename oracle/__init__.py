"""CPU oracle for the 1-bit Adam step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  The product library (``adam_ob_compress_amd``) never imports, links or runs it, and it
imports nothing from the product.  Arithmetic lives in ``ob_oracle.c`` (plain single-threaded C,
double-precision arithmetic on fp32 state, built with ``-ffp-contract=off``); this module only
marshals numpy arrays and holds the host-side step schedules.

Pages cited (by title and section):
  [P1] "1bit Adam" tutorial (intelliparadigm.com article 2150495), sections 2.1, 2.2, 3.1, 3.2, 6.1.
  [P2] "DeepSpeed Communication Compression and Hiding", sections "1-bit Adam: warmup, frozen
       variance, error feedback" and "0/1 Adam".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ob_oracle.c")
_LIB = os.path.join(_HERE, "libob_oracle.so")
# A test may point the wrapper at a rebuilt copy of the oracle (the planted-mistake test does).
_LIB_OVERRIDE = os.environ.get("OB_ORACLE_LIB")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]

_lib = None


def build(verbose: bool = False) -> str:
    """Compile ob_oracle.c into libob_oracle.so with gcc (always recompiles)."""
    cmd = ["gcc", *CFLAGS, "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    global _lib
    _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    F = ctypes.c_float
    I = ctypes.c_int
    lib.or_pack.argtypes = [P, I, I64, P]
    lib.or_unpack.argtypes = [P, I64, I64, P, P, P]
    lib.or_compress_step.argtypes = [I64, I64, P, P, I, P, I, P, P, P, P, P, P, P,
                                     F, F, F, F, I, F]
    lib.or_lamb_compress_step.argtypes = [I64, I64, P, P, I, P, I, P, P, P, P, P, P, P, P,
                                          F, F, F, F, I, F]
    lib.or_lamb_warmup_step.argtypes = [I64, I64, P, P, I, P, P, P, P, F, F, F, F, I, I64]
    lib.or_diagnostics.argtypes = [I64, I64, P, P, I, P, P, P]
    U64 = ctypes.c_uint64
    lib.or_philox4x32.argtypes = [P, P, P]
    lib.or_philox4x32.restype = None
    lib.or_to_format_sr.argtypes = [P, I64, I, U64, U64, I64, P]
    lib.or_worker_compress.argtypes = [I64, I64, P, P, I, P, I, P, P, P, P, F, I, F, I, U64, U64, I64]
    lib.or_worker_update.argtypes = [I64, I64, P, P, P, P, P, P, F, F, F]
    lib.or_lamb_worker_update.argtypes = [I64, I64, P, P, P, P, P, P, P, F, F, F]
    lib.or_compress_step_sr.argtypes = [I64, I64, P, P, I, P, I, P, P, P, P, P, P, P,
                                        F, F, F, F, I, F, I, P, U64, U64, I64]
    lib.or_to_format.argtypes = [P, I64, I, P]
    lib.or_from_format.argtypes = [P, I64, I, P]
    lib.or_warmup_step.argtypes = [I64, P, I, P, P, P, F, F, F, F, I, I64]
    lib.or_server_reduce.argtypes = [I64, I64, P, I, P, P, P, P, P]
    lib.or_server_average.argtypes = [I64, I64, P, I, P, P, P]
    lib.or_chunk_sumsq.argtypes = [P, I64, I64]
    lib.or_chunk_sumsq.restype = ctypes.c_double
    lib.or_chunk_scale.argtypes = [P, I64, I64]
    lib.or_chunk_scale.restype = ctypes.c_float
    for name in ("or_pack", "or_unpack", "or_compress_step", "or_warmup_step",
                 "or_server_reduce", "or_server_average", "or_to_format", "or_from_format",
                 "or_lamb_compress_step", "or_lamb_warmup_step", "or_diagnostics", "or_to_format_sr",
                 "or_compress_step_sr"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _grad(g):
    """Return (array, is_bf16).  bf16 gradients travel as their raw uint16 bit patterns."""
    if g.dtype == np.float32:
        return g, 0
    if g.dtype == np.uint16:
        return g, 1
    raise TypeError(f"gradient must be float32 or uint16 (bf16 bits), got {g.dtype}")


# Storage formats of the error buffer (reading R15 in ob_oracle.c).  fp16 travels as numpy float16,
# bf16 as its raw uint16 bit patterns.
ERR_FORMATS = {"f32": 0, "bf16": 1, "f16": 2}


def _err(e):
    """Return (array, format code) of an error buffer: float32, float16, or uint16 (bf16 bits)."""
    if e.dtype == np.float32:
        return e, 0
    if e.dtype == np.uint16:
        return e, 1
    if e.dtype == np.float16:
        return e, 2
    raise TypeError(f"error buffer must be float32, float16 or uint16 (bf16 bits), got {e.dtype}")


def to_format(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round fp32 values to "bf16" (uint16 bits) or "f16" (float16), nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = np.zeros(x.size, dtype=np.uint16)
    _check(_load().or_to_format(_ptr(x), x.size, ERR_FORMATS[fmt], _ptr(bits)), "to_format")
    return bits.view(np.float16) if fmt == "f16" else bits


def philox4x32(counter, key) -> np.ndarray:
    """Philox4x32-10 of a 4 x uint32 counter under a 2 x uint32 key (reading R18)."""
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    _load().or_philox4x32(_ptr(c), _ptr(k), _ptr(out))
    return out


def to_format_sr(x: np.ndarray, fmt: str, seed: int, step: int, index0: int = 0) -> np.ndarray:
    """Stochastic rounding (R18) of fp32 values stored as flat elements index0.. of a "bf16" (uint16 bits)
    or "f16" (float16) error buffer, with the random bits of (seed, step)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = np.zeros(x.size, dtype=np.uint16)
    _check(_load().or_to_format_sr(_ptr(x), x.size, ERR_FORMATS[fmt], seed, step, index0, _ptr(bits)),
           "to_format_sr")
    return bits.view(np.float16) if fmt == "f16" else bits


def from_format(bits: np.ndarray, fmt: str) -> np.ndarray:
    """Widen "bf16" bits (uint16) or "f16" values (float16 or their uint16 bits) to fp32, exactly."""
    bits = np.ascontiguousarray(bits).view(np.uint16)
    out = np.zeros(bits.size, dtype=np.float32)
    _check(_load().or_from_format(_ptr(bits), bits.size, ERR_FORMATS[fmt], _ptr(out)), "from_format")
    return out


# ----------------------------------------------------------------------------------------------
# chunk tables
# ----------------------------------------------------------------------------------------------

def uniform_offsets(n: int, chunk: int) -> np.ndarray:
    """Offsets of uniform chunks of `chunk` elements; the last chunk ends at n."""
    k = (n + chunk - 1) // chunk
    off = [min(c * chunk, n) for c in range(k)] + [n]
    return np.asarray(off, dtype=np.int64)


def n_words(n: int) -> int:
    return (n + 31) // 32


# ----------------------------------------------------------------------------------------------
# the method
# ----------------------------------------------------------------------------------------------

def pack(x: np.ndarray) -> np.ndarray:
    x, bf = _grad(np.ascontiguousarray(x))
    out = np.zeros(n_words(x.size), dtype=np.uint32)
    _check(_load().or_pack(_ptr(x), bf, x.size, _ptr(out)), "pack")
    return out


def unpack(words: np.ndarray, n: int, offsets: np.ndarray | None = None,
           scales: np.ndarray | None = None) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    k = 0 if offsets is None else offsets.size - 1
    _check(_load().or_unpack(_ptr(words), n, k, _ptr(offsets), _ptr(scales), _ptr(out)), "unpack")
    return out


def chunk_sumsq(x: np.ndarray, begin: int, end: int) -> float:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return _load().or_chunk_sumsq(_ptr(x), begin, end)


def chunk_scale(x: np.ndarray, begin: int, end: int) -> float:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return _load().or_chunk_scale(_ptr(x), begin, end)


def compress_step(g, err, m, v, p, offsets, *, lr, beta1, eps, clip=0.0, ef_mode=0, ef_beta=0.9,
                  want_signs=False, count_nonfinite=False, stochastic=False, sr_seed=0, sr_step=0,
                  sr_index0=0):
    """One compressed step.  err, m, p are updated in place; v is read only.  m, v, p are fp32; the
    error buffer is fp32, fp16 (numpy float16) or bf16 (uint16 bits), see R15.

    Returns (words uint32[ceil(n/32)], scales fp32[K], signs int8[n] or None, nonfinite int or None).
    """
    g, bf = _grad(np.ascontiguousarray(g))
    n = g.size
    err, efmt = _err(err)
    assert err.size == n and err.flags["C_CONTIGUOUS"]
    for a in (m, v, p):
        assert a.dtype == np.float32 and a.size == n and a.flags["C_CONTIGUOUS"]
    k = offsets.size - 1
    words = np.zeros(n_words(n), dtype=np.uint32)
    scales = np.zeros(max(k, 0), dtype=np.float32)
    signs = np.zeros(n, dtype=np.int8) if want_signs else None
    nf = np.zeros(1, dtype=np.int64) if count_nonfinite else None
    if stochastic:      # R18: stochastic rounding of a 16-bit error buffer
        rc = _load().or_compress_step_sr(n, k, _ptr(offsets), _ptr(g), bf, _ptr(err), efmt, _ptr(m),
                                         _ptr(v), _ptr(p), _ptr(words), _ptr(scales), _ptr(signs),
                                         _ptr(nf), lr, beta1, eps, clip, ef_mode, ef_beta, 0, None,
                                         sr_seed, sr_step, sr_index0)
    else:
        rc = _load().or_compress_step(n, k, _ptr(offsets), _ptr(g), bf, _ptr(err), efmt, _ptr(m), _ptr(v),
                                      _ptr(p), _ptr(words), _ptr(scales), _ptr(signs), _ptr(nf),
                                      lr, beta1, eps, clip, ef_mode, ef_beta)
    _check(rc, "compress_step")
    return words, scales, signs, (int(nf[0]) if nf is not None else None)


def worker_compress(g, err, offsets, *, clip=0.0, ef_mode=0, ef_beta=0.9, want_signs=False,
                    count_nonfinite=False, stochastic=False, sr_seed=0, sr_step=0, sr_index0=0):
    """The worker's half before the exchange (reading R19 (a)): err updated in place with the worker's
    own g_hat.  Returns (words, scales, signs or None, nonfinite or None)."""
    g, bf = _grad(np.ascontiguousarray(g))
    n = g.size
    err, efmt = _err(err)
    assert err.size == n and err.flags["C_CONTIGUOUS"]
    k = offsets.size - 1
    words = np.zeros(n_words(n), dtype=np.uint32)
    scales = np.zeros(max(k, 0), dtype=np.float32)
    signs = np.zeros(n, dtype=np.int8) if want_signs else None
    nf = np.zeros(1, dtype=np.int64) if count_nonfinite else None
    _check(_load().or_worker_compress(n, k, _ptr(offsets), _ptr(g), bf, _ptr(err), efmt, _ptr(words),
                                      _ptr(scales), _ptr(signs), _ptr(nf), clip, ef_mode, ef_beta,
                                      1 if stochastic else 0, sr_seed, sr_step, sr_index0), "worker_compress")
    return words, scales, signs, (int(nf[0]) if nf is not None else None)


def worker_update(words, scales, m, v, p, offsets, *, lr, beta1, eps):
    """The worker's half after the exchange (reading R19 (b)): g_hat from the exchanged words and scales,
    then m and p in place (v read only)."""
    n = m.size
    for a in (m, v, p):
        assert a.dtype == np.float32 and a.size == n and a.flags["C_CONTIGUOUS"]
    words = np.ascontiguousarray(words, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    assert words.size == n_words(n) and scales.size == offsets.size - 1
    _check(_load().or_worker_update(n, offsets.size - 1, _ptr(offsets), _ptr(words), _ptr(scales), _ptr(m),
                                    _ptr(v), _ptr(p), lr, beta1, eps), "worker_update")


def lamb_worker_update(words, scales, m, v, p, offsets, *, lr, beta1, eps):
    """1-bit LAMB's half after the exchange (readings R16, R19): m on the exchanged g_hat, then the
    per-layer trust ratio and the update.  m, p in place; returns the ratios fp32[K]."""
    n = m.size
    for a in (m, v, p):
        assert a.dtype == np.float32 and a.size == n and a.flags["C_CONTIGUOUS"]
    words = np.ascontiguousarray(words, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    k = offsets.size - 1
    assert words.size == n_words(n) and scales.size == k
    ratios = np.zeros(max(k, 0), dtype=np.float32)
    _check(_load().or_lamb_worker_update(n, k, _ptr(offsets), _ptr(words), _ptr(scales), _ptr(m), _ptr(v),
                                         _ptr(p), _ptr(ratios), lr, beta1, eps), "lamb_worker_update")
    return ratios


def warmup_step(g, m, v, p, *, lr, beta1, beta2, eps, bias_correction=False, step=0):
    """One dense Adam step; m, v, p updated in place."""
    g, bf = _grad(np.ascontiguousarray(g))
    n = g.size
    for a in (m, v, p):
        assert a.dtype == np.float32 and a.size == n and a.flags["C_CONTIGUOUS"]
    rc = _load().or_warmup_step(n, _ptr(g), bf, _ptr(m), _ptr(v), _ptr(p), lr, beta1, beta2, eps,
                                1 if bias_correction else 0, step)
    _check(rc, "warmup_step")


def diagnostics(err_before, words, offsets):
    """Per-chunk diagnostics of a compressed step (reading R17): (sum of squares of the error buffer
    the step read, float64[K]; number of +1 signs in the step's words, int64[K])."""
    err_before, efmt = _err(np.ascontiguousarray(err_before))
    k = offsets.size - 1
    ss = np.zeros(max(k, 0), dtype=np.float64)
    plus = np.zeros(max(k, 0), dtype=np.int64)
    words = np.ascontiguousarray(words, dtype=np.uint32)
    _check(_load().or_diagnostics(err_before.size, k, _ptr(offsets), _ptr(err_before), efmt, _ptr(words),
                                  _ptr(ss), _ptr(plus)), "diagnostics")
    return ss, plus


def lamb_compress_step(g, err, m, v, p, offsets, *, lr, beta1, eps, clip=0.0, ef_mode=0, ef_beta=0.9,
                       want_signs=False, count_nonfinite=False, stochastic=False, sr_seed=0, sr_step=0,
                       sr_index0=0):
    """One compressed 1-bit LAMB step (reading R16): as compress_step up to the momentum, then the
    per-chunk (layer) trust ratio and update.  err, m, p in place; v read only.

    Returns (words, scales fp32[K], ratios fp32[K], signs or None, nonfinite or None)."""
    g, bf = _grad(np.ascontiguousarray(g))
    n = g.size
    err, efmt = _err(err)
    assert err.size == n and err.flags["C_CONTIGUOUS"]
    for a in (m, v, p):
        assert a.dtype == np.float32 and a.size == n and a.flags["C_CONTIGUOUS"]
    k = offsets.size - 1
    words = np.zeros(n_words(n), dtype=np.uint32)
    scales = np.zeros(max(k, 0), dtype=np.float32)
    ratios = np.zeros(max(k, 0), dtype=np.float32)
    signs = np.zeros(n, dtype=np.int8) if want_signs else None
    nf = np.zeros(1, dtype=np.int64) if count_nonfinite else None
    if stochastic:
        rc = _load().or_compress_step_sr(n, k, _ptr(offsets), _ptr(g), bf, _ptr(err), efmt, _ptr(m),
                                         _ptr(v), _ptr(p), _ptr(words), _ptr(scales), _ptr(signs),
                                         _ptr(nf), lr, beta1, eps, clip, ef_mode, ef_beta, 1, _ptr(ratios),
                                         sr_seed, sr_step, sr_index0)
    else:
        rc = _load().or_lamb_compress_step(n, k, _ptr(offsets), _ptr(g), bf, _ptr(err), efmt, _ptr(m),
                                           _ptr(v), _ptr(p), _ptr(words), _ptr(scales), _ptr(ratios),
                                           _ptr(signs), _ptr(nf), lr, beta1, eps, clip, ef_mode, ef_beta)
    _check(rc, "lamb_compress_step")
    return words, scales, ratios, signs, (int(nf[0]) if nf is not None else None)


def lamb_warmup_step(g, m, v, p, offsets, *, lr, beta1, beta2, eps, bias_correction=False, step=0):
    """One dense LAMB step (the warmup of 1-bit LAMB); m, v, p in place.  Returns ratios fp32[K]."""
    g, bf = _grad(np.ascontiguousarray(g))
    n = g.size
    for a in (m, v, p):
        assert a.dtype == np.float32 and a.size == n and a.flags["C_CONTIGUOUS"]
    k = offsets.size - 1
    ratios = np.zeros(max(k, 0), dtype=np.float32)
    rc = _load().or_lamb_warmup_step(n, k, _ptr(offsets), _ptr(g), bf, _ptr(m), _ptr(v), _ptr(p),
                                     _ptr(ratios), lr, beta1, beta2, eps, 1 if bias_correction else 0,
                                     step)
    _check(rc, "lamb_warmup_step")
    return ratios


def server_reduce(worker_words, worker_scales, server_err, offsets):
    """Server half on one share: worker_words uint32[W, ceil(n/32)], worker_scales fp32[W, K].

    server_err (fp32[n]) is updated in place; returns (words_out, scales_out)."""
    n = server_err.size
    k = offsets.size - 1
    W = worker_words.shape[0]
    assert worker_words.shape == (W, n_words(n)) and worker_words.dtype == np.uint32
    assert worker_scales.shape == (W, k) and worker_scales.dtype == np.float32
    words = np.zeros(n_words(n), dtype=np.uint32)
    scales = np.zeros(k, dtype=np.float32)
    rc = _load().or_server_reduce(n, k, _ptr(offsets), W, _ptr(np.ascontiguousarray(worker_words)),
                                  _ptr(np.ascontiguousarray(worker_scales)), _ptr(server_err),
                                  _ptr(words), _ptr(scales))
    _check(rc, "server_reduce")
    return words, scales


def server_average(worker_words, worker_scales, n, offsets):
    k = offsets.size - 1
    W = worker_words.shape[0]
    out = np.empty(n, dtype=np.float32)
    rc = _load().or_server_average(n, k, _ptr(offsets), W,
                                   _ptr(np.ascontiguousarray(worker_words)),
                                   _ptr(np.ascontiguousarray(worker_scales)), _ptr(out))
    _check(rc, "server_average")
    return out


# ----------------------------------------------------------------------------------------------
# host schedules
# ----------------------------------------------------------------------------------------------

def one_bit_adam_kind(step: int, freeze_step: int) -> str:
    """[P2] 1-bit Adam: dense Adam while step < freeze_step, compressed afterwards (step from 0)."""
    return "dense" if step < freeze_step else "compressed"


def zero_one_adam_kind(t: int, period: int) -> str:
    """[P2] 0/1 Adam: a full-precision variance refresh on every period-th step (t from 1)."""
    return "dense" if t % period == 0 else "compressed"
