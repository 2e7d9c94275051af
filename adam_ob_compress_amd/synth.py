"""Seeded synthetic workloads for the 1-bit Adam step.

This module only draws inputs: shapes, chunk tables and random state with the distributions of the
workloads below.  It holds none of the optimizer's arithmetic, and it is the one module that both the
HIP path's callers and the CPU oracle's callers take their inputs from.

Workloads (shapes stand in for the models the pages train; no dataset or weights are involved):
  single-1M-fp32        one fp32 tensor of 2^20 elements, one chunk.
  bert-base-110M-fp32   the 197 parameter tensors of BERT-base (no pooler) in one flat fp32 buffer,
                        one chunk per tensor (the BERT-base experiment of the "1bit Adam" tutorial,
                        sec. 5.1).
  server-2^28-W8        the server share: n = 2^28, W = 8 simulated workers, chunks of 2^20.
  gpt2-1.5B-bf16        a flat 1,557,611,200-element buffer, bf16 gradients, chunks of 2^24.
  llama2-7B-bf16-ema    a flat 6,738,415,616-element buffer, bf16 gradients, chunks of 2^24, with
                        the tutorial's clip / EMA error / int8 variant and a variance refresh every
                        16th step.
"""
from __future__ import annotations

import dataclasses
import numpy as np
import torch

SEED = 0x1B17ADA3
SLICE = 1 << 26  # elements drawn per generator call: bounds temporary memory on large buffers

# stream ids: one independent random stream per state array
S_GRAD, S_ERR, S_M, S_V, S_P, S_SIGMA, S_OUTLIER, S_WORDS, S_WSCALES = range(9)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int
    offsets: tuple | None  # per-tensor chunk offsets (K+1), or None for uniform chunks
    chunk: int             # uniform chunk size (ignored when offsets is given)
    grad_dtype: str        # "f32" | "bf16"
    grad_sigma: float | None   # None: per-tensor log-uniform sigma in [1e-4, 1e-2]
    outlier_frac: float = 0.0  # fraction of gradient elements scaled by outlier_mult before bf16 rounding
    outlier_mult: float = 100.0
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    clip: float = 0.0
    ef_mode: int = 0           # 0 plain, 1 EMA
    ef_beta: float = 0.9
    int8_signs: bool = False
    freeze_step: int = 0       # dense steps s < freeze_step first (s from 0)
    refresh_period: int = 0    # dense refresh when t % period == 0 (t from 1); 0 = never
    steps: int = 10
    workers: int = 0           # > 0: server-stage workload
    err_dtype: str = "f32"     # storage of the error buffer: "f32" | "bf16" | "f16"
    optimizer: str = "adam"    # "adam" | "lamb" (1-bit LAMB: the chunks are the layers)
    err_rounding: str = "nearest"  # 16-bit error buffers: "nearest" | "stochastic"

    @property
    def n_chunks(self) -> int:
        if self.offsets is not None:
            return len(self.offsets) - 1
        return (self.n + self.chunk - 1) // self.chunk

    def chunk_offsets(self) -> np.ndarray:
        if self.offsets is not None:
            return np.asarray(self.offsets, dtype=np.int64)
        k = self.n_chunks
        return np.asarray([min(c * self.chunk, self.n) for c in range(k)] + [self.n], dtype=np.int64)


def bert_base_tensor_sizes() -> list[int]:
    """Element counts of BERT-base's 197 trainable tensors (pooler excluded), in model order."""
    h, ff, vocab, pos, types, layers = 768, 3072, 30522, 512, 2, 12
    sizes = [vocab * h, pos * h, types * h, h, h]          # embeddings + embedding LayerNorm
    for _ in range(layers):
        for _ in range(4):                                  # Q, K, V, attention-output projections
            sizes += [h * h, h]
        sizes += [h, h]                                     # attention LayerNorm
        sizes += [ff * h, ff]                               # FFN in
        sizes += [h * ff, h]                                # FFN out
        sizes += [h, h]                                     # output LayerNorm
    return sizes


def llama2_7b_tensor_sizes() -> list[int]:
    """Element counts of Llama-2-7B's 291 tensors, in model order."""
    h, ff, vocab, layers = 4096, 11008, 32000, 32
    sizes = [vocab * h]                                     # token embedding
    for _ in range(layers):
        sizes += [h * h] * 4                                # q, k, v, o projections
        sizes += [ff * h, ff * h, h * ff]                   # gate, up, down projections
        sizes += [h, h]                                     # the two RMSNorm weights
    sizes += [h, vocab * h]                                 # final norm, output head
    return sizes


def _offsets_from_sizes(sizes) -> tuple:
    off = [0]
    for s in sizes:
        off.append(off[-1] + s)
    return tuple(off)


SINGLE_1M = Workload("single-1M-fp32", 1 << 20, None, 1 << 20, "f32", 1e-3, steps=10)
BERT_BASE = Workload("bert-base-110M-fp32", 108_891_648, _offsets_from_sizes(bert_base_tensor_sizes()),
                     0, "f32", None, freeze_step=5, steps=25)
SERVER_W8 = Workload("server-2^28-W8", 1 << 28, None, 1 << 20, "f32", None, workers=8, steps=10)
GPT2_XL = Workload("gpt2-1.5B-bf16", 1_557_611_200, None, 1 << 24, "bf16", 1e-3, outlier_frac=0.01,
                   steps=10)
LLAMA2_7B = Workload("llama2-7B-bf16-ema", 6_738_415_616, None, 1 << 24, "bf16", 1e-3,
                     outlier_frac=0.01, clip=5.0, ef_mode=1, ef_beta=0.9, int8_signs=True,
                     refresh_period=16, steps=48)

# 1-bit LAMB: the layers are the model's tensors (one chunk each)
BERT_BASE_LAMB = dataclasses.replace(BERT_BASE, name="bert-base-110M-fp32-lamb", optimizer="lamb")
LLAMA2_7B_LAMB = Workload("llama2-7B-bf16-lamb", 6_738_415_616, _offsets_from_sizes(llama2_7b_tensor_sizes()),
                          0, "bf16", 1e-3, outlier_frac=0.01, clip=5.0, ef_mode=1, ef_beta=0.9,
                          int8_signs=True, freeze_step=2, steps=10, optimizer="lamb")

WORKLOADS = {w.name: w for w in (SINGLE_1M, BERT_BASE, SERVER_W8, GPT2_XL, LLAMA2_7B, BERT_BASE_LAMB,
                                 LLAMA2_7B_LAMB)}
# the same optimizer workloads with the error buffer stored in 16 bits ("<name>-err-bf16", "-err-f16")
WORKLOADS.update({f"{w.name}-err-{e}": dataclasses.replace(w, name=f"{w.name}-err-{e}", err_dtype=e)
                  for w in (BERT_BASE, GPT2_XL, LLAMA2_7B) for e in ("bf16", "f16")})
# ... and stored with stochastic rounding ("<name>-err-bf16-sr", "<name>-err-f16-sr")
WORKLOADS.update({f"{w.name}-err-{e}-sr": dataclasses.replace(w, name=f"{w.name}-err-{e}-sr", err_dtype=e,
                                                              err_rounding="stochastic")
                  for w in (BERT_BASE, GPT2_XL, LLAMA2_7B) for e in ("bf16", "f16")})
SR_SEED = 0x0B1AD  # the stochastic-rounding key of every workload


def scaled(w: Workload, n: int, chunk: int | None = None) -> Workload:
    """The same recipe on a smaller flat buffer (uniform chunks), for tests the oracle finishes fast."""
    return dataclasses.replace(w, name=f"{w.name}@{n}", n=n, offsets=None,
                               chunk=chunk if chunk is not None else (w.chunk or n))


# ----------------------------------------------------------------------------------------------
# drawing
# ----------------------------------------------------------------------------------------------

def _gen(device, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    h = SEED
    for k in key:
        h = (h * 0x9E3779B1 + int(k) + 1) & 0x7FFFFFFFFFFFFFFF
    g.manual_seed(h)
    return g


def _slice_normal(device, sigma: float, key: tuple, s0: int, s1: int) -> torch.Tensor:
    """Slice [s0, s1) of the N(0, sigma) stream `key` (s0 a multiple of SLICE): its values depend on
    (key, slice index) only, so one slice can be drawn again on its own."""
    g = _gen(device, *key, s0 // SLICE)
    return torch.randn(s1 - s0, generator=g, device=device, dtype=torch.float32) * sigma


def _fill_normal(out: torch.Tensor, sigma: float, *key):
    """out[:] = N(0, sigma) drawn slice by slice; values depend on (key, slice index)."""
    n = out.numel()
    for s0 in range(0, n, SLICE):
        s1 = min(n, s0 + SLICE)
        out[s0:s1] = _slice_normal(out.device, sigma, key, s0, s1)


def _window(n: int, a: int, b: int, draw_slice) -> torch.Tensor:
    """Elements [a, b) of an n-element stream drawn slice by slice: every slice that overlaps the window
    is drawn again whole by draw_slice(s0, s1), and the overlap is kept."""
    parts = []
    for s0 in range(a // SLICE * SLICE, b, SLICE):
        s1 = min(n, s0 + SLICE)
        parts.append(draw_slice(s0, s1)[max(a, s0) - s0:min(b, s1) - s0])
    return parts[0] if len(parts) == 1 else torch.cat(parts)


def _sigma_per_tensor(w: Workload) -> np.ndarray:
    """Per-chunk gradient sigma, log-uniform in [1e-4, 1e-2] (fixed for the run)."""
    rng = np.random.default_rng([SEED, S_SIGMA])
    return 10.0 ** rng.uniform(-4.0, -2.0, size=w.n_chunks)


def _grad_slice(w: Workload, step: int, device, s0: int, s1: int) -> torch.Tensor:
    """Slice [s0, s1) of a uniform-sigma gradient: N(0, sigma) with outliers, in w's gradient dtype."""
    t = _slice_normal(device, w.grad_sigma, (S_GRAD, step), s0, s1)
    if w.outlier_frac > 0:
        go = _gen(device, S_OUTLIER, step, s0 // SLICE)
        hit = torch.rand(s1 - s0, generator=go, device=device) < w.outlier_frac
        t = torch.where(hit, t * w.outlier_mult, t)
    return t.to(torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32)


def draw_grad(w: Workload, step: int, device, out: torch.Tensor | None = None) -> torch.Tensor:
    """A fresh gradient for `step`: fp32, or bf16 with outliers scaled before rounding."""
    dt = torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32
    if out is None:
        out = torch.empty(w.n, dtype=dt, device=device)
    if w.grad_sigma is None:
        off = w.chunk_offsets()
        sig = _sigma_per_tensor(w)
        tmp = torch.empty(w.n, dtype=torch.float32, device=device) if dt != torch.float32 else out
        for c in range(w.n_chunks):
            a, b = int(off[c]), int(off[c + 1])
            _fill_normal(tmp[a:b], float(sig[c]), S_GRAD, step, c)
        if tmp is not out:
            out.copy_(tmp)
        return out
    for s0 in range(0, w.n, SLICE):
        s1 = min(w.n, s0 + SLICE)
        out[s0:s1] = _grad_slice(w, step, device, s0, s1)
    return out


def draw_grad_window(w: Workload, step: int, a: int, b: int, device) -> torch.Tensor:
    """Elements [a, b) of draw_grad(w, step), drawn on their own (a per-tensor-sigma workload: [a, b)
    must lie in one chunk)."""
    if w.grad_sigma is not None:
        return _window(w.n, a, b, lambda s0, s1: _grad_slice(w, step, device, s0, s1))
    off = w.chunk_offsets()
    c = int(np.searchsorted(off, a, side="right")) - 1
    o0, o1 = int(off[c]), int(off[c + 1])
    assert o0 <= a <= b <= o1, "a per-tensor-sigma window must lie in one chunk"
    sig = float(_sigma_per_tensor(w)[c])
    t = _window(o1 - o0, a - o0, b - o0,
                lambda s0, s1: _slice_normal(device, sig, (S_GRAD, step, c), s0, s1))
    return t.to(torch.bfloat16) if w.grad_dtype == "bf16" else t


ERR_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _state_slice(w: Workload, which: str, device, s0: int, s1: int, err_sigma: float, m_sigma: float):
    if which == "err":
        t = (_slice_normal(device, err_sigma, (S_ERR, 0, 0), s0, s1) if err_sigma > 0
             else torch.zeros(s1 - s0, dtype=torch.float32, device=device))
        return t.to(ERR_TORCH_DTYPES[w.err_dtype])
    if which == "m":
        return (_slice_normal(device, m_sigma, (S_M, 0, 0), s0, s1) if m_sigma > 0
                else torch.zeros(s1 - s0, dtype=torch.float32, device=device))
    if which == "v":
        return _slice_normal(device, 1e-6, (S_V, 0, 0), s0, s1).abs_().add_(1e-8)
    return _slice_normal(device, 0.02, (S_P, 0, 0), s0, s1)


def draw_state(w: Workload, device, err_sigma: float = 0.0, m_sigma: float = 0.0, out=None):
    """Initial (err, m, v, p): err = 0 (in w.err_dtype), m = 0, v = |N(0,1e-6)| + 1e-8, p ~ N(0, 0.02).
    err_sigma / m_sigma > 0 draw err ~ N(0, err_sigma) (rounded to w.err_dtype) and m ~ N(0, m_sigma)
    instead, for checks from a state with every term non-zero.  out: four tensors of n elements (err in
    w.err_dtype, the others fp32) to fill in place instead of allocating."""
    n = w.n
    given = out
    out = []
    for k, (which, dt) in enumerate((("err", ERR_TORCH_DTYPES[w.err_dtype]), ("m", torch.float32),
                                     ("v", torch.float32), ("p", torch.float32))):
        t = torch.empty(n, dtype=dt, device=device) if given is None else given[k]
        assert t.dtype == dt and t.numel() == n
        if (which == "err" and err_sigma <= 0) or (which == "m" and m_sigma <= 0):
            t.zero_()
        else:
            for s0 in range(0, n, SLICE):
                s1 = min(n, s0 + SLICE)
                t[s0:s1] = _state_slice(w, which, device, s0, s1, err_sigma, m_sigma)
        out.append(t)
    return tuple(out)


def draw_state_window(w: Workload, a: int, b: int, device, err_sigma: float = 0.0, m_sigma: float = 0.0):
    """Elements [a, b) of draw_state(w, device, err_sigma, m_sigma), drawn on their own."""
    return tuple(_window(w.n, a, b, lambda s0, s1, k=k: _state_slice(w, k, device, s0, s1, err_sigma, m_sigma))
                 for k in ("err", "m", "v", "p"))


def draw_worker_words(w: Workload, rnd: int, device) -> torch.Tensor:
    """W rows of ceil(n/32) uint32 words of fair random bits (returned as int32 storage)."""
    nw = (w.n + 31) // 32
    out = torch.empty((w.workers, nw), dtype=torch.int32, device=device)
    for k in range(w.workers):
        g = _gen(device, S_WORDS, rnd, k)
        out[k] = torch.randint(-(1 << 31), (1 << 31) - 1, (nw,), generator=g, device=device,
                               dtype=torch.int64).to(torch.int32)
        if w.n % 32:
            out[k, -1] &= (1 << (w.n % 32)) - 1
    return out


def draw_worker_scales(w: Workload, rnd: int, device) -> torch.Tensor:
    """W rows of K fp32 scales, U(1e-4, 1e-2)."""
    g = _gen(device, S_WSCALES, rnd)
    u = torch.rand((w.workers, w.n_chunks), generator=g, device=device, dtype=torch.float64)
    return (1e-4 + u * (1e-2 - 1e-4)).to(torch.float32)


def draw_values(n: int, seed: int, pattern: str = "normal") -> np.ndarray:
    """Small host-side fp32 test vectors with edge patterns (for brute-force checks)."""
    rng = np.random.default_rng([SEED, seed, n])
    if pattern == "normal":
        return rng.standard_normal(n).astype(np.float32) * np.float32(1e-3)
    if pattern == "zeros":
        return np.zeros(n, dtype=np.float32)
    if pattern == "signed_zeros":
        return np.where(rng.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    if pattern == "denormals":
        mag = rng.integers(1, 1 << 23, size=n).astype(np.uint32)
        sgn = (rng.random(n) < 0.5).astype(np.uint32) << 31
        return (mag | sgn).view(np.float32)
    if pattern == "alternating":
        return np.where(np.arange(n) % 2 == 0, 1.0, -1.0).astype(np.float32)
    if pattern == "special":
        pool = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-45, -1e-45, 3.0, -3.0],
                        dtype=np.float32)
        return pool[rng.integers(0, pool.size, size=n)]
    if pattern == "wide":
        return (rng.standard_normal(n) * 20.0).astype(np.float32)
    raise ValueError(pattern)


def host(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy of a tensor (bf16 travels as its uint16 bits)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16).copy()
    if t.dtype == torch.int32:
        return t.cpu().numpy().view(np.uint32).copy()
    return t.cpu().numpy().copy()
