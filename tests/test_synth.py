"""Host checks of the seeded input generators: a window drawn on its own equals the same elements of
the whole draw (the full-size parity checks regenerate one chunk's inputs at a time this way)."""
import dataclasses

import pytest
import torch

from adam_ob_compress_amd import synth


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


@pytest.mark.parametrize("w", [
    dataclasses.replace(synth.GPT2_XL, n=50_000, chunk=1 << 13),
    dataclasses.replace(synth.LLAMA2_7B, n=40_001, chunk=1 << 12, err_dtype="bf16"),
    dataclasses.replace(synth.LLAMA2_7B, n=9_000, chunk=1 << 12, err_dtype="f16"),
    synth.scaled(synth.BERT_BASE, 20_000, 4096),
], ids=lambda w: w.name)
def test_windows_equal_the_whole_draw(w, monkeypatch):
    monkeypatch.setattr(synth, "SLICE", 1 << 12)          # several generator slices per chunk
    g = synth.draw_grad(w, 3, "cpu")
    for sig in ((0.0, 0.0), (1e-4, 2e-4)):
        full = synth.draw_state(w, "cpu", *sig)
        assert (full[0] != 0).any() == (sig[0] > 0) and (full[1] != 0).any() == (sig[1] > 0)
        off = w.chunk_offsets()
        for c in range(w.n_chunks):
            a, b = int(off[c]), int(off[c + 1])
            assert torch.equal(_bits(synth.draw_grad_window(w, 3, a, b, "cpu")), _bits(g[a:b])), c
            for t, win in zip(full, synth.draw_state_window(w, a, b, "cpu", *sig)):
                assert t.dtype == win.dtype and torch.equal(_bits(t[a:b]), _bits(win)), c
    if w.grad_sigma is not None:                          # windows that straddle slices
        for a, b in ((5, 9000), (4095, 4097), (0, w.n)):
            assert torch.equal(_bits(synth.draw_grad_window(w, 3, a, b, "cpu")), _bits(g[a:b]))
