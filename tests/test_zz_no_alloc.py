"""The allocation-free clip + AdamW (gpt2k_clip_adamw_noalloc) against the entry
point that takes a caller's scratch buffer (gpt2k_clip_adamw), through the C ABI.

Both run the same three kernels (sum of squares, norm, AdamW) on the same inputs,
so every output is compared bit for bit: parameters, both moments, the zeroed
gradient, the bf16 shadow and the norm.  Two calls in a row, the second on a
smaller input, show that the static scratch left by the first call does not leak
into the second."""
import numpy as np
import pytest

from transformer_lm_pretraining_amd import synth
from gpu_util import to_dev_f32

pytestmark = pytest.mark.gpu


def _state(n, seed, gscale):
    return (synth.normal((n,), std=0.02, seed=300 + seed),
            synth.normal((n,), std=gscale, seed=310 + seed),
            synth.normal((n,), std=1e-3, seed=320 + seed),
            np.abs(synth.normal((n,), std=1e-4, seed=330 + seed)))


def test_noalloc_clip_adamw_matches_the_scratch_entry_point(gpu_lib):
    import torch
    from transformer_lm_pretraining_amd import lib
    norm_b = torch.zeros(1, dtype=torch.float32, device="cuda")
    # (n, n_decay, seed, gradient scale, t): a clipped call on 1M elements, then an
    # unclipped one on 4,004 (fewer elements than the sum-of-squares kernel has threads)
    for n, n_decay, seed, gscale, t in ((1 << 20, 700 * 1024, 0, 1.0, 5), (4004, 2400, 1, 1e-4, 2)):
        print("noalloc clip_adamw n", n, "n_decay", n_decay, flush=True)
        p, g, m, v = _state(n, seed, gscale)
        pa, ga, ma, va = (to_dev_f32(x) for x in (p, g, m, v))
        pb, gb, mb, vb = (to_dev_f32(x) for x in (p, g, m, v))
        sha = torch.empty(n_decay, dtype=torch.bfloat16, device="cuda")
        shb = torch.empty(n_decay, dtype=torch.bfloat16, device="cuda")
        norm_a = lib.clip_adamw(pa, ga, ma, va, sha, n_decay, 3e-4, t)
        lib.clip_adamw_noalloc(pb, gb, mb, vb, shb, n_decay, 3e-4, t, norm=norm_b)
        torch.cuda.synchronize()
        assert float(norm_a.item()) > 0
        assert torch.equal(norm_a, norm_b), (float(norm_a.item()), float(norm_b.item()))
        for name, a, b in (("p", pa, pb), ("m", ma, mb), ("v", va, vb), ("g", ga, gb)):
            assert torch.equal(a, b), name
        assert torch.all(gb == 0)
        assert torch.equal(sha.view(torch.int16), shb.view(torch.int16))
        clipped = float(np.linalg.norm(g.astype(np.float64))) > 1.0
        assert clipped == (gscale == 1.0)


def test_noalloc_clip_adamw_rejects_bad_arguments(gpu_lib):
    """Invalid sizes are refused before any device work, with the same codes as the
    scratch entry point."""
    import ctypes
    import torch
    from transformer_lm_pretraining_amd import lib
    L = lib.load()
    x = torch.zeros(16, dtype=torch.float32, device="cuda")
    a = lib.AdamwArgs(1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, 1)
    P = lib._ptr
    assert L.gpt2k_clip_adamw_noalloc(P(x), P(x), P(x), P(x), None, 14, 0, ctypes.byref(a), None,
                                      lib._stream()) == lib.GPT2_E_INVALID  # n % 4
    assert L.gpt2k_clip_adamw_noalloc(P(x), P(x), P(x), P(x), None, 16, 20, ctypes.byref(a), None,
                                      lib._stream()) == lib.GPT2_E_INVALID  # n_decay > n
    bad_t = lib.AdamwArgs(1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, 0)
    assert L.gpt2k_clip_adamw_noalloc(P(x), P(x), P(x), P(x), None, 16, 0, ctypes.byref(bad_t), None,
                                      lib._stream()) == lib.GPT2_E_INVALID  # t < 1
    torch.cuda.synchronize()
    assert torch.all(x == 0)
