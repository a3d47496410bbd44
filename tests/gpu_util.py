"""Helpers for the GPU tests: device buffers with guard bands, the parity bar.

Parity bar for bf16 attention outputs (a reading of "max-abs 1e-2 / max-rel
2e-2"): an element passes when |gpu - oracle| <= 1e-2 + 2e-2 * |oracle|.  A
pure absolute bound would reject correctly rounded outputs of magnitude >= 2
(bf16 half-ulp there is 0.0078, plus the error of rounding P to bf16), so the
relative term is part of the bar.  KV-cache bytes, untouched guard bands and
outputs that are exact copies are compared bit for bit.
"""
import sys

import numpy as np
import torch

ATOL = 1e-2
RTOL = 2e-2
SENTINEL = 0x7FC1  # a bf16 NaN pattern no N(0,1) draw produces
GUARD = 4096       # guard elements on each side (a multiple of 8: keeps 16-B alignment)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_f64(t):
    return t.detach().float().cpu().double().numpy()


def bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def guarded(n, fill=SENTINEL, device="cuda"):
    """A bf16 device buffer of n elements inside sentinel guard bands.

    Returns (view, whole) where view is the n-element slice."""
    whole = torch.full((n + 2 * GUARD,), fill - 65536 if fill > 32767 else fill,
                       dtype=torch.int16, device=device)
    view = whole[GUARD:GUARD + n].view(torch.bfloat16)
    return view, whole


def guards_intact(whole):
    g = whole.detach().cpu().numpy().view(np.uint16)
    return bool(np.all(g[:GUARD] == SENTINEL) and np.all(g[-GUARD:] == SENTINEL))


def assert_close(gpu, ref, what=""):
    """gpu: bf16/float tensor or array; ref: float64 array."""
    g = to_f64(gpu) if torch.is_tensor(gpu) else np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), "%s: non-finite outputs" % what
    err = np.abs(g - ref)
    bound = ATOL + RTOL * np.abs(ref)
    big = np.abs(ref) >= 1e-2
    max_abs = float(err.max()) if err.size else 0.0
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    bad = int(np.count_nonzero(err > bound))
    say("  %s: max_abs=%.3e max_rel=%.3e (elements %d, failing %d)"
        % (what, max_abs, max_rel, err.size, bad))
    assert bad == 0, "%s: %d elements outside |d| <= %g + %g|ref|; max_abs %.3e" % (
        what, bad, ATOL, RTOL, max_abs)
    return max_abs, max_rel
