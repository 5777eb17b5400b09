"""Parity tolerance for the bf16 layer output.

The layer output must match the oracle within max relative error 1e-2, with a
max absolute error of 2e-2 at unit-scale outputs.  Reading used here, element
by element over the valid rows:

    |gpu - ref| <= 2e-2 * rms(ref) + 1e-2 * |ref|

i.e. the absolute term is 2e-2 in units of the output's own scale.  On its
own, the largest error must also stay within 1e-2 of the largest reference
magnitude (max |gpu - ref| <= 1e-2 * max |ref|), the stricter whole-tensor
reading of "max relative error 1e-2".
"""

import numpy as np

RTOL = 1e-2
ATOL_UNIT = 2e-2


def bf16_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def check_close(gpu_bits, ref_bits, what="output"):
    g = bf16_to_f64(gpu_bits)
    r = bf16_to_f64(ref_bits)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values in GPU output"
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    bound = ATOL_UNIT * max(rms, 1e-30) + RTOL * np.abs(r)
    err = np.abs(g - r)
    bad = err > bound
    stats = dict(max_abs=float(err.max(initial=0.0)), rms_ref=rms,
                 max_rel_to_max=float(err.max(initial=0.0) / max(np.abs(r).max(initial=0.0), 1e-30)),
                 rel_fro=float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)),
                 n_bad=int(bad.sum()))
    assert not bad.any(), f"{what}: {stats}; first bad at {np.argwhere(bad)[:5].tolist()}"
    if r.size:
        assert stats["max_rel_to_max"] <= RTOL, f"{what}: {stats}"
    return stats
