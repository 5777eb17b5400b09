"""Seeded generators for MoE-layer inputs (numpy PCG64 streams).

Everything here is data synthesis: random draws, routing of synthetic logits,
and the integer re-layouts that an upstream dispatcher would hand to the
grouped entry points.  The layer's arithmetic lives elsewhere.

Conventions shared by every consumer:
  * bf16 tensors are numpy ``uint16`` arrays holding raw bf16 bits;
  * packed weights are ``int32`` words ``[E, N, K/8]``; code ``k`` of a row sits
    in bits ``4*(k % 8) .. 4*(k % 8)+3`` of word ``k // 8`` (low nibble first);
  * scales are bf16 ``[E, N, K/32]`` (one per group of 32 along K);
  * ``topk_ids`` are global expert ids, int32 ``[T, k]``; ``topk_weights`` fp32.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

GROUP = 32


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (torch's conversion) and return the raw bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def draw_activations(rng: np.random.Generator, rows: int, H: int) -> np.ndarray:
    """bf16 activations ~ N(0, 1), shape [rows, H]."""
    return bf16_bits_from_f32(rng.standard_normal((rows, H), dtype=np.float32))


def draw_weights(rng: np.random.Generator, E: int, N: int, K: int,
                 scale_lo: float = 0.005, scale_hi: float = 0.02,
                 scale_mult: float = 1.0):
    """uint4 codes (uniform 0..15, packed 8 per int32 along K) and bf16 scales.

    Returns ``(qweight int32 [E,N,K/8], scales uint16 [E,N,K/32])``.  Codes come
    from uniform random 32-bit words, so every nibble is uniform on 0..15.
    Scales are U(scale_lo, scale_hi) * scale_mult, rounded to bf16.
    """
    assert K % GROUP == 0
    words = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32)
    s = rng.uniform(scale_lo, scale_hi, size=(E, N, K // GROUP)).astype(np.float32)
    if scale_mult != 1.0:
        s = (s * np.float32(scale_mult)).astype(np.float32)
    return words.view(np.int32), bf16_bits_from_f32(s)


def draw_routing(rng: np.random.Generator, T: int, E_g: int, k: int,
                 dist: str = "normal"):
    """Synthetic router: fp32 softmax over E_g logits, top-k, renormalise.

    Ties in the top-k go to the lower expert index (stable sort).  Returns
    ``(topk_ids int32 [T,k], topk_weights fp32 [T,k])``.
    """
    if dist == "normal":
        logits = rng.standard_normal((T, E_g), dtype=np.float32)
    elif dist == "uniform":
        logits = rng.random((T, E_g), dtype=np.float32)
    else:
        raise ValueError(dist)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z, dtype=np.float32)
    p = (p / p.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :k].astype(np.int32)
    w = np.take_along_axis(p, ids, axis=1).astype(np.float32)
    w = (w / w.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(w)


def build_contiguous(topk_ids: np.ndarray, x_bits: np.ndarray, expert_begin: int,
                     E_l: int, align: int = 128):
    """Dispatch routed rows into the contiguous grouped layout.

    Segments in ascending local expert, each padded to a multiple of ``align``
    rows; inside a segment the rows keep ascending flat index ``t*k + j``.
    Returns ``(a [M,H] bf16 bits, m_indices int32 [M] (-1 = padding),
    flat_to_row int32 [T*k] (-1 = not local), valid_rows)``.
    """
    T, k = topk_ids.shape
    H = x_bits.shape[1]
    flat = topk_ids.reshape(-1).astype(np.int64) - expert_begin
    local = (flat >= 0) & (flat < E_l)
    counts = np.bincount(flat[local], minlength=E_l)
    padded = ((counts + align - 1) // align) * align
    M = int(padded.sum())
    m_indices = np.full(M, -1, dtype=np.int32)
    flat_to_row = np.full(T * k, -1, dtype=np.int32)
    a = np.zeros((M, H), dtype=np.uint16)
    start = 0
    for e in range(E_l):
        ids = np.nonzero(local & (flat == e))[0]  # ascending flat index
        n = ids.size
        m_indices[start:start + n] = e
        flat_to_row[ids] = np.arange(start, start + n, dtype=np.int32)
        a[start:start + n] = x_bits[ids // k]
        start += int(padded[e])
    return a, m_indices, flat_to_row, int(counts.sum())


def draw_masked(rng: np.random.Generator, E_l: int, max_m: int, H: int,
                zipf_s: float = 1.2):
    """Masked grouped layout with Zipf-skewed per-expert counts.

    Expert popularity is proportional to rank^-zipf_s over a seeded random
    ranking; the total is chosen so that the hottest expert's expected count
    equals ``max_m``; counts are a multinomial draw clipped at ``max_m``.
    Valid rows are N(0,1) bf16, the rest of the buffer is zero.
    Returns ``(a3 [E,max_m,H] bf16 bits, masked_m int32 [E], expected_m,
    n_clipped)``.
    """
    ranks = rng.permutation(E_l) + 1
    p = ranks.astype(np.float64) ** (-zipf_s)
    p /= p.sum()
    R = int(round(max_m / p.max()))
    m = rng.multinomial(R, p)
    n_clipped = int(np.maximum(m - max_m, 0).sum())
    m = np.minimum(m, max_m).astype(np.int32)
    a3 = np.zeros((E_l, max_m, H), dtype=np.uint16)
    for e in range(E_l):
        if m[e]:
            a3[e, :m[e]] = draw_activations(rng, int(m[e]), H)
    expected_m = max(1, int(math.ceil(int(m.sum()) / E_l)))
    return a3, m, expected_m, n_clipped


@dataclasses.dataclass
class MoEWorkload:
    """One synthetic layer invocation (host arrays)."""
    name: str
    T: int
    H: int
    I: int
    E_g: int
    E_l: int
    k: int
    expert_begin: int
    layout: str
    q13: np.ndarray          # int32 [E_l, 2I, H/8]   (gate rows 0..I-1, up rows I..2I-1)
    s13: np.ndarray          # bf16  [E_l, 2I, H/32]
    q2: np.ndarray           # int32 [E_l, H, I/8]
    s2: np.ndarray           # bf16  [E_l, H, I/32]
    x: Optional[np.ndarray] = None             # bf16 [T, H]
    topk_ids: Optional[np.ndarray] = None      # int32 [T, k]
    topk_weights: Optional[np.ndarray] = None  # fp32  [T, k]
    a3: Optional[np.ndarray] = None            # masked: bf16 [E_l, max_m, H]
    masked_m: Optional[np.ndarray] = None
    expected_m: Optional[int] = None
    max_m: Optional[int] = None
    n_clipped: int = 0


def make_workload(spec) -> MoEWorkload:
    """Draw a workload from a spec (see ``configs.py``) in the fixed order
    x, logits, q13, s13, q2, s2 (masked: a3 counts/rows first, then weights)."""
    rng = _rng(spec.seed)
    H, I, E_l = spec.H, spec.I, spec.E_l
    if spec.scale_normalize:
        m13, m2 = math.sqrt(256.0 / H), math.sqrt(256.0 / I)
    else:
        m13 = m2 = 1.0
    wl = dict(name=spec.name, T=spec.T, H=H, I=I, E_g=spec.E_g, E_l=E_l, k=spec.k,
              expert_begin=spec.expert_begin, layout=spec.layout)
    if spec.layout == "masked":
        a3, mm, em, nclip = draw_masked(rng, E_l, spec.max_m, H, spec.zipf_s)
        wl.update(a3=a3, masked_m=mm, expected_m=em, max_m=spec.max_m, n_clipped=nclip)
    else:
        wl["x"] = draw_activations(rng, spec.T, H)
        wl["topk_ids"], wl["topk_weights"] = draw_routing(rng, spec.T, spec.E_g, spec.k,
                                                          spec.logits)
    q13, s13 = draw_weights(rng, E_l, 2 * I, H, scale_mult=m13)
    q2, s2 = draw_weights(rng, E_l, H, I, scale_mult=m2)
    return MoEWorkload(q13=q13, s13=s13, q2=q2, s2=s2, **wl)
