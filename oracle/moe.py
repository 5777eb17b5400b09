"""CPU oracle for the W4A16 mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP path.

Sources (the pages are cited by title and section):
  [Novita]  "vLLM x Novita AI: Chord W4A16 INT4 MoE Kernel für Kimi K2.x"
            (novita.ai/de blog).
  [aihirek] "A Novita AI új INT4 MoE-kernelt nyílt forráskódúvá tett a Kimi
            K2.x-hez" (aihirek.info).
  [picx]    "vLLM and Novita AI Announce Chord, an INT4 MoE Backend for Kimi
            K2.x" (picx.dev news).
  [prism]   INT4 vs NVFP4 video transcript (prism.simon-ai.net).

What the layer computes (the plain MoE-FFN definition; the pages' kernels reach
it up to rounding order).  For token t and routing slot j whose expert e is
local:

    W[e,n,k] = bf16_rne((q[e,n,k] - 8) * s[e,n,k // 32])            (dequant)
    g, u     = W1_e x_t, W3_e x_t      with W13_e = [W1_e ; W3_e]    (gate_up)
    h        = bf16_rne(silu(g) * u)                                 (act)
    y_tj     = W2_e h                                                (down)
    out[t]   = bf16_rne(sum_j w[t,j] * y_tj)   (ascending j, local j only)

Precision: the pages fix the bf16/uint4 operand formats, the bf16 rounding of
the dequantised weight ([Novita] §"H200 und Blackwell indexierter Decode": the
fused subtract-then-scale keeps the unfused bf16 rounding order), the 16-bit
activation operand of the down GEMM (W4A16, [prism]) and the bf16 output.  They
leave the accumulation precision open; the oracle accumulates in fp64.

Pins: every function here is pinned in ``tests/test_oracle_pins.py`` against
brute force, closed forms and library routines (see that file's header).
"""

from __future__ import annotations

import numpy as np

GROUP = 32
ZERO_POINT = 8


# ----------------------------------------------------------------------------
# bf16 helpers (round-to-nearest-even, written out)
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Raw bf16 bits (uint16) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits with a single round-to-nearest-even.

    bf16 has 8 significant bits and fp32's exponent range; below 2^-126 the
    quantum is fixed at 2^-133 (subnormals).  Overflow rounds to +-inf.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    fin = np.isfinite(v)
    x = v[fin]
    _, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(x / q) * q                   # rint = round half to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    out[fin] = r
    out[~fin] = v[~fin]
    # The rounded value is exactly representable in fp32 (and in bf16).
    b = out.astype(np.float32).view(np.uint32)
    nan = np.isnan(out)
    res = (b >> 16).astype(np.uint16)
    res[nan] = 0x7FC0
    return res


def f32_to_bf16(v: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round-to-nearest-even on the raw bits."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(v, dtype=np.float32))
    r[nan] = 0x7FC0
    return r


# ----------------------------------------------------------------------------
# uint4 codes and dequantisation
# ----------------------------------------------------------------------------

def unpack_codes(qweight: np.ndarray) -> np.ndarray:
    """int32 words [..., K/8] -> uint4 codes [..., K].

    Code k of a row is bits 4*(k%8)..4*(k%8)+3 of word k//8 (low nibble first,
    8 codes per int32 along K: the packing stated for the tiny workload).
    """
    w = np.asarray(qweight).view(np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    codes = (w[..., None] >> shifts) & np.uint32(0xF)
    return codes.reshape(*w.shape[:-1], w.shape[-1] * 8).astype(np.uint8)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Inverse of ``unpack_codes``: uint4 codes [..., K] -> int32 words [..., K/8]."""
    c = np.asarray(codes, dtype=np.uint32)
    K = c.shape[-1]
    assert K % 8 == 0 and int(c.max(initial=0)) < 16
    c = c.reshape(*c.shape[:-1], K // 8, 8)
    w = np.zeros(c.shape[:-1], dtype=np.uint32)
    for i in range(8):
        w |= c[..., i] << np.uint32(4 * i)
    return w.view(np.int32)


def dequant(qweight: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W4A16 dequantisation -> bf16 bits [..., N, K].

    ``(q - 8) * s`` for the group of 32 along K that k falls in, then one
    round-to-nearest-even to bf16 ([Novita] §"H200 und Blackwell indexierter
    Decode": subtract-then-scale with the unfused bf16 rounding order; zero
    point 8 for unsigned 4-bit codes; groups of 32 with bf16 scales, [picx]).
    """
    q = unpack_codes(qweight).astype(np.float64) - ZERO_POINT
    s = bf16_to_f64(scales)
    K = q.shape[-1]
    assert s.shape[-1] * GROUP == K, (s.shape, K)
    s_full = np.repeat(s, GROUP, axis=-1)
    return f64_to_bf16(q * s_full)


def dequant_f64(qweight: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return bf16_to_f64(dequant(qweight, scales))


# ----------------------------------------------------------------------------
# expert MLP and the layer
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)), fp64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_mlp(xrows: np.ndarray, w13: np.ndarray, w2: np.ndarray,
               unfused: bool = False) -> np.ndarray:
    """One expert on a set of rows (all fp64 values of bf16 numbers).

    xrows [R,H], w13 [2I,H] (gate rows first, then up rows), w2 [H,I].
    Returns y [R,H] fp64 (not rounded).  ``unfused=True`` rounds g, u and y to
    bf16 as separate kernels with bf16 outputs would.
    """
    I = w13.shape[0] // 2
    gu = xrows @ w13.T                       # [R, 2I]
    g, u = gu[:, :I], gu[:, I:]
    if unfused:
        g, u = bf16_to_f64(f64_to_bf16(g)), bf16_to_f64(f64_to_bf16(u))
    h = bf16_to_f64(f64_to_bf16(silu(g) * u))
    y = h @ w2.T
    if unfused:
        y = bf16_to_f64(f64_to_bf16(y))
    return y


def routed_y(x_bits, topk_ids, q13, s13, q2, s2, expert_begin, tokens=None,
             unfused=False):
    """y for every (token, slot) pair with a local expert.

    Returns ``dict[(t, j)] -> y fp64 [H]`` over ``tokens`` (default: all).
    Dequantises each needed expert once.
    """
    T, k = topk_ids.shape
    E_l = q13.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    x = bf16_to_f64(x_bits)
    pairs = {}
    for t in tokens:
        for j in range(k):
            e = int(topk_ids[t, j]) - expert_begin
            if 0 <= e < E_l:
                pairs.setdefault(e, []).append((int(t), j))
    ys = {}
    for e in sorted(pairs):
        w13 = dequant_f64(q13[e], s13[e])
        w2 = dequant_f64(q2[e], s2[e])
        rows = pairs[e]
        xr = x[[t for t, _ in rows]]
        y = expert_mlp(xr, w13, w2, unfused=unfused)
        for i, tj in enumerate(rows):
            ys[tj] = y[i]
    return ys


def combine(ys: dict, topk_ids, topk_weights, expert_begin, E_l, H, tokens):
    """out[t] = bf16_rne(sum over local j, ascending, of w[t,j] * y_tj); 0 if none."""
    out = np.zeros((len(tokens), H), dtype=np.float64)
    for i, t in enumerate(tokens):
        acc = np.zeros(H, dtype=np.float64)
        for j in range(topk_ids.shape[1]):
            e = int(topk_ids[t, j]) - expert_begin
            if 0 <= e < E_l:
                acc = acc + np.float64(topk_weights[t, j]) * ys[(int(t), j)]
        out[i] = acc
    return f64_to_bf16(out)


def moe_layer(x_bits, topk_ids, topk_weights, q13, s13, q2, s2, expert_begin=0,
              tokens=None, unfused=False):
    """The W4A16 MoE layer output (bf16 bits) for ``tokens`` (default all)."""
    T = topk_ids.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    H = x_bits.shape[1]
    ys = routed_y(x_bits, topk_ids, q13, s13, q2, s2, expert_begin, tokens, unfused)
    return combine(ys, topk_ids, topk_weights, expert_begin, q13.shape[0], H, tokens)


# ----------------------------------------------------------------------------
# routing alignment (indexed layout)
# ----------------------------------------------------------------------------

def moe_align(topk_ids: np.ndarray, expert_begin: int, E_l: int, block_m: int,
              max_padded: int):
    """Per-expert alignment of routed slots for the indexed layout.

    The indexed family consumes ``sorted_ids / expert_ids /
    num_tokens_padded``; activations stay unpadded and the index list carries
    a padding sentinel ([Novita] §"Zwei Kernel-Familien" and Abb. 3; [aihirek]
    §"Két külön kernelcsalád").  Oversize buffers are allowed ([Novita]
    §"vLLM-Integration").  Readings where the pages are silent: entries in a
    segment keep ascending flat index ``i = t*k + j``; the sentinel is ``T*k``;
    a zero-count expert gets no block; ``expert_ids`` holds the local expert
    index (0..E_l-1) and -1 for blocks past the padded total.

    Returns ``(sorted_ids int32 [max_padded], expert_ids int32
    [ceil(max_padded/block_m)], num_tokens_post_padded int)``.
    """
    T, k = topk_ids.shape
    n = T * k
    sentinel = n
    flat = topk_ids.reshape(-1).astype(np.int64) - expert_begin
    # 1. count the local entries per expert
    counts = [0] * E_l
    for i in range(n):
        if 0 <= flat[i] < E_l:
            counts[int(flat[i])] += 1
    # 2. pad each count to a multiple of block_m
    padded = [((c + block_m - 1) // block_m) * block_m for c in counts]
    total = sum(padded)
    assert max_padded >= total, "buffer smaller than the padded total"
    n_blocks = (max_padded + block_m - 1) // block_m
    sorted_ids = np.full(max_padded, sentinel, dtype=np.int32)
    expert_ids = np.full(n_blocks, -1, dtype=np.int32)
    # 3. segments in ascending expert order, entries in ascending flat index
    start = 0
    for e in range(E_l):
        members = [i for i in range(n) if flat[i] == e]
        sorted_ids[start:start + len(members)] = members
        for b in range(start // block_m, (start + padded[e]) // block_m):
            expert_ids[b] = e
        start += padded[e]
    return sorted_ids, expert_ids, total


def layer_from_alignment(x_bits, topk_ids, topk_weights, q13, s13, q2, s2,
                         expert_begin, sorted_ids, expert_ids, ntpp, block_m):
    """The layer evaluated block by block through the alignment tensors
    (used to pin that the indexed encoding reproduces the definition)."""
    T, k = topk_ids.shape
    H = x_bits.shape[1]
    x = bf16_to_f64(x_bits)
    ys = {}
    for b in range(ntpp // block_m):
        e = int(expert_ids[b])
        ids = [int(i) for i in sorted_ids[b * block_m:(b + 1) * block_m] if i < T * k]
        if not ids:
            continue
        w13 = dequant_f64(q13[e], s13[e])
        w2 = dequant_f64(q2[e], s2[e])
        y = expert_mlp(x[[i // k for i in ids]], w13, w2)
        for r, i in enumerate(ids):
            ys[(i // k, i % k)] = y[r]
    return combine(ys, topk_ids, topk_weights, expert_begin, q13.shape[0], H, np.arange(T))


# ----------------------------------------------------------------------------
# grouped layouts
# ----------------------------------------------------------------------------

def grouped_contiguous(a_bits, m_indices, q13, s13, q2, s2, row_weights=None,
                       rows=None):
    """Contiguous grouped layout: rows concatenated per expert in 128-row
    segments, ``m_indices`` gives each row's local expert, -1 marks padding
    ([Novita] §"Gruppierte SM90-Kernel", Abb. 3).  Output per row: bf16 of
    ``y`` (times ``row_weights`` if given); padding rows are left 0 here (the
    entry point leaves them unspecified).  ``rows`` restricts the computed rows.
    """
    M, H = a_bits.shape
    rows = np.arange(M) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), H), dtype=np.uint16)
    x = bf16_to_f64(a_bits)
    by_e = {}
    for i, r in enumerate(rows):
        e = int(m_indices[r])
        if e >= 0:
            by_e.setdefault(e, []).append((i, int(r)))
    for e in sorted(by_e):
        w13 = dequant_f64(q13[e], s13[e])
        w2 = dequant_f64(q2[e], s2[e])
        idx = by_e[e]
        y = expert_mlp(x[[r for _, r in idx]], w13, w2)
        if row_weights is not None:
            y = y * np.asarray(row_weights, dtype=np.float64)[[r for _, r in idx]][:, None]
        out[[i for i, _ in idx]] = f64_to_bf16(y)
    return out


def grouped_masked(a3_bits, masked_m, q13, s13, q2, s2, row_weights=None):
    """Masked grouped layout: a fixed budget of ``max_m`` rows per expert,
    ``masked_m[e]`` valid ([Novita] §"Gruppierte SM90-Kernel", Abb. 3).  The
    output is flat ``[E*max_m, H]``; rows past an expert's count are left 0
    here (unspecified at the entry point)."""
    E, max_m, H = a3_bits.shape
    out = np.zeros((E * max_m, H), dtype=np.uint16)
    for e in range(E):
        m = int(min(masked_m[e], max_m))
        if m <= 0:
            continue
        w13 = dequant_f64(q13[e], s13[e])
        w2 = dequant_f64(q2[e], s2[e])
        y = expert_mlp(bf16_to_f64(a3_bits[e, :m]), w13, w2)
        if row_weights is not None:
            y = y * np.asarray(row_weights, dtype=np.float64)[e, :m, None]
        out[e * max_m:e * max_m + m] = f64_to_bf16(y)
    return out


def combine_rows(out_rows_bits, flat_to_row, topk_weights, H):
    """Token outputs from per-row grouped outputs: out[t] = bf16(sum_j w * y_row)
    over the slots with a row (``flat_to_row >= 0``), ascending j."""
    T, k = topk_weights.shape
    y = bf16_to_f64(out_rows_bits)
    out = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            r = int(flat_to_row[t * k + j])
            if r >= 0:
                out[t] += np.float64(topk_weights[t, j]) * y[r]
    return f64_to_bf16(out)


# ----------------------------------------------------------------------------
# dispatch into the grouped layouts (the step before the grouped GEMMs)
# ----------------------------------------------------------------------------

def dispatch_contiguous(x_bits, topk_ids, expert_begin, E_l, max_rows, align=128):
    """Permute-gather of routed token rows into the contiguous grouped layout
    ([Novita] §"Gruppierte SM90-Kernel", Abb. 3: per-expert segments padded
    to the 128-row M-tile, ``m_indices`` marking each row's expert).  Readings:
    segments in ascending local expert, rows in ascending flat index
    ``t*k + j`` (the same stable order as the indexed alignment); padding rows
    and rows past the used total carry ``m_indices = -1`` and zero data;
    ``flat_to_row`` maps each local slot to its row and other slots to -1.

    Returns ``(a [max_rows, H] bf16 bits, m_indices int32 [max_rows],
    flat_to_row int32 [T*k], num_rows)``.
    """
    T, k = topk_ids.shape
    H = x_bits.shape[1]
    flat = topk_ids.reshape(-1).astype(np.int64) - expert_begin
    a = np.zeros((max_rows, H), dtype=np.uint16)
    m_indices = np.full(max_rows, -1, dtype=np.int32)
    flat_to_row = np.full(T * k, -1, dtype=np.int32)
    row = 0
    for e in range(E_l):
        members = [i for i in range(T * k) if flat[i] == e]
        if not members:
            continue
        for r, i in enumerate(members):
            m_indices[row + r] = e
            flat_to_row[i] = row + r
            a[row + r] = x_bits[i // k]
        row += ((len(members) + align - 1) // align) * align
    assert row <= max_rows, "buffer smaller than the padded total"
    return a, m_indices, flat_to_row, row


def dispatch_masked(x_bits, topk_ids, expert_begin, E_l, max_m):
    """Permute-gather into the masked grouped layout ([Novita]
    §"Gruppierte SM90-Kernel": a fixed ``[E, max_m, H]`` buffer with the valid
    row count ``masked_m[e]`` per expert).  Readings: rows of an expert keep
    ascending flat index; an expert with more than ``max_m`` slots keeps the
    first ``max_m`` and the others are dropped (their ``flat_to_row`` is -1, so
    a combine treats them like non-local slots) and counted; rows past
    ``masked_m[e]`` are left zero.

    Returns ``(a3 [E_l, max_m, H] bf16 bits, masked_m int32 [E_l],
    flat_to_row int32 [T*k] (row e*max_m + r, or -1), dropped)``.
    """
    T, k = topk_ids.shape
    H = x_bits.shape[1]
    flat = topk_ids.reshape(-1).astype(np.int64) - expert_begin
    a3 = np.zeros((E_l, max_m, H), dtype=np.uint16)
    masked_m = np.zeros(E_l, dtype=np.int32)
    flat_to_row = np.full(T * k, -1, dtype=np.int32)
    dropped = 0
    for e in range(E_l):
        members = [i for i in range(T * k) if flat[i] == e]
        for r, i in enumerate(members):
            if r < max_m:
                a3[e, r] = x_bits[i // k]
                flat_to_row[i] = e * max_m + r
            else:
                dropped += 1
        masked_m[e] = min(len(members), max_m)
    return a3, masked_m, flat_to_row, dropped
