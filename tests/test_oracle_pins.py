"""Pins for the CPU oracle, against things other than the oracle itself.

Each pin is chosen so that a plausible mistake in the oracle fails it:

  * bf16 rounding   -- exact rational rounding (fractions) and torch's fp32->bf16
                       conversion (library).
  * dequant         -- exhaustive: 16 codes x every finite bf16 scale, against
                       torch's conversion of the exact product; q == 8 gives 0.
  * nibble packing  -- hand-built words decode to known code sequences;
                       round trip.
  * SiLU            -- scipy's expit (library) and limits.
  * layer           -- closed forms with selection-matrix weights (catch a
                       transposed operand, swapped gate/up, a wrong scale group,
                       a wrong nibble, a wrong combine slot); the dense one-expert
                       case via numpy fp64 matmul; brute-force scalar fp64 loops
                       on tiny layers; zero weights give exactly zero.
  * combine         -- identical experts reproduce the single-expert MLP;
                       token permutation permutes outputs; routing weights sum
                       to 1.
  * alignment       -- brute-force sort and the invariants (each local slot once,
                       segments multiples of block_m, blocks belong to their
                       expert, padded total, sentinel fill).
  * layouts         -- indexed, contiguous and masked give the same per-slot
                       rows, bit for bit.
  * planted mistakes -- a mutated oracle fails the pins.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from oracle import moe as om
from moe_inputs import gen as G


# ----------------------------------------------------------------------------
# helpers written independently of the oracle
# ----------------------------------------------------------------------------

def bf16_round_exact(v: float) -> float:
    """Round an fp64 number to bf16 (8 significant bits, RNE) with exact
    rational arithmetic."""
    if v == 0 or math.isnan(v) or math.isinf(v):
        return v
    _, e = math.frexp(v)
    qe = max(e - 8, -133)
    r = round(Fraction(v) / Fraction(2) ** qe)  # Fraction.__round__: half to even
    out = float(r * Fraction(2) ** qe)
    if abs(out) >= 2.0 ** 128:
        return math.copysign(math.inf, out)
    return out


def bits_to_float(b: int) -> float:
    return float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])


def nibble(word: int, pos: int) -> int:
    """Code at position pos (0..7) of an int32 word, low nibble first, read
    from the word's hex spelling."""
    hexs = f"{word & 0xFFFFFFFF:08x}"
    return int(hexs[7 - pos], 16)


def torch_bf16_bits(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def brute_layer(x_bits, topk_ids, topk_w, q13, s13, q2, s2, expert_begin):
    """Scalar fp64 loops straight from the definition (tiny shapes only)."""
    T, H = x_bits.shape
    E, N13, _ = q13.shape
    I = N13 // 2
    k = topk_ids.shape[1]
    xv = [[bits_to_float(int(b)) for b in row] for row in x_bits]
    cache = {}

    def W(q, s, e, n, kk):
        key = (id(q), e, n, kk)
        if key not in cache:
            code = nibble(int(q[e, n, kk // 8]), kk % 8)
            sc = bits_to_float(int(s[e, n, kk // 32]))
            cache[key] = bf16_round_exact((code - 8) * sc)
        return cache[key]

    out = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        acc = [0.0] * H
        for j in range(k):
            e = int(topk_ids[t, j]) - expert_begin
            if not (0 <= e < E):
                continue
            gu = [sum(W(q13, s13, e, n, kk) * xv[t][kk] for kk in range(H)) for n in range(2 * I)]
            h = []
            for i in range(I):
                g, u = gu[i], gu[I + i]
                h.append(bf16_round_exact(g / (1.0 + math.exp(-g)) * u))
            for n in range(H):
                y = sum(W(q2, s2, e, n, i) * h[i] for i in range(I))
                acc[n] += float(topk_w[t, j]) * y
        out[t] = [bf16_round_exact(a) for a in acc]
    return out


def tiny_workload(seed, T=6, H=64, I=32, E_g=8, E_l=4, k=2, expert_begin=2):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = G.draw_activations(rng, T, H)
    ids, w = G.draw_routing(rng, T, E_g, k)
    q13, s13 = G.draw_weights(rng, E_l, 2 * I, H)
    q2, s2 = G.draw_weights(rng, E_l, H, I)
    return x, ids, w, q13, s13, q2, s2, expert_begin


# ----------------------------------------------------------------------------
# bf16
# ----------------------------------------------------------------------------

def test_f64_to_bf16_matches_exact_rational_rounding():
    rng = np.random.default_rng(123)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    # exact ties and near-ties around bf16 halfway points
    for b in rng.integers(0x0080, 0x7F00, 500):
        lo, hi = bits_to_float(int(b)), bits_to_float(int(b) + 1)
        mid = (lo + hi) / 2
        vals += [mid, np.nextafter(mid, 0), np.nextafter(mid, 1e300), -mid]
    vals += [0.0, -0.0, 1e-45, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 3.3e38, 3.4e38, 1e39]
    got = om.bf16_to_f64(om.f64_to_bf16(np.array(vals)))
    exp = np.array([bf16_round_exact(float(v)) for v in vals])
    assert np.array_equal(got, exp, equal_nan=True)


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    assert np.array_equal(om.f32_to_bf16(f), torch_bf16_bits(f))


# ----------------------------------------------------------------------------
# codes and dequant
# ----------------------------------------------------------------------------

def test_unpack_known_words():
    w = np.array([0x76543210, 0xFEDCBA98 - 2 ** 32], dtype=np.int64).astype(np.int32)
    c = om.unpack_codes(w)
    assert c.tolist() == list(range(8)) + list(range(8, 16))


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, (3, 5, 64), dtype=np.uint8)
    assert np.array_equal(om.unpack_codes(om.pack_codes(codes)), codes)
    words = rng.integers(-2 ** 31, 2 ** 31, (4, 9), dtype=np.int64).astype(np.int32)
    assert np.array_equal(om.pack_codes(om.unpack_codes(words)), words)
    # independent nibble reader agrees
    for r in range(4):
        for c in range(9):
            for p in range(8):
                assert om.unpack_codes(words)[r, c * 8 + p] == nibble(int(words[r, c]), p)


def test_dequant_exhaustive_all_codes_all_finite_bf16_scales():
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    sf = om.bf16_to_f64(all_bits)
    scales = all_bits[np.isfinite(sf)]
    n = scales.size
    # one row per code value; 32 columns share each scale
    for code in range(16):
        word = 0
        for p in range(8):
            word |= code << (4 * p)
        q = np.full((n, 4), np.uint32(word)).view(np.int32)      # K = 32
        s = scales.reshape(n, 1)
        got = om.dequant(q, s)                                   # [n, 32]
        assert np.all(got == got[:, :1])
        prod = ((code - 8) * om.bf16_to_f64(scales)).astype(np.float32)  # exact in fp32
        exp = torch_bf16_bits(prod)
        assert np.array_equal(got[:, 0], exp), code


def test_dequant_zero_point_gives_zero():
    q = np.full((2, 3, 4), 0x88888888 - 2 ** 32, dtype=np.int64).astype(np.int32)
    s = G.bf16_bits_from_f32(np.full((2, 3, 1), 0.37, np.float32))
    assert np.all(om.bf16_to_f64(om.dequant(q, s)) == 0.0)


def test_dequant_scale_group_indexing():
    # K = 96 -> three groups; scales 1, 2, 4 per group, every code 9 -> +1 * s
    q = np.full((1, 12), 0x99999999 - 2 ** 32, dtype=np.int64).astype(np.int32)
    s = G.bf16_bits_from_f32(np.array([[1.0, 2.0, 4.0]], np.float32))
    w = om.bf16_to_f64(om.dequant(q, s))
    assert w[0, :32].tolist() == [1.0] * 32
    assert w[0, 32:64].tolist() == [2.0] * 32
    assert w[0, 64:].tolist() == [4.0] * 32


# ----------------------------------------------------------------------------
# SiLU
# ----------------------------------------------------------------------------

def test_silu_against_library_and_limits():
    z = np.linspace(-30, 30, 2001)
    assert np.allclose(om.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert om.silu(np.array([0.0]))[0] == 0.0
    assert om.silu(np.array([800.0]))[0] == 800.0
    assert om.silu(np.array([-800.0]))[0] == 0.0


# ----------------------------------------------------------------------------
# layer: closed forms
# ----------------------------------------------------------------------------

def selection_weights(rng, E, N, K, mult_codes):
    """Codes with exactly one non-8 code per row (at a random column), scales
    powers of two per group.  Returns (q, s, col[E,N], val[E,N]) where the
    dequantised row n has value val at column col and 0 elsewhere."""
    codes = np.full((E, N, K), 8, dtype=np.uint8)
    col = np.stack([rng.permutation(K)[:N] if N <= K else rng.integers(0, K, N) for _ in range(E)])
    c = rng.choice(mult_codes, size=(E, N))
    for e in range(E):
        codes[e, np.arange(N), col[e]] = c[e]
    sexp = rng.integers(-3, 3, size=(E, N, K // 32))
    s = G.bf16_bits_from_f32((2.0 ** sexp).astype(np.float32))
    grp = col // 32
    sval = 2.0 ** np.take_along_axis(sexp, grp[..., None], axis=2)[..., 0]
    val = (c.astype(np.float64) - 8) * sval
    return om.pack_codes(codes), s, col, val


def closed_form_selection_layer(x_bits, ids, w, eb, c13, v13, c2, v2, I):
    """out[t,m] for selection weights, computed by indexing (no matmul)."""
    T, H = x_bits.shape
    x = om.bf16_to_f64(x_bits)
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j]) - eb
            if not (0 <= e < c13.shape[0]):
                continue
            g = v13[e, :I] * x[t, c13[e, :I]]
            u = v13[e, I:] * x[t, c13[e, I:]]
            h = np.array([bf16_round_exact(float(a)) for a in g / (1 + np.exp(-g)) * u])
            y = v2[e] * h[c2[e]]
            out[t] += float(w[t, j]) * y
    return np.array([[bf16_round_exact(float(a)) for a in row] for row in out])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_layer_closed_form_selection_weights(seed):
    rng = np.random.default_rng(seed)
    T, H, I, E_g, E_l, k, eb = 7, 96, 64, 6, 4, 3, 1
    x = G.draw_activations(rng, T, H)
    ids, w = G.draw_routing(rng, T, E_g, k)
    q13, s13, c13, v13 = selection_weights(rng, E_l, 2 * I, H, [0, 3, 5, 6, 7, 9, 11, 13, 15])
    q2, s2, c2, v2 = selection_weights(rng, E_l, H, I, [1, 4, 9, 10, 12, 15])
    got = om.bf16_to_f64(oracle.moe_layer(x, ids, w, q13, s13, q2, s2, eb))
    exp = closed_form_selection_layer(x, ids, w, eb, c13, v13, c2, v2, I)
    assert np.array_equal(got, exp)


def test_layer_dense_single_expert_matches_numpy_matmul():
    rng = np.random.default_rng(5)
    T, H, I = 9, 128, 64
    x = G.draw_activations(rng, T, H)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    q13, s13 = G.draw_weights(rng, 1, 2 * I, H)
    q2, s2 = G.draw_weights(rng, 1, H, I)
    got = om.bf16_to_f64(oracle.moe_layer(x, ids, w, q13, s13, q2, s2, 0))
    # library route: torch dequant of the exact product, numpy fp64 matmul
    def deq(q, s):
        codes = np.array([[[nibble(int(q[0, n, kk // 8]), kk % 8) for kk in range(q.shape[2] * 8)]
                           for n in range(q.shape[1])]], dtype=np.float64)[0]
        sf = np.repeat(om.bf16_to_f64(s[0]), 32, axis=1)
        return om.bf16_to_f64(torch_bf16_bits(((codes - 8) * sf).astype(np.float32)))
    W13, W2 = deq(q13, s13), deq(q2, s2)
    xf = om.bf16_to_f64(x)
    gu = np.matmul(xf, W13.T)
    g, u = gu[:, :I], gu[:, I:]
    h = np.array([[bf16_round_exact(float(a)) for a in r] for r in g * expit(g) * u])
    y = np.matmul(h, W2.T)
    exp = np.array([[bf16_round_exact(float(a)) for a in r] for r in y])
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("seed", [11, 12])
def test_layer_brute_force_tiny(seed):
    args = tiny_workload(seed)
    got = om.bf16_to_f64(oracle.moe_layer(*args))
    exp = brute_layer(*args)
    assert np.array_equal(got, exp)


@pytest.mark.slow
def test_layer_brute_force_tiny_workload_config():
    from moe_inputs.configs import TINY
    wl = G.make_workload(TINY)
    args = (wl.x, wl.topk_ids, wl.topk_weights, wl.q13, wl.s13, wl.q2, wl.s2, wl.expert_begin)
    tokens = [0, 5, 15]
    got = om.bf16_to_f64(oracle.moe_layer(*args, tokens=tokens))
    exp = brute_layer(wl.x[tokens], wl.topk_ids[tokens], wl.topk_weights[tokens], *args[3:])
    assert np.array_equal(got, exp)


def test_zero_weights_give_exact_zero():
    x, ids, w, q13, s13, q2, s2, eb = tiny_workload(3)
    q13z = np.full_like(q13, 0x88888888 - 2 ** 32)
    out = oracle.moe_layer(x, ids, w, q13z, s13, q2, s2, eb)
    assert np.all(om.bf16_to_f64(out) == 0.0)


# ----------------------------------------------------------------------------
# combine and routing
# ----------------------------------------------------------------------------

def test_routing_weights_sum_to_one():
    rng = np.random.default_rng(9)
    for dist in ("normal", "uniform"):
        ids, w = G.draw_routing(rng, 257, 384, 8, dist)
        assert np.allclose(w.sum(1), 1.0, atol=1e-6)
        assert np.all(np.diff(w, axis=1) <= 0)                   # descending
        assert all(len(set(r)) == 8 for r in ids.tolist())       # distinct experts


def test_identical_experts_reproduce_single_mlp():
    rng = np.random.default_rng(4)
    T, H, I, E, k = 5, 64, 32, 6, 3
    x = G.draw_activations(rng, T, H)
    ids, w = G.draw_routing(rng, T, E, k)
    q13, s13 = G.draw_weights(rng, 1, 2 * I, H)
    q2, s2 = G.draw_weights(rng, 1, H, I)
    rep = lambda a: np.repeat(a, E, axis=0)
    out = om.bf16_to_f64(oracle.moe_layer(x, ids, w, rep(q13), rep(s13), rep(q2), rep(s2), 0))
    single = om.bf16_to_f64(oracle.moe_layer(x, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32),
                                             q13, s13, q2, s2, 0))
    # sum_j w_j y = y * (sum_j w_j) with sum_j w_j = 1 up to fp32 rounding: one bf16 ulp at most
    assert np.all(np.abs(out - single) <= np.abs(single) * 2.0 ** -7 + 1e-30)


def test_token_permutation_permutes_output():
    x, ids, w, q13, s13, q2, s2, eb = tiny_workload(6, T=9)
    perm = np.random.default_rng(0).permutation(9)
    a = oracle.moe_layer(x, ids, w, q13, s13, q2, s2, eb)
    b = oracle.moe_layer(x[perm], ids[perm], w[perm], q13, s13, q2, s2, eb)
    assert np.array_equal(a[perm], b)


def test_nonlocal_tokens_give_zero_rows():
    x, ids, w, q13, s13, q2, s2, eb = tiny_workload(8, T=8, E_g=16, E_l=2, expert_begin=0)
    out = om.bf16_to_f64(oracle.moe_layer(x, ids, w, q13, s13, q2, s2, eb))
    none_local = ~np.any((ids >= 0) & (ids < 2), axis=1)
    assert np.all(out[none_local] == 0.0)


# ----------------------------------------------------------------------------
# alignment
# ----------------------------------------------------------------------------

def check_alignment_invariants(ids, eb, E_l, bm, sorted_ids, expert_ids, ntpp, max_padded):
    T, k = ids.shape
    flat = ids.reshape(-1) - eb
    local = np.nonzero((flat >= 0) & (flat < E_l))[0]
    valid = sorted_ids[sorted_ids < T * k]
    # each local slot exactly once, nothing else
    assert sorted(valid.tolist()) == local.tolist()
    assert np.all((sorted_ids == T * k) | (sorted_ids < T * k))
    counts = np.bincount(flat[local], minlength=E_l)
    assert ntpp == int((((counts + bm - 1) // bm) * bm).sum())
    assert ntpp % bm == 0
    assert np.all(sorted_ids[ntpp:] == T * k)
    nb = ntpp // bm
    assert np.all(expert_ids[nb:] == -1)
    assert len(expert_ids) == (max_padded + bm - 1) // bm
    # blocks belong to their expert, experts ascending, segments multiples of bm
    assert np.all(np.diff(expert_ids[:nb]) >= 0)
    for b in range(nb):
        blk = sorted_ids[b * bm:(b + 1) * bm]
        blk = blk[blk < T * k]
        assert blk.size > 0
        assert np.all(flat[blk] == expert_ids[b])
        assert np.all(np.diff(blk) > 0)


@pytest.mark.parametrize("T,k,E_g,E_l,eb,bm,extra", [
    (16, 2, 8, 8, 0, 16, 0), (64, 8, 384, 48, 0, 16, 7), (33, 8, 384, 384, 0, 8, 100),
    (1, 8, 384, 384, 0, 16, 0), (50, 4, 32, 8, 8, 32, 1), (0, 8, 384, 48, 0, 16, 0)])
def test_align_brute_force_and_invariants(T, k, E_g, E_l, eb, bm, extra):
    rng = np.random.default_rng(T + bm)
    ids, _ = G.draw_routing(rng, T, E_g, k) if T else (np.zeros((0, k), np.int32), None)
    max_padded = T * k + E_l * (bm - 1) + extra
    s, e, n = oracle.moe_align(ids, eb, E_l, bm, max_padded)
    # brute force: python sorted() on (expert, flat index), then pad
    pairs = sorted((int(ids.reshape(-1)[i]) - eb, i) for i in range(T * k)
                   if 0 <= int(ids.reshape(-1)[i]) - eb < E_l)
    exp = []
    for ex in range(E_l):
        seg = [i for (ee, i) in pairs if ee == ex]
        if seg:
            exp += seg + [T * k] * ((-len(seg)) % bm)
    assert n == len(exp)
    assert s[:n].tolist() == exp
    check_alignment_invariants(ids, eb, E_l, bm, s, e, n, max_padded)


def test_layer_from_alignment_equals_definition():
    x, ids, w, q13, s13, q2, s2, eb = tiny_workload(21, T=11)
    E_l, bm = q13.shape[0], 4
    s, e, n = oracle.moe_align(ids, eb, E_l, bm, ids.size + E_l * (bm - 1) + 5)
    a = oracle.layer_from_alignment(x, ids, w, q13, s13, q2, s2, eb, s, e, n, bm)
    b = oracle.moe_layer(x, ids, w, q13, s13, q2, s2, eb)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------
# layouts
# ----------------------------------------------------------------------------

def test_indexed_contiguous_masked_rows_agree():
    x, ids, w, q13, s13, q2, s2, eb = tiny_workload(31, T=10, E_l=4, E_g=6, k=3)
    E_l, H = q13.shape[0], x.shape[1]
    T, k = ids.shape
    ys = oracle.routed_y(x, ids, q13, s13, q2, s2, eb)
    a, m_idx, f2r, nvalid = G.build_contiguous(ids, x, eb, E_l, align=16)
    rows = oracle.grouped_contiguous(a, m_idx, q13, s13, q2, s2)
    assert len(ys) == nvalid
    for (t, j), y in ys.items():
        assert np.array_equal(rows[f2r[t * k + j]], om.f64_to_bf16(y))
    # masked: expert e's rows are its slots in ascending flat order
    max_m = 12
    a3 = np.zeros((E_l, max_m, H), np.uint16)
    mm = np.zeros(E_l, np.int32)
    where = {}
    for i in range(T * k):
        e = int(ids.reshape(-1)[i]) - eb
        if 0 <= e < E_l:
            a3[e, mm[e]] = x[i // k]
            where[(i // k, i % k)] = e * max_m + mm[e]
            mm[e] += 1
    out = oracle.grouped_masked(a3, mm, q13, s13, q2, s2)
    for tj, y in ys.items():
        assert np.array_equal(out[where[tj]], om.f64_to_bf16(y))
    # combining the contiguous rows equals the layer with y rounded to bf16
    comb = oracle.combine_rows(rows, f2r, w, H)
    ref = oracle.moe_layer(x, ids, w, q13, s13, q2, s2, eb)
    assert np.max(np.abs(om.bf16_to_f64(comb) - om.bf16_to_f64(ref))) <= \
        2 ** -7 * np.max(np.abs(om.bf16_to_f64(ref)))


def test_unfused_variant_within_tolerance():
    from tests.tolerance import check_close
    x, ids, w, q13, s13, q2, s2, eb = tiny_workload(41, T=12, H=256, I=128)
    a = oracle.moe_layer(x, ids, w, q13, s13, q2, s2, eb)
    b = oracle.moe_layer(x, ids, w, q13, s13, q2, s2, eb, unfused=True)
    check_close(b, a)


# ----------------------------------------------------------------------------
# planted mistakes: a mutated oracle must fail the pins above
# ----------------------------------------------------------------------------

def _selection_case():
    rng = np.random.default_rng(77)
    T, H, I, E_g, E_l, k, eb = 5, 64, 32, 4, 4, 2, 0
    x = G.draw_activations(rng, T, H)
    ids, w = G.draw_routing(rng, T, E_g, k)
    q13, s13, c13, v13 = selection_weights(rng, E_l, 2 * I, H, [3, 5, 7, 9, 13])
    q2, s2, c2, v2 = selection_weights(rng, E_l, H, I, [1, 4, 10, 12])
    exp = closed_form_selection_layer(x, ids, w, eb, c13, v13, c2, v2, I)
    return (x, ids, w, q13, s13, q2, s2, eb), exp


@pytest.mark.parametrize("mutation", ["zero_point", "swap_gate_up", "transpose_down",
                                      "nibble_order", "scale_group", "combine_slot"])
def test_planted_mistakes_fail_pins(monkeypatch, mutation):
    args, exp = _selection_case()
    if mutation == "zero_point":
        monkeypatch.setattr(om, "ZERO_POINT", 7)
    elif mutation == "swap_gate_up":
        orig = om.expert_mlp
        def bad(xr, w13, w2, unfused=False):
            I = w13.shape[0] // 2
            return orig(xr, np.concatenate([w13[I:], w13[:I]]), w2, unfused)
        monkeypatch.setattr(om, "expert_mlp", bad)
    elif mutation == "transpose_down":
        orig = om.expert_mlp
        def bad(xr, w13, w2, unfused=False):
            I = w13.shape[0] // 2
            w2b = w2.reshape(-1)[:w2.size].reshape(w2.shape[1], w2.shape[0]).T
            return orig(xr, w13, w2b, unfused)
        monkeypatch.setattr(om, "expert_mlp", bad)
    elif mutation == "nibble_order":
        orig = om.unpack_codes
        def bad(q):
            c = orig(q)
            return c.reshape(*c.shape[:-1], -1, 8)[..., ::-1].reshape(c.shape)
        monkeypatch.setattr(om, "unpack_codes", bad)
    elif mutation == "scale_group":
        orig = om.dequant
        def bad(q, s):
            return orig(q, np.roll(s, 1, axis=-1))
        monkeypatch.setattr(om, "dequant", bad)
    elif mutation == "combine_slot":
        orig = om.combine
        def bad(ys, ids, w, eb, E_l, H, tokens):
            return orig(ys, ids, w[:, ::-1].copy(), eb, E_l, H, tokens)
        monkeypatch.setattr(om, "combine", bad)
    got = om.bf16_to_f64(om.moe_layer(*args))
    assert not np.array_equal(got, exp)


# ----------------------------------------------------------------------------
# grouped layouts: per-row weights and the row subset
# ----------------------------------------------------------------------------

def brute_row(x_row_bits, e, q13, s13, q2, s2):
    """y of one row through expert e by scalar fp64 loops from the definition
    (dequant with exact rational rounding, gate rows first, h rounded to bf16).
    Returns the unrounded fp64 y [H]."""
    H = x_row_bits.shape[0]
    I = q13.shape[1] // 2
    xv = [bits_to_float(int(b)) for b in x_row_bits]

    def W(q, s, n, kk):
        code = nibble(int(q[e, n, kk // 8]), kk % 8)
        return bf16_round_exact((code - 8) * bits_to_float(int(s[e, n, kk // 32])))

    gu = [sum(W(q13, s13, n, kk) * xv[kk] for kk in range(H)) for n in range(2 * I)]
    h = [bf16_round_exact(gu[i] / (1.0 + math.exp(-gu[i])) * gu[I + i]) for i in range(I)]
    return [sum(W(q2, s2, n, i) * h[i] for i in range(I)) for n in range(H)]


def _row_weight_case():
    rng = np.random.default_rng(91)
    E, H, I = 3, 64, 32
    x, ids, _, q13, s13, q2, s2, eb = tiny_workload(92, T=9, H=H, I=I, E_g=3, E_l=E, k=2,
                                                    expert_begin=0)
    a, m_idx, _, _ = G.build_contiguous(ids, x, 0, E, align=8)
    # fp32 weights that are not powers of two, so rounding y before the
    # weight (double rounding) differs from rounding once after it
    rw = rng.uniform(0.1, 1.0, a.shape[0]).astype(np.float32)
    valid = np.nonzero(m_idx >= 0)[0]
    rows = rng.permutation(valid)[: max(4, valid.size // 2)]   # shuffled subset
    return a, m_idx, q13, s13, q2, s2, rw, rows


def _contiguous_row_pin_holds(fn):
    """fn = grouped_contiguous (or a mutation of it) against brute force:
    output i is row rows[i] of expert m_indices[rows[i]], times the weight of
    that absolute row, rounded to bf16 once."""
    a, m_idx, q13, s13, q2, s2, rw, rows = _row_weight_case()
    got = om.bf16_to_f64(fn(a, m_idx, q13, s13, q2, s2, row_weights=rw, rows=rows))
    if got.shape != (len(rows), a.shape[1]):
        return False
    for i, r in enumerate(rows):
        y = brute_row(a[r], int(m_idx[r]), q13, s13, q2, s2)
        exp = [bf16_round_exact(float(rw[r]) * v) for v in y]
        if not np.array_equal(got[i], np.array(exp)):
            return False
    return True


def test_contiguous_row_weights_and_row_subset_brute_force():
    assert _contiguous_row_pin_holds(oracle.grouped_contiguous)


def test_contiguous_row_subset_without_weights_brute_force():
    """rows= alone: each listed row (shuffled order) equals the brute-force
    y of that row, rounded once; unlisted rows are not in the output."""
    a, m_idx, q13, s13, q2, s2, _, rows = _row_weight_case()
    got = om.bf16_to_f64(oracle.grouped_contiguous(a, m_idx, q13, s13, q2, s2, rows=rows))
    assert got.shape == (len(rows), a.shape[1])
    for i, r in enumerate(rows):
        exp = [bf16_round_exact(v) for v in brute_row(a[r], int(m_idx[r]), q13, s13, q2, s2)]
        assert np.array_equal(got[i], np.array(exp))


def _masked_row_pin_holds(fn):
    rng = np.random.default_rng(93)
    E, max_m, H, I = 3, 5, 64, 32
    a3 = G.draw_activations(rng, E * max_m, H).reshape(E, max_m, H)
    mm = np.array([5, 0, 3], np.int32)
    q13, s13 = G.draw_weights(rng, E, 2 * I, H)
    q2, s2 = G.draw_weights(rng, E, H, I)
    rw = rng.uniform(0.1, 1.0, (E, max_m)).astype(np.float32)
    got = om.bf16_to_f64(fn(a3, mm, q13, s13, q2, s2, row_weights=rw))
    for e in range(E):
        for r in range(max_m):
            row = got[e * max_m + r]
            if r >= mm[e]:
                if not np.all(row == 0):           # the oracle leaves invalid rows 0
                    return False
                continue
            y = brute_row(a3[e, r], e, q13, s13, q2, s2)
            exp = [bf16_round_exact(float(rw[e, r]) * v) for v in y]
            if not np.array_equal(row, np.array(exp)):
                return False
    return True


def test_masked_row_weights_brute_force():
    assert _masked_row_pin_holds(oracle.grouped_masked)


def _mutated_contiguous(kind):
    orig = om.grouped_contiguous

    def by_position(a, m, q13, s13, q2, s2, row_weights=None, rows=None):
        # weight i of the subset taken for row rows[i]
        rw = np.array(row_weights, copy=True)
        rw[np.asarray(rows)] = np.asarray(row_weights)[: len(rows)]
        return orig(a, m, q13, s13, q2, s2, row_weights=rw, rows=rows)

    def after_rounding(a, m, q13, s13, q2, s2, row_weights=None, rows=None):
        y = orig(a, m, q13, s13, q2, s2, rows=rows)
        w = np.asarray(row_weights, dtype=np.float64)[np.asarray(rows)][:, None]
        return om.f64_to_bf16(om.bf16_to_f64(y) * w)

    def subset_ignored(a, m, q13, s13, q2, s2, row_weights=None, rows=None):
        return orig(a, m, q13, s13, q2, s2, row_weights=row_weights, rows=np.sort(rows))

    return {"by_position": by_position, "after_rounding": after_rounding,
            "subset_order": subset_ignored}[kind]


def _mutated_masked(kind):
    orig = om.grouped_masked

    def flat_index(a3, mm, q13, s13, q2, s2, row_weights=None):
        # weight of row r of expert e read as the (e + r)-th weight of a flat list
        E, max_m = np.asarray(row_weights).shape
        flat = np.asarray(row_weights).reshape(-1)
        rw = np.array([[flat[e + r] for r in range(max_m)] for e in range(E)], np.float32)
        return orig(a3, mm, q13, s13, q2, s2, row_weights=rw)

    def after_rounding(a3, mm, q13, s13, q2, s2, row_weights=None):
        y = om.bf16_to_f64(orig(a3, mm, q13, s13, q2, s2))
        w = np.asarray(row_weights, dtype=np.float64).reshape(-1)[:, None]
        return om.f64_to_bf16(y * w)

    return {"flat_index": flat_index, "after_rounding": after_rounding}[kind]


@pytest.mark.parametrize("kind", ["by_position", "after_rounding", "subset_order"])
def test_planted_row_weight_mistakes_fail_the_contiguous_pin(kind):
    assert not _contiguous_row_pin_holds(_mutated_contiguous(kind))


@pytest.mark.parametrize("kind", ["flat_index", "after_rounding"])
def test_planted_row_weight_mistakes_fail_the_masked_pin(kind):
    assert not _masked_row_pin_holds(_mutated_masked(kind))


# ----------------------------------------------------------------------------
# dispatch into the grouped layouts
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E_g,E_l,eb", [(30, 4, 16, 6, 3), (7, 8, 8, 8, 0), (50, 2, 64, 5, 60)])
def test_dispatch_contiguous_against_generator_and_invariants(T, k, E_g, E_l, eb):
    """Pinned against the input generator's independent builder, plus the
    layout's invariants (every local slot once, 128-row segments of one
    expert in ascending order, gathered rows equal the token rows)."""
    rng = np.random.default_rng(T * 100 + E_l)
    x = G.draw_activations(rng, T, 32)
    ids, _ = G.draw_routing(rng, T, E_g, k)
    a_g, m_g, f_g, _ = G.build_contiguous(ids, x, eb, E_l)
    M = a_g.shape[0]
    a, m, f, rows = om.dispatch_contiguous(x, ids, eb, E_l, M + 256)
    assert rows == M
    assert np.array_equal(a[:M], a_g) and np.array_equal(m[:M], m_g) and np.array_equal(f, f_g)
    assert (m[M:] == -1).all() and (a[M:] == 0).all()
    flat = ids.reshape(-1) - eb
    local = (flat >= 0) & (flat < E_l)
    assert sorted(f[local].tolist()) == sorted(set(f[local].tolist()))          # one row per slot
    assert (f[~local] == -1).all()
    for i in np.nonzero(local)[0]:
        assert m[f[i]] == flat[i] and np.array_equal(a[f[i]], x[i // k])
    for c in range(M // 128):                                                   # one expert per chunk
        vals = set(m[c * 128:(c + 1) * 128].tolist()) - {-1}
        assert len(vals) <= 1
    assert (np.diff(m[m >= 0]) >= 0).all()                                      # ascending experts


@pytest.mark.parametrize("max_m", [64, 3])
def test_dispatch_masked_brute_force(max_m):
    """Brute force over the slots: rank of a slot among its expert's slots in
    flat order decides its row; ranks >= max_m are dropped and counted."""
    rng = np.random.default_rng(5 + max_m)
    T, k, E_g, E_l, eb = 40, 4, 12, 5, 2
    x = G.draw_activations(rng, T, 16)
    ids, _ = G.draw_routing(rng, T, E_g, k)
    a3, mm, f, dropped = om.dispatch_masked(x, ids, eb, E_l, max_m)
    flat = (ids.reshape(-1) - eb).tolist()
    seen = [0] * E_l
    exp_drop = 0
    for i, e in enumerate(flat):
        if not 0 <= e < E_l:
            assert f[i] == -1
            continue
        r = seen[e]
        seen[e] += 1
        if r < max_m:
            assert f[i] == e * max_m + r and np.array_equal(a3[e, r], x[i // k])
        else:
            assert f[i] == -1
            exp_drop += 1
    assert dropped == exp_drop and mm.tolist() == [min(c, max_m) for c in seen]
    for e in range(E_l):
        assert (a3[e, mm[e]:] == 0).all()
    if max_m == 3:
        assert dropped > 0


def test_dispatch_then_grouped_layers_equal_the_definition():
    """Dispatch + grouped layer + row combine reproduce the layer exactly
    (fp64 oracle arithmetic in both; the grouped rows are bf16, so the
    reference combines bf16-rounded y) when nothing is dropped."""
    x, ids, w, q13, s13, q2, s2, eb = tiny_workload(11)
    T, k = ids.shape
    E_l = q13.shape[0]
    ys = om.routed_y(x, ids, q13, s13, q2, s2, eb)
    ys = {tj: om.bf16_to_f64(om.f64_to_bf16(y)) for tj, y in ys.items()}
    ref = om.combine(ys, ids, w, eb, E_l, x.shape[1], np.arange(T))
    a, m, f, rows = om.dispatch_contiguous(x, ids, eb, E_l, T * k + E_l * 128)
    yc = om.grouped_contiguous(a, m, q13, s13, q2, s2)
    assert np.array_equal(om.combine_rows(yc, f, w, x.shape[1]), ref)
    a3, mm, f3, dropped = om.dispatch_masked(x, ids, eb, E_l, T * k)
    assert dropped == 0
    ym = om.grouped_masked(a3, mm, q13, s13, q2, s2)
    assert np.array_equal(om.combine_rows(ym, f3, w, x.shape[1]), ref)
