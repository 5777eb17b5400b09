"""GPU parity of the dispatch into the grouped layouts and of the standalone
combine, through the C ABI, against the oracle.

Dispatch is byte and index work, so it must match bit for bit: row counts,
m_indices / masked_m, flat_to_row, the drop count, and every row the layout
defines (rows the contract leaves unwritten are not compared).  The chains
dispatch -> grouped layer -> combine are floating point and are held to the
layer tolerance (tests/tolerance.py).
"""

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import gen as G
from tests.gpu_util import banner, dev, dev_bf16, host, host_bf16
from tests.tolerance import check_close

pytestmark = pytest.mark.gpu

C = None


def setup_module(module):
    global C
    from quantized_moe_amd import chord
    C = chord
    banner(f"dispatch tests: library {C.version()}")


def routing_case(seed, T, H, E_g, k, skew=None):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = G.draw_activations(rng, T, H) if T else np.zeros((0, H), np.uint16)
    if T == 0:
        return x, np.zeros((0, k), np.int32), np.zeros((0, k), np.float32)
    if skew is None:
        ids, w = G.draw_routing(rng, T, E_g, k)
    else:   # a few hot experts: k distinct picks with probability ~ skew
        p = np.asarray(skew, np.float64)
        p /= p.sum()
        ids = np.stack([rng.choice(E_g, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
        w = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
        w /= w.sum(axis=1, keepdims=True)
    return x, ids, w


def dev_ids(ids):
    return dev(ids) if ids.shape[0] else torch.zeros(ids.shape, dtype=torch.int32, device="cuda")


def dev_x(x):
    return dev_bf16(x) if x.shape[0] else torch.zeros(x.shape, dtype=torch.bfloat16, device="cuda")


CONTIG_CASES = [
    # seed, T, H, E_g, E_l, k, expert_begin
    (1, 90, 200, 12, 6, 3, 0),          # H not a multiple of 256 bf16: ragged row copy
    (2, 64, 7168, 384, 48, 8, 96),      # decode EP share of another rank
    (3, 8192, 7168, 384, 48, 8, 0),     # prefill EP share: multi-workgroup alignment
    (4, 300, 64, 1024, 700, 4, 5),      # more than 512 local experts
    (5, 40, 256, 16, 4, 2, 100),        # no local expert at all
    (6, 0, 256, 8, 8, 2, 0),            # no tokens
]


@pytest.mark.parametrize("seed,T,H,E_g,E_l,k,eb", CONTIG_CASES)
def test_dispatch_contiguous_bit_exact(seed, T, H, E_g, E_l, k, eb):
    banner(f"dispatch contiguous T={T} H={H} E_g={E_g} E_l={E_l} k={k} eb={eb}")
    x, ids, _ = routing_case(seed, T, H, E_g, k)
    max_rows = C.chord_moe_dispatch_contiguous_rows(T, k, E_l)
    # poison the outputs so unwritten entries cannot pass by accident
    a = torch.full((max_rows, H), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    m_idx = torch.full((max_rows,), 99, dtype=torch.int32, device="cuda")
    f2r = torch.full((T * k,), 99, dtype=torch.int32, device="cuda")
    nrows = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    C.chord_moe_dispatch_contiguous(dev_x(x), dev_ids(ids), eb, E_l, max_rows,
                                    out=(a, m_idx, f2r, nrows))
    torch.cuda.synchronize()
    ra, rm, rf, rn = oracle.dispatch_contiguous(x, ids, eb, E_l, max_rows)
    n = int(host(nrows)[0])
    assert n == rn
    assert np.array_equal(host(m_idx), rm)
    assert np.array_equal(host(f2r), rf)
    assert np.array_equal(host_bf16(a[:n]), ra[:n])


def test_dispatch_contiguous_reuses_buffers_across_calls():
    """A second, smaller routing into the same buffers and workspace: the
    outputs follow the new routing only (row count, m_indices tail, slots)."""
    banner("dispatch contiguous: two calls, shared buffers")
    T0, H, E_g, E_l, k = 200, 256, 16, 8, 4
    max_rows = C.chord_moe_dispatch_contiguous_rows(T0, k, E_l)
    ws = torch.empty(C.chord_moe_dispatch_workspace_bytes(C.MODE_CONTIGUOUS, T0, k, E_l),
                     dtype=torch.uint8, device="cuda")
    a = torch.empty((max_rows, H), dtype=torch.bfloat16, device="cuda")
    m_idx = torch.empty(max_rows, dtype=torch.int32, device="cuda")
    f2r_big = torch.empty(T0 * k, dtype=torch.int32, device="cuda")
    nrows = torch.empty(1, dtype=torch.int32, device="cuda")
    for seed, T in ((61, T0), (62, 50)):
        x, ids, _ = routing_case(seed, T, H, E_g, k)
        f2r = f2r_big[:T * k]
        C.chord_moe_dispatch_contiguous(dev_x(x), dev_ids(ids), 0, E_l, max_rows,
                                        out=(a, m_idx, f2r, nrows), workspace=ws)
        torch.cuda.synchronize()
        ra, rm, rf, rn = oracle.dispatch_contiguous(x, ids, 0, E_l, max_rows)
        n = int(host(nrows)[0])
        assert n == rn
        assert np.array_equal(host(m_idx), rm)
        assert np.array_equal(host(f2r), rf)
        assert np.array_equal(host_bf16(a[:n]), ra[:n])


MASKED_CASES = [
    # seed, T, H, E_g, E_l, k, expert_begin, max_m, skew
    (11, 90, 200, 12, 6, 3, 0, 16, None),            # ~22 slots per expert: drops
    (12, 64, 7168, 384, 48, 8, 96, 64, None),        # decode EP share
    (13, 256, 512, 8, 8, 2, 0, 48, [40, 20, 10, 5, 3, 2, 0, 0]),  # hot experts, two empty
    (14, 8192, 7168, 384, 48, 8, 0, 160, None),      # prefill-sized routing, about half drop
    (15, 40, 256, 16, 4, 2, 100, 8, None),           # no local expert
    (16, 0, 256, 8, 8, 2, 0, 8, None),               # no tokens
]


@pytest.mark.parametrize("seed,T,H,E_g,E_l,k,eb,max_m,skew", MASKED_CASES)
def test_dispatch_masked_bit_exact(seed, T, H, E_g, E_l, k, eb, max_m, skew):
    banner(f"dispatch masked T={T} H={H} E_g={E_g} E_l={E_l} k={k} eb={eb} max_m={max_m}")
    x, ids, _ = routing_case(seed, T, H, E_g, k, skew)
    a3 = torch.full((E_l, max_m, H), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    mm = torch.full((E_l,), 99, dtype=torch.int32, device="cuda")
    f2r = torch.full((T * k,), 99, dtype=torch.int32, device="cuda")
    dropped = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    C.chord_moe_dispatch_masked(dev_x(x), dev_ids(ids), eb, E_l, max_m,
                                out=(a3, mm, f2r, dropped))
    torch.cuda.synchronize()
    ra3, rmm, rf, rd = oracle.dispatch_masked(x, ids, eb, E_l, max_m)
    if skew is not None:
        assert rd > 0 and (rmm == 0).sum() == 2
    assert int(host(dropped)[0]) == rd
    assert np.array_equal(host(mm), rmm)
    assert np.array_equal(host(f2r), rf)
    got = host_bf16(a3)
    for e in range(E_l):
        assert np.array_equal(got[e, :rmm[e]], ra3[e, :rmm[e]]), f"expert {e}"


def test_dispatch_contiguous_layer_combine_matches_the_layer():
    """dispatch -> grouped contiguous layer (with its token combine) equals the
    MoE layer's definition on the same routing."""
    from quantized_moe_amd.moe import W4A16MoE
    banner("dispatch contiguous -> grouped layer -> combine")
    rng = np.random.Generator(np.random.PCG64(41))
    T, H, I, E_g, E_l, k, eb = 120, 256, 128, 12, 6, 3, 3
    x = G.draw_activations(rng, T, H)
    ids, w = G.draw_routing(rng, T, E_g, k)
    q13, s13 = G.draw_weights(rng, E_l, 2 * I, H, scale_mult=(256.0 / H) ** 0.5)
    q2, s2 = G.draw_weights(rng, E_l, H, I, scale_mult=(256.0 / I) ** 0.5)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2), mode=C.MODE_CONTIGUOUS)
    a, m_idx, f2r, _ = C.chord_moe_dispatch_contiguous(dev_bf16(x), dev(ids), eb, E_l)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    layer.contiguous(a, m_idx, T * k * E_l // E_g, flat_to_row=f2r, topk_weights=dev(w),
                     out_tokens=out, flags=C.FLAG_VALIDATE)
    torch.cuda.synchronize()
    check_close(host_bf16(out), oracle.moe_layer(x, ids, w, q13, s13, q2, s2, eb),
                "dispatch + contiguous layer")


def test_dispatch_masked_layer_combine_matches_the_oracle_chain():
    """dispatch -> grouped masked layer -> standalone combine, with dropped
    slots, against the oracle's dispatch, masked layer and row combine."""
    from quantized_moe_amd.moe import W4A16MoE
    banner("dispatch masked -> grouped layer -> combine")
    T, H, I, E, k, max_m = 200, 256, 128, 8, 2, 40
    x, ids, w = routing_case(42, T, H, E, k, [30, 20, 10, 5, 3, 2, 1, 1])
    rng = np.random.Generator(np.random.PCG64(43))
    q13, s13 = G.draw_weights(rng, E, 2 * I, H, scale_mult=(256.0 / H) ** 0.5)
    q2, s2 = G.draw_weights(rng, E, H, I, scale_mult=(256.0 / I) ** 0.5)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2), mode=C.MODE_MASKED)
    a3, mm, f2r, dropped = C.chord_moe_dispatch_masked(dev_bf16(x), dev(ids), 0, E, max_m)
    rows = layer.masked(a3, mm, T * k // E, flags=C.FLAG_VALIDATE)
    out = C.chord_moe_combine(rows, f2r, dev(w))
    torch.cuda.synchronize()
    ra3, rmm, rf, rd = oracle.dispatch_masked(x, ids, 0, E, max_m)
    assert rd > 0 and int(host(dropped)[0]) == rd
    ref_rows = oracle.grouped_masked(ra3, rmm, q13, s13, q2, s2)
    ref = oracle.combine_rows(ref_rows, rf, w, H)
    check_close(host_bf16(out), ref, "dispatch + masked layer + combine")


@pytest.mark.parametrize("T,k,H,n_rows", [
    (77, 5, 72, 50),          # fewer waves than SIMDs: all slots in one batch
    (1100, 5, 72, 50),        # more waves: slots in batches of two
    (40, 5, 7168, 18800),     # row buffer above 256 MB (non-temporal loads), few waves
    (1100, 5, 7168, 18800),   # row buffer above 256 MB, more waves
])
def test_combine_is_exact_on_representable_sums(T, k, H, n_rows):
    """The standalone combine on small-integer rows and power-of-two weights:
    every product and partial sum is exact in fp32, so the output must be the
    exact weighted sum rounded once to bf16, bit for bit.  Slots mapped to -1
    or past n_rows are left out; a token with no slot gets 0."""
    banner(f"combine: exact sums T={T} k={k} H={H} n_rows={n_rows}")
    rng = np.random.default_rng(44)
    f2r = rng.integers(-1, n_rows + 3, T * k).astype(np.int32)
    f2r[:k] = -1                                          # token 0: no slot
    used = np.unique(f2r[(f2r >= 0) & (f2r < n_rows)])
    vals = rng.integers(-8, 9, (used.size, H)).astype(np.float32)   # rows in `used` order
    rows_bits = np.zeros((n_rows, H), np.uint16)
    rows_bits[used] = oracle.f32_to_bf16(vals)
    w = (2.0 ** rng.integers(-3, 2, (T, k))).astype(np.float32)
    out = C.chord_moe_combine(dev_bf16(rows_bits), dev(f2r), dev(w))
    torch.cuda.synchronize()
    exact = np.zeros((T, H), np.float64)
    for t in range(T):
        for j in range(k):
            r = f2r[t * k + j]
            if 0 <= r < n_rows:
                exact[t] += float(w[t, j]) * vals[np.searchsorted(used, r)]
    assert np.array_equal(host_bf16(out), oracle.f32_to_bf16(exact.astype(np.float32)))
