"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Alignment tensors must match bit for bit; the bf16 layer output must match
within |gpu - ref| <= 2e-2 * rms(ref) + 1e-2 * |ref| (tests/tolerance.py).
The full-size workloads are covered by tests/test_gpu_full_size.py against
expected values the oracle wrote beforehand.
"""

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import gen as G
from moe_inputs.configs import TINY
from tests.gpu_util import banner, dev, dev_bf16, host, host_bf16
from tests.tolerance import check_close

pytestmark = pytest.mark.gpu

C = None


def setup_module(module):
    global C
    from quantized_moe_amd import chord
    C = chord
    banner(f"library {C.version()} on {torch.cuda.get_device_name(0)}")


def small_case(seed, T, H, I, E_g, E_l, k, expert_begin=0, logits="normal"):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = G.draw_activations(rng, T, H)
    ids, w = G.draw_routing(rng, T, E_g, k, logits)
    q13, s13 = G.draw_weights(rng, E_l, 2 * I, H, scale_mult=(256.0 / H) ** 0.5)
    q2, s2 = G.draw_weights(rng, E_l, H, I, scale_mult=(256.0 / I) ** 0.5)
    return x, ids, w, q13, s13, q2, s2, expert_begin


def run_indexed(x, ids, w, q13, s13, q2, s2, eb, E_g, bm=16, extra=0, override=None, flags=0,
                layer=None):
    from quantized_moe_amd.moe import W4A16MoE
    if layer is None:
        layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2))
    T, k = ids.shape
    ids_d = dev(ids)
    mp = C.chord_moe_align_max_padded(T, k, q13.shape[0], bm) + extra
    al = C.chord_moe_align(ids_d, eb, q13.shape[0], bm, max_padded=mp)
    out = layer.indexed(dev_bf16(x), ids_d, dev(w), expert_begin=eb, num_global_experts=E_g,
                        align=(*al, bm), override=override, flags=flags)
    torch.cuda.synchronize()
    return host_bf16(out), layer, al


# ---------------------------------------------------------------------------
# alignment: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E_g,E_l,eb,bm,extra", [
    (16, 2, 8, 8, 0, 16, 0),            # tiny layer
    (64, 8, 384, 48, 0, 16, 0),         # decode EP share
    (64, 8, 384, 48, 96, 32, 1000),     # another rank, oversize buffers
    (8192, 8, 384, 48, 0, 16, 0),       # prefill: multi-workgroup path
    (1, 8, 384, 384, 0, 16, 0),         # TP slice, one token
    (4096, 8, 384, 384, 0, 64, 33),     # TP slice, multi-workgroup
    (300, 4, 1024, 700, 5, 128, 7),     # more than 512 local experts
    (0, 8, 384, 48, 0, 16, 5),          # no tokens
])
def test_align_bit_exact(T, k, E_g, E_l, eb, bm, extra):
    banner(f"align T={T} k={k} E_g={E_g} E_l={E_l} eb={eb} bm={bm} extra={extra}")
    rng = np.random.default_rng(T * 7 + bm)
    ids = G.draw_routing(rng, T, E_g, k)[0] if T else np.zeros((0, k), np.int32)
    mp = C.chord_moe_align_max_padded(T, k, E_l, bm) + extra
    s, e, n = C.chord_moe_align(dev(ids) if T else torch.zeros((0, k), dtype=torch.int32, device="cuda"),
                                eb, E_l, bm, max_padded=mp)
    torch.cuda.synchronize()
    rs, re_, rn = oracle.moe_align(ids, eb, E_l, bm, mp)
    assert int(host(n)[0]) == rn
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(e), re_)


def test_align_deterministic_repeat():
    banner("align repeat determinism T=8192")
    rng = np.random.default_rng(3)
    ids = dev(G.draw_routing(rng, 8192, 384, 8, "uniform")[0])
    a = [host(t).copy() for t in C.chord_moe_align(ids, 0, 48, 16)]
    b = [host(t).copy() for t in C.chord_moe_align(ids, 0, 48, 16)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# indexed layer
# ---------------------------------------------------------------------------

def test_indexed_tiny_workload_full_output():
    wl = G.make_workload(TINY)
    banner(f"indexed {TINY.name}")
    got, _, _ = run_indexed(wl.x, wl.topk_ids, wl.topk_weights, wl.q13, wl.s13, wl.q2, wl.s2, 0,
                            wl.E_g, bm=16)
    ref = oracle.moe_layer(wl.x, wl.topk_ids, wl.topk_weights, wl.q13, wl.s13, wl.q2, wl.s2, 0)
    st = check_close(got, ref, TINY.name)
    banner(f"  {st}")


@pytest.mark.parametrize("T,H,I,E_g,E_l,k,eb", [
    (37, 256, 128, 16, 6, 4, 3),        # ragged tokens, expert_begin != 0, non-local slots
    (5, 384, 256, 8, 8, 8, 0),          # k = E: every expert active
    (129, 512, 384, 32, 32, 2, 0),      # several 16-row tiles, I not a power of two
    (1, 256, 128, 64, 4, 8, 0),         # single token, likely no local hit
])
def test_indexed_small_shapes(T, H, I, E_g, E_l, k, eb):
    banner(f"indexed small T={T} H={H} I={I} E_g={E_g} E_l={E_l} k={k} eb={eb}")
    case = small_case(T * 31 + H, T, H, I, E_g, E_l, k, eb)
    got, _, _ = run_indexed(*case, E_g=E_g, bm=16)
    ref = oracle.moe_layer(*case)
    check_close(got, ref)


@pytest.mark.parametrize("tokens", [16, 32])
def test_indexed_schedule_overrides_bit_identical(tokens):
    """Schedules differ only in tiling of tokens: results must be bit-identical."""
    banner(f"indexed schedule override tokens={tokens}")
    case = small_case(99, 70, 256, 128, 8, 8, 4)
    base, layer, _ = run_indexed(*case, E_g=8, bm=16, override={"kernel": 1, "tokens": 16})
    got, _, _ = run_indexed(*case, E_g=8, bm=16, override={"kernel": 1, "tokens": tokens},
                            layer=layer)
    assert np.array_equal(got, base)
    check_close(got, oracle.moe_layer(*case))


@pytest.mark.parametrize("bm,extra", [(32, 0), (64, 500), (128, 1)])
def test_indexed_block_m_and_oversize_buffers(bm, extra):
    banner(f"indexed bm={bm} extra={extra}")
    case = small_case(5 + bm, 40, 256, 128, 16, 16, 4)
    got, _, _ = run_indexed(*case, E_g=16, bm=bm, extra=extra)
    check_close(got, oracle.moe_layer(*case))


def test_indexed_no_local_tokens_give_zero():
    banner("indexed: no local slots")
    case = small_case(11, 9, 256, 128, 64, 4, 2, expert_begin=60)
    x, ids, w, *rest = case
    ids = np.where(ids >= 60, ids - 8, ids).astype(np.int32)  # nothing in [60, 64)
    got, _, _ = run_indexed(x, ids, w, *rest, E_g=64)
    assert np.all(got == 0)


def test_indexed_repeat_is_bitwise_deterministic():
    banner("indexed determinism")
    case = small_case(12, 64, 512, 256, 16, 16, 4)
    a, layer, _ = run_indexed(*case, E_g=16)
    b, _, _ = run_indexed(*case, E_g=16, layer=layer)
    assert np.array_equal(a, b)


def test_indexed_validate_flag_passes_good_routing():
    banner("indexed validate flag")
    case = small_case(13, 20, 256, 128, 8, 8, 2)
    got, _, _ = run_indexed(*case, E_g=8, flags=C.FLAG_VALIDATE)
    check_close(got, oracle.moe_layer(*case))


def test_indexed_validate_flag_reports_bad_expert_ids():
    """A corrupted expert_ids entry is skipped in trusted mode and reported as
    CHORD_ERR_ROUTING with validation on (forced from the host; the kernels
    never index out of bounds)."""
    from quantized_moe_amd.moe import W4A16MoE
    banner("indexed validate flag with corrupted expert_ids")
    x, ids, w, q13, s13, q2, s2, eb = small_case(14, 20, 256, 128, 8, 8, 2)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2))
    ids_d = dev(ids)
    s, e, n = C.chord_moe_align(ids_d, 0, 8, 16)
    e[0] = 99
    with pytest.raises(C.ChordError) as ei:
        layer.indexed(dev_bf16(x), ids_d, dev(w), 0, 8, align=(s, e, n, 16), flags=C.FLAG_VALIDATE)
    assert ei.value.status == 5
    layer.indexed(dev_bf16(x), ids_d, dev(w), 0, 8, align=(s, e, n, 16))  # trusted: no error
    torch.cuda.synchronize()


def test_streaming_ring_runs_on_across_items_and_skipped_tiles():
    """More gate_up work items than the persistent grid holds (64 experts x 64
    weight-tile groups), so each workgroup's load ring runs on from one item
    into the next; one alignment block is corrupted in trusted mode, so a
    workgroup meets a skipped item between two others and must restart its
    ring there.  Every token without a slot in the corrupted block matches the
    oracle, and the same call without the corruption matches it everywhere."""
    banner("streaming ring across items, one skipped alignment block")
    T, H, I, E, k = 64, 512, 2048, 64, 8
    case = small_case(61, T, H, I, E, E, k)
    x, ids, w, q13, s13, q2, s2, eb = case
    ref = oracle.moe_layer(*case)
    got, layer, al = run_indexed(*case, E_g=E, bm=16, override={"kernel": 1})
    assert "gate_up nt=4 wk=1 pf=4" in C.last_plan(), C.last_plan()
    check_close(got, ref, "all blocks")
    s_ids, e_ids, ntpp = al
    bad = 5
    slots = host(s_ids)[bad * 16:(bad + 1) * 16]
    hit = np.unique(slots[slots < T * k] // k)
    e_ids[bad] = 999
    out = layer.indexed(dev_bf16(x), dev(ids), dev(w), expert_begin=0, num_global_experts=E,
                        align=(s_ids, e_ids, ntpp, 16), override={"kernel": 1})
    torch.cuda.synchronize()
    got2 = host_bf16(out)
    keep = np.setdiff1d(np.arange(T), hit)
    assert 0 < hit.size < T
    check_close(got2[keep], ref[keep], "tokens outside the skipped block")


def test_streaming_ring_with_uneven_wave_ranges():
    """A routed gate_up with 25 K chunks split over two waves (12 and 13
    chunks) and more work items (44 experts x 64 weight-tile groups) than the
    persistent grid holds: the wave with an even chunk count runs its load
    ring on into the next item, the other restarts it, inside the same
    workgroups; the layer matches the oracle."""
    banner("streaming ring, uneven wave ranges, H=3200")
    case = small_case(63, 48, 3200, 1024, 192, 48, 8)
    got, _ = run_routed(*case, E_g=192)
    assert "gate_up nt=2 wk=2 pf=2" in C.last_plan(), C.last_plan()
    check_close(got, oracle.moe_layer(*case), "uneven wave ranges")


@pytest.mark.parametrize("H,I,k", [(4224, 128, 2), (4096, 256, 1)])
def test_single_token_deep_k_split(H, I, k):
    """One routed token on a deep-K gate_up: the planner takes one weight
    tile per item over 8 K-split waves (33 chunks at H = 4224: uneven wave
    ranges of 4 and 5 chunks); the layer matches the oracle."""
    banner(f"single token deep-K split H={H} I={I} k={k}")
    case = small_case(31, 1, H, I, 8, 8, k)
    got, _, _ = run_indexed(*case, E_g=8, bm=16)
    assert "gate_up nt=1 wk=8 pf=4" in C.last_plan(), C.last_plan()
    check_close(got, oracle.moe_layer(*case), what=f"single token H={H}")


# ---------------------------------------------------------------------------
# grouped layouts
# ---------------------------------------------------------------------------

def test_contiguous_small_with_token_combine():
    from quantized_moe_amd.moe import W4A16MoE
    banner("contiguous small + combine")
    x, ids, w, q13, s13, q2, s2, eb = small_case(21, 90, 256, 128, 12, 6, 3)
    a, m_idx, f2r, nvalid = G.build_contiguous(ids, x, eb, 6)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2), mode=C.MODE_CONTIGUOUS)
    T = ids.shape[0]
    out_tokens = torch.empty((T, 256), dtype=torch.bfloat16, device="cuda")
    rows, tok = layer.contiguous(dev_bf16(a), dev(m_idx), nvalid, flat_to_row=dev(f2r),
                                 topk_weights=dev(w), out_tokens=out_tokens)
    torch.cuda.synchronize()
    rows_h = host_bf16(rows)
    ref_rows = oracle.grouped_contiguous(a, m_idx, q13, s13, q2, s2)
    valid = m_idx >= 0
    check_close(rows_h[valid], ref_rows[valid], "contiguous rows")
    check_close(host_bf16(tok), oracle.moe_layer(x, ids, w, q13, s13, q2, s2, eb), "contiguous tokens")


def test_contiguous_row_weights():
    from quantized_moe_amd.moe import W4A16MoE
    banner("contiguous row weights")
    x, ids, w, q13, s13, q2, s2, eb = small_case(22, 30, 256, 128, 4, 4, 2)
    a, m_idx, f2r, nvalid = G.build_contiguous(ids, x, eb, 4)
    rw = np.random.default_rng(0).uniform(0.1, 1.0, a.shape[0]).astype(np.float32)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2), mode=C.MODE_CONTIGUOUS)
    rows, _ = layer.contiguous(dev_bf16(a), dev(m_idx), nvalid, row_weights=dev(rw))
    torch.cuda.synchronize()
    ref = oracle.grouped_contiguous(a, m_idx, q13, s13, q2, s2, row_weights=rw)
    valid = m_idx >= 0
    check_close(host_bf16(rows)[valid], ref[valid])


def test_masked_small():
    from quantized_moe_amd.moe import W4A16MoE
    banner("masked small")
    rng = np.random.default_rng(31)
    E, max_m, H, I = 6, 40, 256, 128
    a3, mm, em, _ = G.draw_masked(rng, E, max_m, H)
    mm[2] = 0
    mm[3] = max_m
    q13, s13 = G.draw_weights(rng, E, 2 * I, H)
    q2, s2 = G.draw_weights(rng, E, H, I)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2), mode=C.MODE_MASKED)
    out = layer.masked(dev_bf16(a3), dev(mm), em)
    torch.cuda.synchronize()
    got = host_bf16(out)
    ref = oracle.grouped_masked(a3, mm, q13, s13, q2, s2)
    valid = np.zeros(E * max_m, bool)
    for e in range(E):
        valid[e * max_m:e * max_m + mm[e]] = True
    check_close(got[valid], ref[valid], "masked")


def test_masked_expected_m_is_only_a_hint():
    from quantized_moe_amd.moe import W4A16MoE
    banner("masked expected_m hint")
    rng = np.random.default_rng(32)
    E, max_m, H, I = 4, 64, 256, 128
    a3, mm, em, _ = G.draw_masked(rng, E, max_m, H)
    q13, s13 = G.draw_weights(rng, E, 2 * I, H)
    q2, s2 = G.draw_weights(rng, E, H, I)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2), mode=C.MODE_MASKED)
    outs = []
    for hint in (1, em, 64):
        o = layer.masked(dev_bf16(a3), dev(mm), hint)
        torch.cuda.synchronize()
        outs.append(host_bf16(o))
    ref = oracle.grouped_masked(a3, mm, q13, s13, q2, s2)
    for e in range(E):
        sl = slice(e * max_m, e * max_m + mm[e])
        for o in outs:
            check_close(o[sl], ref[sl])


def test_masked_validate_reports_overflowing_counts():
    from quantized_moe_amd.moe import W4A16MoE
    banner("masked validate: masked_m > max_m")
    rng = np.random.default_rng(33)
    E, max_m, H, I = 3, 16, 256, 128
    a3, mm, em, _ = G.draw_masked(rng, E, max_m, H)
    q13, s13 = G.draw_weights(rng, E, 2 * I, H)
    q2, s2 = G.draw_weights(rng, E, H, I)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2), mode=C.MODE_MASKED)
    bad = mm.copy()
    bad[1] = max_m + 5
    with pytest.raises(C.ChordError) as ei:
        layer.masked(dev_bf16(a3), dev(bad), em, flags=C.FLAG_VALIDATE)
    assert ei.value.status == 5
    out = layer.masked(dev_bf16(a3), dev(bad), em)       # trusted: clamped to max_m
    torch.cuda.synchronize()
    clamped = np.minimum(bad, max_m)
    ref = oracle.grouped_masked(a3, clamped, q13, s13, q2, s2)
    got = host_bf16(out)
    for e in range(E):
        sl = slice(e * max_m, e * max_m + clamped[e])
        check_close(got[sl], ref[sl])


# ---------------------------------------------------------------------------
# LDS-tiled kernel (many rows per expert)
# ---------------------------------------------------------------------------

def test_tile_kernel_bit_identical_to_streaming_kernel():
    """With one wave per K range both kernels accumulate every output over the
    same chunks and MFMA steps in the same order, so they must agree bit for
    bit; several 128-row tiles per expert and ragged tails."""
    banner("tile kernel vs streaming kernel: indexed T=300 H=512 I=256")
    case = small_case(301, 300, 512, 256, 16, 8, 4, 4)
    tiled, layer, _ = run_indexed(*case, E_g=16, bm=16, override={"kernel": 2, "tile_split": 1})
    stream, _, _ = run_indexed(*case, E_g=16, bm=16, layer=layer,
                               override={"kernel": 1, "gate_up_wk": 1, "down_wk": 1})
    assert np.array_equal(tiled, stream)
    check_close(tiled, oracle.moe_layer(*case))


def test_tile_kernel_masked_tile_boundaries():
    from quantized_moe_amd.moe import W4A16MoE
    banner("tile kernel: masked rows at tile boundaries")
    rng = np.random.default_rng(34)
    E, max_m, H, I = 6, 300, 256, 256
    a3, _, _, _ = G.draw_masked(rng, E, max_m, H)
    mm = np.array([0, 1, 128, 129, 300, 255], np.int32)
    q13, s13 = G.draw_weights(rng, E, 2 * I, H)
    q2, s2 = G.draw_weights(rng, E, H, I)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2), mode=C.MODE_MASKED)
    out = layer.masked(dev_bf16(a3), dev(mm), 200)   # hint >= 48 rows: tiled kernel
    torch.cuda.synchronize()
    assert "tile" in C.last_plan()
    got = host_bf16(out)
    ref = oracle.grouped_masked(a3, mm, q13, s13, q2, s2)
    for e in range(E):
        sl = slice(e * max_m, e * max_m + mm[e])
        check_close(got[sl], ref[sl], f"masked e={e}")


def skewed_case(seed, T, H, I, E, k, popularity):
    """Routing with a few hot experts: each token picks k distinct experts with
    probability proportional to `popularity`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = G.draw_activations(rng, T, H)
    p = np.asarray(popularity, dtype=np.float64)
    p /= p.sum()
    ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    q13, s13 = G.draw_weights(rng, E, 2 * I, H, scale_mult=(256.0 / H) ** 0.5)
    q2, s2 = G.draw_weights(rng, E, H, I, scale_mult=(256.0 / I) ** 0.5)
    return x, ids, w, q13, s13, q2, s2, 0


def test_split_kernels_indexed_bit_identical_and_oracle():
    """Kernel 3 sends experts with >= 48 rows to the tiled kernel and the rest
    to the streaming kernel; with one wave per K range every output keeps the
    same accumulation order, so it must equal the streaming-only run bit for
    bit (hot expert of ~250 rows: two big tiles)."""
    banner("split kernels: indexed, skewed routing")
    case = skewed_case(77, 256, 512, 256, 8, 2, [40, 20, 10, 5, 3, 2, 1, 1])
    counts = np.bincount(case[1].ravel(), minlength=8)
    assert counts.max() > 192 and (counts >= 48).sum() >= 2 and (counts < 48).sum() >= 2, counts
    split, layer, _ = run_indexed(*case, E_g=8, bm=16, override={"kernel": 3, "tile_split": 1})
    assert "experts with >= 48 rows" in C.last_plan()
    stream, _, _ = run_indexed(*case, E_g=8, bm=16, layer=layer,
                               override={"kernel": 1, "gate_up_wk": 1, "down_wk": 1})
    assert np.array_equal(split, stream)
    check_close(split, oracle.moe_layer(*case))


def test_contiguous_validate_flags_bad_m_indices():
    """An out-of-range m_indices value is reported with validation on; in
    trusted mode the rows of intact segments are still computed."""
    from quantized_moe_amd.moe import W4A16MoE
    banner("contiguous validate: bad m_indices")
    x, ids, w, q13, s13, q2, s2, eb = small_case(23, 200, 256, 128, 6, 6, 2)
    a, m_idx, f2r, nvalid = G.build_contiguous(ids, x, eb, 6)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2), mode=C.MODE_CONTIGUOUS)
    good, _ = layer.contiguous(dev_bf16(a), dev(m_idx), nvalid, flags=C.FLAG_VALIDATE)
    torch.cuda.synchronize()
    bad = m_idx.copy()
    seg = np.nonzero(bad == 3)[0]
    bad[seg[0]] = 17                                   # out of range
    with pytest.raises(C.ChordError) as ei:
        layer.contiguous(dev_bf16(a), dev(bad), nvalid, flags=C.FLAG_VALIDATE)
    assert ei.value.status == 5
    rows, _ = layer.contiguous(dev_bf16(a), dev(bad), nvalid)
    torch.cuda.synchronize()
    keep = (bad >= 0) & (bad < 6) & (bad != 3)        # rows of intact experts
    check_close(host_bf16(rows)[keep], host_bf16(good)[keep], "trusted rows of other experts")
    ref = oracle.grouped_contiguous(a, m_idx, q13, s13, q2, s2)
    check_close(host_bf16(good)[m_idx >= 0], ref[m_idx >= 0], "validated run")


@pytest.mark.parametrize("kernel", [1, 2])
def test_indexed_layer_replays_in_a_hip_graph(kernel):
    """Alignment + layer captured once in a HIP graph (no host sync, no
    allocation, no memset on the default path) and replayed on new inputs
    written into the same buffers: every replay equals an eager call bit for
    bit, with eager work and synchronisations between the replays."""
    from quantized_moe_amd.moe import W4A16MoE
    banner(f"graph replay, kernel {kernel}")
    T, H, I, E, k, bm = 80, 512, 256, 8, 4, 16
    base = small_case(500, T, H, I, E, E, k)
    layer = W4A16MoE(dev(base[3]), dev_bf16(base[4]), dev(base[5]), dev_bf16(base[6]))
    mp = C.chord_moe_align_max_padded(T, k, E, bm)
    al = (torch.empty(mp, dtype=torch.int32, device="cuda"),
          torch.empty((mp + bm - 1) // bm, dtype=torch.int32, device="cuda"),
          torch.empty(1, dtype=torch.int32, device="cuda"))
    al_ws = torch.empty(max(1, C.lib.chord_moe_align_workspace_bytes(T, k, E, bm)),
                        dtype=torch.uint8, device="cuda")
    x, ids, w = dev_bf16(base[0]), dev(base[1]), dev(base[2])
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ov = {"kernel": kernel}

    def step(o):
        C.chord_moe_align(ids, 0, E, bm, max_padded=mp, out=al, workspace=al_ws)
        layer.indexed(x, ids, w, 0, E, align=(*al, bm), out=o, override=ov)

    step(out)                      # warm-up: plan and workspace exist before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    torch.cuda.synchronize()
    for r in range(3):
        case = small_case(600 + r, T, H, I, E, E, k)
        x.copy_(dev_bf16(case[0]))
        ids.copy_(dev(case[1]))
        w.copy_(dev(case[2]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = host_bf16(out)
        eager_out = torch.empty_like(out)
        step(eager_out)
        torch.cuda.synchronize()
        assert np.array_equal(replayed, host_bf16(eager_out)), f"replay {r}"
        check_close(replayed, oracle.moe_layer(case[0], case[1], case[2], base[3], base[4],
                                               base[5], base[6], 0), f"replay {r}")


def test_tile_k_split_of_a_hot_expert_is_deterministic_and_close():
    """A masked call with one expert far above the others: the tile builder
    splits that expert's tiles along K and the last part adds the fp32
    partials in part order, so repeats are bit-identical; the result matches
    the oracle and the unsplit indexed path (same rows) within tolerance."""
    from quantized_moe_amd.moe import W4A16MoE
    banner("tiled K split: masked hot expert")
    rng = np.random.default_rng(35)
    E, max_m, H, I = 8, 192, 512, 512
    a3, _, _, _ = G.draw_masked(rng, E, max_m, H)
    mm = np.array([192, 9, 12, 7, 16, 5, 11, 8], np.int32)   # mean 16 groups 2.5, hot 12
    q13, s13 = G.draw_weights(rng, E, 2 * I, H, scale_mult=(256.0 / H) ** 0.5)
    q2, s2 = G.draw_weights(rng, E, H, I, scale_mult=(256.0 / I) ** 0.5)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2), mode=C.MODE_MASKED)
    outs = []
    for _ in range(3):
        o = layer.masked(dev_bf16(a3), dev(mm), 32)    # hint >= 24 rows: tiled kernel
        torch.cuda.synchronize()
        outs.append(host_bf16(o))
    assert "tile" in C.last_plan()
    ref = oracle.grouped_masked(a3, mm, q13, s13, q2, s2)
    for e in range(E):    # rows past masked_m[e] are unspecified: compare valid rows only
        sl = slice(e * max_m, e * max_m + mm[e])
        assert np.array_equal(outs[0][sl], outs[1][sl]) and np.array_equal(outs[0][sl], outs[2][sl])
        check_close(outs[0][sl], ref[sl], f"masked e={e}")


# ---------------------------------------------------------------------------
# routed calls: rows from topk_ids inside the gate_up launch (no alignment)
# ---------------------------------------------------------------------------

def run_routed(x, ids, w, q13, s13, q2, s2, eb, E_g, layer=None, flags=0):
    """The planner's own choice with no alignment (block_m 0)."""
    from quantized_moe_amd.moe import W4A16MoE
    if layer is None:
        layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2))
    T, k = ids.shape
    E_l, H, I = q13.shape[0], x.shape[1], q2.shape[2] * 8
    assert C.chord_w4a16_moe_indexed_block_m(T, k, E_g, E_l, H, I) == 0
    out = layer.indexed(dev_bf16(x), dev(ids), dev(w), expert_begin=eb, num_global_experts=E_g,
                        block_m=0, flags=flags)
    torch.cuda.synchronize()
    return host_bf16(out), layer


@pytest.mark.parametrize("T,H,I,E_g,E_l,k,eb", [
    (64, 1024, 512, 64, 16, 8, 8),      # decode-like: ~1 row per expert, non-local slots
    (160, 512, 512, 64, 24, 8, 0),      # ~20 rows per expert: 32-row token tiles
    (300, 640, 256, 384, 384, 2, 0),    # TP-like, short-K down GEMM
    (256, 384, 384, 384, 64, 8, 0),     # 2048 slots, the routed maximum
])
def test_routed_equals_aligned_bit_identical(T, H, I, E_g, E_l, k, eb):
    """A routed call and the same schedule on the alignment (kernel-1
    override) compute every row from the same chunks in the same order, so
    they agree bit for bit; the rows of an expert may share tiles in another
    order, which changes no row."""
    banner(f"routed vs aligned T={T} H={H} I={I} E_g={E_g} E_l={E_l} k={k}")
    case = small_case(T * 13 + I, T, H, I, E_g, E_l, k, eb)
    routed, layer = run_routed(*case, E_g=E_g)
    plan = C.last_plan()
    assert "tiles=routed" in plan and "down+combine" not in plan, plan
    aligned, _, _ = run_indexed(*case, E_g=E_g, bm=16, layer=layer, override={"kernel": 1})
    assert "tiles=blocks" in C.last_plan() or "tiles=list" in C.last_plan()
    assert np.array_equal(routed, aligned)
    check_close(routed, oracle.moe_layer(*case))
    again, _ = run_routed(*case, E_g=E_g, layer=layer)
    assert np.array_equal(again, routed)


def test_routed_hot_experts_span_many_tiles():
    """Skewed routing: hot experts hold up to ~150 rows, i.e. several 16-row
    tiles of one routed expert."""
    banner("routed: skewed experts over many tiles")
    case = skewed_case(78, 300, 512, 512, 64, 2, [60, 30, 20] + [1] * 61)
    counts = np.bincount(case[1].ravel(), minlength=64)
    assert counts.max() > 64, counts.max()
    routed, layer = run_routed(*case, E_g=64)
    assert "tiles=routed" in C.last_plan()
    aligned, _, _ = run_indexed(*case, E_g=64, bm=16, layer=layer, override={"kernel": 1})
    assert np.array_equal(routed, aligned)
    check_close(routed, oracle.moe_layer(*case))


def test_routed_validate_flag_and_no_local_slot():
    banner("routed: validate flag, tokens without a local slot")
    case = small_case(79, 40, 512, 512, 128, 16, 4, expert_begin=100)
    x, ids, w, *rest = case
    got, _ = run_routed(x, ids, w, *rest, E_g=128, flags=C.FLAG_VALIDATE)
    ref = oracle.moe_layer(x, ids, w, *rest)
    check_close(got, ref)
    none = ~np.any((ids >= 100) & (ids < 116), axis=1)
    assert none.any() and np.all(got[none] == 0)


@pytest.mark.parametrize("T,H,I,E_g,E_l,k,eb", [
    (1, 1024, 256, 384, 384, 8, 0),     # the single-token TP slice, small H
    (2, 512, 512, 64, 16, 8, 4),        # some slots non-local
    (16, 384, 128, 16, 16, 4, 0),       # 64 slots, 16 tokens: the fused maximum
    (5, 384, 256, 32, 32, 1, 0),        # top-1
    (3, 384, 128, 64, 4, 8, 60),        # likely tokens without a local slot
])
def test_fused_down_combine_matches_the_oracle(T, H, I, E_g, E_l, k, eb):
    """T <= 16 and T*k <= 64: the down GEMM and the combine run as one launch
    that sums w * y in fp32 without rounding y first (the oracle's reading);
    the aligned path rounds y to bf16 before its combine, so the two agree
    within the tolerance, not bit for bit."""
    banner(f"fused down+combine T={T} H={H} I={I} E_g={E_g} E_l={E_l} k={k} eb={eb}")
    case = small_case(T * 17 + H + k, T, H, I, E_g, E_l, k, eb)
    fused, layer = run_routed(*case, E_g=E_g)
    assert "down+combine" in C.last_plan(), C.last_plan()
    ref = oracle.moe_layer(*case)
    st = check_close(fused, ref, "fused")
    banner(f"  {st}")
    aligned, _, _ = run_indexed(*case, E_g=E_g, bm=16, layer=layer, override={"kernel": 1})
    check_close(fused, aligned, "fused vs aligned")
    ids = case[1]
    none = ~np.any((ids >= eb) & (ids < eb + E_l), axis=1)
    assert np.all(fused[none] == 0)
    again, _ = run_routed(*case, E_g=E_g, layer=layer)
    assert np.array_equal(again, fused)


@pytest.mark.parametrize("T,k,I", [(12, 4, 512), (64, 8, 512), (48, 8, 1024)])
def test_routed_layer_replays_in_a_hip_graph(T, k, I):
    """A routed call (no alignment launch; fused down+combine at T = 12)
    captured in a HIP graph and replayed on new inputs in the same buffers:
    every replay equals an eager call bit for bit."""
    from quantized_moe_amd.moe import W4A16MoE
    banner(f"graph replay, routed T={T} k={k} I={I}")
    H, E_g, E_l = 512, 64, 16
    base = small_case(800 + T, T, H, I, E_g, E_l, k)
    layer = W4A16MoE(dev(base[3]), dev_bf16(base[4]), dev(base[5]), dev_bf16(base[6]))
    x, ids, w = dev_bf16(base[0]), dev(base[1]), dev(base[2])
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step(o):
        layer.indexed(x, ids, w, 0, E_g, block_m=0, out=o)

    step(out)
    torch.cuda.synchronize()
    assert "tiles=routed" in C.last_plan()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    torch.cuda.synchronize()
    for r in range(3):
        case = small_case(900 + r, T, H, I, E_g, E_l, k)
        x.copy_(dev_bf16(case[0]))
        ids.copy_(dev(case[1]))
        w.copy_(dev(case[2]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = host_bf16(out)
        eager_out = torch.empty_like(out)
        step(eager_out)
        torch.cuda.synchronize()
        assert np.array_equal(replayed, host_bf16(eager_out)), f"replay {r}"
        check_close(replayed, oracle.moe_layer(case[0], case[1], case[2], base[3], base[4],
                                               base[5], base[6], 0), f"replay {r}")


# ---------------------------------------------------------------------------
# producer/consumer form of the LDS-tiled GEMMs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,I,pop", [
    (512, 384, [300, 177, 176, 100, 17, 1, 40, 64]),    # edges of the 176-row tiles
    (640, 512, [40, 30, 20, 10, 5, 3, 2, 1]),           # skewed, ragged token groups
])
def test_tile_producer_consumer_form_bit_identical(H, I, pop):
    """Kernel 5 (waves that only issue MFMAs on LDS operands, waves that only
    load and dequantise) and kernel 4 (every wave does both) sum every output
    over the same chunks and steps in the same order: bit-identical, whatever
    tiles the rows fall in (176- vs 192-row tiles)."""
    banner(f"tiled producer/consumer vs single-role H={H} I={I}")
    E, k = len(pop), 2
    T = sum(pop) // k + 1
    case = skewed_case(91 + H, T, H, I, E, k, pop)
    counts = np.bincount(case[1].ravel(), minlength=E)
    banner(f"  rows per expert {counts.tolist()}")
    pc, layer, _ = run_indexed(*case, E_g=E, bm=16, override={"kernel": 5})
    assert "producer/consumer" in C.last_plan(), C.last_plan()
    single, _, _ = run_indexed(*case, E_g=E, bm=16, layer=layer, override={"kernel": 4})
    assert "8 waves" in C.last_plan(), C.last_plan()
    assert np.array_equal(pc, single)
    check_close(pc, oracle.moe_layer(*case))
    again, _, _ = run_indexed(*case, E_g=E, bm=16, layer=layer, override={"kernel": 5})
    assert np.array_equal(again, pc)
