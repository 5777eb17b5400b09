"""CPU tests of the planner through the host-only query entry point: the
schedule each benchmark-shaped call would get, the effect of overrides and of
the compute-unit count, and the query's own argument checks.  No GPU: the
query makes no HIP call."""

import ctypes

import pytest

from quantized_moe_amd import chord as C


def indexed(T, k, E_g, E_l, H, I, **kw):
    bm = C.chord_w4a16_moe_indexed_block_m(T, k, E_g, E_l, H, I)
    mp = C.chord_moe_align_max_padded(T, k, E_l, bm)
    return C.chord_w4a16_moe_plan(C.MODE_INDEXED, T, k, E_g, E_l, H, I, bm, mp, **kw)


def test_decode_streams_weights_with_split_k_gate_up():
    # 64 tokens over 48 of 384 experts: about one token per expert, so every
    # GEMM streams its weights once; gate_up splits K over two waves.
    p = indexed(64, 8, 384, 48, 7168, 2048)
    assert p.startswith("indexed: ") and "| stream tiles=routed" in p
    assert "gate_up nt=2 wk=2" in p and "down nt=4 wk=1" in p


@pytest.mark.parametrize("T,k,over,fused", [
    (16, 4, None, True),                  # 64 slots, 16 tokens: the fused maximum
    (1, 8, None, True),                   # the single-token TP slice shape
    (17, 4, None, False),                 # 68 slots
    (8, 8, None, True),
    (8, 8, {"down_nt": 4}, False),        # a down override keeps the separate launches
    (8, 8, {"gate_up_nt": 4}, True),
])
def test_fused_down_combine_only_for_a_handful_of_tokens(T, k, over, fused):
    p = indexed(T, k, 384, 384, 7168, 256, override=over)
    assert "tiles=routed" in p, p
    assert ("down+combine" in p) == fused, p
def test_prefill_and_large_tp_slices_take_the_tiled_kernel():
    assert "| tile 256x192" in indexed(8192, 8, 384, 48, 7168, 2048)
    for T in (512, 4096):
        assert "| tile 256x192" in indexed(T, 8, 384, 384, 7168, 256), T


def test_single_token_tp_slice_splits_gate_up_eight_ways():
    # I = 256: 32 weight tiles of gate_up per expert and 8 routed rows; with
    # so few tiles the gate_up K split goes to eight waves and each item
    # takes one weight tile, so every CU gets a workgroup.
    p = indexed(1, 8, 384, 384, 7168, 256)
    assert "| stream " in p and "gate_up nt=1 wk=8 pf=4" in p
    # Twice the routed rows fill the CUs with 2 weight tiles and 4 waves.
    assert "gate_up nt=2 wk=4" in indexed(2, 8, 384, 384, 7168, 256)


def test_small_tp_slice_streams():
    assert "| stream " in indexed(32, 8, 384, 384, 7168, 256)


def test_grouped_layouts_plan_the_tiled_kernel():
    M = 8192 * 8 * 48 // 384
    p = C.chord_w4a16_moe_plan(C.MODE_CONTIGUOUS, 8192, 8, 0, 48, 7168, 2048, M, M + 48 * 128)
    assert p.startswith("contiguous: ") and "| tile 256x192" in p
    for E in (24, 48, 96):
        p = C.chord_w4a16_moe_plan(C.MODE_MASKED, 0, 0, 0, E, 7168, 2048, 100, E * 256)
        assert p.startswith("masked: ") and "| tile 256x192" in p, E


def test_overrides_select_the_kernel_family():
    assert "| tile " in indexed(64, 8, 384, 48, 7168, 2048, override={"kernel": 2})
    assert "| stream " in indexed(8192, 8, 384, 48, 7168, 2048, override={"kernel": 1})
    p = indexed(64, 8, 384, 48, 7168, 2048, override={"gate_up_wk": 4, "down_nt": 2})
    assert "gate_up nt=2 wk=4" in p and "down nt=2" in p


def test_plans_are_deterministic_and_accept_other_cu_counts():
    a = indexed(64, 8, 384, 48, 7168, 2048)
    assert indexed(64, 8, 384, 48, 7168, 2048) == a
    assert indexed(64, 8, 384, 48, 7168, 2048, num_cus=256) == a
    for cus in (1, 80, 304):
        assert indexed(64, 8, 384, 48, 7168, 2048, num_cus=cus).startswith("indexed: ")


@pytest.mark.parametrize("args, override", [
    ((3, 64, 8, 384, 48, 7168, 2048, 16, 1024), None),                 # mode
    ((0, 64, 8, 384, 48, 7100, 2048, 16, 1024), None),                 # H % 128
    ((0, 64, 8, 384, 48, 7168, 2048, 24, 1024), None),                 # block_m
    ((0, 0, 8, 384, 48, 7168, 2048, 16, 1024), None),                  # T
    ((0, 64, 8, 384, 0, 7168, 2048, 16, 1024), None),                  # E_l
    ((0, 64, 8, 384, 48, 7168, 2048, 16, -1), None),                   # rows
    ((2, 0, 0, 0, 48, 7168, 2048, 100, 48 * 256), {"kernel": 1}),      # grouped override
    ((0, 64, 8, 384, 48, 7168, 2048, 16, 1024), {"gate_up_wk": 3}),    # out of range
])
def test_query_rejects_bad_descriptors(args, override):
    with pytest.raises(C.ChordError) as e:
        C.chord_w4a16_moe_plan(*args, override=override)
    assert e.value.status == 1


def test_query_rejects_null_buffer():
    st = C.lib.chord_w4a16_moe_plan(0, 64, 8, 384, 48, 7168, 2048, 16, 1024, 0, None, None, 16)
    assert st == 1
    buf = ctypes.create_string_buffer(8)
    st = C.lib.chord_w4a16_moe_plan(0, 64, 8, 384, 48, 7168, 2048, 16, 1024, 0, None, buf, 0)
    assert st == 1
    # A short buffer is filled and terminated, not overrun.
    assert C.lib.chord_w4a16_moe_plan(0, 64, 8, 384, 48, 7168, 2048, 16, 1024, 0, None, buf, 8) == 0
    assert buf.value == b"indexed"


def test_plan_cache_holds_one_entry_per_descriptor():
    """Identical descriptors hit the memoised plan whatever the caller's stack
    held before (the key has no indeterminate bytes): in a fresh process with
    CHORD_LOG=1, which logs each plan the cache computes, repeated queries from
    different call depths and with stack garbage in between compute each
    distinct descriptor once."""
    import os
    import subprocess
    import sys
    code = r'''
import ctypes, random
from quantized_moe_amd import chord as C
def q(T):
    return C.chord_w4a16_moe_plan(C.MODE_INDEXED, T, 8, 384, 48, 7168, 2048, 16,
                                  C.chord_moe_align_max_padded(T, 8, 48, 16))
def deep(n, T):
    junk = ctypes.create_string_buffer(bytes(random.getrandbits(8) for _ in range(256)))
    return q(T) if n == 0 else deep(n - 1, T)
for i in range(60):
    deep(i % 13, 64 if i % 2 else 8192)
    C.chord_w4a16_moe_plan(C.MODE_MASKED, 0, 0, 0, 48, 7168, 2048, 18, 48 * 256)
'''
    env = dict(os.environ, CHORD_LOG="1")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("[chord] plan")]
    assert len(lines) == 3, lines


def test_routed_calls_need_a_gate_up_k_over_two_chunks():
    """Routed calls (no alignment) need the general streaming kernel for the
    gate_up: at H <= 256 the short-K variant would run, which reads its tiles
    from the alignment, so such calls align."""
    assert C.chord_w4a16_moe_indexed_block_m(256, 8, 384, 64, 256, 384) != 0
    assert C.chord_w4a16_moe_indexed_block_m(256, 8, 384, 64, 384, 384) == 0
    assert "tiles=routed" not in C.chord_w4a16_moe_plan(C.MODE_INDEXED, 256, 8, 384, 64, 256, 384,
                                                       0, 0)
    assert "tiles=routed" in C.chord_w4a16_moe_plan(C.MODE_INDEXED, 256, 8, 384, 64, 384, 384, 0,
                                                   0)


def test_routed_tables_fit_their_lds_share():
    # The tables take (4 E + 2 + 2 n) ints of the launch's LDS, at most 32 KB:
    # at 2,048 slots routed up to 1,022 local experts, aligned at the
    # 1,024-expert limit; fewer slots leave room for every expert count.
    assert C.chord_w4a16_moe_indexed_block_m(256, 8, 1022, 1022, 7168, 256) == 0
    assert C.chord_w4a16_moe_indexed_block_m(256, 8, 1024, 1024, 7168, 256) != 0
    assert C.chord_w4a16_moe_indexed_block_m(8, 8, 1024, 1024, 7168, 256) == 0
