"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, and rejects misuse on the host before any HIP call (no GPU needed:
every call here fails validation first)."""

import ctypes
import os
import re

import pytest

from quantized_moe_amd import chord as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def header_functions():
    txt = open(os.path.join(ROOT, "include", "chord.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(chord_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(C.lib, n), n
    assert sorted(C.EXPORTED) == names


def test_status_strings_and_version():
    assert C.lib.chord_status_string(0) == b"CHORD_OK"
    assert C.lib.chord_status_string(3) == b"CHORD_ERR_LAYOUT_MISMATCH"
    assert b"gfx950" in C.lib.chord_version()


def test_packed_bytes_and_bounds():
    assert C.chord_w4a16_packed_bytes(0, 0, 48, 4096, 7168) == 48 * 4096 * 7168 * 9 // 16
    assert C.chord_w4a16_packed_bytes(0, 1, 1, 16, 100) == 0        # K % 128
    assert C.chord_w4a16_packed_bytes(0, 0, 1, 24, 128) == 0        # I % 8 for gate_up
    assert C.chord_moe_align_max_padded(64, 8, 48, 16) == 512 + 48 * 15
    # decode: routed inside the GEMM, no alignment (block_m 0); prefill aligns
    assert C.chord_w4a16_moe_indexed_block_m(64, 8, 384, 48, 7168, 2048) == 0
    assert C.chord_w4a16_moe_indexed_block_m(8192, 8, 384, 48, 7168, 2048) in (16, 32, 64, 128)


def _handle(mode, role, E=2, N=256, K=256):
    h = C.Weight()
    h.magic, h.version, h.mode, h.role = 0x43573441, 1, mode, role
    h.num_experts, h.n, h.k, h.group_size = E, N, K, 32
    h.data, h.bytes = 0x2000, E * N * K * 9 // 16
    return h


def _indexed(h13, h2, T=4, H=256, I=128, k=2, bm=16, max_padded=None, ws=1 << 30, ov=None, null_x=False):
    mp = max_padded if max_padded is not None else T * k + 2 * (bm - 1)
    return C.lib.chord_w4a16_moe_indexed(
        None if null_x else FAKE, T, H, I, ctypes.byref(h13), ctypes.byref(h2), FAKE, FAKE, k, 0, 8,
        FAKE, FAKE, FAKE, mp, bm, FAKE, FAKE, ws, ov, 0, None)


def test_pack_rejects_unsupported_schemes_on_host():
    h = C.Weight()
    assert C.lib.chord_w4a16_pack(0, 0, FAKE, FAKE, 1, 256, 256, 64, FAKE, 1 << 20, ctypes.byref(h), None) == 2
    assert C.lib.chord_w4a16_pack(0, 0, FAKE, FAKE, 1, 256, 200, 32, FAKE, 1 << 20, ctypes.byref(h), None) == 2
    assert C.lib.chord_w4a16_pack(0, 1, None, FAKE, 1, 256, 256, 32, FAKE, 1 << 20, ctypes.byref(h), None) == 1
    assert C.lib.chord_w4a16_pack(0, 1, FAKE, FAKE, 1, 256, 256, 32, FAKE, 10, ctypes.byref(h), None) == 1
    assert C.lib.chord_w4a16_pack(7, 1, FAKE, FAKE, 1, 256, 256, 32, FAKE, 1 << 20, ctypes.byref(h), None) == 1
    assert C.lib.chord_w4a16_pack(0, 0, FAKE, FAKE, 1, 256, 256, 16, FAKE, 1 << 20,
                                  ctypes.byref(h), None) == 2
    assert b"group size" in C.lib.chord_last_error()


def test_layer_rejects_wrong_mode_and_role():
    assert _indexed(_handle(1, 0), _handle(0, 1, N=256, K=128)) == 3      # contiguous weight, indexed call
    assert b"mode" in C.lib.chord_last_error()
    assert _indexed(_handle(0, 1), _handle(0, 1, N=256, K=128)) == 3      # role mismatch


def _aligned():
    # a kernel-1 override keeps a small call on the alignment (not routed)
    s = C.Schedule()
    s.kernel = 1
    return s


def test_layer_host_validation():
    h13, h2 = _handle(0, 0), _handle(0, 1, N=256, K=128)
    ov = _aligned()
    assert _indexed(h13, h2, null_x=True) == 1
    assert _indexed(h13, h2, bm=24, ov=ctypes.byref(ov)) == 1
    assert _indexed(h13, h2, max_padded=3, ov=ctypes.byref(ov)) == 1
    assert _indexed(h13, h2, ws=16) == 4
    assert _indexed(h13, h2, I=64) == 1                                   # shape mismatch with handle
    bad = C.Schedule()
    bad.kernel = 9
    assert _indexed(h13, h2, ov=ctypes.byref(bad)) == 1
    # T == 0 is a no-op that never touches the device
    assert _indexed(h13, h2, T=0) == 0


def test_grouped_rejects_overrides_and_bad_expected_m():
    s = C.Schedule()
    hc13, hc2 = _handle(1, 0), _handle(1, 1, N=256, K=128)
    assert C.lib.chord_w4a16_moe_grouped_contiguous(
        FAKE, 128, FAKE, 0, ctypes.byref(hc13), ctypes.byref(hc2), 256, 128, None, None, 0, 1, None,
        FAKE, None, FAKE, 1 << 30, ctypes.byref(s), 0, None) == 1
    assert b"override" in C.lib.chord_last_error()
    assert C.lib.chord_w4a16_moe_grouped_contiguous(
        FAKE, 100, FAKE, 0, ctypes.byref(hc13), ctypes.byref(hc2), 256, 128, None, None, 0, 1, None,
        FAKE, None, FAKE, 1 << 30, None, 0, None) == 1                    # M % 128
    hm13, hm2 = _handle(2, 0), _handle(2, 1, N=256, K=128)
    assert C.lib.chord_w4a16_moe_grouped_masked(
        FAKE, 2, 16, FAKE, 0, ctypes.byref(hm13), ctypes.byref(hm2), 256, 128, None, FAKE, FAKE,
        1 << 30, None, 0, None) == 1                                      # expected_m <= 0
    assert C.lib.chord_w4a16_moe_grouped_masked(
        FAKE, 2, 16, FAKE, 4, ctypes.byref(hc13), ctypes.byref(hc2), 256, 128, None, FAKE, FAKE,
        1 << 30, None, 0, None) == 3                                      # prefill weight in decode
    assert C.lib.chord_w4a16_moe_grouped_masked(
        FAKE, 3, 16, FAKE, 4, ctypes.byref(hm13), ctypes.byref(hm2), 256, 128, None, FAKE, FAKE,
        1 << 30, None, 0, None) == 1                                      # E mismatch
    assert C.lib.chord_w4a16_moe_grouped_masked(
        FAKE, 2, 16, FAKE, 4, ctypes.byref(hm13), ctypes.byref(hm2), 256, 128, None, FAKE, FAKE,
        64, None, 0, None) == 4                                           # workspace


def test_align_host_validation():
    assert C.lib.chord_moe_align(FAKE, 4, 2, 0, 8, 16, FAKE, FAKE, FAKE, 3, FAKE, 1 << 20, 0, None) == 1
    assert C.lib.chord_moe_align(FAKE, 4, 2, 0, 8, 12, FAKE, FAKE, FAKE, 1000, FAKE, 1 << 20, 0, None) == 1
    assert C.lib.chord_moe_align(FAKE, 4, 2, 0, 0, 16, FAKE, FAKE, FAKE, 1000, FAKE, 1 << 20, 0, None) == 1
    # large inputs need a workspace
    assert C.lib.chord_moe_align(FAKE, 8192, 8, 0, 48, 16, FAKE, FAKE, FAKE, 70000, None, 0, 0, None) == 4


def test_workspace_query_grows_with_rows():
    a = C.chord_w4a16_moe_workspace_bytes(0, 64, 8, 48, 7168, 2048, 1232)
    b = C.chord_w4a16_moe_workspace_bytes(0, 64, 8, 48, 7168, 2048, 5000)
    assert 0 < a < b
    assert C.chord_w4a16_moe_workspace_bytes(0, 64, 8, 0, 7168, 2048, 1232) == 0


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "quantized_moe_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", txt, re.M), f
                assert "oracle/" not in txt, f


def test_dispatch_and_combine_host_validation():
    L = C.lib
    assert C.chord_moe_dispatch_contiguous_rows(64, 8, 48) == (512 + 48 * 127 + 127) // 128 * 128
    ws_c = C.chord_moe_dispatch_workspace_bytes(C.MODE_CONTIGUOUS, 64, 8, 48)
    ws_m = C.chord_moe_dispatch_workspace_bytes(C.MODE_MASKED, 64, 8, 48)
    assert ws_c > 0 and ws_m > 0
    assert C.chord_moe_dispatch_workspace_bytes(C.MODE_INDEXED, 64, 8, 48) == 0
    rows = C.chord_moe_dispatch_contiguous_rows(4, 2, 8)

    def contig(H=256, max_rows=rows, ws=1 << 20, x=FAKE, E=8):
        return L.chord_moe_dispatch_contiguous(x, 4, H, FAKE, 2, 0, E, FAKE, FAKE, max_rows, FAKE,
                                               FAKE, FAKE, ws, None)

    assert contig(max_rows=rows - 128) == 1                 # below the routing-independent bound
    assert contig(max_rows=rows + 1) == 1                   # not a multiple of 128
    assert contig(H=100) == 2                               # H % 8
    assert contig(ws=16) == 4
    assert contig(x=ctypes.c_void_p(0x1008)) == 1           # misaligned rows
    assert contig(E=0) == 1

    def masked(max_m=16, ws=1 << 20, E=8):
        return L.chord_moe_dispatch_masked(FAKE, 4, 256, FAKE, 2, 0, E, max_m, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, ws, None)

    assert masked(max_m=0) == 1
    assert masked(ws=16) == 4
    assert masked(E=1 << 20) in (1, 2)
    assert L.chord_moe_combine(FAKE, 16, 100, FAKE, FAKE, 4, 2, FAKE, None) == 2
    assert L.chord_moe_combine(FAKE, 16, 256, None, FAKE, 4, 2, FAKE, None) == 1
    assert L.chord_moe_combine(FAKE, 1 << 22, 1024, FAKE, FAKE, 4, 2, FAKE, None) == 2
    assert L.chord_moe_combine(FAKE, 16, 256, FAKE, FAKE, 0, 2, FAKE, None) == 0   # no tokens: no-op


def _indexed_noalloc(h13, h2, T=4, H=256, I=128, k=2, bm=16, max_padded=None, ov=None):
    mp = max_padded if max_padded is not None else T * k + h13.num_experts * (bm - 1)
    return C.lib.chord_w4a16_moe_indexed_noalloc(
        FAKE, T, H, I, ctypes.byref(h13), ctypes.byref(h2), FAKE, FAKE, k, 0, 8,
        FAKE, FAKE, FAKE, mp, bm, FAKE, ov, 0, None)


def test_noalloc_entry_point_rejects_misuse_and_oversize_calls_on_the_host():
    """The allocation-free call validates like the workspace one, and a call
    whose scratch would exceed CHORD_NOALLOC_SCRATCH_BYTES (64 MiB) is
    refused before anything touches the device."""
    h13, h2 = _handle(0, 0), _handle(0, 1, N=256, K=128)
    ov = _aligned()
    assert _indexed_noalloc(h13, h2, bm=24, ov=ctypes.byref(ov)) == 1
    assert _indexed_noalloc(h13, h2, max_padded=3, ov=ctypes.byref(ov)) == 1
    assert _indexed_noalloc(_handle(1, 0), h2) == 3
    three = C.Schedule()
    three.kernel = 3
    assert _indexed_noalloc(h13, h2, ov=ctypes.byref(three)) == 1
    assert b"side stream" in C.lib.chord_last_error()
    assert _indexed_noalloc(h13, h2, T=0) == 0
    # the prefill EP share: h and the per-slot rows need far more than 64 MiB
    g13 = _handle(0, 0, E=48, N=4096, K=7168)
    g2 = _handle(0, 1, E=48, N=7168, K=2048)
    need = C.chord_w4a16_moe_workspace_bytes(0, 8192, 8, 48, 7168, 2048,
                                             C.chord_moe_align_max_padded(8192, 8, 48, 16))
    assert need > 64 << 20
    assert _indexed_noalloc(g13, g2, T=8192, H=7168, I=2048, k=8) == 4
    assert b"scratch" in C.lib.chord_last_error()


def test_routed_call_reads_no_alignment():
    """A small indexed call is routed inside the GEMM: null alignment
    pointers pass host validation (the call then stops at the device check,
    CHORD_ERR_HIP here without a GPU), while an aligned schedule override
    still requires them."""
    h13, h2 = _handle(0, 0, N=256, K=384), _handle(0, 1, N=384, K=128)
    assert C.chord_w4a16_moe_indexed_block_m(4, 2, 8, 2, 384, 128) == 0
    r = C.lib.chord_w4a16_moe_indexed(FAKE, 4, 384, 128, ctypes.byref(h13), ctypes.byref(h2),
                                      FAKE, FAKE, 2, 0, 8, None, None, None, 0, 0, FAKE, FAKE,
                                      1 << 30, None, 0, None)
    assert r == 6, C.lib.chord_last_error()
    ov = _aligned()
    r = C.lib.chord_w4a16_moe_indexed(FAKE, 4, 384, 128, ctypes.byref(h13), ctypes.byref(h2),
                                      FAKE, FAKE, 2, 0, 8, None, None, None, 0, 0, FAKE, FAKE,
                                      1 << 30, ctypes.byref(ov), 0, None)
    assert r == 1 and b"alignment" in C.lib.chord_last_error()
