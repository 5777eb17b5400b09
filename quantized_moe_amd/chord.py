"""ctypes binding of libchord.so (see include/chord.h for the contract).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  If the
library is missing this module raises on import -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libchord.so")

CHORD_OK = 0
STATUS_NAMES = {0: "CHORD_OK", 1: "CHORD_ERR_INVALID_ARGUMENT", 2: "CHORD_ERR_UNSUPPORTED",
                3: "CHORD_ERR_LAYOUT_MISMATCH", 4: "CHORD_ERR_WORKSPACE", 5: "CHORD_ERR_ROUTING",
                6: "CHORD_ERR_HIP"}
MODE_INDEXED, MODE_CONTIGUOUS, MODE_MASKED = 0, 1, 2
ROLE_GATE_UP, ROLE_DOWN = 0, 1
FLAG_VALIDATE = 1

EXPORTED = [
    "chord_status_string", "chord_last_error", "chord_last_plan", "chord_version",
    "chord_profile_enable", "chord_profile_reset", "chord_profile_read",
    "chord_w4a16_packed_bytes", "chord_w4a16_pack", "chord_moe_align_max_padded",
    "chord_moe_align_workspace_bytes", "chord_moe_align", "chord_w4a16_moe_indexed_block_m",
    "chord_w4a16_moe_workspace_bytes", "chord_w4a16_moe_indexed", "chord_w4a16_moe_indexed_noalloc",
    "chord_w4a16_moe_grouped_contiguous", "chord_w4a16_moe_grouped_masked",
    "chord_moe_dispatch_contiguous_rows", "chord_moe_dispatch_workspace_bytes",
    "chord_moe_dispatch_contiguous", "chord_moe_dispatch_masked", "chord_moe_combine",
    "chord_w4a16_moe_plan",
]


class ChordError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


class Weight(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("mode", ctypes.c_int32),
                ("role", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("group_size", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("bytes", ctypes.c_size_t)]


class Schedule(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("tokens", ctypes.c_int32),
                ("gate_up_nt", ctypes.c_int32), ("gate_up_wk", ctypes.c_int32),
                ("down_nt", ctypes.c_int32), ("down_wk", ctypes.c_int32),
                ("prefetch", ctypes.c_int32), ("tile_split", ctypes.c_int32)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m quantized_moe_amd.build` "
                          "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, I64, SZ, U32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint32
    WP = ctypes.POINTER(Weight)
    sig = {
        "chord_status_string": (ctypes.c_char_p, [I]),
        "chord_last_error": (ctypes.c_char_p, []),
        "chord_last_plan": (I, [ctypes.c_char_p, SZ]),
        "chord_version": (ctypes.c_char_p, []),
        "chord_profile_enable": (I, [I]),
        "chord_profile_reset": (I, []),
        "chord_profile_read": (I, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
        "chord_w4a16_packed_bytes": (SZ, [I, I, I, I, I]),
        "chord_w4a16_pack": (I, [I, I, P, P, I, I, I, I, P, SZ, WP, P]),
        "chord_moe_align_max_padded": (I64, [I, I, I, I]),
        "chord_moe_align_workspace_bytes": (SZ, [I, I, I, I]),
        "chord_moe_align": (I, [P, I, I, I, I, I, P, P, P, I64, P, SZ, U32, P]),
        "chord_w4a16_moe_indexed_block_m": (I, [I, I, I, I, I, I]),
        "chord_w4a16_moe_workspace_bytes": (SZ, [I, I, I, I, I, I, I64]),
        "chord_w4a16_moe_indexed": (I, [P, I, I, I, WP, WP, P, P, I, I, I, P, P, P, I64, I, P, P, SZ,
                                        ctypes.POINTER(Schedule), U32, P]),
        "chord_w4a16_moe_indexed_noalloc": (I, [P, I, I, I, WP, WP, P, P, I, I, I, P, P, P, I64, I, P,
                                                ctypes.POINTER(Schedule), U32, P]),
        "chord_w4a16_moe_grouped_contiguous": (I, [P, I64, P, I64, WP, WP, I, I, P, P, I, I, P, P, P,
                                                   P, SZ, ctypes.POINTER(Schedule), U32, P]),
        "chord_w4a16_moe_grouped_masked": (I, [P, I, I, P, I, WP, WP, I, I, P, P, P, SZ,
                                               ctypes.POINTER(Schedule), U32, P]),
        "chord_moe_dispatch_contiguous_rows": (I64, [I, I, I]),
        "chord_moe_dispatch_workspace_bytes": (SZ, [I, I, I, I]),
        "chord_moe_dispatch_contiguous": (I, [P, I, I, P, I, I, I, P, P, I64, P, P, P, SZ, P]),
        "chord_moe_dispatch_masked": (I, [P, I, I, P, I, I, I, I, P, P, P, P, P, SZ, P]),
        "chord_moe_combine": (I, [P, I64, I, P, P, I, I, P, P]),
        "chord_w4a16_moe_plan": (I, [I, I, I, I, I, I, I, I, I64, I, ctypes.POINTER(Schedule),
                                     ctypes.c_char_p, SZ]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int):
    if status != CHORD_OK:
        raise ChordError(status, lib.chord_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def last_plan() -> str:
    buf = ctypes.create_string_buffer(512)
    lib.chord_last_plan(buf, 512)
    return buf.value.decode()


def chord_profile_enable(on: bool = True):
    _check(lib.chord_profile_enable(1 if on else 0))


def chord_profile_reset():
    _check(lib.chord_profile_reset())


def chord_profile_read():
    """Returns (stage_ms[4] summed over calls: tiles, gate_up, down, combine; calls)."""
    ms = (ctypes.c_double * 4)()
    n = ctypes.c_int64()
    _check(lib.chord_profile_read(ms, ctypes.byref(n)))
    return list(ms), n.value


def version() -> str:
    return lib.chord_version().decode()


class PackedWeight:
    """A packed weight: the host handle plus the torch buffer that owns its bytes."""

    def __init__(self, handle: Weight, buf: torch.Tensor):
        self.handle = handle
        self.buf = buf

    @property
    def num_experts(self):
        return self.handle.num_experts


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def chord_w4a16_packed_bytes(mode: int, role: int, E: int, N: int, K: int) -> int:
    return lib.chord_w4a16_packed_bytes(mode, role, E, N, K)


def chord_w4a16_pack(mode: int, role: int, qweight: torch.Tensor, scales: torch.Tensor,
                     group_size: int = 32, stream=None) -> PackedWeight:
    """qweight int32 [E,N,K/8], scales bf16 [E,N,K/32] (device tensors)."""
    E, N, K8 = qweight.shape
    K = K8 * 8
    nbytes = lib.chord_w4a16_packed_bytes(mode, role, E, N, K)
    buf = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=qweight.device)
    h = Weight()
    _check(lib.chord_w4a16_pack(mode, role, _ptr(qweight), _ptr(scales), E, N, K, group_size,
                                _ptr(buf), nbytes, ctypes.byref(h), _stream(stream)))
    return PackedWeight(h, buf)


def chord_moe_align_max_padded(T: int, k: int, E_l: int, block_m: int) -> int:
    return lib.chord_moe_align_max_padded(T, k, E_l, block_m)


def chord_moe_align(topk_ids: torch.Tensor, expert_begin: int, num_local_experts: int,
                    block_m: int, max_padded: Optional[int] = None, out=None, workspace=None,
                    flags: int = 0, stream=None):
    """Returns (sorted_ids, expert_ids, num_tokens_post_padded) device int32 tensors."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    if max_padded is None:
        max_padded = lib.chord_moe_align_max_padded(T, k, num_local_experts, block_m)
    if out is None:
        sorted_ids = torch.empty(max_padded, dtype=torch.int32, device=dev)
        expert_ids = torch.empty((max_padded + block_m - 1) // block_m, dtype=torch.int32, device=dev)
        ntpp = torch.empty(1, dtype=torch.int32, device=dev)
    else:
        sorted_ids, expert_ids, ntpp = out
    ws_bytes = lib.chord_moe_align_workspace_bytes(T, k, num_local_experts, block_m)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(lib.chord_moe_align(_ptr(topk_ids), T, k, expert_begin, num_local_experts, block_m,
                               _ptr(sorted_ids), _ptr(expert_ids), _ptr(ntpp), max_padded,
                               _ptr(workspace), workspace.numel(), flags, _stream(stream)))
    return sorted_ids, expert_ids, ntpp


def chord_w4a16_moe_indexed_block_m(T, k, E_g, E_l, H, I) -> int:
    return lib.chord_w4a16_moe_indexed_block_m(T, k, E_g, E_l, H, I)


def chord_w4a16_moe_workspace_bytes(mode, T, k, E_l, H, I, rows) -> int:
    return lib.chord_w4a16_moe_workspace_bytes(mode, T, k, E_l, H, I, rows)


def _sched(override):
    if override is None:
        return None
    s = Schedule()
    for name, _ in Schedule._fields_:
        setattr(s, name, int(override.get(name, 0)))
    return ctypes.byref(s)


def chord_w4a16_moe_plan(mode, T, k, num_global_experts, E_l, H, I, hint, rows, num_cus=0,
                         override=None) -> str:
    """The schedule a layer call with this descriptor would choose (host only)."""
    buf = ctypes.create_string_buffer(512)
    _check(lib.chord_w4a16_moe_plan(mode, T, k, num_global_experts, E_l, H, I, hint, rows,
                                    num_cus, _sched(override), buf, 512))
    return buf.value.decode()


def chord_w4a16_moe_indexed(x, w13: PackedWeight, w2: PackedWeight, topk_ids, topk_weights,
                            expert_begin, num_global_experts, sorted_ids, expert_ids, ntpp,
                            block_m, out=None, workspace=None, override=None, flags=0, stream=None):
    T, H = x.shape
    I = w2.handle.k
    k = topk_ids.shape[1]
    max_padded = 0 if sorted_ids is None else sorted_ids.numel()
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    ws_bytes = lib.chord_w4a16_moe_workspace_bytes(MODE_INDEXED, T, k, w13.num_experts, H, I,
                                                   max_padded)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    _check(lib.chord_w4a16_moe_indexed(
        _ptr(x), T, H, I, ctypes.byref(w13.handle), ctypes.byref(w2.handle), _ptr(topk_ids),
        _ptr(topk_weights), k, expert_begin, num_global_experts, _ptr(sorted_ids), _ptr(expert_ids),
        _ptr(ntpp), max_padded, block_m, _ptr(out), _ptr(workspace), workspace.numel(),
        _sched(override), flags, _stream(stream)))
    return out


def chord_w4a16_moe_indexed_noalloc(x, w13: PackedWeight, w2: PackedWeight, topk_ids,
                                    topk_weights, expert_begin, num_global_experts, sorted_ids,
                                    expert_ids, ntpp, block_m, out, override=None, flags=0,
                                    stream=None):
    """The allocation-free indexed layer: no workspace, and `out` must be
    given (this wrapper allocates nothing either)."""
    T, H = x.shape
    I = w2.handle.k
    k = topk_ids.shape[1]
    _check(lib.chord_w4a16_moe_indexed_noalloc(
        _ptr(x), T, H, I, ctypes.byref(w13.handle), ctypes.byref(w2.handle), _ptr(topk_ids),
        _ptr(topk_weights), k, expert_begin, num_global_experts, _ptr(sorted_ids), _ptr(expert_ids),
        _ptr(ntpp), 0 if sorted_ids is None else sorted_ids.numel(), block_m, _ptr(out),
        _sched(override), flags, _stream(stream)))
    return out


def chord_w4a16_moe_grouped_contiguous(a, m_indices, w13: PackedWeight, w2: PackedWeight,
                                       valid_m_hint=0, row_weights=None, flat_to_row=None,
                                       topk_weights=None, out_rows=None, out_tokens=None,
                                       workspace=None, override=None, flags=0, stream=None):
    M, H = a.shape
    I = w2.handle.k
    T, k = (topk_weights.shape if topk_weights is not None else (0, 1))
    if out_rows is None:
        out_rows = torch.empty((M, H), dtype=torch.bfloat16, device=a.device)
    ws_bytes = lib.chord_w4a16_moe_workspace_bytes(MODE_CONTIGUOUS, T, k, w13.num_experts, H, I, M)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=a.device)
    _check(lib.chord_w4a16_moe_grouped_contiguous(
        _ptr(a), M, _ptr(m_indices), valid_m_hint, ctypes.byref(w13.handle), ctypes.byref(w2.handle),
        H, I, _ptr(row_weights), _ptr(flat_to_row), T, k, _ptr(topk_weights), _ptr(out_rows),
        _ptr(out_tokens), _ptr(workspace), workspace.numel(), _sched(override), flags,
        _stream(stream)))
    return out_rows, out_tokens


def chord_w4a16_moe_grouped_masked(a3, masked_m, expected_m, w13: PackedWeight, w2: PackedWeight,
                                   row_weights=None, out=None, workspace=None, override=None,
                                   flags=0, stream=None):
    E, max_m, H = a3.shape
    I = w2.handle.k
    if out is None:
        out = torch.empty((E * max_m, H), dtype=torch.bfloat16, device=a3.device)
    ws_bytes = lib.chord_w4a16_moe_workspace_bytes(MODE_MASKED, 0, 0, E, H, I, E * max_m)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=a3.device)
    _check(lib.chord_w4a16_moe_grouped_masked(
        _ptr(a3), E, max_m, _ptr(masked_m), expected_m, ctypes.byref(w13.handle),
        ctypes.byref(w2.handle), H, I, _ptr(row_weights), _ptr(out), _ptr(workspace),
        workspace.numel(), _sched(override), flags, _stream(stream)))
    return out


def chord_moe_dispatch_contiguous_rows(T: int, k: int, E_l: int) -> int:
    return lib.chord_moe_dispatch_contiguous_rows(T, k, E_l)


def chord_moe_dispatch_workspace_bytes(mode: int, T: int, k: int, E_l: int) -> int:
    return lib.chord_moe_dispatch_workspace_bytes(mode, T, k, E_l)


def chord_moe_dispatch_contiguous(x, topk_ids, expert_begin: int, num_local_experts: int,
                                  max_rows: Optional[int] = None, out=None, workspace=None,
                                  stream=None):
    """Returns (a [max_rows, H], m_indices [max_rows], flat_to_row [T*k], num_rows [1])."""
    T, H = x.shape
    k = topk_ids.shape[1]
    dev = x.device
    if max_rows is None:
        max_rows = lib.chord_moe_dispatch_contiguous_rows(T, k, num_local_experts)
    if out is None:
        a = torch.empty((max_rows, H), dtype=torch.bfloat16, device=dev)
        m_indices = torch.empty(max_rows, dtype=torch.int32, device=dev)
        flat_to_row = torch.empty(T * k, dtype=torch.int32, device=dev)
        num_rows = torch.empty(1, dtype=torch.int32, device=dev)
    else:
        a, m_indices, flat_to_row, num_rows = out
    if workspace is None:
        ws = lib.chord_moe_dispatch_workspace_bytes(MODE_CONTIGUOUS, T, k, num_local_experts)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    _check(lib.chord_moe_dispatch_contiguous(
        _ptr(x), T, H, _ptr(topk_ids), k, expert_begin, num_local_experts, _ptr(a),
        _ptr(m_indices), max_rows, _ptr(flat_to_row), _ptr(num_rows), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return a, m_indices, flat_to_row, num_rows


def chord_moe_dispatch_masked(x, topk_ids, expert_begin: int, num_local_experts: int, max_m: int,
                              out=None, workspace=None, stream=None):
    """Returns (a3 [E_l, max_m, H], masked_m [E_l], flat_to_row [T*k], dropped [1])."""
    T, H = x.shape
    k = topk_ids.shape[1]
    dev = x.device
    if out is None:
        a3 = torch.empty((num_local_experts, max_m, H), dtype=torch.bfloat16, device=dev)
        masked_m = torch.empty(num_local_experts, dtype=torch.int32, device=dev)
        flat_to_row = torch.empty(T * k, dtype=torch.int32, device=dev)
        dropped = torch.empty(1, dtype=torch.int32, device=dev)
    else:
        a3, masked_m, flat_to_row, dropped = out
    if workspace is None:
        ws = lib.chord_moe_dispatch_workspace_bytes(MODE_MASKED, T, k, num_local_experts)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    _check(lib.chord_moe_dispatch_masked(
        _ptr(x), T, H, _ptr(topk_ids), k, expert_begin, num_local_experts, max_m, _ptr(a3),
        _ptr(masked_m), _ptr(flat_to_row), _ptr(dropped), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return a3, masked_m, flat_to_row, dropped


def chord_moe_combine(rows, flat_to_row, topk_weights, out=None, stream=None):
    """out[t] = bf16(sum_j topk_weights[t,j] * rows[flat_to_row[t*k+j]]) over slots with a row."""
    n_rows, H = rows.shape
    T, k = topk_weights.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=rows.device)
    _check(lib.chord_moe_combine(_ptr(rows), n_rows, H, _ptr(flat_to_row), _ptr(topk_weights), T, k,
                                 _ptr(out), _stream(stream)))
    return out
