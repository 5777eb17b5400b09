"""Python-side convenience over the C ABI: a layer object that owns its packed
weights and a reusable workspace.  Marshalling only -- every step runs in
libchord.so's kernels.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import chord as C


class W4A16MoE:
    """One GPU's share of a W4A16 MoE layer.

    q13: int32 [E_l, 2I, H/8], s13: bf16 [E_l, 2I, H/32]  (gate rows first)
    q2:  int32 [E_l, H, I/8],  s2:  bf16 [E_l, H, I/32]
    Canonical packing: 8 codes per int32 along K, low nibble first; weight =
    (code - 8) * scale per group of 32.  ``mode`` is the entry point the packed
    weights are prepared for (indexed, contiguous or masked).
    """

    def __init__(self, q13, s13, q2, s2, mode: int = C.MODE_INDEXED):
        self.E_l, n13, h8 = q13.shape
        self.I = n13 // 2
        self.H = h8 * 8
        self.mode = mode
        self.w13 = C.chord_w4a16_pack(mode, C.ROLE_GATE_UP, q13, s13)
        self.w2 = C.chord_w4a16_pack(mode, C.ROLE_DOWN, q2, s2)
        self._ws: Optional[torch.Tensor] = None

    def workspace(self, nbytes: int, device) -> torch.Tensor:
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        return self._ws

    def indexed(self, x, topk_ids, topk_weights, expert_begin=0, num_global_experts=0,
                block_m: Optional[int] = None, align=None, out=None, override=None, flags=0,
                stream=None):
        """Aligns the routing (unless ``align`` = (sorted_ids, expert_ids,
        ntpp, block_m) is given, or the planner routes the call inside the
        GEMM: block_m 0) and runs the indexed layer."""
        assert self.mode == C.MODE_INDEXED
        T, k = topk_ids.shape
        if align is None:
            bm = block_m if block_m is not None else C.chord_w4a16_moe_indexed_block_m(
                T, k, num_global_experts or self.E_l, self.E_l, self.H, self.I)
            if bm == 0 and override is None:
                sorted_ids = expert_ids = ntpp = None
            else:
                bm = bm or 16
                sorted_ids, expert_ids, ntpp = C.chord_moe_align(topk_ids, expert_begin, self.E_l,
                                                                 bm, stream=stream)
        else:
            sorted_ids, expert_ids, ntpp, bm = align
        ws = self.workspace(C.chord_w4a16_moe_workspace_bytes(
            C.MODE_INDEXED, T, k, self.E_l, self.H, self.I,
            0 if sorted_ids is None else sorted_ids.numel()), x.device)
        return C.chord_w4a16_moe_indexed(x, self.w13, self.w2, topk_ids, topk_weights, expert_begin,
                                         num_global_experts, sorted_ids, expert_ids, ntpp, bm,
                                         out=out, workspace=ws, override=override, flags=flags,
                                         stream=stream)

    def contiguous(self, a, m_indices, valid_m_hint=0, row_weights=None, flat_to_row=None,
                   topk_weights=None, out_rows=None, out_tokens=None, flags=0, stream=None):
        assert self.mode == C.MODE_CONTIGUOUS
        M = a.shape[0]
        T, k = (topk_weights.shape if topk_weights is not None else (0, 1))
        ws = self.workspace(C.chord_w4a16_moe_workspace_bytes(C.MODE_CONTIGUOUS, T, k, self.E_l,
                                                             self.H, self.I, M), a.device)
        return C.chord_w4a16_moe_grouped_contiguous(
            a, m_indices, self.w13, self.w2, valid_m_hint, row_weights, flat_to_row, topk_weights,
            out_rows, out_tokens, workspace=ws, flags=flags, stream=stream)

    def masked(self, a3, masked_m, expected_m, row_weights=None, out=None, flags=0, stream=None):
        assert self.mode == C.MODE_MASKED
        E, max_m, _ = a3.shape
        ws = self.workspace(C.chord_w4a16_moe_workspace_bytes(C.MODE_MASKED, 0, 0, E, self.H,
                                                             self.I, E * max_m), a3.device)
        return C.chord_w4a16_moe_grouped_masked(a3, masked_m, expected_m, self.w13, self.w2,
                                                row_weights, out, workspace=ws, flags=flags,
                                                stream=stream)
