"""GPU parity at the full workload sizes, in the launch configuration the
benchmark uses, against expected outputs the CPU oracle wrote beforehand
(``tests/golden/make_full_size.py``; those files record which rows or tokens
they cover and a digest of the generated inputs).

Indexed workloads: every token of the decode batch and of the small TP
slices; for the larger ones the tokens that hold each active expert's first
and last routed row and the rows at the 16-row group and 192-row tile edges.
Every token without a local slot must be exactly zero.  Contiguous and masked
layouts: the same row positions of every expert with rows.
"""

import numpy as np
import pytest
import torch

from moe_inputs import gen as G
from moe_inputs.configs import workload_by_name
from tests.golden import make_full_size as golden
from tests.gpu_util import banner, dev, dev_bf16, host_bf16
from tests.tolerance import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C():
    from quantized_moe_amd import chord
    return chord


def _load_checked(name, wl):
    kind, index, expected, digest = golden.load(name)
    assert digest == golden.input_digest(wl), \
        f"{name}: the generated inputs no longer match the stored expected values " \
        "(re-run tests/golden/make_full_size.py)"
    return kind, index, expected


def _run_indexed(C, wl):
    from quantized_moe_amd.moe import W4A16MoE
    layer = W4A16MoE(dev(wl.q13), dev_bf16(wl.s13), dev(wl.q2), dev_bf16(wl.s2))
    bm = C.chord_w4a16_moe_indexed_block_m(wl.T, wl.k, wl.E_g, wl.E_l, wl.H, wl.I)
    ids = dev(wl.topk_ids)
    if bm:
        mp = C.chord_moe_align_max_padded(wl.T, wl.k, wl.E_l, bm)
        al = C.chord_moe_align(ids, wl.expert_begin, wl.E_l, bm, max_padded=mp)
    else:                                # routed inside the GEMM: no alignment
        al = (None, None, None)
    out = layer.indexed(dev_bf16(wl.x), ids, dev(wl.topk_weights), wl.expert_begin, wl.E_g,
                        align=(*al, bm))
    torch.cuda.synchronize()
    plan = C.last_plan()
    got = host_bf16(out)
    del layer, out, al
    torch.cuda.empty_cache()
    return got, plan


@pytest.mark.parametrize("name", [n for n in golden.FULL_SIZE
                                  if workload_by_name(n).layout == "indexed"])
def test_indexed_full_size(C, name):
    spec = workload_by_name(name)
    banner(f"full size {name}: drawing inputs")
    wl = G.make_workload(spec)
    kind, toks, exp = _load_checked(name, wl)
    assert kind == "tokens"
    banner(f"full size {name}: GPU run")
    got, plan = _run_indexed(C, wl)
    banner(f"  plan {plan}; comparing {len(toks)} tokens")
    st = check_close(got[toks], exp, name)
    banner(f"  {st}")
    assert np.all(np.isfinite(got.view(np.int16).astype(np.float64)))
    local = (wl.topk_ids >= wl.expert_begin) & (wl.topk_ids < wl.expert_begin + wl.E_l)
    none = ~np.any(local, axis=1)
    assert np.all(got[none] == 0)
    # every active expert is represented by at least one compared token
    flat = (wl.topk_ids[toks] - wl.expert_begin).reshape(-1)
    active = set(np.unique((wl.topk_ids - wl.expert_begin)[local]).tolist())
    assert active <= set(flat[(flat >= 0) & (flat < wl.E_l)].tolist())


def test_contiguous_prefill_full_size(C):
    from quantized_moe_amd.moe import W4A16MoE
    name = "kimi_prefill_T8192_ep48of384_top8_contiguous"
    banner(f"full size {name}: drawing inputs")
    wl = G.make_workload(workload_by_name(name))
    kind, rows, exp = _load_checked(name, wl)
    assert kind == "rows"
    a, m_idx, _, nvalid = G.build_contiguous(wl.topk_ids, wl.x, wl.expert_begin, wl.E_l)
    layer = W4A16MoE(dev(wl.q13), dev_bf16(wl.s13), dev(wl.q2), dev_bf16(wl.s2),
                     mode=C.MODE_CONTIGUOUS)
    banner(f"full size {name}: GPU run M={a.shape[0]}")
    out_rows, _ = layer.contiguous(dev_bf16(a), dev(m_idx), nvalid)
    torch.cuda.synchronize()
    got = host_bf16(out_rows)
    del layer, out_rows
    torch.cuda.empty_cache()
    banner(f"  comparing {len(rows)} rows")
    st = check_close(got[rows], exp, name)
    banner(f"  {st}")
    assert set(np.unique(m_idx[rows]).tolist()) == set(np.unique(m_idx[m_idx >= 0]).tolist())
    valid = m_idx >= 0
    assert np.all(np.isfinite(got[valid].view(np.int16).astype(np.float64)))


@pytest.mark.parametrize("name", [n for n in golden.FULL_SIZE
                                  if workload_by_name(n).layout == "masked"])
def test_masked_full_size(C, name):
    from quantized_moe_amd.moe import W4A16MoE
    banner(f"full size {name}: drawing inputs")
    wl = G.make_workload(workload_by_name(name))
    kind, rows, exp = _load_checked(name, wl)
    assert kind == "rows"
    layer = W4A16MoE(dev(wl.q13), dev_bf16(wl.s13), dev(wl.q2), dev_bf16(wl.s2),
                     mode=C.MODE_MASKED)
    banner(f"full size {name}: GPU run")
    out = layer.masked(dev_bf16(wl.a3), dev(wl.masked_m), wl.expected_m)
    torch.cuda.synchronize()
    banner(f"  plan {C.last_plan()}; comparing {len(rows)} rows")
    got = host_bf16(out)
    del layer, out
    torch.cuda.empty_cache()
    st = check_close(got[rows], exp, name)
    banner(f"  {st}")
    with_rows = set(np.nonzero(wl.masked_m > 0)[0].tolist())
    assert set((np.asarray(rows) // wl.max_m).tolist()) == with_rows
