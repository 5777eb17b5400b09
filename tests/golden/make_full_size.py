"""Writes the expected layer outputs of the full-size workloads for the GPU
parity tests (``tests/golden/full_size/<workload>.npz``).

    python tests/golden/make_full_size.py [--jobs 4] [workload ...]

Test infrastructure: it imports only the CPU oracle (``oracle/``) and the
seeded input generators (``moe_inputs/``); no value comes from the HIP path.
Each file holds, for one workload, the rows or tokens it covers, their
expected bf16 outputs from the oracle, and a digest of the generated inputs so
a test can tell when the generators have drifted from the file.

Coverage per workload (positions count an expert's routed rows in the stable
order of the alignment: ascending flat slot id t*k + j):
  * indexed, at most 64 tokens: every token;
  * indexed, more tokens: for every active expert its first and last routed
    row, plus positions 15, 16, 191 and 192 (the edges of the 16-row token
    groups and of the 192-row tiles) for all experts of the EP share and for
    the 8 busiest experts of the TP slices; the outputs are the tokens those
    rows belong to;
  * contiguous: for every expert rows 0, 191, 192 and its last row, plus 15,
    16, 127 and 128 for the 8 busiest experts (rows of the layout);
  * masked: for every expert with rows its first and last row, plus 15, 16,
    191 and 192 for the 8 busiest (rows of the flat output).
"""

from __future__ import annotations

import argparse
import hashlib
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

OUT_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "full_size")
EDGES = (15, 16, 191, 192)
CONTIG_EDGES = (15, 16, 127, 128)


def input_digest(wl) -> str:
    """sha256 over the routing, the activations and the first and last words
    of every weight and scale row (enough to notice a changed generator)."""
    h = hashlib.sha256()
    for a in (wl.x, wl.topk_ids, wl.topk_weights, wl.a3, wl.masked_m):
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    for a in (wl.q13, wl.s13, wl.q2, wl.s2):
        h.update(np.ascontiguousarray(a[..., :2]).tobytes())
        h.update(np.ascontiguousarray(a[..., -2:]).tobytes())
    return h.hexdigest()


def _busiest(counts, n=8):
    return set(int(e) for e in np.argsort(-np.asarray(counts), kind="stable")[:n] if counts[e] > 0)


def indexed_tokens(wl):
    if wl.T <= 64:
        return list(range(wl.T))
    flat = wl.topk_ids.reshape(-1).astype(np.int64) - wl.expert_begin
    counts = np.bincount(flat[(flat >= 0) & (flat < wl.E_l)], minlength=wl.E_l)
    hot = set(range(wl.E_l)) if wl.E_l <= 48 else _busiest(counts)
    toks = set()
    for e in range(wl.E_l):
        members = np.nonzero(flat == e)[0]
        c = members.size
        if c == 0:
            continue
        pos = {0, c - 1} | (set(EDGES) if e in hot else set())
        toks |= {int(members[p]) // wl.k for p in pos if p < c}
    return sorted(toks)


def contiguous_rows(m_idx, E_l):
    counts = np.bincount(m_idx[m_idx >= 0], minlength=E_l)
    hot = _busiest(counts)
    rows = set()
    for e in range(E_l):
        seg = np.nonzero(m_idx == e)[0]
        c = seg.size
        if c == 0:
            continue
        pos = {0, 191, 192, c - 1} | (set(CONTIG_EDGES) if e in hot else set())
        rows |= {int(seg[p]) for p in pos if p < c}
    return sorted(rows)


def masked_rows(masked_m, max_m):
    hot = _busiest(masked_m)
    rows = []
    for e, m in enumerate(np.asarray(masked_m).tolist()):
        if m <= 0:
            continue
        pos = {0, m - 1} | (set(EDGES) if e in hot else set())
        rows += [e * max_m + p for p in sorted(pos) if p < m]
    return rows


def expected(spec):
    """(kind, index, expected bf16 rows, digest) of one workload."""
    import oracle
    from moe_inputs import gen as G
    wl = G.make_workload(spec)
    if wl.layout == "indexed":
        toks = indexed_tokens(wl)
        ref = oracle.moe_layer(wl.x, wl.topk_ids, wl.topk_weights, wl.q13, wl.s13, wl.q2, wl.s2,
                               wl.expert_begin, tokens=toks)
        return "tokens", np.asarray(toks, np.int64), ref, input_digest(wl)
    if wl.layout == "contiguous":
        a, m_idx, _, _ = G.build_contiguous(wl.topk_ids, wl.x, wl.expert_begin, wl.E_l)
        rows = contiguous_rows(m_idx, wl.E_l)
        ref = oracle.grouped_contiguous(a, m_idx, wl.q13, wl.s13, wl.q2, wl.s2, rows=rows)
        return "rows", np.asarray(rows, np.int64), ref, input_digest(wl)
    rows = masked_rows(wl.masked_m, wl.max_m)
    ref = np.zeros((len(rows), wl.H), np.uint16)
    # masked rows are independent: each expert's selected rows go through the
    # oracle as a small masked layer of their own
    by_e = {}
    for i, r in enumerate(rows):
        by_e.setdefault(r // wl.max_m, []).append((i, r % wl.max_m))
    for e, lst in sorted(by_e.items()):
        sub = wl.a3[e:e + 1, [p for _, p in lst]]
        out = oracle.grouped_masked(sub, np.array([len(lst)], np.int32), wl.q13[e:e + 1],
                                    wl.s13[e:e + 1], wl.q2[e:e + 1], wl.s2[e:e + 1])
        ref[[i for i, _ in lst]] = out[:len(lst)]
    return "rows", np.asarray(rows, np.int64), ref, input_digest(wl)


def path_for(name):
    return os.path.join(OUT_DIR, f"{name}.npz")


def write_one(name):
    from moe_inputs.configs import workload_by_name
    t0 = time.time()
    kind, index, ref, digest = expected(workload_by_name(name))
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = path_for(name) + ".tmp.npz"
    np.savez_compressed(tmp, kind=np.array(kind), index=index, expected=ref,
                        digest=np.array(digest))
    os.replace(tmp, path_for(name))
    return f"{name}: {len(index)} {kind}, {os.path.getsize(path_for(name)) / 1e6:.2f} MB, " \
           f"{time.time() - t0:.0f} s"


def load(name):
    """(kind, index, expected, digest) stored for a workload."""
    with np.load(path_for(name), allow_pickle=False) as z:
        return str(z["kind"]), z["index"], z["expected"], str(z["digest"])


FULL_SIZE = ["kimi_decode_T64_ep48of384_top8", "kimi_prefill_T8192_ep48of384_top8",
             "kimi_prefill_T8192_ep48of384_top8_contiguous",
             "kimi_tp8slice_T1_all384_I256_top8", "kimi_tp8slice_T32_all384_I256_top8",
             "kimi_tp8slice_T512_all384_I256_top8", "kimi_tp8slice_T4096_all384_I256_top8",
             "kimi_masked_zipf_E48_maxm256", "kimi_masked_zipf_E96_maxm256",
             "kimi_masked_zipf_E24_maxm256"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("names", nargs="*", default=FULL_SIZE)
    args = ap.parse_args()
    os.environ.setdefault("OMP_NUM_THREADS", "2")
    with mp.get_context("spawn").Pool(args.jobs) as pool:
        for line in pool.imap_unordered(write_one, args.names):
            print(line, flush=True)


if __name__ == "__main__":
    main()
