"""GPU parity on randomly drawn small shapes: the indexed layer through the C
ABI against the CPU oracle, over ragged token counts, hidden and
intermediate sizes (multiples of 128), expert windows, top-k, alignment
block sizes and all kernel-family choices of the planner (automatic,
streaming, tiled, both split at the row threshold).  Every case is seeded;
the banner names it before the GPU runs it.
"""

import numpy as np
import pytest

import oracle
import tests.test_gpu_parity as parity
from tests.gpu_util import banner
from tests.test_gpu_parity import small_case, run_indexed
from tests.tolerance import check_close

pytestmark = pytest.mark.gpu

import os

# Cases per sweep; CHORD_RANDOM_CASES widens them for a longer run.
N_CASES = int(os.environ.get("CHORD_RANDOM_CASES", "16"))
N_MASKED = max(12, N_CASES * 3 // 4)


def setup_module(module):
    # run_indexed reaches the library through the parity module's handle.
    from quantized_moe_amd import chord
    parity.C = chord


def draw_case(seed):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    H = int(rng.choice([128, 256, 384, 512, 640]))
    I = int(rng.choice([128, 256, 384]))
    E_g = int(rng.integers(2, 65))
    E_l = int(rng.integers(1, E_g + 1))
    eb = int(rng.integers(0, E_g - E_l + 1))
    k = int(rng.integers(1, min(8, E_g) + 1))
    T = int(rng.integers(1, 301))
    bm = int(rng.choice([16, 32, 64]))
    kernel = int(rng.integers(0, 4))
    extra = int(rng.choice([0, 0, 37]))
    return dict(T=T, H=H, I=I, E_g=E_g, E_l=E_l, k=k, eb=eb, bm=bm, kernel=kernel, extra=extra)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_indexed_random_shapes(seed):
    c = draw_case(seed)
    banner(f"random indexed case {seed}: {c}")
    case = small_case(2000 + seed, c["T"], c["H"], c["I"], c["E_g"], c["E_l"], c["k"], c["eb"])
    override = {"kernel": c["kernel"]} if c["kernel"] else None
    got, _, al = run_indexed(*case, E_g=c["E_g"], bm=c["bm"], extra=c["extra"], override=override)
    ref = oracle.moe_layer(*case)
    check_close(got, ref, what=f"random case {seed}")
    # The alignment that fed the layer equals the oracle's, bit for bit.
    sorted_ids, expert_ids, ntpp = (a.cpu().numpy() for a in al)
    ref_sorted, ref_experts, ref_ntpp = oracle.moe_align(case[1], c["eb"], c["E_l"], c["bm"],
                                                         sorted_ids.shape[0])
    assert int(ntpp[0]) == int(ref_ntpp)
    assert np.array_equal(sorted_ids, ref_sorted)
    assert np.array_equal(expert_ids, ref_experts)
    # The host-only planner query names the schedule the call took.
    import torch
    C = parity.C
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert C.last_plan() == C.chord_w4a16_moe_plan(
        C.MODE_INDEXED, c["T"], c["k"], c["E_g"], c["E_l"], c["H"], c["I"], c["bm"],
        sorted_ids.shape[0], num_cus=cus, override=override)
    # A call the planner routes inside the GEMM gives the same output bit for
    # bit without any alignment.
    if override is None and C.chord_w4a16_moe_indexed_block_m(
            c["T"], c["k"], c["E_g"], c["E_l"], c["H"], c["I"]) == 0:
        assert "tiles=routed" in C.last_plan()
        bare, _ = parity.run_routed(*case, E_g=c["E_g"])
        assert np.array_equal(bare, got)


def draw_masked_case(seed):
    rng = np.random.Generator(np.random.PCG64(5000 + seed))
    E = int(rng.integers(1, 25))
    max_m = int(rng.choice([16, 40, 64, 200, 256]))
    H = int(rng.choice([128, 384, 512, 768]))
    I = int(rng.choice([128, 256, 384, 512]))
    pattern = int(rng.integers(0, 3))  # 0: uniform, 1: one hot expert, 2: empty and full experts
    if pattern == 0:
        mm = rng.integers(0, max_m + 1, E)
    elif pattern == 1:
        mm = rng.integers(0, max(2, max_m // 8), E)
        mm[int(rng.integers(0, E))] = max_m
    else:
        mm = rng.choice([0, max_m, int(rng.integers(1, max_m + 1))], E)
    expected_m = int(rng.integers(1, max_m + 1))
    return dict(E=E, max_m=max_m, H=H, I=I, mm=mm.astype(np.int32), expected_m=expected_m,
                pattern=pattern)


@pytest.mark.parametrize("seed", range(N_MASKED))
def test_masked_random_shapes(seed):
    from quantized_moe_amd import chord as C
    from quantized_moe_amd.moe import W4A16MoE
    from moe_inputs import gen as G
    from tests.gpu_util import dev, dev_bf16, host_bf16
    c = draw_masked_case(seed)
    banner(f"random masked case {seed}: E={c['E']} max_m={c['max_m']} H={c['H']} I={c['I']} "
           f"pattern={c['pattern']} expected_m={c['expected_m']} masked_m={c['mm'].tolist()}")
    rng = np.random.Generator(np.random.PCG64(7000 + seed))
    E, max_m, H, I, mm = c["E"], c["max_m"], c["H"], c["I"], c["mm"]
    a3 = G.draw_activations(rng, E * max_m, H).reshape(E, max_m, H)
    q13, s13 = G.draw_weights(rng, E, 2 * I, H, scale_mult=(256.0 / H) ** 0.5)
    q2, s2 = G.draw_weights(rng, E, H, I, scale_mult=(256.0 / I) ** 0.5)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2), mode=C.MODE_MASKED)
    got = host_bf16(layer.masked(dev_bf16(a3), dev(mm), c["expected_m"]))
    ref = oracle.grouped_masked(a3, mm, q13, s13, q2, s2)
    valid = np.zeros(E * max_m, bool)
    for e in range(E):
        valid[e * max_m:e * max_m + int(mm[e])] = True
    check_close(got[valid], ref[valid], what=f"random masked case {seed}")


def draw_routed_case(seed):
    rng = np.random.Generator(np.random.PCG64(9000 + seed))
    H = int(rng.choice([384, 512, 640, 1024]))
    I = int(rng.choice([128, 256, 384, 512, 1024]))
    E_g = int(rng.integers(4, 129))
    E_l = int(rng.integers(1, E_g + 1))
    eb = int(rng.integers(0, E_g - E_l + 1))
    k = int(rng.integers(1, min(8, E_g) + 1))
    T = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 257))]))
    return dict(T=T, H=H, I=I, E_g=E_g, E_l=E_l, k=k, eb=eb)


N_ROUTED = max(8, N_CASES // 2)


@pytest.mark.parametrize("seed", range(N_ROUTED))
def test_routed_random_shapes(seed):
    """Calls the planner routes inside the GEMM, with no alignment at all:
    within tolerance of the oracle; unless the down GEMM and the combine are
    fused, bit for bit equal to the same schedule run on an alignment."""
    C = parity.C
    c = draw_routed_case(seed)
    banner(f"random routed case {seed}: {c}")
    case = small_case(3000 + seed, c["T"], c["H"], c["I"], c["E_g"], c["E_l"], c["k"], c["eb"])
    bm = C.chord_w4a16_moe_indexed_block_m(c["T"], c["k"], c["E_g"], c["E_l"], c["H"], c["I"])
    if bm:  # the planner aligns this shape: the aligned call against the oracle
        got, _, _ = run_indexed(*case, E_g=c["E_g"], bm=bm)
        check_close(got, oracle.moe_layer(*case), what=f"random routed-draw case {seed}")
        return
    got, layer = parity.run_routed(*case, E_g=c["E_g"])
    plan = C.last_plan()
    assert "tiles=routed" in plan, plan
    check_close(got, oracle.moe_layer(*case), what=f"random routed case {seed}")
    if "down+combine" not in plan:
        aligned, _, _ = run_indexed(*case, E_g=c["E_g"], bm=16, layer=layer,
                                    override={"kernel": 1})
        assert np.array_equal(got, aligned)
