"""The allocation-free indexed entry point (chord_w4a16_moe_indexed_noalloc)
against the workspace entry point it mirrors, through the C ABI: two calls in
a row with the second on a smaller input, for the weight-streaming and the
LDS-tiled kernel families.  Both entry points run the same kernels with the
same schedule, so their outputs must agree bit for bit; each is also checked
against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import gen as G
from tests.gpu_util import banner, dev, dev_bf16, host_bf16
from tests.tolerance import check_close

pytestmark = pytest.mark.gpu


def _draw(rng, T, H, E_g, k):
    x = G.draw_activations(rng, T, H)
    ids, w = G.draw_routing(rng, T, E_g, k)
    return x, ids, w


@pytest.mark.parametrize("kernel", [0, 2])
def test_noalloc_matches_the_workspace_entry_point(kernel):
    from quantized_moe_amd import chord as C
    from quantized_moe_amd.moe import W4A16MoE
    H, I, E_g, E_l, k, eb = 1024, 512, 64, 16, 8, 4
    rng = np.random.Generator(np.random.PCG64(700 + kernel))
    q13, s13 = G.draw_weights(rng, E_l, 2 * I, H, scale_mult=(256.0 / H) ** 0.5)
    q2, s2 = G.draw_weights(rng, E_l, H, I, scale_mult=(256.0 / I) ** 0.5)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2))
    ov = {"kernel": kernel} if kernel else None
    # the second call is smaller; with the planner's choice both are routed
    # inside the GEMM (no alignment), the third also fuses down and combine
    for T in ((160, 23, 5) if not kernel else (160, 23)):
        banner(f"no-alloc kernel={kernel} T={T} H={H} I={I} E_l={E_l} k={k}")
        x, ids, w = _draw(rng, T, H, E_g, k)
        x_d, ids_d, w_d = dev_bf16(x), dev(ids), dev(w)
        bm = C.chord_w4a16_moe_indexed_block_m(T, k, E_g, E_l, H, I) if not kernel else 16
        al = C.chord_moe_align(ids_d, eb, E_l, bm) if bm else (None, None, None)
        ref = layer.indexed(x_d, ids_d, w_d, eb, E_g, align=(*al, bm), override=ov)
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        C.chord_w4a16_moe_indexed_noalloc(x_d, layer.w13, layer.w2, ids_d, w_d, eb, E_g, *al, bm,
                                          out, override=ov)
        torch.cuda.synchronize()
        got, want = host_bf16(out), host_bf16(ref)
        assert np.array_equal(got, want), f"T={T}: differs from the workspace entry point"
        st = check_close(got, oracle.moe_layer(x, ids, w, q13, s13, q2, s2, eb), f"no-alloc T={T}")
        banner(f"  {st}; plan {C.last_plan()}")


def test_noalloc_call_replays_in_a_hip_graph():
    """The callers this entry point is for capture it: a routed decode-shaped
    call captured once in a HIP graph and replayed on new inputs written into
    the same buffers equals the eager allocation-free call bit for bit, replay
    after replay, with eager work and synchronisations in between."""
    from quantized_moe_amd import chord as C
    from quantized_moe_amd.moe import W4A16MoE
    H, I, E_g, E_l, k, T = 1024, 512, 64, 16, 8, 40
    rng = np.random.Generator(np.random.PCG64(777))
    q13, s13 = G.draw_weights(rng, E_l, 2 * I, H, scale_mult=(256.0 / H) ** 0.5)
    q2, s2 = G.draw_weights(rng, E_l, H, I, scale_mult=(256.0 / I) ** 0.5)
    layer = W4A16MoE(dev(q13), dev_bf16(s13), dev(q2), dev_bf16(s2))
    assert C.chord_w4a16_moe_indexed_block_m(T, k, E_g, E_l, H, I) == 0
    x, ids, w = _draw(rng, T, H, E_g, k)
    x_d, ids_d, w_d = dev_bf16(x), dev(ids), dev(w)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def call(o):
        C.chord_w4a16_moe_indexed_noalloc(x_d, layer.w13, layer.w2, ids_d, w_d, 0, E_g, None,
                                          None, None, 0, o)

    banner("no-alloc call under HIP graph capture")
    call(out)  # plans and looks up the scratch array outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    torch.cuda.synchronize()
    for r in range(3):
        x2, ids2, w2 = _draw(rng, T, H, E_g, k)
        x_d.copy_(dev_bf16(x2))
        ids_d.copy_(dev(ids2))
        w_d.copy_(dev(w2))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = host_bf16(out)
        eager = torch.empty_like(out)
        call(eager)
        torch.cuda.synchronize()
        assert np.array_equal(replayed, host_bf16(eager)), f"replay {r}"
        check_close(replayed, oracle.moe_layer(x2, ids2, w2, q13, s13, q2, s2, 0), f"replay {r}")
