"""moe_layer_decode_noalloc (the fused decode on the library's static scratch, for callers
that cannot allocate) against moe_layer_decode with a caller workspace: bit-identical
outputs, on two calls in a row, the second with a smaller input, for the small-batch and the
large-batch kernels and for MXFP4 routed experts; and the size check."""
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_softmax_amd as M
import synth
from bit_quantized_moe_softmax_amd.layer import bf16_experts
from tests.helpers import layer_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print("[no-alloc]", *a, file=sys.__stderr__, flush=True)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _routed(c, inp, tiled):
    fmt = M.MOE_W_STQ1_0 if c.fmt == "stq1" else M.MOE_W_MXFP4
    tens = [(dev(cd), dev(sc)) for cd, sc in inp["routed"]]
    if tiled:
        out = []
        for (cd, sc), (codes, _) in zip(tens, inp["routed"]):
            tc, ts = torch.empty_like(cd), torch.empty_like(sc)
            M.moe_mxfp4_pack_tiles(cd, sc, codes.shape[0] * codes.shape[1], 2 * codes.shape[-1], tc, ts)
            out.append((tc, ts))
        return M.Experts(M.MOE_W_MXFP4_TILED, *out)
    return M.Experts(fmt, *tens)


def _outputs(c, T):
    f32, i32 = torch.float32, torch.int32
    P = T * c.k
    return [torch.full((T, c.E), 7.0, dtype=f32, device="cuda"),
            torch.full((T, c.k), -5, dtype=i32, device="cuda"),
            torch.full((T, c.k), 7.0, dtype=f32, device="cuda"),
            torch.full((P,), -5, dtype=i32, device="cuda"),
            torch.full((c.E + 1,), -5, dtype=i32, device="cuda"),
            torch.full((P,), -5, dtype=i32, device="cuda"),
            torch.full((P, c.H), 7.0, dtype=f32, device="cuda"),
            torch.full((T, c.H), 7.0, dtype=f32, device="cuda"),
            torch.full((T, c.H), 7.0, dtype=f32, device="cuda"),
            torch.full((T, c.H), 7, dtype=torch.int16, device="cuda")]


def _run(c, inp, routed, shared, T, noalloc, residual):
    d = M.Dims(T, c.H, c.I, c.E, c.k)
    o = _outputs(c, T)
    x = dev(inp["x"][:T])
    wr = dev(inp["wr"])
    bias = dev(inp["bias"]) if inp["bias"] is not None else None
    res = residual[:T].contiguous() if residual is not None else None
    ysh = o[7] if shared is not None else None
    if noalloc:
        M.moe_layer_decode_noalloc(d, routed, shared, x, wr, bias, o[0], o[1], o[2], o[3], o[4], o[5], o[6],
                                   ysh, res, o[8], o[9])
    else:
        ws = torch.zeros(M.moe_layer_decode_workspace_size(d, shared is not None), dtype=torch.uint8,
                         device="cuda")
        M.moe_layer_decode(d, routed, shared, x, wr, bias, o[0], o[1], o[2], o[3], o[4], o[5], o[6],
                           ysh, res, o[8], o[9], ws)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in o]


CASES = {
    # Hy4 shape, STQ1_0, the small-batch kernels: 4 tokens then 1
    "hy4-stq1-t4-then-t1": (synth.LayerCfg("na", 4, 6144, 2048, 256, 8, True, "stq1", False, False, 1, 81), (4, 1), False),
    # the large-batch kernels (router ticket in the scratch): 64 tokens then 9, Zipf bias
    "h1024-stq1-t64-then-t9": (synth.LayerCfg("na", 64, 1024, 512, 64, 8, True, "stq1", True, False, 1, 82), (64, 9), False),
    # MXFP4 tiled routed experts: 4 tokens then 2
    "h1024-mxfp4-t4-then-t2": (synth.LayerCfg("na", 4, 1024, 512, 16, 4, True, "mxfp4", False, False, 1, 83), (4, 2), True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_equals_workspace_entry_point(name):
    c, Ts, tiled = CASES[name]
    inp = layer_inputs(c)
    routed = _routed(c, inp, tiled)
    shared = bf16_experts(*(dev(w) for w in inp["shared"]))
    g = np.random.default_rng(84)
    residual = torch.from_numpy(g.standard_normal((c.T, c.H)).astype(np.float32)).cuda()
    for T in Ts:
        say(name, "T", T)
        a = _run(c, inp, routed, shared, T, True, residual)
        b = _run(c, inp, routed, shared, T, False, residual)
        for i, (u, v) in enumerate(zip(a, b)):
            assert u.shape == v.shape
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), f"output {i} differs at T={T}"
        assert np.isfinite(a[8]).all()


def test_noalloc_rejects_what_exceeds_the_scratch():
    """64 tokens x top-32 at hidden 8192: the workspace exceeds the 8 MiB scratch, so the call
    is refused before anything is enqueued (the same call with a workspace is valid)."""
    d = M.Dims(64, 8192, 2048, 256, 32)
    assert M.moe_layer_decode_workspace_size(d, True) > 8 << 20
    z = torch.zeros(16, dtype=torch.int32, device="cuda")
    routed = M.Experts(M.MOE_W_STQ1_0, (z, z), (z, z), (z, z))
    shared = bf16_experts(z, z, z)
    with pytest.raises(M.MoeError, match="unsupported"):
        M.moe_layer_decode_noalloc(d, routed, shared, z, z, None, z, z, z, z, z, z, z, z, None, z, None)
