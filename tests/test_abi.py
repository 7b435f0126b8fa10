"""The C-ABI library loads, exports every symbol its header declares, and its host-side
argument checks and workspace arithmetic behave (no device work; CPU only)."""
import ctypes
import os
import re

import pytest

import bit_quantized_moe_softmax_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_MI355X_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", txt)))


def test_header_symbols_exported():
    names = _declared()
    assert len(names) >= 15
    L = M.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(M.EXPORTED)


def test_status_and_version():
    assert M.moe_status_str(0) == "ok"
    assert "workspace" in M.moe_status_str(3)
    assert "gfx950" in M.moe_version()


def test_counters_roundtrip():
    M.moe_reset_counters()
    c = M.moe_get_counters()
    assert set(c) == set(M.COUNTER_NAMES) and all(v == 0 for v in c.values())


def test_workspace_layout():
    d = M.Dims(T=4, H=256, I=128, E=8, k=2)
    n = M.moe_workspace_size(d, M.MOE_W_STQ1_0, False)
    assert n == 8 * 128 * 4                      # h of 8 pairs x 128, fp32, 256-aligned
    offs = M.moe_workspace_offsets(d, M.MOE_W_STQ1_0, True)
    # routed h, shared h, then the shared expert's bf16 staging of h (hi | lo, or its MXFP8
    # values) and of x (MXFP8)
    assert offs[0] == 0 and offs[1] == 4096 and offs[2] is None and offs[6] == 4096 + 2048 + 2048 + 2048
    d = M.Dims(T=4096, H=6144, I=2048, E=256, k=8)
    offs = M.moe_workspace_offsets(d, M.MOE_W_MXFP4, True)
    P = 4096 * 8
    assert offs[0] is None
    assert offs[1] == 0 and offs[2] == 4096 * 2048 * 4
    assert offs[3] == offs[2] + 4096 * 6144
    assert offs[4] == offs[3] + 4096 * 6144 // 32
    assert offs[5] == offs[4] + P * 2048
    # the shared expert's staging (h as bf16 hi | lo, x as MXFP8 values) closes the workspace
    assert offs[6] == offs[5] + P * 2048 // 32 + 4096 * 2 * 2048 * 2 + 4096 * 6144 * 2
    # STQ1_0 at prefill size: x and h (hi | lo) as fp16 rows with their row exponents, then the
    # shared expert's hi | lo h (each region 256-byte aligned)
    up = lambda v: (v + 255) // 256 * 256
    offs = M.moe_workspace_offsets(d, M.MOE_W_STQ1_0, True)
    assert offs[0] == 0 and offs[1] == P * 2048 * 4 and offs[2] is None
    ext = (up(4096 * 6144 * 2) + up(4096 * 4) + up(P * 2 * 2048 * 2) + up(P * 4) + up(4096 * 2 * 2048 * 2)
           + up(4096 * 6144 * 2))
    assert offs[6] == offs[1] + 4096 * 2048 * 4 + ext


def _raw(name, *args):
    return getattr(M.lib(), name)(*args)


def test_size_limits_hold_at_their_boundaries():
    """moe_expert_ffn refuses a call whose grouped-GEMM operands pass 2^31 bytes, and moe_route
    one with more 8-token tiles than a grid dimension holds.  A call just inside a limit stops
    at the (deliberately short) workspace instead, so nothing is launched."""
    w = ((1 << 20, 1 << 20),) * 3
    stq, mx = M.Experts(M.MOE_W_STQ1_0, *w), M.Experts(M.MOE_W_MXFP4, *w)
    bf = M.Experts(M.MOE_W_BF16, *(((1 << 20, None),) * 3))

    def ffn(T, routed, shared=None, k=8):
        d = M.Dims(T=T, H=6144, I=2048, E=256, k=k)
        return _raw("moe_expert_ffn", d.ref(), routed.ref(), shared.ref() if shared else None,
                    1 << 20, 1 << 20, 1 << 20, 1 << 20, (1 << 20) if shared else None, 1 << 20,
                    ctypes.c_size_t(16), None)

    # STQ1_0: h as fp16 hi | lo, 4 P I bytes = 2^31 at 32768 tokens
    assert ffn(32768, stq) == 3 and ffn(32769, stq) == 2
    # MXFP4: h as E4M3, P I bytes = 2^31 at 131072 tokens
    assert ffn(131072, mx) == 3 and ffn(131073, mx) == 2
    # a bf16 shared expert on the GEMMs: x bf16, 2 T H bytes (top-1 keeps the routed side inside)
    assert ffn(174762, mx, bf, k=1) == 3 and ffn(174763, mx, bf, k=1) == 2
    d = M.Dims(T=8 * 65535 + 1, H=6144, I=2048, E=256, k=8)
    assert _raw("moe_route", d.ref(), 1 << 20, 1 << 20, None, None, 1 << 20, 1 << 20, 1 << 20,
                None) == 2


def test_argument_checks_need_no_gpu():
    bad = M.Dims(T=1, H=6144, I=2048, E=256, k=40)          # k > 32
    assert _raw("moe_route", bad.ref(), None, None, None, None, None, None, None, None) == 1
    d = M.Dims(T=1, H=6144, I=2048, E=256, k=8)
    # missing outputs
    assert _raw("moe_route", d.ref(), None, None, None, None, None, None, None, None) == 1
    assert _raw("moe_permute", d.ref(), None, None, None, None, None) == 1
    assert _raw("moe_combine", d.ref(), None, None, None, None, None, None, None, None) == 1
    # expert_ffn: short workspace is reported before any launch
    routed = M.Experts(M.MOE_W_STQ1_0, (1 << 20, 1 << 20), (1 << 20, 1 << 20), (1 << 20, 1 << 20))
    st = _raw("moe_expert_ffn", d.ref(), routed.ref(), None, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
              None, 1 << 20, ctypes.c_size_t(16), None)
    assert st == 3
    # unsupported MXFP4 shape (H not a multiple of 128)
    d2 = M.Dims(T=1, H=96, I=128, E=8, k=2)
    mx = M.Experts(M.MOE_W_MXFP4, (1 << 20, 1 << 20), (1 << 20, 1 << 20), (1 << 20, 1 << 20))
    st = _raw("moe_expert_ffn", d2.ref(), mx.ref(), None, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
              None, 1 << 20, ctypes.c_size_t(1 << 30), None)
    assert st == 2
    # a shared expert must be bf16
    sh = M.Experts(M.MOE_W_STQ1_0, (1 << 20, None), (1 << 20, None), (1 << 20, None))
    st = _raw("moe_expert_ffn", d.ref(), routed.ref(), sh.ref(), 1 << 20, 1 << 20, 1 << 20, 1 << 20,
              1 << 20, 1 << 20, ctypes.c_size_t(1 << 30), None)
    assert st == 1
    assert _raw("moe_mx_quant_act", 4, 30, None, None, None, None, None) == 1
    assert _raw("moe_mx_quant_act", 4, 32, 1 << 20, 1 << 20, 1 << 20, 1 << 20, None) == 1
    assert _raw("moe_rmsnorm_bf16", 2, 64, ctypes.c_float(-1.0), 1 << 20, 1 << 20, None) == 1
    assert _raw("moe_stq1_pack", None, None, None, -1, None, None, None) == 1
    # tiled MXFP4 repack: shape, alignment and overlap checks come before any launch
    pk = "moe_mxfp4_pack_tiles"
    assert _raw(pk, 1 << 20, 1 << 21, 24, 128, 1 << 22, 1 << 23, None) == 1     # rows % 16
    assert _raw(pk, 1 << 20, 1 << 21, 32, 96, 1 << 22, 1 << 23, None) == 1      # K % 128
    assert _raw(pk, (1 << 20) + 8, 1 << 21, 32, 128, 1 << 22, 1 << 23, None) == 1  # codes align
    assert _raw(pk, 1 << 20, (1 << 21) + 2, 32, 128, 1 << 22, 1 << 23, None) == 1  # scales align
    assert _raw(pk, 1 << 20, 1 << 21, 32, 128, (1 << 20) + 1024, 1 << 23, None) == 1  # overlap
    assert _raw(pk, None, None, 0, 128, None, None, None) == 0                   # nothing to do
    # the tiled format shares the MXFP4 workspace layout
    d3 = M.Dims(T=64, H=512, I=256, E=8, k=2)
    assert M.moe_workspace_offsets(d3, M.MOE_W_MXFP4_TILED, True) == \
        M.moe_workspace_offsets(d3, M.MOE_W_MXFP4, True)


def test_new_entry_point_checks_need_no_gpu():
    F = 1 << 20   # a fake device address: every call below returns before any launch
    # STQ1_0 encoder: whole 256-weight blocks, a positive K, a known method, aligned pointers
    enc = "moe_stq1_encode"
    assert _raw(enc, F, None, 300, 256, 0, F, F, None) == 1             # n_weights % 256
    assert _raw(enc, F, None, 512, 0, 0, F, F, None) == 1               # K <= 0
    assert _raw(enc, F, None, 512, 256, 7, F, F, None) == 1             # unknown method
    assert _raw(enc, F + 4, None, 512, 256, 1, F, F, None) == 1         # x not 16-byte aligned
    assert _raw(enc, F, None, 512, 256, 1, F + 4, F, None) == 1         # codes not 8-byte aligned
    assert _raw(enc, None, None, 0, 256, 1, None, None, None) == 0      # nothing to do
    d = M.Dims(T=4, H=512, I=256, E=8, k=2)
    routed = M.Experts(M.MOE_W_STQ1_0, (F, F), (F, F), (F, F))
    # an MXFP8 shared expert needs its scale bytes
    sh8 = M.Experts(M.MOE_W_MXFP8, (F, None), (F, F), (F, F))
    assert _raw("moe_expert_ffn", d.ref(), routed.ref(), sh8.ref(), F, F, F, F, F, F,
                ctypes.c_size_t(1 << 30), None) == 1
    # the fused decode takes only a bf16 shared expert, and MXFP4 routed experts up to 64 tokens
    # (up to 4 only while every pair's FP8 h fits the small-batch down kernel)
    sh8 = M.Experts(M.MOE_W_MXFP8, (F, F), (F, F), (F, F))
    args = (F,) * 11 + (None, F, None, F, ctypes.c_size_t(1 << 30), None)
    assert _raw("moe_layer_decode", d.ref(), routed.ref(), sh8.ref(), *args) == 2
    mx = M.Experts(M.MOE_W_MXFP4_TILED, (F, F), (F, F), (F, F))
    d65 = M.Dims(T=65, H=512, I=256, E=8, k=2)
    assert _raw("moe_layer_decode", d65.ref(), mx.ref(), None, *args) == 2
    d4 = M.Dims(T=4, H=6144, I=2048, E=256, k=32)                   # FP8 h of 128 pairs: too big
    assert _raw("moe_layer_decode", d4.ref(), mx.ref(), None, *args) == 2
    # a routed format that is no routed format at all is an invalid argument, in both calls
    bad = M.Experts(M.MOE_W_BF16, (F, F), (F, F), (F, F))
    assert _raw("moe_layer_decode", d.ref(), bad.ref(), None, *args) == 1
    assert _raw("moe_expert_ffn", d.ref(), bad.ref(), None, F, F, F, F, None, F,
                ctypes.c_size_t(1 << 30), None) == 1
    offs = M.moe_layer_decode_workspace_offsets(d, True)
    assert offs[10] == M.moe_layer_decode_workspace_size(d, True)
    assert offs[9] >= offs[8] and offs[10] - offs[9] >= d.T * (d.H + d.H // 32)


def test_zero_tokens_enqueue_nothing():
    d = M.Dims(T=0, H=256, I=128, E=8, k=2)
    # T == 0 returns before touching the (fake) pointers or the GPU
    assert _raw("moe_route", d.ref(), 8, 8, None, None, 8, 8, 8, None) == 0
    assert _raw("moe_combine", d.ref(), 8, 8, 8, None, None, 8, None, None) == 0
