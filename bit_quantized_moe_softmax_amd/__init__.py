"""Python binding of libmoe_mi355x (gfx950 routed-expert MoE FFN on packed low-bit weights).

Thin ctypes marshalling over the C ABI declared in include/moe_mi355x.h: every function
here has the C entry point's name and arguments, takes torch tensors (device memory) or
None (NULL) for the pointers, and raises MoeError on a non-zero status.  All compute runs
in the HIP kernels of the shared library; there is no fallback path -- importing fails
loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MoeError", "lib", "Dims", "Experts", "MOE_W_STQ1_0", "MOE_W_MXFP4", "MOE_W_BF16",
    "MOE_W_MXFP4_TILED", "MOE_W_MXFP8", "moe_mxfp4_pack_tiles",
    "COUNTER_NAMES", "moe_status_str", "moe_version", "moe_get_counters", "moe_reset_counters",
    "moe_route", "moe_permute", "moe_workspace_size", "moe_workspace_offsets", "moe_expert_ffn",
    "moe_combine", "moe_stq1_pack", "moe_stq1_dequant", "moe_mxfp4_dequant", "moe_mx_quant_act",
    "moe_mx_quant_f32_hwcvt",
    "moe_rmsnorm_bf16", "moe_layer_decode_workspace_size", "moe_layer_decode_workspace_offsets",
    "moe_layer_decode", "moe_layer_decode_noalloc", "moe_stq1_encode", "SlotBank", "moe_remap_ids", "MOE_STQ1_ENC_UPSTREAM", "MOE_STQ1_ENC_WLS",
    "moe_profile_enable", "moe_profile_read", "PROFILE_SLOTS",
]

PROFILE_SLOTS = ["decode_k1_route", "decode_k2_gateup",
                 "decode_k3_down_combine", "decode_k4_combine", "mx_quant", "mx_gateup", "mx_down",
                 "stq_gateup", "stq_down", "shared_gateup", "shared_down", "act_prep"]

MOE_W_STQ1_0, MOE_W_MXFP4, MOE_W_BF16, MOE_W_MXFP4_TILED, MOE_W_MXFP8 = 1, 2, 3, 4, 5
COUNTER_NAMES = ["route_gemv", "route_topk", "permute", "stq_gateup_mfma", "stq_down_mfma",
                 "stq_generic", "mx_quant", "mx_gateup_mfma", "mx_down_mfma", "bf16_gateup",
                 "bf16_down", "combine", "rmsnorm", "dequant", "bf16_gemm", "decode_fused",
                 "stq_gemm", "rowscale", "mxfp8_shared"]

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")


class MoeError(RuntimeError):
    pass


class _Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32)]


class _Mat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class _Experts(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("gate", _Mat), ("up", _Mat), ("down", _Mat)]


_P = ctypes.c_void_p
_SIGS = {
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_version": (ctypes.c_char_p, []),
    "moe_get_counters": (ctypes.c_int, [_P]),
    "moe_reset_counters": (ctypes.c_int, []),
    "moe_route": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_permute": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "moe_workspace_size": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, _P]),
    "moe_workspace_offsets": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, _P]),
    "moe_expert_ffn": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_combine": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_stq1_pack": (ctypes.c_int, [_P, _P, _P, ctypes.c_int64, _P, _P, _P]),
    "moe_stq1_dequant": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P, _P]),
    "moe_mxfp4_dequant": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, _P, _P]),
    "moe_mxfp4_pack_tiles": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P]),
    "moe_mx_quant_act": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P, _P]),
    "moe_mx_quant_f32_hwcvt": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P]),
    "moe_rmsnorm_bf16": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, _P, _P]),
    "moe_layer_decode_workspace_size": (ctypes.c_int, [_P, ctypes.c_int32, _P]),
    "moe_layer_decode_workspace_offsets": (ctypes.c_int, [_P, ctypes.c_int32, _P]),
    "moe_stq1_encode": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "moe_slot_bank_create": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P]),
    "moe_slot_bank_destroy": (ctypes.c_int, [_P]),
    "moe_slot_bank_plan": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P, _P]),
    "moe_slot_bank_fetch": (ctypes.c_int, [_P, _P, _P, _P]),
    "moe_slot_bank_stats": (ctypes.c_int, [_P, _P, _P]),
    "moe_remap_ids": (ctypes.c_int, [_P, ctypes.c_int64, _P, _P, _P]),
    "moe_layer_decode": (ctypes.c_int, [_P, _P, _P] + [_P] * 15 + [ctypes.c_size_t, _P]),
    "moe_layer_decode_noalloc": (ctypes.c_int, [_P, _P, _P] + [_P] * 15),
    "moe_profile_enable": (ctypes.c_int, [ctypes.c_int32]),
    "moe_profile_read": (ctypes.c_int, [_P, _P]),
}
EXPORTED = tuple(_SIGS)

_lib = None


def lib():
    """The loaded shared library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise MoeError(f"{_LIB_PATH} is missing: build it first (python -m "
                           "bit_quantized_moe_softmax_amd.build or __graft_entry__.build())")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st):
    if st != 0:
        raise MoeError(f"moe_mi355x error {st}: {lib().moe_status_str(st).decode()}")


class Dims:
    """moe_dims: T tokens, hidden H, expert intermediate I, E routed experts, k per token."""

    def __init__(self, T, H, I, E, k):
        self.T, self.H, self.I, self.E, self.k = int(T), int(H), int(I), int(E), int(k)
        self._c = _Dims(self.T, self.H, self.I, self.E, self.k)

    @property
    def P(self):
        return self.T * self.k

    def ref(self):
        return ctypes.byref(self._c)


class Experts:
    """moe_experts: fmt plus (codes, scales) tensors of gate, up and down (scales None for
    bf16).  Keeps the tensors alive while the struct is in use."""

    def __init__(self, fmt, gate, up, down):
        self.fmt = fmt
        self.tensors = (gate, up, down)
        m = [_Mat(_ptr(c), _ptr(s)) for c, s in (gate, up, down)]
        self._c = _Experts(fmt, 0, m[0], m[1], m[2])

    def ref(self):
        return ctypes.byref(self._c)


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_version() -> str:
    return lib().moe_version().decode()


def moe_get_counters() -> dict:
    buf = (ctypes.c_uint64 * len(COUNTER_NAMES))()
    _check(lib().moe_get_counters(ctypes.cast(buf, _P)))
    return {n: int(v) for n, v in zip(COUNTER_NAMES, buf)}


def moe_reset_counters() -> None:
    _check(lib().moe_reset_counters())


def moe_route(d: Dims, x_bf16, wr_bf16, logit_bias, logits_in, logits_out, topk_ids, topk_w,
              stream=None):
    _check(lib().moe_route(d.ref(), _ptr(x_bf16), _ptr(wr_bf16), _ptr(logit_bias), _ptr(logits_in),
                           _ptr(logits_out), _ptr(topk_ids), _ptr(topk_w), _stream(stream)))


def moe_permute(d: Dims, topk_ids, sorted_pair, expert_offsets, pair_pos, stream=None):
    _check(lib().moe_permute(d.ref(), _ptr(topk_ids), _ptr(sorted_pair), _ptr(expert_offsets),
                             _ptr(pair_pos), _stream(stream)))


def moe_workspace_size(d: Dims, routed_fmt: int, has_shared: bool) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(d.ref(), routed_fmt, int(bool(has_shared)), ctypes.byref(out)))
    return out.value


def moe_workspace_offsets(d: Dims, routed_fmt: int, has_shared: bool) -> list:
    buf = (ctypes.c_size_t * 7)()
    _check(lib().moe_workspace_offsets(d.ref(), routed_fmt, int(bool(has_shared)), ctypes.cast(buf, _P)))
    return [None if v == ctypes.c_size_t(-1).value else int(v) for v in buf]


def moe_expert_ffn(d: Dims, routed: Experts, shared, x_bf16, sorted_pair, expert_offsets, y_pairs,
                   y_shared, ws, stream=None):
    _check(lib().moe_expert_ffn(d.ref(), routed.ref(), shared.ref() if shared is not None else None,
                                _ptr(x_bf16), _ptr(sorted_pair), _ptr(expert_offsets), _ptr(y_pairs),
                                _ptr(y_shared), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(stream)))


def moe_combine(d: Dims, y_pairs, topk_w, pair_pos, y_shared, residual, out_f32, out_bf16,
                stream=None):
    _check(lib().moe_combine(d.ref(), _ptr(y_pairs), _ptr(topk_w), _ptr(pair_pos), _ptr(y_shared),
                             _ptr(residual), _ptr(out_f32), _ptr(out_bf16), _stream(stream)))


def moe_stq1_pack(zpos, signs, d_f16, n_blocks, codes, scales, stream=None):
    _check(lib().moe_stq1_pack(_ptr(zpos), _ptr(signs), _ptr(d_f16), int(n_blocks), _ptr(codes),
                               _ptr(scales), _stream(stream)))


def moe_stq1_dequant(codes, scales, n_blocks, out, stream=None):
    _check(lib().moe_stq1_dequant(_ptr(codes), _ptr(scales), int(n_blocks), _ptr(out), _stream(stream)))


def moe_mxfp4_dequant(codes, scales, rows, K, out, stream=None):
    _check(lib().moe_mxfp4_dequant(_ptr(codes), _ptr(scales), int(rows), int(K), _ptr(out),
                                   _stream(stream)))


def moe_mxfp4_pack_tiles(codes, scales, rows, K, tcodes, tscales, stream=None):
    _check(lib().moe_mxfp4_pack_tiles(_ptr(codes), _ptr(scales), int(rows), int(K), _ptr(tcodes),
                                      _ptr(tscales), _stream(stream)))


def moe_mx_quant_act(rows, K, x_bf16, x_f32, q, s, stream=None):
    _check(lib().moe_mx_quant_act(int(rows), int(K), _ptr(x_bf16), _ptr(x_f32), _ptr(q), _ptr(s),
                                  _stream(stream)))


def moe_mx_quant_f32_hwcvt(rows, K, x_f32, q, s, stream=None):
    _check(lib().moe_mx_quant_f32_hwcvt(int(rows), int(K), _ptr(x_f32), _ptr(q), _ptr(s), _stream(stream)))


def moe_rmsnorm_bf16(T, H, eps, r, a, stream=None):
    _check(lib().moe_rmsnorm_bf16(int(T), int(H), float(eps), _ptr(r), _ptr(a), _stream(stream)))


MOE_STQ1_ENC_UPSTREAM, MOE_STQ1_ENC_WLS = 0, 1


class SlotBank:
    """Host handle of an expert slot bank (E experts, S device slots): plan() returns the
    slot of every resident expert for a step's expert ids (a host int32 array), fetch()
    enqueues the planned host -> device copies."""

    def __init__(self, E: int, S: int, bytes_per_expert, io_split: int = 4):
        b = (ctypes.c_uint64 * 6)(*[int(v) for v in bytes_per_expert])
        h = ctypes.c_void_p()
        _check(lib().moe_slot_bank_create(E, S, ctypes.cast(b, _P), io_split, ctypes.byref(h)))
        self._h = h
        self.E, self.S = E, S

    def plan(self, ids_host):
        import numpy as np
        ids = np.ascontiguousarray(ids_host, dtype=np.int32).reshape(-1)
        slot_of = np.empty(self.E, dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib().moe_slot_bank_plan(self._h, ids.ctypes.data, ids.size, slot_of.ctypes.data,
                                        ctypes.byref(n)))
        return slot_of, n.value

    def fetch(self, host_src, dev_slots, stream=None):
        _check(lib().moe_slot_bank_fetch(self._h, host_src.ref(), dev_slots.ref(), _stream(stream)))

    def stats(self):
        h, m = ctypes.c_uint64(), ctypes.c_uint64()
        _check(lib().moe_slot_bank_stats(self._h, ctypes.byref(h), ctypes.byref(m)))
        return h.value, m.value

    def close(self):
        if self._h:
            lib().moe_slot_bank_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter teardown
            pass


def moe_remap_ids(ids, n: int, slot_of, out, stream=None) -> None:
    _check(lib().moe_remap_ids(_ptr(ids), n, _ptr(slot_of), _ptr(out), _stream(stream)))


def moe_stq1_encode(x_f32, imatrix_f32, n_weights: int, K: int, method: int, codes, scales, stream=None):
    """Encode a float32 matrix (flattened [N][K]) into STQ1_0 codes / fp16 scale bits."""
    _check(lib().moe_stq1_encode(_ptr(x_f32), _ptr(imatrix_f32), n_weights, K, method, _ptr(codes),
                                 _ptr(scales), _stream(stream)))


def moe_layer_decode_workspace_offsets(d: Dims, has_shared: bool) -> list:
    buf = (ctypes.c_size_t * 11)()
    _check(lib().moe_layer_decode_workspace_offsets(d.ref(), int(bool(has_shared)), ctypes.cast(buf, _P)))
    return [int(v) for v in buf]


def moe_layer_decode_workspace_size(d: Dims, has_shared: bool) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().moe_layer_decode_workspace_size(d.ref(), int(bool(has_shared)), ctypes.byref(out)))
    return out.value


def moe_layer_decode(d: Dims, routed: Experts, shared, x_bf16, wr_bf16, logit_bias, logits_out,
                     topk_ids, topk_w, sorted_pair, expert_offsets, pair_pos, y_pairs, y_shared,
                     residual, out_f32, out_bf16, ws, stream=None):
    _check(lib().moe_layer_decode(
        d.ref(), routed.ref(), shared.ref() if shared is not None else None, _ptr(x_bf16),
        _ptr(wr_bf16), _ptr(logit_bias), _ptr(logits_out), _ptr(topk_ids), _ptr(topk_w),
        _ptr(sorted_pair), _ptr(expert_offsets), _ptr(pair_pos), _ptr(y_pairs), _ptr(y_shared),
        _ptr(residual), _ptr(out_f32), _ptr(out_bf16), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer_decode_noalloc(d: Dims, routed: Experts, shared, x_bf16, wr_bf16, logit_bias, logits_out,
                             topk_ids, topk_w, sorted_pair, expert_offsets, pair_pos, y_pairs, y_shared,
                             residual, out_f32, out_bf16, stream=None):
    _check(lib().moe_layer_decode_noalloc(
        d.ref(), routed.ref(), shared.ref() if shared is not None else None, _ptr(x_bf16),
        _ptr(wr_bf16), _ptr(logit_bias), _ptr(logits_out), _ptr(topk_ids), _ptr(topk_w),
        _ptr(sorted_pair), _ptr(expert_offsets), _ptr(pair_pos), _ptr(y_pairs), _ptr(y_shared),
        _ptr(residual), _ptr(out_f32), _ptr(out_bf16), _stream(stream)))


def moe_profile_enable(on: bool) -> None:
    _check(lib().moe_profile_enable(int(bool(on))))


def moe_profile_read() -> dict:
    """{slot name: (average microseconds, launches)} of the events recorded since the last read."""
    avg = (ctypes.c_double * 16)()
    cnt = (ctypes.c_int64 * 16)()
    _check(lib().moe_profile_read(ctypes.cast(avg, _P), ctypes.cast(cnt, _P)))
    return {n: (float(avg[i]), int(cnt[i])) for i, n in enumerate(PROFILE_SLOTS)}
