"""One MoE layer as the four C-ABI calls (route -> permute -> expert_ffn -> combine).

Plumbing only: allocates the device buffers the calls write (torch is the allocator) and
enqueues the four library calls on one stream.  Every step runs in the library's kernels.
"""
from __future__ import annotations

import torch

from . import (MOE_W_BF16, Dims, Experts, moe_combine, moe_expert_ffn, moe_permute, moe_route,
               moe_workspace_size)


class LayerBuffers:
    """Outputs and workspace of one layer call for dims d (device tensors)."""

    def __init__(self, d: Dims, routed_fmt: int, has_shared: bool, device="cuda"):
        i32, f32 = torch.int32, torch.float32
        self.d = d
        self.logits = torch.empty((d.T, d.E), dtype=f32, device=device)
        self.topk_ids = torch.empty((d.T, d.k), dtype=i32, device=device)
        self.topk_w = torch.empty((d.T, d.k), dtype=f32, device=device)
        self.sorted_pair = torch.empty(d.P, dtype=i32, device=device)
        self.offsets = torch.empty(d.E + 1, dtype=i32, device=device)
        self.pair_pos = torch.empty(d.P, dtype=i32, device=device)
        self.y_pairs = torch.empty((d.P, d.H), dtype=f32, device=device)
        self.y_shared = torch.empty((d.T, d.H), dtype=f32, device=device) if has_shared else None
        self.out = torch.empty((d.T, d.H), dtype=f32, device=device)
        ws = moe_workspace_size(d, routed_fmt, has_shared)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)


def run_layer(d: Dims, bufs: LayerBuffers, x_bf16, routed: Experts, shared: Experts | None = None,
              wr_bf16=None, logit_bias=None, logits_in=None, residual=None, out_f32=None,
              out_bf16=None, stream=None):
    """Enqueue the whole layer; returns the fp32 output tensor."""
    out = bufs.out if out_f32 is None else out_f32
    moe_route(d, x_bf16, wr_bf16, logit_bias, logits_in, bufs.logits, bufs.topk_ids, bufs.topk_w,
              stream)
    moe_permute(d, bufs.topk_ids, bufs.sorted_pair, bufs.offsets, bufs.pair_pos, stream)
    moe_expert_ffn(d, routed, shared, x_bf16, bufs.sorted_pair, bufs.offsets, bufs.y_pairs,
                   bufs.y_shared if shared is not None else None, bufs.ws, stream)
    moe_combine(d, bufs.y_pairs, bufs.topk_w, bufs.pair_pos,
                bufs.y_shared if shared is not None else None, residual, out, out_bf16, stream)
    return out


def bf16_experts(gate, up, down) -> Experts:
    return Experts(MOE_W_BF16, (gate, None), (up, None), (down, None))
