"""Device-resident latent-MoE layer for the C ABI's ``k2_moe_layer``.

PyTorch only allocates device memory here.  Dense weights are the seeded
bf16 draws of ``synth``; every routed expert is its seeded bf16 window of the
expert pool, quantized to MXFP4 on the device by the library's own
``k2_quantize_mxfp4``.  Every step of the layer runs in libk2.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Tuple

import numpy as np
import torch

from . import k2
from .model import upload


class MoeLayer:
    """All buffers of one latent-MoE layer (a ``synth.MoeConfig``) on the GPU
    plus the ``k2_moe_layer_weights`` struct that points at them."""

    def __init__(self, cfg, device="cuda", max_tokens: Optional[int] = None):
        import synth
        self.cfg = cfg
        self.device = torch.device(device)
        dev = self.device
        H, Lt, I, E = cfg.hidden, cfg.latent, cfg.inter, cfg.n_experts
        self.w_router = upload(synth.moe_dense_weight(cfg, "router"), dev)
        self.bias = upload(synth.moe_router_bias(cfg), dev)
        self.w_down = upload(synth.moe_dense_weight(cfg, "down"), dev)
        self.w_up = upload(synth.moe_dense_weight(cfg, "up"), dev)
        self.gamma = torch.ones(Lt, dtype=torch.float32, device=dev)
        self.sh_w13 = upload(synth.moe_dense_weight(cfg, "shared_w13"), dev)
        self.sh_w2 = upload(synth.moe_dense_weight(cfg, "shared_w2"), dev)
        # routed experts: MXFP4 codes + E8M0 scales for all experts back to back
        self.w13q = torch.empty((E, 2 * I, Lt // 2), dtype=torch.uint8, device=dev)
        self.w13s = torch.empty((E, 2 * I, Lt // 32), dtype=torch.uint8, device=dev)
        self.w2q = torch.empty((E, Lt, I // 2), dtype=torch.uint8, device=dev)
        self.w2s = torch.empty((E, Lt, I // 32), dtype=torch.uint8, device=dev)
        pool = upload(synth.moe_expert_pool(cfg), dev)
        n13, n2 = 2 * I * Lt, Lt * I
        for e in range(E):
            o13, o2 = synth.moe_expert_offsets(cfg, e)
            k2.check(k2.k2_quantize_mxfp4(pool[o13:o13 + n13], self.w13q[e], self.w13s[e],
                                          2 * I, Lt))
            k2.check(k2.k2_quantize_mxfp4(pool[o2:o2 + n2], self.w2q[e], self.w2s[e], Lt, I))
        torch.cuda.current_stream().synchronize()
        del pool
        c = k2.k2_moe_config(H, Lt, I, E, cfg.top_k, cfg.n_shared, cfg.routed_scale, cfg.eps)
        self.weights = k2.k2_moe_layer_weights(
            c, k2.ptr(self.w_router), k2.ptr(self.bias), k2.ptr(self.w_down), k2.ptr(self.gamma),
            k2.ptr(self.w_up), k2.ptr(self.w13q), k2.ptr(self.w13s), k2.ptr(self.w2q),
            k2.ptr(self.w2s), k2.ptr(self.sh_w13), k2.ptr(self.sh_w2))
        self.max_tokens = max(cfg.tokens) if max_tokens is None else max_tokens
        self.ws_bytes = k2.k2_moe_layer_workspace_bytes(c, self.max_tokens)
        if self.ws_bytes == 0:
            raise k2.K2Error(k2.K2_EUNSUPPORTED)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)

    # --------------------------------------------------------------------
    def expert_bytes(self) -> int:
        """Bytes of one routed expert (W1, W3, W2 codes and scales)."""
        return (self.w13q[0].numel() + self.w13s[0].numel() + self.w2q[0].numel()
                + self.w2s[0].numel())

    def dense_bytes(self) -> int:
        """Bytes of the bf16 router, down, up and shared-expert weights."""
        return 2 * (self.w_router.numel() + self.w_down.numel() + self.w_up.numel()
                    + self.sh_w13.numel() + self.sh_w2.numel())

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """Enqueue the layer on x [T][hidden] fp32.  Returns (y, topk_idx,
        topk_w) device tensors."""
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError(f"T={T} exceeds the workspace's {self.max_tokens} tokens")
        cfg = self.cfg
        if y is None:
            y = torch.empty((T, cfg.hidden), dtype=torch.float32, device=self.device)
        if topk_idx is None:
            topk_idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=self.device)
        if topk_w is None:
            topk_w = torch.empty((T, cfg.top_k), dtype=torch.float32, device=self.device)
        k2.check(k2.k2_moe_layer(self.weights, x, T, y, topk_idx, topk_w, self.err, self.ws,
                                 self.ws_bytes, stream))
        return y, topk_idx, topk_w
