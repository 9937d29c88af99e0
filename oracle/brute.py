"""Full-recompute decoder in torch fp64 -- TEST INFRASTRUCTURE ONLY.

An independent second formulation of the same model, used to pin the C
oracle (``liboracle``): it keeps no KV cache and recomputes every position
of the prompt at once, the way the K3 engine's default decode re-runs the
whole prefix (k3_run.c header, "DECODE STRATEGY"; its GATE 3 requires the
incremental path to give the same tokens).  It is written with library
routines wherever one exists:

* storage decoders: torch's bfloat16 / float8_e4m3fn / float8_e8m0fnu views,
  and the E2M1 magnitude table of the OCP Microscaling spec;
* grouped RMSNorm: ``F.rms_norm`` on the [groups][hidden/groups] view;
* split-half RoPE: complex multiplication by ``torch.polar(1, angle)``, pairing
  element i with i + hd/2 as real and imaginary parts;
* attention: ``F.scaled_dot_product_attention`` (causal, ``enable_gqa``);
* SwiGLU: ``F.silu``.

The KV-cache storage rounding (fp32, then bf16 or the int8 block codec) is
applied to every position's k and v before attention, since the cached path
reads stored values.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np
import torch
import torch.nn.functional as F

# OCP MX v1.0, FP4 (E2M1) element encodings 0b0000 .. 0b0111
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def dequant(dtype: str, w: np.ndarray, s: Optional[np.ndarray] = None) -> torch.Tensor:
    """Storage-format matrix -> fp64 torch tensor [N][K]."""
    if dtype == "f32":
        return torch.from_numpy(np.asarray(w, np.float32)).double()
    if dtype == "bf16":
        return torch.from_numpy(np.asarray(w, np.uint16).view(np.int16)).view(torch.bfloat16).double()
    if dtype == "fp8":
        v = torch.from_numpy(np.asarray(w, np.uint8)).view(torch.float8_e4m3fn).double()
        return v * torch.from_numpy(np.asarray(s, np.float32)).double()[:, None]
    if dtype == "mxfp4":
        q = torch.from_numpy(np.asarray(w, np.uint8)).long()
        lo, hi = q & 15, q >> 4
        nib = torch.stack([lo, hi], dim=-1).reshape(q.shape[0], -1)       # even k = low nibble
        table = torch.tensor(E2M1_MAGNITUDES + [-m for m in E2M1_MAGNITUDES], dtype=torch.float64)
        vals = table[nib]
        sc = torch.from_numpy(np.asarray(s, np.uint8)).view(torch.float8_e8m0fnu).double()
        return vals * sc.repeat_interleave(32, dim=1)
    if dtype == "q4s":
        q = torch.from_numpy(np.asarray(w, np.uint8)).long()
        nib = torch.stack([q & 15, q >> 4], dim=-1).reshape(q.shape[0], -1)   # even k = low nibble
        vals = torch.where(nib >= 8, nib - 16, nib).double()                 # two's complement
        sc = torch.from_numpy(np.asarray(s, np.float32)).double()
        return vals * sc.repeat_interleave(64, dim=1)
    raise ValueError(dtype)


def grouped_rmsnorm(h: torch.Tensor, gamma: torch.Tensor, groups: int, eps: float) -> torch.Tensor:
    shp = h.shape
    hg = h.reshape(*shp[:-1], groups, shp[-1] // groups)
    return F.rms_norm(hg, (shp[-1] // groups,), eps=eps).reshape(shp) * gamma


def rope(u: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """u [T][heads][hd]; pos [T]."""
    hd = u.shape[-1]
    half = hd // 2
    inv = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / hd)
    ang = pos.double()[:, None] * inv[None, :]                    # [T][half]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]       # [T][1][half]
    z = torch.complex(u[..., :half], u[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def kv_store_roundtrip(x: torch.Tensor, kvdt: str) -> torch.Tensor:
    """x [T][n_kv][hd] fp64 -> the values a cached path reads back."""
    x32 = x.float()
    if kvdt == "f32":
        return x32.double()
    if kvdt == "bf16":
        return x32.to(torch.bfloat16).double()
    if kvdt == "i8":
        a = x32.abs().amax(dim=-1, keepdim=True)
        s = a / torch.tensor(127.0, dtype=torch.float32)
        safe = torch.where(a > 0, s, torch.ones_like(s))
        codes = torch.round(x32 / safe).clamp(-127, 127)
        codes = torch.where(a > 0, codes, torch.zeros_like(codes))
        return (codes * s).float().double()
    raise ValueError(kvdt)


def forward_full(cfg, w: Dict[str, torch.Tensor], tokens: List[int]) -> torch.Tensor:
    """Logits [T][vocab] (fp64) for every position of ``tokens``.

    ``w`` holds fp64 dequantized tensors: embed, lm_head, g_final and per
    layer l: ``l.wqkv``, ``l.wo``, ``l.wgu``, ``l.wd``, ``l.g_in``,
    ``l.g_post``."""
    T = len(tokens)
    H, nq, nkv, hd, I = cfg.hidden, cfg.n_qh, cfg.n_kv, cfg.head_dim, cfg.inter
    pos = torch.arange(T)
    h = w["embed"][torch.tensor(tokens, dtype=torch.long)]
    for l in range(cfg.n_layers):
        x = grouped_rmsnorm(h, w[f"{l}.g_in"], cfg.groups, cfg.eps)
        qkv = x @ w[f"{l}.wqkv"].T
        q = qkv[:, : nq * hd].reshape(T, nq, hd)
        k = qkv[:, nq * hd: (nq + nkv) * hd].reshape(T, nkv, hd)
        v = qkv[:, (nq + nkv) * hd:].reshape(T, nkv, hd)
        q = rope(q, pos, cfg.theta)
        k = kv_store_roundtrip(rope(k, pos, cfg.theta), cfg.kvdt)
        v = kv_store_roundtrip(v, cfg.kvdt)
        o = F.scaled_dot_product_attention(
            q.transpose(0, 1)[None].contiguous(), k.transpose(0, 1)[None].contiguous(),
            v.transpose(0, 1)[None].contiguous(), is_causal=True, enable_gqa=True)
        o = o[0].transpose(0, 1).reshape(T, nq * hd)
        h = h + o @ w[f"{l}.wo"].T
        x = grouped_rmsnorm(h, w[f"{l}.g_post"], cfg.groups, cfg.eps)
        gu = x @ w[f"{l}.wgu"].T
        h = h + (F.silu(gu[:, :I]) * gu[:, I:]) @ w[f"{l}.wd"].T
    x = grouped_rmsnorm(h, w["g_final"], cfg.groups, cfg.eps)
    return x @ w["lm_head"].T


def weights_from_decoder(dec) -> Dict[str, torch.Tensor]:
    """fp64 tensors from the storage-format arrays held by an
    ``oracle.Decoder`` (the same input bytes, decoded here independently)."""
    cfg = dec.cfg
    w = {}
    emb = dec.embed
    w["embed"] = dequant("f32" if cfg.embed_dt == "f32" else "bf16", emb)
    w["lm_head"] = dequant(dec.lm.dtype, dec.lm.w, dec.lm.s)
    w["g_final"] = torch.from_numpy(dec.g_final).double()
    for l, mats in enumerate(dec.layers):
        for name, m in mats.items():
            w[f"{l}.{name}"] = dequant(m.dtype, m.w, m.s)
        w[f"{l}.g_in"] = torch.from_numpy(dec.g_in[l]).double()
        w[f"{l}.g_post"] = torch.from_numpy(dec.g_post[l]).double()
    return w
