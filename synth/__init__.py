"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only *draws* inputs: workload shapes, weight tensors, prompt ids,
KV-cache prefixes and MoE activations.  It holds none of the decode method's
arithmetic (no norm, GEMV, RoPE, attention, quantizer or cache codec); the
oracle under ``oracle/`` and the HIP library each implement those on their own.

Weights follow the K2-Horizon model card on the k2-burn page ("Model shape"):
hidden 2560, 36 layers, 32 query / 8 key-value heads, head_dim 128, SwiGLU
intermediate 10240, two RMSNorm groups, eps 1e-6, vocab 250624, untied
lm_head.  Every projection is drawn as 0.02 * N(0, 1) in fp32 and stored as
bf16 with round-to-nearest-even (a storage format of the input, done here by
torch's own cast); norm gains are ones, as in the synthetic builder of the
avarok ``cpu_weights.rs`` page (``ones(..)`` for every norm).

Draws are reproducible on any machine: a tensor is cut into fixed chunks of
2**22 elements, and chunk ``c`` of tensor ``name`` under workload seed ``s``
uses its own ``torch.Generator`` seeded from BLAKE2b(s, name, c).  The chunks
are drawn on host threads, so the values do not depend on the thread count.
"""
from __future__ import annotations

import dataclasses
import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

CHUNK = 1 << 22
WEIGHT_STD = 0.02


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def sub_seed(seed: int, name: str, chunk: int = 0) -> int:
    h = hashlib.blake2b(f"{seed}/{name}/{chunk}".encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _normal_chunk(seed: int, name: str, c: int, n: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(sub_seed(seed, name, c))
    return torch.randn(n, generator=g, dtype=torch.float32)


def normal_f32(seed: int, name: str, shape, std: float = 1.0) -> torch.Tensor:
    """fp32 CPU tensor of ``std * N(0, 1)`` for tensor ``name``."""
    numel = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(numel, dtype=torch.float32)
    nchunks = (numel + CHUNK - 1) // CHUNK

    def work(c):
        lo = c * CHUNK
        hi = min(numel, lo + CHUNK)
        t = _normal_chunk(seed, name, c, hi - lo)
        if std != 1.0:
            t.mul_(std)
        out[lo:hi] = t

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.view(*shape)


def normal_bf16_bits(seed: int, name: str, shape, std: float = WEIGHT_STD) -> np.ndarray:
    """bf16 weights as a uint16 numpy array of bit patterns.

    The fp32 draw is cast to bf16 by torch (round to nearest even)."""
    numel = int(np.prod(shape))
    out = torch.empty(numel, dtype=torch.bfloat16)
    nchunks = (numel + CHUNK - 1) // CHUNK

    def work(c):
        lo = c * CHUNK
        hi = min(numel, lo + CHUNK)
        t = _normal_chunk(seed, name, c, hi - lo)
        t.mul_(std)
        out[lo:hi] = t.to(torch.bfloat16)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nchunks)))
    return out.view(torch.int16).numpy().view(np.uint16).reshape(shape)


def uniform_ids(seed: int, name: str, n: int, vocab: int) -> np.ndarray:
    g = torch.Generator().manual_seed(sub_seed(seed, name))
    return torch.randint(0, vocab, (n,), generator=g, dtype=torch.int64).numpy().astype(np.int32)


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class DecoderConfig:
    """Shape of a dense decoder-only model and of one greedy decode run."""
    name: str
    hidden: int
    n_layers: int
    n_qh: int
    n_kv: int
    head_dim: int
    inter: int
    vocab: int
    groups: int
    eps: float
    theta: float
    cap: int
    wdt: str            # "f32" | "bf16" | "fp8" | "mxfp4" | "q4s"  (projection + lm_head storage)
    kvdt: str           # "f32" | "bf16" | "i8"
    prompt_len: int
    n_decode: int
    seed: int = 0
    prefix_lens: Tuple[int, ...] = ()

    @property
    def embed_dt(self) -> str:
        return "f32" if self.wdt == "f32" else "bf16"

    @property
    def qkv_rows(self) -> int:
        return (self.n_qh + 2 * self.n_kv) * self.head_dim

    def replace(self, **kw) -> "DecoderConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    """One latent-MoE layer: hidden -> latent down-projection -> norm -> routed
    SwiGLU experts (top-k, renormalised) -> up-projection, plus shared experts
    on the hidden input (Kimi K3 numbers from the k3_run.c page's hard-coded
    configuration: 7168 / 3584 / 3072, 896 experts, top-16, 2 shared)."""
    name: str
    hidden: int
    latent: int
    inter: int
    n_experts: int
    top_k: int
    n_shared: int
    routed_scale: float
    eps: float
    tokens: Tuple[int, ...]
    seed: int = 0
    expert_pool: int = 1 << 25      # bf16 values shared by the routed experts' windows

    def replace(self, **kw) -> "MoeConfig":
        return dataclasses.replace(self, **kw)


TINY = DecoderConfig(
    name="tiny-dense-fp32", hidden=64, n_layers=2, n_qh=4, n_kv=2, head_dim=16,
    inter=256, vocab=512, groups=2, eps=1e-6, theta=1e4, cap=32, wdt="f32",
    kvdt="f32", prompt_len=16, n_decode=16)

K2H_BF16 = DecoderConfig(
    name="k2h-3.7b-bf16-kvbf16-ctx4096", hidden=2560, n_layers=36, n_qh=32, n_kv=8,
    head_dim=128, inter=10240, vocab=250624, groups=2, eps=1e-6, theta=1e4,
    cap=4096, wdt="bf16", kvdt="bf16", prompt_len=512, n_decode=256)

K2H_BF16_I8_LONG = K2H_BF16.replace(
    name="k2h-3.7b-bf16-kvi8-ctx32768", cap=32768, kvdt="i8",
    prefix_lens=(1024, 8192, 32768))

K2H_FP8 = K2H_BF16.replace(name="k2h-3.7b-fp8-kvi8-ctx4096", wdt="fp8", kvdt="i8")
K2H_MXFP4 = K2H_BF16.replace(name="k2h-3.7b-mxfp4-kvi8-ctx4096", wdt="mxfp4", kvdt="i8")
K2H_Q4S = K2H_BF16.replace(name="k2h-3.7b-q4s-kvi8-ctx4096", wdt="q4s", kvdt="i8")

K3_MOE = MoeConfig(
    name="k3-latent-moe-layer", hidden=7168, latent=3584, inter=3072, n_experts=896,
    top_k=16, n_shared=2, routed_scale=1.0, eps=1e-5, tokens=(1, 8, 32))

CONFIGS: Dict[str, object] = {c.name: c for c in
                              (TINY, K2H_BF16, K2H_BF16_I8_LONG, K2H_FP8, K2H_MXFP4, K2H_Q4S,
                               K3_MOE)}


# --------------------------------------------------------------------------
# Dense decoder weights
# --------------------------------------------------------------------------

def layer_shapes(cfg: DecoderConfig) -> Dict[str, Tuple[int, int]]:
    """Projection matrices of one layer, row-major [out][in].

    ``wqkv`` stacks the q rows (n_qh*head_dim), then k, then v; ``wgu``
    stacks the gate rows (inter), then the up rows (inter)."""
    H, D = cfg.hidden, cfg.head_dim
    return {
        "wqkv": (cfg.qkv_rows, H),
        "wo": (H, cfg.n_qh * D),
        "wgu": (2 * cfg.inter, H),
        "wd": (H, cfg.inter),
    }


def dense_weight(cfg: DecoderConfig, name: str, shape) -> np.ndarray:
    """The unquantized draw of one matrix: fp32 for fp32 models, bf16 bits
    (uint16) otherwise.  fp8 / MXFP4 models quantize this bf16 draw."""
    if cfg.wdt == "f32":
        return normal_f32(cfg.seed, name, shape, WEIGHT_STD).numpy()
    return normal_bf16_bits(cfg.seed, name, shape)


def layer_weight(cfg: DecoderConfig, layer: int, which: str) -> np.ndarray:
    return dense_weight(cfg, f"layers.{layer}.{which}", layer_shapes(cfg)[which])


def embed_weight(cfg: DecoderConfig) -> np.ndarray:
    return dense_weight(cfg, "embed", (cfg.vocab, cfg.hidden))


def lm_head_weight(cfg: DecoderConfig) -> np.ndarray:
    return dense_weight(cfg, "lm_head", (cfg.vocab, cfg.hidden))


def norm_gain(cfg: DecoderConfig) -> np.ndarray:
    return np.ones(cfg.hidden, dtype=np.float32)


def prompt(cfg: DecoderConfig, n: Optional[int] = None) -> np.ndarray:
    return uniform_ids(cfg.seed, "prompt", cfg.prompt_len if n is None else n, cfg.vocab)


def int8_kv_prefix(cfg: DecoderConfig, layer: int, length: int):
    """A seeded stand-in for a long int8 KV history (positions < length).

    Codes are uniform on [-127, 127]; per-(kv-head, position) scales are
    |0.05 * N(0, 1)| in fp32.  Returns (kcodes, vcodes) int8 [n_kv][length][hd]
    and (kscale, vscale) fp32 [n_kv][length]."""
    shp = (cfg.n_kv, length, cfg.head_dim)
    out = []
    for which in ("k", "v"):
        g = torch.Generator().manual_seed(sub_seed(cfg.seed, f"kvprefix.{layer}.{which}"))
        codes = torch.randint(-127, 128, shp, generator=g, dtype=torch.int16).to(torch.int8)
        out.append(codes.numpy())
    for which in ("k", "v"):
        s = normal_f32(cfg.seed, f"kvprefix.{layer}.{which}.scale", (cfg.n_kv, length), 0.05)
        out.append(s.abs().numpy())
    return out[0], out[1], out[2], out[3]


# --------------------------------------------------------------------------
# Latent-MoE layer
# --------------------------------------------------------------------------

def moe_dense_weight(cfg: MoeConfig, name: str) -> np.ndarray:
    H, Lt, I = cfg.hidden, cfg.latent, cfg.inter
    shapes = {
        "down": (Lt, H), "up": (H, Lt), "router": (cfg.n_experts, H),
        "shared_w13": (cfg.n_shared * 2 * I, H), "shared_w2": (cfg.n_shared * H, I),
    }
    return normal_bf16_bits(cfg.seed, f"moe.{name}", shapes[name])


def moe_router_bias(cfg: MoeConfig) -> np.ndarray:
    return normal_f32(cfg.seed, "moe.router_bias", (cfg.n_experts,), WEIGHT_STD).numpy()


def moe_expert_pool(cfg: MoeConfig) -> np.ndarray:
    """Routed-expert weights are windows of one seeded pool of bf16 draws
    (896 full-size experts are 29.6e9 values, too many to draw one by one;
    each window has the same 0.02 * N(0, 1) bf16 distribution).  Returned
    with its head repeated after its end, so that every window is one
    contiguous slice: length expert_pool + 2 * inter * latent."""
    base = normal_bf16_bits(cfg.seed, "moe.expert_pool", (cfg.expert_pool,))
    return np.concatenate([base, np.resize(base, 2 * cfg.inter * cfg.latent)])


def moe_expert_offsets(cfg: MoeConfig, e: int) -> Tuple[int, int]:
    """Pool offsets (multiples of 64 values) of expert e's W13 and W2."""
    slots = cfg.expert_pool // 64
    o13 = (sub_seed(cfg.seed, f"moe.expert.{e}.w13") % slots) * 64
    o2 = (sub_seed(cfg.seed, f"moe.expert.{e}.w2") % slots) * 64
    return o13, o2


def moe_expert_draw(cfg: MoeConfig, e: int, pool: Optional[np.ndarray] = None
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """bf16 draws of expert e: w13 [2*inter][latent] (gate rows, then up rows)
    and w2 [latent][inter], as views of the pool."""
    pool = moe_expert_pool(cfg) if pool is None else pool
    o13, o2 = moe_expert_offsets(cfg, e)
    n13, n2 = 2 * cfg.inter * cfg.latent, cfg.latent * cfg.inter
    return (pool[o13:o13 + n13].reshape(2 * cfg.inter, cfg.latent),
            pool[o2:o2 + n2].reshape(cfg.latent, cfg.inter))


def moe_activations(cfg: MoeConfig, T: int, rep: int = 0) -> np.ndarray:
    return normal_f32(cfg.seed, f"moe.x.{T}.{rep}", (T, cfg.hidden), 1.0).numpy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact: a bit shift)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)
