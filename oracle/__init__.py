"""CPU fp64 oracle of the batch-1 decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It wraps ``liboracle.so``
(plain C, fp64, built from ``oracle.c`` with gcc) through ctypes, and
``oracle.brute`` holds an independent full-recompute decoder written with
torch fp64 library routines.  Neither shares code with the HIP library.

Parity is pinned per function by the ``-m "not gpu"`` tests (codec tables
against torch's own fp8/e8m0 decoders and the OCP E2M1 table, closed forms,
invariants, library special cases, incremental-vs-full recompute).  End-to-end
logit *values* have no printed worked example on the pages: beyond those
invariants they are "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None

F32, BF16, FP8, MXFP4, I8, Q4S = 0, 1, 2, 3, 4, 5
DT = {"f32": F32, "bf16": BF16, "fp8": FP8, "mxfp4": MXFP4, "i8": I8, "q4s": Q4S}

_dp = C.POINTER(C.c_double)
_vp = C.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        L.orc_bf16_value.restype = C.c_double
        L.orc_bf16_value.argtypes = [C.c_uint16]
        L.orc_bf16_round.restype = C.c_uint16
        L.orc_bf16_round.argtypes = [C.c_float]
        for n in ("orc_fp8_value", "orc_e2m1_value", "orc_e8m0_value"):
            getattr(L, n).restype = C.c_double
            getattr(L, n).argtypes = [C.c_uint8]
        for n in ("orc_fp8_encode", "orc_e2m1_encode"):
            getattr(L, n).restype = C.c_uint8
            getattr(L, n).argtypes = [C.c_float]
        L.orc_quant_fp8_rows.argtypes = [_vp, C.c_int64, C.c_int64, _vp, _vp]
        L.orc_quant_mxfp4.argtypes = [_vp, C.c_int64, C.c_int64, _vp, _vp]
        L.orc_quant_q4s.argtypes = [_vp, C.c_int64, C.c_int64, _vp, _vp]
        L.orc_q4s_value.argtypes = [C.c_uint8]
        L.orc_q4s_value.restype = C.c_double
        L.orc_kv_quant_int8.argtypes = [_vp, C.c_int, _vp, _vp]
        L.orc_int8_dequant.restype = C.c_double
        L.orc_int8_dequant.argtypes = [C.c_int8, C.c_float]
        L.orc_matvec.argtypes = [C.c_int, _vp, _vp, _vp, _vp, C.c_int64, C.c_int64]
        L.orc_rmsnorm_grouped.argtypes = [_vp, _vp, _vp, C.c_int, C.c_int, C.c_double]
        L.orc_rope.argtypes = [_vp, C.c_int, C.c_int, C.c_int, C.c_double]
        L.orc_silu.restype = C.c_double
        L.orc_silu.argtypes = [C.c_double]
        L.orc_kv_store.argtypes = [C.c_int, _vp, _vp, _vp, C.c_int, C.c_int, C.c_int, C.c_int]
        L.orc_attention.argtypes = [C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int, C.c_int,
                                    C.c_int, C.c_int, C.c_int, _vp]
        L.orc_argmax.restype = C.c_int64
        L.orc_argmax.argtypes = [_vp, C.c_int64]
        L.orc_decode_step.restype = C.c_int64
        L.orc_decode_step.argtypes = [_vp, C.c_int, C.c_int, _vp]
        L.orc_moe_route.argtypes = [_vp, _vp, _vp, C.c_int, C.c_int, C.c_int, C.c_double,
                                    _vp, _vp]
        L.orc_swiglu_expert.argtypes = [_vp, _vp, _vp, C.c_int, C.c_int, C.c_int, _vp]
        L.orc_moe_apply.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, C.c_int, _vp, C.c_int,
                                    C.c_int, C.c_int, C.c_double, _vp, _vp, C.c_int, _vp]
        L.orc_num_threads.restype = C.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def num_threads() -> int:
    return lib().orc_num_threads()


# ---------------------------------------------------------------- codecs ---

def bf16_value(bits) -> np.ndarray:
    L = lib()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.orc_bf16_value(int(x)) for x in b]).reshape(np.shape(bits))


def bf16_round(x) -> np.ndarray:
    L = lib()
    a = np.asarray(x, dtype=np.float32).ravel()
    return np.array([L.orc_bf16_round(float(v)) for v in a], dtype=np.uint16).reshape(np.shape(x))


def fp8_value(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.orc_fp8_value(int(v)) for v in c]).reshape(np.shape(codes))


def e2m1_value(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.orc_e2m1_value(int(v)) for v in c]).reshape(np.shape(codes))


def e8m0_value(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.orc_e8m0_value(int(v)) for v in c]).reshape(np.shape(codes))


def fp8_encode(x) -> np.ndarray:
    L = lib()
    a = np.asarray(x, dtype=np.float32).ravel()
    return np.array([L.orc_fp8_encode(float(v)) for v in a], dtype=np.uint8).reshape(np.shape(x))


def e2m1_encode(x) -> np.ndarray:
    L = lib()
    a = np.asarray(x, dtype=np.float32).ravel()
    return np.array([L.orc_e2m1_encode(float(v)) for v in a], dtype=np.uint8).reshape(np.shape(x))


def quant_fp8_rows(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    N, K = w.shape
    codes = np.empty((N, K), np.uint8)
    scale = np.empty(N, np.float32)
    lib().orc_quant_fp8_rows(_p(w), N, K, _p(codes), _p(scale))
    return codes, scale


def quant_mxfp4(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    N, K = w.shape
    assert K % 32 == 0
    q = np.empty((N, K // 2), np.uint8)
    e = np.empty((N, K // 32), np.uint8)
    lib().orc_quant_mxfp4(_p(w), N, K, _p(q), _p(e))
    return q, e


def q4s_value(codes) -> np.ndarray:
    """Signed value of Q4S nibbles (two's complement, [-8, 7])."""
    L = lib()
    a = np.asarray(codes, dtype=np.uint8)
    return np.array([L.orc_q4s_value(int(c)) for c in a.ravel()], np.float64).reshape(a.shape)


def quant_q4s(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Q4S: int4 codes on [-7, 7] packed two per byte (low nibble = even k)
    and one fp32 scale per 64 consecutive k of a row."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    N, K = w.shape
    assert K % 64 == 0
    q = np.empty((N, K // 2), np.uint8)
    s = np.empty((N, K // 64), np.float32)
    lib().orc_quant_q4s(_p(w), N, K, _p(q), _p(s))
    return q, s


def kv_quant_int8(x) -> Tuple[np.ndarray, float]:
    a = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(a.shape, np.int8)
    s = np.zeros(1, np.float32)
    lib().orc_kv_quant_int8(_p(a), a.size, _p(codes), _p(s))
    return codes, float(s[0])


def int8_dequant(code: int, scale: float) -> float:
    return lib().orc_int8_dequant(int(code), float(scale))


# ------------------------------------------------------------- matrices ---

class _Mat(C.Structure):
    _fields_ = [("dtype", C.c_int), ("w", _vp), ("s", _vp)]


class Mat:
    """A projection matrix in storage format (keeps its arrays alive)."""

    def __init__(self, dtype: str, w: np.ndarray, s: Optional[np.ndarray] = None,
                 shape: Optional[Tuple[int, int]] = None):
        self.dtype = dtype
        self.w = np.ascontiguousarray(w)
        self.s = None if s is None else np.ascontiguousarray(s)
        if shape is None:
            N = self.w.shape[0]
            K = self.w.shape[1] * (2 if dtype in ("mxfp4", "q4s") else 1)
            shape = (N, K)
        self.shape = shape
        self.c = _Mat(DT[dtype], _p(self.w), _p(self.s))

    @staticmethod
    def from_draw(wdt: str, draw: np.ndarray) -> "Mat":
        """Storage-format matrix from a draw: fp32 / bf16 as is; fp8 and
        MXFP4 quantized by the oracle's own quantizers from the bf16 draw."""
        if wdt == "f32":
            return Mat("f32", np.asarray(draw, np.float32))
        if wdt == "bf16":
            return Mat("bf16", np.asarray(draw, np.uint16))
        if wdt == "fp8":
            c, s = quant_fp8_rows(draw)
            return Mat("fp8", c, s, draw.shape)
        if wdt == "mxfp4":
            q, e = quant_mxfp4(draw)
            return Mat("mxfp4", q, e, draw.shape)
        if wdt == "q4s":
            q, sc = quant_q4s(draw)
            return Mat("q4s", q, sc, draw.shape)
        raise ValueError(wdt)

    def matvec(self, x: np.ndarray) -> np.ndarray:
        N, K = self.shape
        xx = np.ascontiguousarray(x, dtype=np.float64)
        assert xx.size == K
        y = np.empty(N, np.float64)
        lib().orc_matvec(self.c.dtype, self.c.w, self.c.s, _p(xx), _p(y), N, K)
        return y


def rmsnorm_grouped(h, gamma, groups: int, eps: float) -> np.ndarray:
    hh = np.ascontiguousarray(h, dtype=np.float64)
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    y = np.empty_like(hh)
    lib().orc_rmsnorm_grouped(_p(hh), _p(g), _p(y), hh.size, groups, eps)
    return y


def rope(u, n_heads: int, head_dim: int, pos: int, theta: float) -> np.ndarray:
    uu = np.array(u, dtype=np.float64, copy=True).ravel()
    lib().orc_rope(_p(uu), n_heads, head_dim, pos, theta)
    return uu


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


def argmax(v) -> int:
    vv = np.ascontiguousarray(v, dtype=np.float64)
    return int(lib().orc_argmax(_p(vv), vv.size))


class KVCache:
    """One layer's cache in storage format: [n_kv][cap][hd] (+ int8 scales
    [n_kv][cap])."""

    def __init__(self, kvdt: str, n_kv: int, cap: int, hd: int):
        npdt = {"f32": np.float32, "bf16": np.uint16, "i8": np.int8}[kvdt]
        self.kvdt = kvdt
        self.n_kv, self.cap, self.hd = n_kv, cap, hd
        self.k = np.zeros((n_kv, cap, hd), npdt)
        self.v = np.zeros((n_kv, cap, hd), npdt)
        self.ks = np.zeros((n_kv, cap), np.float32)
        self.vs = np.zeros((n_kv, cap), np.float32)

    def store(self, k: np.ndarray, v: np.ndarray, pos: int):
        L = lib()
        kk = np.ascontiguousarray(k, np.float64)
        vv = np.ascontiguousarray(v, np.float64)
        L.orc_kv_store(DT[self.kvdt], _p(kk), _p(self.k), _p(self.ks), self.n_kv, self.hd,
                       self.cap, pos)
        L.orc_kv_store(DT[self.kvdt], _p(vv), _p(self.v), _p(self.vs), self.n_kv, self.hd,
                       self.cap, pos)

    def dequant(self, which: str, length: int) -> np.ndarray:
        """Dequantized values [n_kv][length][hd] as the oracle reads them."""
        c = self.k if which == "k" else self.v
        s = self.ks if which == "k" else self.vs
        c = c[:, :length]
        if self.kvdt == "f32":
            return c.astype(np.float64)
        if self.kvdt == "bf16":
            return (c.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return (c.astype(np.float32) * s[:, :length, None]).astype(np.float32).astype(np.float64)


def attention(q, cache: KVCache, n_qh: int, length: int, want_probs: bool = False):
    qq = np.ascontiguousarray(q, np.float64)
    out = np.empty(n_qh * cache.hd, np.float64)
    probs = np.empty((n_qh, length), np.float64) if want_probs else None
    lib().orc_attention(DT[cache.kvdt], _p(qq), _p(cache.k), _p(cache.v), _p(cache.ks),
                        _p(cache.vs), _p(out), n_qh, cache.n_kv, cache.hd, cache.cap, length,
                        _p(probs))
    return (out, probs) if want_probs else out


# --------------------------------------------------------------- decoder ---

class _Cfg(C.Structure):
    _fields_ = [("hidden", C.c_int), ("n_layers", C.c_int), ("n_qh", C.c_int),
                ("n_kv", C.c_int), ("head_dim", C.c_int), ("inter", C.c_int),
                ("vocab", C.c_int), ("groups", C.c_int), ("cap", C.c_int),
                ("kvdt", C.c_int), ("embdt", C.c_int), ("eps", C.c_double),
                ("theta", C.c_double)]


class _Layer(C.Structure):
    _fields_ = [("qkv", _Mat), ("o", _Mat), ("gu", _Mat), ("down", _Mat),
                ("g_in", _vp), ("g_post", _vp), ("kc", _vp), ("vc", _vp),
                ("ks", _vp), ("vs", _vp)]


class _Model(C.Structure):
    _fields_ = [("cfg", _Cfg), ("embed", _vp), ("lm", _Mat), ("g_final", _vp),
                ("layers", C.POINTER(_Layer))]


class Decoder:
    """The dense decoder of a ``synth.DecoderConfig`` with its KV caches.

    ``weights`` maps names to storage-format inputs:
      embed [V][H] (fp32 or bf16 bits), lm_head (Mat), and per layer l the
      Mats ``layers.l.{wqkv,wo,wgu,wd}`` plus gains ``g_in``, ``g_post``,
      ``g_final`` (fp32)."""

    def __init__(self, cfg, embed: np.ndarray, lm: Mat, layers: List[Dict[str, Mat]],
                 g_in: List[np.ndarray], g_post: List[np.ndarray], g_final: np.ndarray):
        self.cfg = cfg
        self.embed = np.ascontiguousarray(embed)
        self.lm = lm
        self.layers = layers
        self.g_in = [np.ascontiguousarray(g, np.float32) for g in g_in]
        self.g_post = [np.ascontiguousarray(g, np.float32) for g in g_post]
        self.g_final = np.ascontiguousarray(g_final, np.float32)
        self.caches = [KVCache(cfg.kvdt, cfg.n_kv, cfg.cap, cfg.head_dim)
                       for _ in range(cfg.n_layers)]
        self._build()

    def _build(self):
        cfg = self.cfg
        arr = (_Layer * cfg.n_layers)()
        for l, (mats, kv) in enumerate(zip(self.layers, self.caches)):
            arr[l].qkv = mats["wqkv"].c
            arr[l].o = mats["wo"].c
            arr[l].gu = mats["wgu"].c
            arr[l].down = mats["wd"].c
            arr[l].g_in = _p(self.g_in[l])
            arr[l].g_post = _p(self.g_post[l])
            arr[l].kc, arr[l].vc = _p(kv.k), _p(kv.v)
            arr[l].ks, arr[l].vs = _p(kv.ks), _p(kv.vs)
        self._layers_arr = arr
        c = _Cfg(cfg.hidden, cfg.n_layers, cfg.n_qh, cfg.n_kv, cfg.head_dim, cfg.inter,
                 cfg.vocab, cfg.groups, cfg.cap, DT[cfg.kvdt], DT[cfg.embed_dt],
                 cfg.eps, cfg.theta)
        self._model = _Model(c, _p(self.embed), self.lm.c, _p(self.g_final),
                             C.cast(arr, C.POINTER(_Layer)))

    @classmethod
    def from_synth(cls, cfg, n_layers: Optional[int] = None, progress=None) -> "Decoder":
        """Build from the seeded draws in ``synth`` (optionally only the first
        ``n_layers`` layers, for partial-depth checks).  ``progress``, if
        given, is called with a short message after each layer is drawn."""
        import synth
        if n_layers is not None:
            cfg = cfg.replace(n_layers=n_layers)
        layers, gi, gp = [], [], []
        for l in range(cfg.n_layers):
            layers.append({w: Mat.from_draw(cfg.wdt, synth.layer_weight(cfg, l, w))
                           for w in ("wqkv", "wo", "wgu", "wd")})
            gi.append(synth.norm_gain(cfg))
            gp.append(synth.norm_gain(cfg))
            if progress is not None:
                progress(f"oracle layer {l + 1}/{cfg.n_layers} drawn")
        lm = Mat.from_draw(cfg.wdt, synth.lm_head_weight(cfg))
        return cls(cfg, synth.embed_weight(cfg), lm, layers, gi, gp, synth.norm_gain(cfg))

    def load_int8_prefix(self, length: int):
        """Fill cache slots [0, length) of every layer with the seeded int8
        history of ``synth.int8_kv_prefix`` (the same bytes the GPU side gets)."""
        import synth
        for l, c in enumerate(self.caches):
            kc, vc, ks, vs = synth.int8_kv_prefix(self.cfg, l, length)
            c.k[:, :length] = kc
            c.v[:, :length] = vc
            c.ks[:, :length] = ks
            c.vs[:, :length] = vs

    def step(self, token: int, pos: int, want_logits: bool = True):
        """Run one position; returns (argmax, fp64 logits) or (-1, None)."""
        if not (0 <= token < self.cfg.vocab) or not (0 <= pos < self.cfg.cap):
            raise ValueError("token or position out of range")
        logits = np.empty(self.cfg.vocab, np.float64) if want_logits else None
        nxt = lib().orc_decode_step(C.addressof(self._model), int(token), int(pos), _p(logits))
        return int(nxt), logits

    def generate(self, prompt: Sequence[int], n_decode: int, teacher: Optional[Sequence[int]] = None):
        """Greedy run: feed the prompt, then n_decode steps.  Returns the emitted
        tokens and the logits of every emitting position.  With ``teacher``
        the fed tokens are taken from it instead of the argmax (teacher
        forcing); the emitted argmaxes are still returned."""
        toks, logits = [], []
        P = len(prompt)
        n_decode = min(n_decode, self.cfg.cap - P)      # clamp the budget
        for p, t in enumerate(prompt):
            last = p == P - 1
            nxt, lg = self.step(int(t), p, want_logits=last)
        toks.append(nxt)
        logits.append(lg)
        for i in range(n_decode - 1):
            feed = toks[-1] if teacher is None else int(teacher[i])
            nxt, lg = self.step(feed, P + i)
            toks.append(nxt)
            logits.append(lg)
        return toks, logits


# ------------------------------------------------------------------- MoE ---

def moe_route(wr: Mat, bias: np.ndarray, x: np.ndarray, top_k: int, routed_scale: float):
    E, H = wr.shape
    xx = np.ascontiguousarray(x, np.float64)
    b = np.ascontiguousarray(bias, np.float32)
    sel = np.empty(top_k, np.int32)
    gate = np.empty(top_k, np.float64)
    lib().orc_moe_route(C.addressof(wr.c), _p(b), _p(xx), H, E, top_k, routed_scale,
                        _p(sel), _p(gate))
    return sel, gate


def swiglu_expert(w13: Mat, w2: Mat, u: np.ndarray) -> np.ndarray:
    """One SwiGLU expert W2 (silu(W1 u) * (W3 u)); W13 stacks W1 then W3."""
    inter = w13.shape[0] // 2
    out_dim = w2.shape[0]
    uu = np.ascontiguousarray(u, np.float64)
    assert uu.size == w13.shape[1] and w2.shape[1] == inter
    out = np.empty(out_dim, np.float64)
    lib().orc_swiglu_expert(C.addressof(w13.c), C.addressof(w2.c), _p(uu), uu.size, inter,
                            out_dim, _p(out))
    return out


def moe_apply(wdn: Mat, wup: Mat, experts13: Dict[int, Mat], experts2: Dict[int, Mat],
              shared13: List[Mat], shared2: List[Mat], x: np.ndarray, latent: int, inter: int,
              eps: float, sel: np.ndarray, gate: np.ndarray) -> np.ndarray:
    """One token row through the latent-MoE layer, with a given routing."""
    H = x.size
    n_exp = int(max(sel)) + 1
    t13 = (_Mat * n_exp)()
    t2 = (_Mat * n_exp)()
    for e in set(int(s) for s in sel):
        t13[e] = experts13[e].c
        t2[e] = experts2[e].c
    ns = len(shared13)
    s13 = (_Mat * max(1, ns))()
    s2 = (_Mat * max(1, ns))()
    for i in range(ns):
        s13[i] = shared13[i].c
        s2[i] = shared2[i].c
    xx = np.ascontiguousarray(x, np.float64)
    s = np.ascontiguousarray(sel, np.int32)
    g = np.ascontiguousarray(gate, np.float64)
    y = np.empty(H, np.float64)
    lib().orc_moe_apply(C.addressof(wdn.c), C.addressof(wup.c), C.addressof(t13),
                        C.addressof(t2), C.addressof(s13), C.addressof(s2), ns, _p(xx), H,
                        latent, inter, eps, _p(s), _p(g), len(sel), _p(y))
    return y
