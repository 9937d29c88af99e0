"""ctypes binding of libk2.so -- argument marshalling only.

Every function has the name and argument order of its C counterpart in
``include/k2.h``.  Device buffers are passed as torch tensors on the GPU (or
None for NULL), sizes as ints; the return value is the ``k2_status`` int.
``check(rc)`` turns a nonzero status into ``K2Error``.  Every computation runs
in the HIP library; when it is missing this module raises instead of falling
back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libk2.so")

K2_OK, K2_EINVAL, K2_ERANGE, K2_EUNSUPPORTED, K2_EHIP = 0, -1, -2, -3, -4
K2_F32, K2_BF16, K2_FP8E4M3, K2_MXFP4, K2_I8, K2_Q4S = 0, 1, 2, 3, 4, 5
DTYPES = {"f32": K2_F32, "bf16": K2_BF16, "fp8": K2_FP8E4M3, "mxfp4": K2_MXFP4, "i8": K2_I8,
          "q4s": K2_Q4S}

_lib = None


class K2Error(RuntimeError):
    def __init__(self, rc: int):
        super().__init__(f"k2 status {rc}: {k2_status_str(rc)}")
        self.rc = rc


def load(build_if_missing: bool = True):
    """Load libk2.so from the package directory (building it once with hipcc
    if it has never been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise RuntimeError(f"{LIB_PATH} is not built")
        from . import build as _b
        _b.build()
    _lib = C.CDLL(LIB_PATH)
    _declare(_lib)
    return _lib


_vp, _i, _f, _d, _sz = C.c_void_p, C.c_int, C.c_float, C.c_double, C.c_size_t

SIGNATURES = {
    "k2_abi_version": (_i, []),
    "k2_status_str": (C.c_char_p, [_i]),
    "k2_quantize_fp8_rows": (_i, [_vp, _vp, _vp, _i, _i, _vp]),
    "k2_quantize_mxfp4": (_i, [_vp, _vp, _vp, _i, _i, _vp]),
    "k2_quantize_q4s": (_i, [_vp, _vp, _vp, _i, _i, _vp]),
    "k2_rmsnorm_grouped": (_i, [_vp, _vp, _vp, _i, _i, _i, _f, _vp]),
    "k2_gemv_qbf16": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "k2_gemv_qfp8": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "k2_gemv_qmxfp4": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "k2_gemv_qq4s": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "k2_gemv_f32": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "k2_norm_gemv": (_i, [_i, _vp, _vp, _vp, _vp, _i, _f, _vp, _i, _i, _vp]),
    "k2_norm_gemv_swiglu": (_i, [_i, _vp, _vp, _vp, _vp, _i, _f, _vp, _i, _i, _vp]),
    "k2_norm_gemv_argmax": (_i, [_i, _vp, _vp, _vp, _vp, _i, _f, _vp, _i, _i, _vp, _vp, _sz, _vp]),
    "k2_rope_table": (_i, [_vp, _i, _i, _d, _vp]),
    "k2_rope": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "k2_kv_append": (_i, [_i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "k2_kv_append_int8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "k2_attn_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "k2_gqa_decode_attn": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp,
                                _sz, _vp]),
    "k2_gqa_decode_attn_scratch_limit": (_sz, []),
    "k2_gqa_decode_attn_noalloc": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                                        _vp]),
    "k2_rope_append_attn": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp,
                                 _sz, _vp]),
    "k2_rope_append_attn_o": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                   _vp, _vp, _vp, _i, _vp, _sz, _vp, _vp]),
    "k2_argmax_workspace_bytes": (_sz, [_i]),
    "k2_sample_workspace_bytes": (_sz, [_i]),
    "k2_sample": (_i, [_vp, _i, _vp, _vp, _i, C.c_uint64, C.c_uint64, _vp, _vp, _sz, _vp]),
    "k2_argmax": (_i, [_vp, _i, _vp, _vp, _sz, _vp]),
    "k2_decode_workspace_bytes": (_sz, [_vp]),
    "k2_model_check": (_i, [_vp]),
    "k2_decode_step": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "k2_prefill_workspace_bytes": (_sz, [_vp, _i]),
    "k2_prefill": (_i, [_vp, _vp, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "k2_verify_workspace_bytes": (_sz, [_vp, _i]),
    "k2_verify": (_i, [_vp, _vp, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "k2_decode_step_dev": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "k2_read_probe": (_i, [_vp, _sz, _i, _vp, _vp]),
    "k2_moe_route_workspace_bytes": (_sz, [_i, _i]),
    "k2_moe_route": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _f, _vp, _vp, _vp, _sz, _vp]),
    "k2_moe_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "k2_moe_expert_gemv": (_i, [_vp, _i, _i, _i, _vp, _vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _sz, _vp]),
    "k2_moe_layer_workspace_bytes": (_sz, [_vp, _i]),
    "k2_moe_layer": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
}


def _declare(L):
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


def ptr(t: Optional[torch.Tensor]):
    """Device address of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("k2 calls take device tensors")
    return t.data_ptr()


def stream_handle(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def check(rc: int) -> int:
    if rc != K2_OK:
        raise K2Error(rc)
    return rc


# --------------------------------------------------------------- wrappers --

def k2_abi_version() -> int:
    return load().k2_abi_version()


def k2_status_str(rc: int) -> str:
    return load().k2_status_str(int(rc)).decode()


def k2_quantize_fp8_rows(W, codes, row_scale, N, K, stream=None):
    return load().k2_quantize_fp8_rows(ptr(W), ptr(codes), ptr(row_scale), N, K, stream_handle(stream))


def k2_quantize_mxfp4(W, q, e8m0, N, K, stream=None):
    return load().k2_quantize_mxfp4(ptr(W), ptr(q), ptr(e8m0), N, K, stream_handle(stream))


def k2_rmsnorm_grouped(x, gamma, y, rows, hidden, groups, eps, stream=None):
    return load().k2_rmsnorm_grouped(ptr(x), ptr(gamma), ptr(y), rows, hidden, groups, eps,
                                     stream_handle(stream))


def k2_gemv_qbf16(W, x, y, residual, N, K, B, stream=None):
    return load().k2_gemv_qbf16(ptr(W), ptr(x), ptr(y), ptr(residual), N, K, B, stream_handle(stream))


def k2_gemv_qfp8(W, row_scale, x, y, residual, N, K, B, stream=None):
    return load().k2_gemv_qfp8(ptr(W), ptr(row_scale), ptr(x), ptr(y), ptr(residual), N, K, B,
                               stream_handle(stream))


def k2_quantize_q4s(W, q, s, N, K, stream=None):
    return load().k2_quantize_q4s(ptr(W), ptr(q), ptr(s), N, K, stream_handle(stream))


def k2_gemv_qq4s(Wq, Ws, x, y, residual, N, K, B, stream=None):
    return load().k2_gemv_qq4s(ptr(Wq), ptr(Ws), ptr(x), ptr(y), ptr(residual), N, K, B,
                               stream_handle(stream))


def k2_gemv_qmxfp4(Wq, We8m0, x, y, residual, N, K, B, stream=None):
    return load().k2_gemv_qmxfp4(ptr(Wq), ptr(We8m0), ptr(x), ptr(y), ptr(residual), N, K, B,
                                 stream_handle(stream))


def k2_gemv_f32(W, x, y, residual, N, K, B, stream=None):
    return load().k2_gemv_f32(ptr(W), ptr(x), ptr(y), ptr(residual), N, K, B, stream_handle(stream))


def k2_norm_gemv(wdt, W, S, h, gamma, groups, eps, y, N, K, stream=None):
    return load().k2_norm_gemv(wdt, ptr(W), ptr(S), ptr(h), ptr(gamma), groups, eps, ptr(y), N, K,
                               stream_handle(stream))


def k2_norm_gemv_swiglu(wdt, W, S, h, gamma, groups, eps, act, inter, K, stream=None):
    return load().k2_norm_gemv_swiglu(wdt, ptr(W), ptr(S), ptr(h), ptr(gamma), groups, eps, ptr(act),
                                      inter, K, stream_handle(stream))


def k2_norm_gemv_argmax(wdt, W, S, h, gamma, groups, eps, logits, N, K, out_idx, ws, ws_bytes,
                        stream=None):
    return load().k2_norm_gemv_argmax(wdt, ptr(W), ptr(S), ptr(h), ptr(gamma), groups, eps,
                                      ptr(logits), N, K, ptr(out_idx), ptr(ws), ws_bytes,
                                      stream_handle(stream))


def k2_rope_table(cos_sin, cap, head_dim, theta, stream=None):
    return load().k2_rope_table(ptr(cos_sin), cap, head_dim, float(theta), stream_handle(stream))


def k2_rope(q, k, cos_sin, n_qh, n_kv, head_dim, pos, cap, stream=None):
    return load().k2_rope(ptr(q), ptr(k), ptr(cos_sin), n_qh, n_kv, head_dim, pos, cap,
                          stream_handle(stream))


def k2_kv_append(kvdt, k, v, kc, vc, n_kv, head_dim, cap, pos, stream=None):
    return load().k2_kv_append(kvdt, ptr(k), ptr(v), ptr(kc), ptr(vc), n_kv, head_dim, cap, pos,
                               stream_handle(stream))


def k2_kv_append_int8(k, v, kc, vc, ks, vs, n_kv, head_dim, cap, pos, stream=None):
    return load().k2_kv_append_int8(ptr(k), ptr(v), ptr(kc), ptr(vc), ptr(ks), ptr(vs), n_kv,
                                    head_dim, cap, pos, stream_handle(stream))


def k2_attn_workspace_bytes(n_qh, n_kv, head_dim, cap) -> int:
    return load().k2_attn_workspace_bytes(n_qh, n_kv, head_dim, cap)


def k2_gqa_decode_attn(kvdt, q, kc, vc, ks, vs, out, n_qh, n_kv, head_dim, cap, length, scale, ws,
                       ws_bytes, stream=None):
    return load().k2_gqa_decode_attn(kvdt, ptr(q), ptr(kc), ptr(vc), ptr(ks), ptr(vs), ptr(out),
                                     n_qh, n_kv, head_dim, cap, length, float(scale), ptr(ws),
                                     ws_bytes, stream_handle(stream))


def k2_gqa_decode_attn_scratch_limit() -> int:
    return load().k2_gqa_decode_attn_scratch_limit()


def k2_gqa_decode_attn_noalloc(kvdt, q, kc, vc, ks, vs, out, n_qh, n_kv, head_dim, cap, length,
                               scale, stream=None):
    return load().k2_gqa_decode_attn_noalloc(kvdt, ptr(q), ptr(kc), ptr(vc), ptr(ks), ptr(vs),
                                             ptr(out), n_qh, n_kv, head_dim, cap, length,
                                             float(scale), stream_handle(stream))


def k2_rope_append_attn(kvdt, qkv, cos_sin, kc, vc, ks, vs, out, n_qh, n_kv, head_dim, cap, pos,
                        ws, ws_bytes, stream=None):
    return load().k2_rope_append_attn(kvdt, ptr(qkv), ptr(cos_sin), ptr(kc), ptr(vc), ptr(ks),
                                      ptr(vs), ptr(out), n_qh, n_kv, head_dim, cap, pos, ptr(ws),
                                      ws_bytes, stream_handle(stream))


def k2_rope_append_attn_o(kvdt, qkv, cos_sin, kc, vc, ks, vs, out, n_qh, n_kv, head_dim, cap, pos,
                          wdt, Wo, Wo_s, h, hidden, ws, ws_bytes, d_err=None, stream=None):
    return load().k2_rope_append_attn_o(kvdt, ptr(qkv), ptr(cos_sin), ptr(kc), ptr(vc), ptr(ks),
                                        ptr(vs), ptr(out), n_qh, n_kv, head_dim, cap, pos, wdt,
                                        ptr(Wo), ptr(Wo_s), ptr(h), hidden, ptr(ws), ws_bytes,
                                        ptr(d_err), stream_handle(stream))


def k2_argmax_workspace_bytes(n) -> int:
    return load().k2_argmax_workspace_bytes(n)


def k2_argmax(x, n, out_idx, ws, ws_bytes, stream=None):
    return load().k2_argmax(ptr(x), n, ptr(out_idx), ptr(ws), ws_bytes, stream_handle(stream))


# ------------------------------------------------------ decode-step structs --

class k2_config(C.Structure):
    _fields_ = [("hidden", _i), ("n_layers", _i), ("n_qh", _i), ("n_kv", _i), ("head_dim", _i),
                ("inter", _i), ("vocab", _i), ("groups", _i), ("cap", _i), ("eps", _f),
                ("rope_theta", _d), ("wdt", _i), ("kvdt", _i), ("embdt", _i)]


class k2_layer(C.Structure):
    _fields_ = [("qkv", _vp), ("qkv_s", _vp), ("o", _vp), ("o_s", _vp), ("gu", _vp),
                ("gu_s", _vp), ("down", _vp), ("down_s", _vp), ("g_in", _vp), ("g_post", _vp),
                ("kc", _vp), ("vc", _vp), ("ks", _vp), ("vs", _vp)]


class k2_model(C.Structure):
    _fields_ = [("cfg", k2_config), ("embed", _vp), ("lm", _vp), ("lm_s", _vp),
                ("g_final", _vp), ("rope", _vp), ("layers", C.POINTER(k2_layer)), ("ws", _vp),
                ("ws_bytes", _sz)]


def k2_decode_workspace_bytes(cfg: k2_config) -> int:
    return load().k2_decode_workspace_bytes(C.addressof(cfg))


def k2_model_check(model: k2_model) -> int:
    return load().k2_model_check(C.addressof(model))


def k2_decode_step(model: k2_model, token: int, pos: int, logits, next_token, stream=None):
    return load().k2_decode_step(C.addressof(model), int(token), int(pos), ptr(logits),
                                 ptr(next_token), stream_handle(stream))


def k2_decode_step_dev(model: k2_model, d_token, d_pos, logits, next_token, d_err,
                       stream=None):
    return load().k2_decode_step_dev(C.addressof(model), ptr(d_token), ptr(d_pos), ptr(logits),
                                     ptr(next_token), ptr(d_err), stream_handle(stream))


# --------------------------------------------------------------- latent MoE --

def k2_moe_route_workspace_bytes(T, n_experts) -> int:
    return load().k2_moe_route_workspace_bytes(T, n_experts)


def k2_moe_route(Wr, bias, x, T, hidden, n_experts, top_k, routed_scale, topk_idx, topk_w, ws,
                 ws_bytes, stream=None):
    return load().k2_moe_route(ptr(Wr), ptr(bias), ptr(x), T, hidden, n_experts, top_k,
                               float(routed_scale), ptr(topk_idx), ptr(topk_w), ptr(ws), ws_bytes,
                               stream_handle(stream))


def k2_moe_workspace_bytes(T, top_k, latent, inter) -> int:
    return load().k2_moe_workspace_bytes(T, top_k, latent, inter)


def k2_moe_expert_gemv(z, T, latent, inter, topk_idx, topk_w, top_k, n_experts, w13q, w13s, w2q,
                       w2s, r, d_err, ws, ws_bytes, stream=None):
    return load().k2_moe_expert_gemv(ptr(z), T, latent, inter, ptr(topk_idx), ptr(topk_w), top_k,
                                     n_experts, ptr(w13q), ptr(w13s), ptr(w2q), ptr(w2s), ptr(r),
                                     ptr(d_err), ptr(ws), ws_bytes, stream_handle(stream))


class k2_moe_config(C.Structure):
    _fields_ = [("hidden", _i), ("latent", _i), ("inter", _i), ("n_experts", _i), ("top_k", _i),
                ("n_shared", _i), ("routed_scale", _f), ("eps", _f)]


class k2_moe_layer_weights(C.Structure):
    _fields_ = [("cfg", k2_moe_config), ("w_router", _vp), ("router_bias", _vp), ("w_down", _vp),
                ("latent_gamma", _vp), ("w_up", _vp), ("w13q", _vp), ("w13s", _vp), ("w2q", _vp),
                ("w2s", _vp), ("sh_w13", _vp), ("sh_w2", _vp)]


def k2_moe_layer_workspace_bytes(cfg: k2_moe_config, T) -> int:
    return load().k2_moe_layer_workspace_bytes(C.addressof(cfg), T)


def k2_moe_layer(weights: k2_moe_layer_weights, x, T, y, topk_idx_out, topk_w_out, d_err, ws,
                 ws_bytes, stream=None):
    return load().k2_moe_layer(C.addressof(weights), ptr(x), T, ptr(y), ptr(topk_idx_out),
                               ptr(topk_w_out), ptr(d_err), ptr(ws), ws_bytes,
                               stream_handle(stream))


def k2_prefill_workspace_bytes(cfg, T) -> int:
    return load().k2_prefill_workspace_bytes(C.addressof(cfg), T)


def k2_prefill(model, tokens, T, pos0, logits, next_token, ws, ws_bytes, stream=None):
    """tokens: a host sequence of T ints (copied into a C array here)."""
    arr = (C.c_int32 * T)(*[int(t) for t in tokens])
    return load().k2_prefill(C.addressof(model), arr, T, pos0, ptr(logits), ptr(next_token), ptr(ws),
                             ws_bytes, stream_handle(stream))


def k2_verify_workspace_bytes(cfg, T) -> int:
    return load().k2_verify_workspace_bytes(C.addressof(cfg), T)


def k2_verify(model, tokens, T, pos0, logits, next_tokens, ws, ws_bytes, stream=None):
    """tokens: a host sequence of T ints; next_tokens: device int32 [T]."""
    arr = (C.c_int32 * T)(*[int(t) for t in tokens])
    return load().k2_verify(C.addressof(model), arr, T, pos0, ptr(logits), ptr(next_tokens), ptr(ws),
                            ws_bytes, stream_handle(stream))


class k2_sampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_k", C.c_int), ("top_p", C.c_float),
                ("min_p", C.c_float), ("repetition_penalty", C.c_float)]


def k2_sample_workspace_bytes(vocab) -> int:
    return load().k2_sample_workspace_bytes(vocab)


def k2_sample(logits, vocab, sp: "k2_sampling", prev, n_prev, seed, counter, out_token, ws, ws_bytes,
              stream=None):
    return load().k2_sample(ptr(logits), vocab, C.addressof(sp), ptr(prev), n_prev, int(seed),
                            int(counter), ptr(out_token), ptr(ws), ws_bytes, stream_handle(stream))


# -------------------------------------------------------------- measurement --

def k2_read_probe(buf, nbytes: int, blocks: int, sink, stream=None):
    return load().k2_read_probe(ptr(buf), int(nbytes), int(blocks), ptr(sink),
                                stream_handle(stream))
