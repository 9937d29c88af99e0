"""Host-side checks of the C ABI (no GPU needed).

* libk2.so loads and exports every function that include/k2.h declares.
* Size queries and status strings work on the host.
* Argument validation refuses bad calls with the documented status before
  anything is launched: fake (but aligned) device addresses are passed, so a
  call that got past validation would try to launch and fail with K2_EHIP on
  this GPU-less host instead of returning the expected status.
* The Python binding raises instead of falling back when the library is absent.
"""
import ctypes as C
import os
import re

import pytest

from quantized_gemv_gqa_decode_amd import k2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "k2.h")
FAKE = 0x10000          # aligned, never dereferenced on the host


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(k2_[a-z0-9_]+)\s*\(", src)
    return sorted(set(n for n in names))


def test_every_declared_symbol_is_exported():
    L = k2.load()
    names = declared_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    # and the binding declares a signature for every one of them
    assert not [n for n in names if n not in k2.SIGNATURES], \
        [n for n in names if n not in k2.SIGNATURES]


def test_version_and_status_strings():
    assert k2.k2_abi_version() == 2
    for rc in (0, -1, -2, -3, -4):
        assert k2.k2_status_str(rc)
    assert "unknown" in k2.k2_status_str(7)


def test_workspace_sizes():
    assert k2.k2_attn_workspace_bytes(32, 8, 128, 4096) > 0
    assert k2.k2_attn_workspace_bytes(32, 7, 128, 4096) == 0          # n_qh % n_kv
    assert k2.k2_argmax_workspace_bytes(250624) > 0
    assert k2.k2_argmax_workspace_bytes(0) == 0
    c = k2.k2_config(2560, 36, 32, 8, 128, 10240, 250624, 2, 4096, 1e-6, 1e4, k2.K2_BF16,
                     k2.K2_BF16, k2.K2_BF16)
    assert k2.k2_decode_workspace_bytes(c) > 0
    bad = k2.k2_config(2560, 36, 32, 8, 96, 10240, 250624, 2, 4096, 1e-6, 1e4, k2.K2_BF16,
                       k2.K2_BF16, k2.K2_BF16)
    assert k2.k2_decode_workspace_bytes(bad) == 0                       # head_dim 96


def test_gemv_validation():
    L = k2.load()
    st = None
    assert L.k2_gemv_qbf16(None, FAKE, FAKE, None, 8, 64, 1, st) == k2.K2_EINVAL
    assert L.k2_gemv_qbf16(FAKE + 2, FAKE, FAKE, None, 8, 64, 1, st) == k2.K2_EINVAL
    assert L.k2_gemv_qbf16(FAKE, FAKE, FAKE, None, 0, 64, 1, st) == k2.K2_EINVAL
    assert L.k2_gemv_qbf16(FAKE, FAKE, FAKE, None, 8, 48, 1, st) == k2.K2_EUNSUPPORTED
    assert L.k2_gemv_qbf16(FAKE, FAKE, FAKE, None, 8, 64, 3, st) == k2.K2_EUNSUPPORTED
    assert L.k2_gemv_qbf16(FAKE, FAKE, FAKE, None, 8, 12288 + 32, 1, st) == k2.K2_EUNSUPPORTED
    assert L.k2_gemv_qfp8(FAKE, None, FAKE, FAKE, None, 8, 64, 1, st) == k2.K2_EINVAL
    assert L.k2_gemv_qmxfp4(FAKE, None, FAKE, FAKE, None, 8, 64, 1, st) == k2.K2_EINVAL
    assert L.k2_gemv_qq4s(FAKE, None, FAKE, FAKE, None, 8, 64, 1, st) == k2.K2_EINVAL
    assert L.k2_gemv_qq4s(FAKE, FAKE, FAKE, FAKE, None, 8, 96, 1, st) == k2.K2_EUNSUPPORTED
    assert L.k2_quantize_q4s(FAKE, FAKE, FAKE, 8, 96, st) == k2.K2_EUNSUPPORTED
    assert L.k2_quantize_q4s(FAKE, FAKE, None, 8, 64, st) == k2.K2_EINVAL
    assert L.k2_quantize_mxfp4(FAKE, FAKE, FAKE, 8, 48, st) == k2.K2_EUNSUPPORTED
    assert L.k2_quantize_fp8_rows(FAKE, FAKE, FAKE, 8, 40, st) == k2.K2_EINVAL


def test_rope_append_attention_validation():
    L = k2.load()
    st = None
    assert L.k2_rope(FAKE, FAKE, FAKE, 32, 8, 128, 4096, 4096, st) == k2.K2_ERANGE
    assert L.k2_rope(FAKE, FAKE, FAKE, 32, 8, 96, 0, 4096, st) == k2.K2_EUNSUPPORTED
    assert L.k2_kv_append(k2.K2_BF16, FAKE, FAKE, FAKE, FAKE, 8, 128, 4096, -1, st) == k2.K2_ERANGE
    assert L.k2_kv_append(k2.K2_I8, FAKE, FAKE, FAKE, FAKE, 8, 128, 4096, 0, st) == k2.K2_EUNSUPPORTED
    assert L.k2_kv_append_int8(FAKE, FAKE, FAKE, FAKE, None, FAKE, 8, 128, 4096, 0, st) == k2.K2_EINVAL
    wsb = k2.k2_attn_workspace_bytes(32, 8, 128, 4096)
    ws = 0x100000
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 8, 128, 4096)
    assert L.k2_gqa_decode_attn(k2.K2_BF16, *args, 0, 0.1, ws, wsb, st) == k2.K2_ERANGE
    assert L.k2_gqa_decode_attn(k2.K2_BF16, *args, 4097, 0.1, ws, wsb, st) == k2.K2_ERANGE
    assert L.k2_gqa_decode_attn(k2.K2_BF16, *args, 10, 0.1, ws, wsb - 4, st) == k2.K2_EINVAL
    assert L.k2_gqa_decode_attn(k2.K2_BF16, *args, 10, 0.1, ws + 16, wsb, st) == k2.K2_EINVAL
    assert L.k2_gqa_decode_attn(k2.K2_FP8E4M3, *args, 10, 0.1, ws, wsb, st) == k2.K2_EUNSUPPORTED
    assert L.k2_gqa_decode_attn(k2.K2_I8, FAKE, FAKE, FAKE, None, None, FAKE, 32, 8, 128, 4096,
                                10, 0.1, ws, wsb, st) == k2.K2_EINVAL
    assert L.k2_rope_append_attn(k2.K2_BF16, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 32, 8, 128,
                                 4096, 4096, ws, wsb, st) == k2.K2_ERANGE
    assert L.k2_argmax(FAKE, 100, FAKE, ws, 16, st) == k2.K2_EINVAL
    # attention + O projection: refusals before any launch
    ao = (FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 32, 8, 128, 4096)
    assert L.k2_rope_append_attn_o(k2.K2_BF16, *ao, 4096, k2.K2_BF16, FAKE, None, FAKE, 2560,
                                   ws, wsb, None, st) == k2.K2_ERANGE
    assert L.k2_rope_append_attn_o(k2.K2_BF16, *ao, 0, k2.K2_FP8E4M3, FAKE, None, FAKE, 2560,
                                   ws, wsb, None, st) == k2.K2_EINVAL       # fp8 needs row scales
    assert L.k2_rope_append_attn_o(k2.K2_BF16, *ao, 0, k2.K2_I8, FAKE, None, FAKE, 2560,
                                   ws, wsb, None, st) == k2.K2_EUNSUPPORTED  # not a weight format
    assert L.k2_rope_append_attn_o(k2.K2_BF16, *ao, 0, k2.K2_BF16, FAKE, None, None, 2560,
                                   ws, wsb, None, st) == k2.K2_EINVAL       # h missing
    assert L.k2_rope_append_attn_o(k2.K2_BF16, *ao, 0, k2.K2_BF16, FAKE, None, FAKE, 0,
                                   ws, wsb, None, st) == k2.K2_EINVAL


def _fake_model(cfg_kw=None):
    c = dict(hidden=64, n_layers=2, n_qh=4, n_kv=2, head_dim=16, inter=256, vocab=512, groups=2,
             cap=32, eps=1e-6, rope_theta=1e4, wdt=k2.K2_F32, kvdt=k2.K2_F32, embdt=k2.K2_F32)
    c.update(cfg_kw or {})
    cfg = k2.k2_config(**c)
    arr = (k2.k2_layer * c["n_layers"])()
    for i in range(c["n_layers"]):
        arr[i] = k2.k2_layer(*([FAKE] * 14))
    ws_b = k2.k2_decode_workspace_bytes(cfg)
    m = k2.k2_model(cfg, FAKE, FAKE, FAKE, FAKE, FAKE, C.cast(arr, C.POINTER(k2.k2_layer)),
                    0x100000, ws_b)
    m._keep = arr
    return m


def test_decode_step_refuses_before_launch():
    m = _fake_model()
    assert k2.k2_model_check(m) == k2.K2_OK
    L = k2.load()
    adr = C.addressof(m)
    assert L.k2_decode_step(adr, 512, 0, FAKE, FAKE, None) == k2.K2_ERANGE
    assert L.k2_decode_step(adr, -1, 0, FAKE, FAKE, None) == k2.K2_ERANGE
    assert L.k2_decode_step(adr, 0, 32, FAKE, FAKE, None) == k2.K2_ERANGE
    assert L.k2_decode_step(adr, 0, -1, FAKE, FAKE, None) == k2.K2_ERANGE
    assert L.k2_decode_step(adr, 0, 0, FAKE + 4, FAKE, None) == k2.K2_EINVAL
    assert L.k2_decode_step_dev(adr, None, FAKE, FAKE, FAKE, None, None) == k2.K2_EINVAL
    assert L.k2_decode_step_dev(adr, FAKE, None, FAKE, FAKE, None, None) == k2.K2_EINVAL
    m.ws_bytes -= 256
    assert L.k2_decode_step(adr, 0, 0, FAKE, FAKE, None) == k2.K2_EINVAL
    assert L.k2_decode_step(None, 0, 0, FAKE, FAKE, None) == k2.K2_EINVAL


def test_prefill_refuses_unsupported_shapes():
    # fp32 weights, and a bf16 model whose hidden size the matrix-core products
    # do not take (64 is not a multiple of 128): no workspace, no launch
    assert k2.k2_prefill_workspace_bytes(_fake_model().cfg, 8) == 0
    m = _fake_model(dict(wdt=k2.K2_BF16))
    assert k2.k2_prefill_workspace_bytes(m.cfg, 8) == 0
    assert k2.load().k2_prefill(C.addressof(m), (C.c_int32 * 8)(*[1] * 8), 8, 0, None, None,
                                0x100000, 1 << 20, None) == k2.K2_EUNSUPPORTED
    ok = dict(hidden=512, n_qh=8, n_kv=2, head_dim=128, inter=1024, vocab=1024, wdt=k2.K2_BF16)
    m = _fake_model(ok)
    assert k2.k2_prefill_workspace_bytes(m.cfg, 8) > 0
    assert k2.k2_prefill_workspace_bytes(m.cfg, 1) == 0
    assert k2.k2_prefill_workspace_bytes(m.cfg, 256) > k2.k2_prefill_workspace_bytes(m.cfg, 33) > 0
    assert k2.k2_prefill_workspace_bytes(m.cfg, 257) == 0
    sizes = [k2.k2_prefill_workspace_bytes(m.cfg, t) for t in range(2, 257)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))       # a chunk's workspace serves smaller chunks
    assert k2.k2_verify_workspace_bytes(m.cfg, 32) > 0
    assert k2.k2_verify_workspace_bytes(m.cfg, 33) == 0
    wsb = k2.k2_prefill_workspace_bytes(m.cfg, 8)
    L = k2.load()
    toks = (C.c_int32 * 8)(*[1] * 8)
    assert L.k2_prefill(C.addressof(m), toks, 8, 30, None, None, 0x100000, wsb, None) == k2.K2_ERANGE
    bad = (C.c_int32 * 8)(*([1] * 7 + [1024]))
    assert L.k2_prefill(C.addressof(m), bad, 8, 0, None, None, 0x100000, wsb, None) == k2.K2_ERANGE
    assert L.k2_prefill(C.addressof(m), toks, 8, 0, None, None, 0x100000, wsb - 1, None) == k2.K2_EINVAL
    assert L.k2_prefill(C.addressof(m), None, 8, 0, None, None, 0x100000, wsb, None) == k2.K2_EINVAL


@pytest.mark.parametrize("wdt", ["fp8", "mxfp4", "q4s"])
def test_prefill_takes_quantized_weights(wdt):
    # the matrix-core products decode fp8 / MXFP4 / Q4S weights: workspace
    # sizes as for bf16 (monotone in T), verification too; MXFP4 and Q4S
    # scale arrays that are not 16-byte aligned are refused before a launch
    ok = dict(hidden=512, n_qh=8, n_kv=2, head_dim=128, inter=1024, vocab=1024, wdt=k2.DTYPES[wdt])
    m = _fake_model(ok)
    sizes = [k2.k2_prefill_workspace_bytes(m.cfg, t) for t in range(2, 257)]
    assert sizes[0] > 0 and all(a <= b for a, b in zip(sizes, sizes[1:]))
    assert k2.k2_prefill_workspace_bytes(m.cfg, 257) == 0
    assert k2.k2_verify_workspace_bytes(m.cfg, 32) > 0
    assert k2.k2_verify_workspace_bytes(m.cfg, 33) == 0
    wsb = sizes[6]
    L = k2.load()
    toks = (C.c_int32 * 8)(*[1] * 8)
    assert L.k2_prefill(C.addressof(m), toks, 8, 30, None, None, 0x100000, wsb, None) == k2.K2_ERANGE
    if wdt != "fp8":
        m._keep[1].gu_s = FAKE + 8
        assert k2.k2_model_check(m) == k2.K2_OK
        assert L.k2_prefill(C.addressof(m), toks, 8, 0, None, None, 0x100000, wsb, None) == k2.K2_EINVAL


@pytest.mark.parametrize("change,rc", [(dict(head_dim=96), -3), (dict(n_kv=3), -3),
                                       (dict(groups=3), -3), (dict(hidden=48), -3),
                                       (dict(wdt=k2.K2_I8), -3), (dict(kvdt=k2.K2_MXFP4), -3),
                                       (dict(vocab=0), -1), (dict(eps=-1.0), -1)])
def test_model_check_rejects_bad_configs(change, rc):
    m = _fake_model(change)
    assert k2.k2_model_check(m) == rc


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(k2, "_lib", None)
    monkeypatch.setattr(k2, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        k2.load(build_if_missing=False)


def test_moe_validation():
    L = k2.load()
    st = None
    assert k2.k2_moe_workspace_bytes(32, 16, 3584, 3072) > 32 * 16 * (3584 + 3072) * 4
    assert k2.k2_moe_workspace_bytes(0, 16, 3584, 3072) == 0
    assert k2.k2_moe_route_workspace_bytes(8, 896) >= 8 * 896 * 4
    nb = k2.k2_moe_workspace_bytes(8, 16, 3584, 3072)

    def ex(T=8, latent=3584, inter=3072, k=16, E=896, z=FAKE, ws=FAKE, wsb=nb):
        return L.k2_moe_expert_gemv(z, T, latent, inter, FAKE, FAKE, k, E, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, None, ws, wsb, st)

    assert ex(z=None) == k2.K2_EINVAL
    assert ex(T=0) == k2.K2_EINVAL
    assert ex(latent=3584 + 16) == k2.K2_EUNSUPPORTED
    assert ex(inter=8192) == k2.K2_EUNSUPPORTED
    assert ex(k=33) == k2.K2_EUNSUPPORTED
    assert ex(E=1025) == k2.K2_EUNSUPPORTED
    assert ex(E=8, k=16) == k2.K2_EUNSUPPORTED                  # top_k > n_experts
    assert ex(T=65) == k2.K2_EUNSUPPORTED                       # 1040 pairs
    assert ex(ws=FAKE + 16) == k2.K2_EINVAL                     # 256-byte alignment
    assert ex(wsb=nb - 1) == k2.K2_EINVAL
    rb = k2.k2_moe_route_workspace_bytes(8, 896)

    def rt(T=8, H=7168, E=896, k=16, ws=FAKE, wsb=rb):
        return L.k2_moe_route(FAKE, None, FAKE, T, H, E, k, 1.0, FAKE, FAKE, ws, wsb, st)

    assert rt(H=12288 + 32) == k2.K2_EUNSUPPORTED
    assert rt(H=7168 + 8) == k2.K2_EUNSUPPORTED
    assert rt(E=2048) == k2.K2_EUNSUPPORTED
    assert rt(E=8) == k2.K2_EUNSUPPORTED
    assert rt(T=0) == k2.K2_EINVAL
    assert rt(wsb=rb - 4) == k2.K2_EINVAL
    cfg = k2.k2_moe_config(7168, 3584, 3072, 896, 16, 2, 1.0, 1e-5)
    lb = k2.k2_moe_layer_workspace_bytes(cfg, 32)
    assert lb > nb
    w = k2.k2_moe_layer_weights(cfg, *([FAKE] * 11))
    assert L.k2_moe_layer(C.addressof(w), FAKE, 32, FAKE, None, None, None, FAKE, lb - 1, st) \
        == k2.K2_EINVAL
    w.sh_w13 = None
    assert L.k2_moe_layer(C.addressof(w), FAKE, 32, FAKE, None, None, None, FAKE, lb, st) \
        == k2.K2_EINVAL                                          # 2 shared experts, no weights
    w.sh_w13 = FAKE
    w.cfg.hidden = 7168 + 16
    assert L.k2_moe_layer(C.addressof(w), FAKE, 32, FAKE, None, None, None, FAKE, lb, st) \
        == k2.K2_EUNSUPPORTED


def test_sample_validation():
    L = k2.load()
    ws = 0x100000
    b = k2.k2_sample_workspace_bytes(250624)
    assert b > 0 and k2.k2_sample_workspace_bytes(300000) > 0
    assert k2.k2_sample_workspace_bytes((1 << 24) + 1) == 0 and k2.k2_sample_workspace_bytes(0) == 0
    out = FAKE

    def call(vocab=1000, n_prev=0, prev=None, wsb=b, **kw):
        p = dict(temperature=1.0, top_k=8, top_p=1.0, min_p=0.0, repetition_penalty=1.0)
        p.update(kw)
        sp = k2.k2_sampling(**p)
        return L.k2_sample(FAKE, vocab, C.addressof(sp), prev, n_prev, 1, 2, out, ws, wsb, None)
    assert call(temperature=0.0) == k2.K2_EINVAL
    assert call(top_k=-1) == k2.K2_EINVAL
    assert call(top_p=0.0) == k2.K2_EINVAL
    assert call(top_p=1.5) == k2.K2_EINVAL
    assert call(min_p=1.0) == k2.K2_EINVAL
    assert call(repetition_penalty=0.9) == k2.K2_EINVAL
    assert call(n_prev=3, prev=None) == k2.K2_EINVAL
    assert call(vocab=(1 << 24) + 1) == k2.K2_EUNSUPPORTED
    assert call(vocab=300000, wsb=b) == k2.K2_EINVAL          # workspace too small for it
    assert call(wsb=16) == k2.K2_EINVAL
