"""k2_gqa_decode_attn_noalloc (workspace in the library's device scratch array,
no allocation) against k2_gqa_decode_attn (caller workspace): the same
kernels and split rule, so the outputs are equal bit for bit -- on two calls
in a row, the second with a smaller input (the array keeps the first call's
contents), for every cache format; sizes beyond the array are refused
before launch."""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import DEV, GPU, say, to_dev, to_host

pytestmark = pytest.mark.gpu
if GPU:
    from quantized_gemv_gqa_decode_amd import k2


def _cache(kvdt, n_kv, cap, hd, L, seed):
    rng = np.random.default_rng(seed)
    oc = oracle.KVCache(kvdt, n_kv, cap, hd)
    if kvdt == "i8":
        oc.k[:, :L] = rng.integers(-127, 128, (n_kv, L, hd))
        oc.v[:, :L] = rng.integers(-127, 128, (n_kv, L, hd))
        oc.ks[:, :L] = np.abs(rng.standard_normal((n_kv, L)) * 0.05).astype(np.float32)
        oc.vs[:, :L] = np.abs(rng.standard_normal((n_kv, L)) * 0.05).astype(np.float32)
    else:
        kk = rng.standard_normal((n_kv, L, hd))
        vv = rng.standard_normal((n_kv, L, hd))
        if kvdt == "f32":
            oc.k[:, :L] = kk
            oc.v[:, :L] = vv
        else:
            bf = lambda a: torch.from_numpy(a).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            oc.k[:, :L] = bf(kk)
            oc.v[:, :L] = bf(vv)
    return oc


def _pair(kvdt, n_qh, n_kv, hd, cap, L, seed):
    """(no-allocation output, workspace output, oracle) for one case."""
    oc = _cache(kvdt, n_kv, cap, hd, L, seed)
    rng = np.random.default_rng(seed + 1)
    q = (rng.standard_normal(n_qh * hd) * 2).astype(np.float32)
    kc, vc, ks, vs = to_dev(oc.k), to_dev(oc.v), to_dev(oc.ks), to_dev(oc.vs)
    qd = to_dev(q)
    scale = 1.0 / math.sqrt(hd)
    dt = k2.DTYPES[kvdt]
    out_na = torch.full((n_qh * hd,), float("nan"), device=DEV)
    k2.check(k2.k2_gqa_decode_attn_noalloc(dt, qd, kc, vc, ks, vs, out_na, n_qh, n_kv, hd, cap, L,
                                           scale))
    ws_b = k2.k2_attn_workspace_bytes(n_qh, n_kv, hd, cap)
    ws = torch.zeros(ws_b, dtype=torch.uint8, device=DEV)
    out_ws = torch.full((n_qh * hd,), float("nan"), device=DEV)
    k2.check(k2.k2_gqa_decode_attn(dt, qd, kc, vc, ks, vs, out_ws, n_qh, n_kv, hd, cap, L, scale,
                                   ws, ws_b))
    torch.cuda.synchronize()
    ref = oracle.attention(q.astype(np.float64), oc, n_qh, L)
    vmax = float(np.abs(oc.dequant("v", L)).max())
    return to_host(out_na), to_host(out_ws), ref, vmax


@pytest.mark.parametrize("kvdt", ["f32", "bf16", "i8"])
def test_noalloc_attention_equals_workspace_form_twice(kvdt):
    cases = [(32, 8, 128, 3000, 2900, 11),     # several splits per kv head
             (8, 2, 128, 200, 70, 12)]         # smaller: fewer heads, two splits
    for n_qh, n_kv, hd, cap, L, seed in cases:
        say(f"no-alloc attention {kvdt} {n_qh}/{n_kv} hd={hd} L={L}")
        na, wsf, ref, vmax = _pair(kvdt, n_qh, n_kv, hd, cap, L, seed)
        assert np.array_equal(na, wsf), float(np.nanmax(np.abs(na - wsf)))
        assert np.abs(na - ref).max() <= 2e-5 * vmax + 1e-6


def test_noalloc_refuses_beyond_the_scratch_array():
    limit = k2.k2_gqa_decode_attn_scratch_limit()
    assert limit == 4 << 20
    # a workspace larger than the array: refused, nothing written
    n_qh, n_kv, hd = 64, 64, 128
    cap = 1 << 19
    assert k2.k2_attn_workspace_bytes(n_qh, n_kv, hd, cap) > limit
    out = torch.full((n_qh * hd,), 7.0, device=DEV)
    dummy = torch.zeros(64, device=DEV)
    rc = k2.k2_gqa_decode_attn_noalloc(k2.K2_F32, dummy, dummy, dummy, None, None, out, n_qh, n_kv,
                                       hd, cap, 10, 1.0)
    assert rc == k2.K2_EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
