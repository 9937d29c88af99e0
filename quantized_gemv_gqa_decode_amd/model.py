"""Device-resident decoder for the C ABI's ``k2_decode_step``.

PyTorch only allocates device memory here; weights are uploaded from the
seeded draws of ``synth`` and quantized on the device by the library's own
``k2_quantize_*`` kernels; every step of the decode runs in libk2.
"""
from __future__ import annotations

import ctypes as C
from typing import List, Optional

import numpy as np
import torch

from . import k2

_NP_TORCH = {np.float32: torch.float32, np.uint16: torch.int16, np.uint8: torch.uint8,
             np.int8: torch.int8}


def upload(a: np.ndarray, device) -> torch.Tensor:
    """Copy a host array to the device, keeping its bytes (uint16 -> int16)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceMat:
    """A projection matrix in the library's storage format on the device."""

    def __init__(self, wdt: str, draw: np.ndarray, device, stream=None):
        N, K = draw.shape
        self.wdt, self.N, self.K = wdt, N, K
        self.s = None
        if wdt in ("f32", "bf16"):
            self.w = upload(draw, device)
        else:
            src = upload(draw, device)
            if wdt == "fp8":
                self.w = torch.empty((N, K), dtype=torch.uint8, device=device)
                self.s = torch.empty(N, dtype=torch.float32, device=device)
                k2.check(k2.k2_quantize_fp8_rows(src, self.w, self.s, N, K, stream))
            elif wdt == "mxfp4":
                self.w = torch.empty((N, K // 2), dtype=torch.uint8, device=device)
                self.s = torch.empty((N, K // 32), dtype=torch.uint8, device=device)
                k2.check(k2.k2_quantize_mxfp4(src, self.w, self.s, N, K, stream))
            elif wdt == "q4s":
                self.w = torch.empty((N, K // 2), dtype=torch.uint8, device=device)
                self.s = torch.empty((N, K // 64), dtype=torch.float32, device=device)
                k2.check(k2.k2_quantize_q4s(src, self.w, self.s, N, K, stream))
            else:
                raise ValueError(wdt)
            torch.cuda.current_stream().synchronize()
            del src

    @property
    def nbytes(self) -> int:
        return self.w.numel() * self.w.element_size() + (
            0 if self.s is None else self.s.numel() * self.s.element_size())


def kv_cache(kvdt: str, n_kv: int, cap: int, hd: int, device):
    dt = {"f32": torch.float32, "bf16": torch.int16, "i8": torch.int8}[kvdt]
    kc = torch.zeros((n_kv, cap, hd), dtype=dt, device=device)
    vc = torch.zeros((n_kv, cap, hd), dtype=dt, device=device)
    if kvdt == "i8":
        ks = torch.zeros((n_kv, cap), dtype=torch.float32, device=device)
        vs = torch.zeros((n_kv, cap), dtype=torch.float32, device=device)
    else:
        ks = vs = None
    return kc, vc, ks, vs


class DecodeModel:
    """All buffers of one dense decoder (a ``synth.DecoderConfig``) on the GPU,
    plus the ``k2_model`` struct that points at them."""

    def __init__(self, cfg, device="cuda", n_layers: Optional[int] = None):
        import synth
        if n_layers is not None:
            cfg = cfg.replace(n_layers=n_layers)
        self.cfg = cfg
        self.device = torch.device(device)
        H = cfg.hidden
        self.embed = upload(synth.embed_weight(cfg), self.device)
        self.lm = DeviceMat(cfg.wdt, synth.lm_head_weight(cfg), self.device)
        self.g_final = upload(synth.norm_gain(cfg), self.device)
        self.layers = []
        for l in range(cfg.n_layers):
            mats = {w: DeviceMat(cfg.wdt, synth.layer_weight(cfg, l, w), self.device)
                    for w in ("wqkv", "wo", "wgu", "wd")}
            kc, vc, ks, vs = kv_cache(cfg.kvdt, cfg.n_kv, cfg.cap, cfg.head_dim, self.device)
            self.layers.append(dict(mats=mats, g_in=upload(synth.norm_gain(cfg), self.device),
                                    g_post=upload(synth.norm_gain(cfg), self.device),
                                    kc=kc, vc=vc, ks=ks, vs=vs))
        self.rope = torch.empty((cfg.cap, cfg.head_dim // 2, 2), dtype=torch.float32,
                                device=self.device)
        k2.check(k2.k2_rope_table(self.rope, cfg.cap, cfg.head_dim, cfg.theta))
        self._build()

    def _build(self):
        cfg = self.cfg
        c = k2.k2_config(cfg.hidden, cfg.n_layers, cfg.n_qh, cfg.n_kv, cfg.head_dim, cfg.inter,
                         cfg.vocab, cfg.groups, cfg.cap, cfg.eps, cfg.theta, k2.DTYPES[cfg.wdt],
                         k2.DTYPES[cfg.kvdt], k2.DTYPES[cfg.embed_dt])
        ws_bytes = k2.k2_decode_workspace_bytes(c)
        if ws_bytes == 0:
            raise k2.K2Error(k2.K2_EUNSUPPORTED)
        self.ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=self.device)
        arr = (k2.k2_layer * cfg.n_layers)()
        for i, L in enumerate(self.layers):
            m = L["mats"]
            arr[i] = k2.k2_layer(
                k2.ptr(m["wqkv"].w), k2.ptr(m["wqkv"].s), k2.ptr(m["wo"].w), k2.ptr(m["wo"].s),
                k2.ptr(m["wgu"].w), k2.ptr(m["wgu"].s), k2.ptr(m["wd"].w), k2.ptr(m["wd"].s),
                k2.ptr(L["g_in"]), k2.ptr(L["g_post"]), k2.ptr(L["kc"]), k2.ptr(L["vc"]),
                k2.ptr(L["ks"]), k2.ptr(L["vs"]))
        self._layers_arr = arr
        self.model = k2.k2_model(c, k2.ptr(self.embed), k2.ptr(self.lm.w), k2.ptr(self.lm.s),
                                 k2.ptr(self.g_final), k2.ptr(self.rope),
                                 C.cast(arr, C.POINTER(k2.k2_layer)), k2.ptr(self.ws), ws_bytes)
        k2.check(k2.k2_model_check(self.model))
        self.logits = torch.zeros(cfg.vocab, dtype=torch.float32, device=self.device)
        self.next = torch.zeros(1, dtype=torch.int32, device=self.device)
        # the position k2_decode_step_dev reads and advances
        self.d_pos = torch.zeros(1, dtype=torch.int32, device=self.device)

    # ------------------------------------------------------------------
    def load_int8_prefix(self, length: int):
        """Fill cache slots [0, length) of every layer with the seeded int8
        history of ``synth.int8_kv_prefix`` (a stand-in for a long prefill)."""
        import synth
        if self.cfg.kvdt != "i8":
            raise ValueError("the synthetic prefix is an int8 KV history")
        for l, L in enumerate(self.layers):
            kc, vc, ks, vs = synth.int8_kv_prefix(self.cfg, l, length)
            L["kc"][:, :length].copy_(torch.from_numpy(kc))
            L["vc"][:, :length].copy_(torch.from_numpy(vc))
            L["ks"][:, :length].copy_(torch.from_numpy(ks))
            L["vs"][:, :length].copy_(torch.from_numpy(vs))
        torch.cuda.synchronize()

    def weight_bytes(self) -> int:
        """Bytes of projection and lm_head weights read by one full step."""
        n = self.lm.nbytes
        for L in self.layers:
            n += sum(m.nbytes for m in L["mats"].values())
        return n

    def step(self, token: int, pos: int, want_logits: bool = True, stream=None):
        """Enqueue one position (host token).  Returns the device tensors
        (logits, next) when want_logits, else (None, None)."""
        lg = self.logits if want_logits else None
        nx = self.next if want_logits else None
        k2.check(k2.k2_decode_step(self.model, token, pos, lg, nx, stream))
        return lg, nx

    def prefill(self, tokens, pos0: int = 0, chunk: int = 256, want_logits: bool = True,
                stream=None):
        """Consume prompt positions pos0 .. pos0+len(tokens)-1 with k2_prefill,
        ``chunk`` (2..256) positions per call; a lone last position goes through
        k2_decode_step.  The logits/next of the last position land in
        self.logits / self.next when want_logits."""
        toks = [int(t) for t in tokens]
        n = len(toks)
        if not hasattr(self, "_pf_ws") or self._pf_chunk != chunk:
            b = k2.k2_prefill_workspace_bytes(self.model.cfg, chunk)
            if b == 0:
                raise k2.K2Error(k2.K2_EUNSUPPORTED)
            self._pf_ws = torch.zeros(b, dtype=torch.uint8, device=self.device)
            self._pf_chunk = chunk
        i = 0
        while i < n:
            T = min(chunk, n - i)
            last = i + T == n
            lg = self.logits if (want_logits and last) else None
            nx = self.next if (want_logits and last) else None
            if T == 1:
                k2.check(k2.k2_decode_step(self.model, toks[i], pos0 + i, lg, nx, stream))
            else:
                k2.check(k2.k2_prefill(self.model, toks[i:i + T], T, pos0 + i, lg, nx, self._pf_ws,
                                       self._pf_ws.numel(), stream))
            i += T

    def verify(self, tokens, pos0: int, logits: Optional[torch.Tensor] = None, stream=None):
        """k2_verify of len(tokens) (2..32) positions from pos0: returns the
        device int32 tensor of the greedy token after every position."""
        T = len(tokens)
        if not hasattr(self, "_vf_ws"):
            b = k2.k2_verify_workspace_bytes(self.model.cfg, 32)
            if b == 0:
                raise k2.K2Error(k2.K2_EUNSUPPORTED)
            self._vf_ws = torch.zeros(b, dtype=torch.uint8, device=self.device)
            self._vf_next = torch.zeros(32, dtype=torch.int32, device=self.device)
        k2.check(k2.k2_verify(self.model, tokens, T, pos0, logits, self._vf_next, self._vf_ws,
                              self._vf_ws.numel(), stream))
        return self._vf_next[:T]

    def generate_speculative(self, prompt, n_decode: int, draft=None, k: int = 8,
                             prefilled: bool = False):
        """Greedy decode with draft-and-verify: after the prompt (prefill),
        each round feeds [last token, drafted tokens] to k2_verify and keeps
        the greedy tokens up to the first draft that disagrees; a round with
        no draft is one plain decode step.  draft(history, k) returns up to k
        proposed tokens (default: the n-gram drafter of ``draft.py``).
        Returns (tokens, rounds); the tokens are those of plain greedy
        decode.  self.spec_stats counts rounds, drafted and accepted tokens.
        prefilled: the caches already hold the prompt and self.next its
        greedy token (the prompt is then only the drafter's history)."""
        from .draft import ngram_draft
        if draft is None:
            draft = ngram_draft
        P = len(prompt)
        n_decode = min(n_decode, self.cfg.cap - P)
        if not prefilled:
            self.prefill(prompt, 0)
        torch.cuda.synchronize()
        toks = [int(self.next.item())]
        rounds = drafted = accepted = 0
        while len(toks) < n_decode:
            pos = P + len(toks) - 1                   # where the last token goes
            kk = min(k, self.cfg.cap - 1 - pos, 31)
            d = [int(t) for t in draft(list(prompt) + toks, kk)][:kk] if kk >= 1 else []
            rounds += 1
            if not d:
                lg, nx = self.step(toks[-1], pos)
                torch.cuda.synchronize()
                toks.append(int(nx.item()))
                continue
            g = self.verify([toks[-1]] + d, pos).cpu().numpy().tolist()
            drafted += len(d)
            new = [g[0]]
            for i in range(1, len(d) + 1):
                if d[i - 1] != new[-1]:
                    break
                new.append(g[i])
            accepted += len(new) - 1
            toks.extend(new[:n_decode - len(toks)])
        self.spec_stats = {"rounds": rounds, "drafted": drafted, "accepted": accepted}
        return toks, rounds

    def set_pos(self, pos: int):
        """Set the device position that the next k2_decode_step_dev reads."""
        self.d_pos.fill_(int(pos))

    def step_dev(self, d_token: torch.Tensor, d_next: torch.Tensor,
                 d_err: Optional[torch.Tensor] = None, want_logits: bool = True, stream=None):
        """Enqueue one position with the token (d_token) and the position
        (self.d_pos, advanced by the step) read on the device."""
        lg = self.logits if want_logits else None
        k2.check(k2.k2_decode_step_dev(self.model, d_token, self.d_pos, lg, d_next, d_err, stream))
        return lg

    def generate_sampled(self, prompt, n_decode: int, sampling, seed: int, window: int = 64):
        """Seeded sampling on the device.  The prompt positions go through
        k2_decode_step; from the last one on, each position's logits go to
        k2_sample (counter = that position), which writes the token into a
        device history buffer that the next k2_decode_step_dev reads, so no
        token makes a host round trip.  The repetition penalty sees the last
        ``window`` (<= 64) tokens of prompt and output.  Returns the tokens."""
        cfg = self.cfg
        P = len(prompt)
        n_decode = min(n_decode, cfg.cap - P)
        window = max(0, min(int(window), 64))
        hist = torch.zeros(P + n_decode, dtype=torch.int32, device=self.device)
        hist[:P] = torch.tensor([int(t) for t in prompt], dtype=torch.int32)
        wsb = k2.k2_sample_workspace_bytes(cfg.vocab)
        if wsb == 0:
            raise k2.K2Error(k2.K2_EUNSUPPORTED)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=self.device)
        greedy = torch.zeros(1, dtype=torch.int32, device=self.device)
        for p, t in enumerate(prompt):
            self.step(int(t), p, want_logits=p == P - 1)
        self.set_pos(P)                                # the first decode position
        for i in range(n_decode):
            n = P + i                                  # the new token goes to hist[n]
            if i > 0:
                self.step_dev(hist[n - 1:n], greedy)   # position n - 1
            lo = max(0, n - window)
            k2.check(k2.k2_sample(self.logits, cfg.vocab, sampling, hist[lo:n] if n > lo else None,
                                  n - lo, seed, n - 1, hist[n:n + 1], ws, wsb))
        torch.cuda.synchronize()
        return hist[P:].cpu().tolist()

    def generate(self, prompt, n_decode: int, teacher=None, collect_logits: bool = True):
        """Greedy run on the device: the prompt positions skip the head, the
        last prompt position and every decode position emit an argmax.  With
        ``teacher`` the fed tokens come from it (teacher forcing).  Returns
        (tokens, [logits as CPU fp32 arrays])."""
        cfg = self.cfg
        P = len(prompt)
        n_decode = min(n_decode, cfg.cap - P)
        toks, lgs = [], []
        for p, t in enumerate(prompt):
            last = p == P - 1
            self.step(int(t), p, want_logits=last)
        torch.cuda.synchronize()
        toks.append(int(self.next.item()))
        if collect_logits:
            lgs.append(self.logits.cpu().numpy().copy())
        for i in range(n_decode - 1):
            feed = toks[-1] if teacher is None else int(teacher[i])
            self.step(feed, P + i)
            torch.cuda.synchronize()
            toks.append(int(self.next.item()))
            if collect_logits:
                lgs.append(self.logits.cpu().numpy().copy())
        return toks, lgs
