"""Shared helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
import os

import numpy as np
import pytest
import torch

GPU = torch.cuda.is_available()
DEV = torch.device("cuda:0") if GPU else None


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor, like=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if like is not None and like == np.uint16:
        return a.view(np.uint16)
    return a


def bf16_draw(shape, std=0.02, seed=0) -> np.ndarray:
    g = torch.Generator().manual_seed(seed)
    w = (torch.randn(*shape, generator=g) * std).to(torch.bfloat16)
    return w.view(torch.int16).numpy().view(np.uint16)


def sumabs_bound(Wd: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Worst-case bound of fp32 recursive summation of a row dot product:
    K * 2^-24 * sum_k |w_k x_k| (plus a tiny absolute floor)."""
    K = Wd.shape[1]
    return K * 2.0 ** -24 * (np.abs(Wd) @ np.abs(x)) + 1e-30


def near_tie_ok(gpu_tok: int, ref_logits: np.ndarray, gap: float = 1e-3) -> bool:
    """The GPU argmax must equal the oracle's, except where the oracle's two
    best logits are closer than `gap` -- then any token whose oracle logit is
    within `gap` of the best is accepted."""
    best = float(ref_logits.max())
    if int(np.argmax(ref_logits)) == gpu_tok:
        return True
    return best - float(ref_logits[gpu_tok]) < gap


def tie_gap(err: float) -> float:
    """Near-tie width for a position whose logits differ from the oracle's by
    at most `err` (max-abs): the GPU can pick token t over the oracle's best b
    only if logit_b - logit_t <= e_t + e_b <= 2 err, so an oracle gap within
    2 err is beyond what the fp32 arithmetic resolves (floor 1e-3)."""
    return max(1e-3, 2.0 * err)


def say(msg: str):
    print(msg, flush=True)
