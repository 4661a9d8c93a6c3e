"""Shared test helpers: metrics, host<->device conversion, cached workloads.

Inputs come from the seeded generator; O and lse from the oracle forward
(rounded as the backward consumes them).  Nothing here computes attention.
"""
from __future__ import annotations

import functools
import math

import numpy as np

from oracle import smla_oracle as orc
from sparse_mla_attention_smla_amd import inputs

SCALE = 1.0 / math.sqrt(512)
REL_L2 = 5e-3      # acceptance bar for dq, dkv, d_sink (and bf16 stage tensors)
COS = 0.9999


def rel_l2(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    return float(num / den) if den > 0 else float(num)


def cosine(got, want) -> float:
    got = np.asarray(got, dtype=np.float64).ravel()
    want = np.asarray(want, dtype=np.float64).ravel()
    den = np.linalg.norm(got) * np.linalg.norm(want)
    return float(np.dot(got, want) / den) if den > 0 else 1.0


def assert_close(name, got, want, tol=REL_L2, cos=COS):
    r, c = rel_l2(got, want), cosine(got, want)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{name}: non-finite values"
    assert r <= tol and c >= cos, f"{name}: rel-L2 {r:.3e} (<= {tol}), cos {c:.6f} (>= {cos})"
    return r, c


@functools.lru_cache(maxsize=4)
def workload(name: str):
    """Seeded inputs plus the oracle forward's rounded O (bf16 bits) and lse (fp32)."""
    x = inputs.make(name, sink=True)
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], SCALE)
    O, lse = orc.emit_forward_outputs(O64, lse64)
    x = dict(x)
    x["O"], x["lse"] = O, lse
    return x


@functools.lru_cache(maxsize=4)
def workload_nosink(name: str):
    x = dict(inputs.make(name, sink=False))
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], None, SCALE)
    x["O"], x["lse"] = orc.emit_forward_outputs(O64, lse64)
    return x


def bf16_to_f64(bits) -> np.ndarray:
    return orc.bf16_to_f64(bits)


# ---- device conversion (torch imported lazily so CPU tests never need it) ----

def dev_bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bf16(t) -> np.ndarray:
    """bf16 device tensor -> float64 numpy (exact)."""
    import torch
    return orc.bf16_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def host_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dsp_to_logical(vals, H):
    """dS/P blocks in the library's piece layout (include/smla.h, smla_dq) ->
    [..., 2H, 32] arrays indexed (row, tile slot).  Pure index bookkeeping."""
    v = np.asarray(vals).reshape(-1, 2 * H // 16, 4, 16, 2, 4)   # chunk, g, row%16, half, i
    return v.transpose(0, 1, 3, 4, 2, 5).reshape(-1, 2 * H, 32)  # chunk, row%16, half, g, i


def dsp_from_logical(blocks, H):
    """Inverse of dsp_to_logical: [..., 2H, 32] -> flat piece-layout values."""
    v = np.asarray(blocks).reshape(-1, 2 * H // 16, 16, 2, 4, 4)  # chunk, row%16, half, g, i
    return v.transpose(0, 1, 4, 2, 3, 5).reshape(-1)


def dsp_map(idx, num_kv, chunk=512, bk=32):
    """Where each valid slot lives in the dS/P block buffer of smla_dq (the layout
    documented in include/smla.h): per token, valid slots in increasing order,
    in runs of `chunk` slots, grouped in tiles of `bk`.  Returns int arrays
    (t, block, col, slot) with one entry per valid slot.  Pure index bookkeeping."""
    T, K = idx.shape
    ts, bs, cs, ks = [], [], [], []
    for t in range(T):
        c = 0
        for k0 in range(0, K, chunk):
            seg = np.arange(k0, min(k0 + chunk, K))
            v = seg[(idx[t, seg] >= 0) & (idx[t, seg] < num_kv)]
            pos = np.arange(v.size)
            ts.append(np.full(v.size, t)); bs.append(c + pos // bk); cs.append(pos % bk); ks.append(v)
            c += (v.size + bk - 1) // bk
    cat = lambda a: np.concatenate(a) if a else np.zeros(0, int)
    return cat(ts), cat(bs), cat(cs), cat(ks)
