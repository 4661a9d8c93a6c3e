"""Seeded synthetic inputs for the sparse-MLA backward workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path's tests/benchmark and the CPU oracle's
tests take their inputs from here, so the two sides see identical bytes.

Workloads follow the shapes of the DSv4 sparse-MLA training backward described
in ROCm/aiter PR 4766 "Sparse MLA training backward" (Contract and Performance
sections): one shared 512-wide kv tensor, per-query top-k row indices with -1
padding, an optional per-head sink, and a "sliding window of 128 + compressed
pool" index structure for the large cases.  The pages do not give the pool
stride or pool selection rule; the recipe below fixes them (window 128, pool row
j summarises tokens 4j..4j+3 and becomes eligible once 4j+3 <= t, up to 384
uniform or Zipf(1.1) picks).

Recipe (seed s = 1000 + workload.index):

* indices -- from ``np.random.default_rng(s)``: per row, sampled without
  replacement with the Efraimidis-Spirakis A-ES method (key = ln(u)/w, keep the
  largest keys); equal weights give uniform sampling.  Valid indices are stored
  ascending, then -1 padding.
* sink -- next from the same generator: float32 standard normal, one value per
  head (always drawn, so the with-sink and without-sink runs of one workload
  share every other tensor).
* q, kv, dO -- float32 standard normal rounded to bfloat16 (nearest, ties to
  even), returned as uint16 bit patterns.  Each tensor is drawn in chunks of
  2**22 values; chunk c of tensor k (q=1, kv=2, dO=3) comes from
  ``np.random.default_rng([s, k, c])``, so chunks can be drawn in parallel
  threads and the result does not depend on the thread count.
* dlse (an optional upstream gradient of lse, [T,H] float32) -- standard normal
  from ``np.random.default_rng([s, 4])``; its spread is that of delta for these
  inputs, so both terms of the shifted delta matter.
* q_pe [T,H,64], k_pe [num_kv,64] (the positional parts of the has_pe=True
  variant) -- standard normal rounded to bf16 like q and kv, tensors 5 and 6
  of the same chunk-seeded scheme.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

D = 512  # fixed head dimension of the op
DPE = 64  # width of the positional part of the has_pe=True variant


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed = 1000 + index
    T: int              # query tokens
    H: int              # heads
    num_kv: int         # kv rows (token rows 0..T-1, then pool rows)
    topk: int           # index slots per query token
    selection: str      # "causal" | "swa_pool" | "swa_pool_zipf"
    window: int = 0     # sliding-window length (swa_pool*)
    pool_stride: int = 0
    pool_picks: int = 0
    zipf_s: float = 1.1

    @property
    def pool_rows(self) -> int:
        return self.num_kv - self.T

    def flops(self) -> float:
        """Nominal backward flop count, 10*T*H*topk*512 (padded slots counted)."""
        return 10.0 * self.T * self.H * self.topk * D


WORKLOADS = {
    "tiny": Workload("tiny", 0, T=64, H=16, num_kv=64, topk=16, selection="causal"),
    "small": Workload("small", 1, T=1024, H=64, num_kv=1024, topk=128, selection="causal"),
    "headline": Workload("headline", 2, T=4096, H=128, num_kv=5120, topk=512,
                         selection="swa_pool", window=128, pool_stride=4, pool_picks=384),
    "skewed": Workload("skewed", 3, T=4096, H=128, num_kv=5120, topk=512,
                       selection="swa_pool_zipf", window=128, pool_stride=4, pool_picks=384),
    "long": Workload("long", 4, T=8192, H=128, num_kv=10240, topk=512,
                     selection="swa_pool", window=128, pool_stride=4, pool_picks=384),
    # the page's correctness runs also use H = 64
    "headline_h64": Workload("headline_h64", 5, T=4096, H=64, num_kv=5120, topk=512,
                             selection="swa_pool", window=128, pool_stride=4, pool_picks=384),
    # mid-size parity case: 640 items of 64 heads (several per persistent
    # workgroup on 256 compute units) and tokens of 1 to 14 tiles of 32 slots
    # (pool of stride 1, so late tokens see up to 320 pool rows)
    "mid": Workload("mid", 6, T=320, H=128, num_kv=640, topk=512,
                    selection="swa_pool", window=128, pool_stride=1, pool_picks=384),
    # the headline's tokens and index recipe at the head counts of a head-sharded
    # model (and H = 48, 96: groups of 64 heads with a partial last one)
    **{f"headline_h{h}": Workload(f"headline_h{h}", 30 + h // 16, T=4096, H=h, num_kv=5120, topk=512,
                                  selection="swa_pool", window=128, pool_stride=4, pool_picks=384)
       for h in (16, 32, 48, 96)},
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs here are finite normal draws, so no NaN/Inf handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _aes_pick(rng: np.random.Generator, weights: np.ndarray | None, n: int, m: int) -> np.ndarray:
    """Pick m of n items without replacement (A-ES keys ln(u)/w, largest m)."""
    if m <= 0:
        return np.zeros(0, dtype=np.int64)
    u = rng.random(n)
    if m >= n:
        return np.arange(n, dtype=np.int64)
    with np.errstate(divide="ignore"):
        keys = np.log(u)
    if weights is not None:
        keys = keys / weights
    part = np.argpartition(-keys, m - 1)[:m]
    return np.sort(part)


def make_indices(w: Workload, rng: np.random.Generator) -> np.ndarray:
    T, K = w.T, w.topk
    idx = np.full((T, K), -1, dtype=np.int32)
    if w.selection == "causal":
        for t in range(T):
            rows = _aes_pick(rng, None, t + 1, min(K, t + 1))
            idx[t, : rows.size] = rows
        return idx
    zipf = w.selection == "swa_pool_zipf"
    P = w.pool_rows
    zw = (np.arange(1, P + 1, dtype=np.float64)) ** (-w.zipf_s) if zipf else None
    for t in range(T):
        lo = max(0, t - w.window + 1)
        win = np.arange(lo, t + 1, dtype=np.int64)
        # pool row j is eligible once the tokens it summarises are all visible
        n_elig = 0 if t < w.pool_stride - 1 else min(P, (t - (w.pool_stride - 1)) // w.pool_stride + 1)
        picks = _aes_pick(rng, None if zw is None else zw[:n_elig], n_elig, min(w.pool_picks, n_elig))
        row = np.concatenate([win, T + picks])
        idx[t, : row.size] = row
    return idx


_CHUNK = 1 << 22


def normal_bf16(shape, seed: int, tensor: int, threads: int | None = None) -> np.ndarray:
    """Standard-normal float32 draws rounded to bf16 bits, chunk-seeded (see recipe)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def fill(c):
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        x = np.random.default_rng([seed, tensor, c]).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = f32_to_bf16_bits(x)

    nchunks = (n + _CHUNK - 1) // _CHUNK
    threads = threads or min(16, os.cpu_count() or 1)
    if nchunks <= 1 or threads <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def make(name_or_workload, sink: bool = True) -> dict:
    """Build the seeded inputs of one workload.

    Returns a dict with numpy arrays: q/kv/dO (uint16 bf16 bits, [T,H,512] /
    [num_kv,512] / [T,H,512]), idx (int32 [T,topk]), sink (float32 [H] or None),
    and the Workload under "workload".
    """
    w = WORKLOADS[name_or_workload] if isinstance(name_or_workload, str) else name_or_workload
    seed = 1000 + w.index
    rng = np.random.default_rng(seed)
    idx = make_indices(w, rng)
    s = rng.standard_normal(w.H).astype(np.float32)
    q = normal_bf16((w.T, w.H, D), seed, 1)
    kv = normal_bf16((w.num_kv, D), seed, 2)
    dO = normal_bf16((w.T, w.H, D), seed, 3)
    return {"workload": w, "q": q, "kv": kv, "dO": dO, "idx": idx, "sink": s if sink else None}


def make_dlse(name_or_workload) -> np.ndarray:
    """Seeded upstream gradient of lse for one workload: float32 [T, H]."""
    w = WORKLOADS[name_or_workload] if isinstance(name_or_workload, str) else name_or_workload
    return np.random.default_rng([1000 + w.index, 4]).standard_normal((w.T, w.H), dtype=np.float32)


def make_pe(name_or_workload) -> tuple:
    """Seeded positional parts for one workload: q_pe [T,H,64] and k_pe [num_kv,64]
    as bf16 bits (uint16)."""
    w = WORKLOADS[name_or_workload] if isinstance(name_or_workload, str) else name_or_workload
    seed = 1000 + w.index
    return normal_bf16((w.T, w.H, DPE), seed, 5), normal_bf16((w.num_kv, DPE), seed, 6)


def shuffle_slots(idx: np.ndarray, seed: int) -> np.ndarray:
    """Return a copy of idx with every row's slots permuted (valid and -1 mixed)."""
    rng = np.random.default_rng(seed)
    out = idx.copy()
    for t in range(out.shape[0]):
        out[t] = out[t, rng.permutation(out.shape[1])]
    return out
