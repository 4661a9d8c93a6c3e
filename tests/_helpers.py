"""Shared test helpers: metrics, host<->device conversion, cached workloads.

Inputs come from the seeded generator; O and lse from the oracle forward
(rounded as the backward consumes them).  Nothing here computes attention; the
rounding bounds below only sum magnitudes of products of the inputs.
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
# Per-row bar (every output row, not only the whole tensor): the relative L2
# error of each row along the last axis, measured against the larger of the
# row's own norm and ROW_FLOOR times the RMS row norm (so that near-zero rows
# are not judged on a relative error).  bf16 rounding of the dS/P operands and
# of the output gives about 2e-3 per row (at most 4e-3 over the small
# workload's 65,536 dq rows when those roundings are emulated in fp64); a
# dropped, zeroed or garbled row gives 1 or more.
ROW_REL = 1e-2
ROW_FLOOR = 0.02


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


def row_errors(got, want, floor=ROW_FLOOR) -> np.ndarray:
    """Relative L2 error of every row (last axis; each element of a 1-D array is
    a row of its own), against max(|row of want|, floor * RMS row norm)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    n = want.shape[-1] if want.ndim >= 2 else 1
    g, w = got.reshape(-1, n), want.reshape(-1, n)
    num = np.linalg.norm(g - w, axis=1)
    den = np.linalg.norm(w, axis=1)
    rms = math.sqrt(float(np.mean(den ** 2))) if den.size else 0.0
    ref = np.maximum(den, floor * rms)
    out = np.where(ref > 0, num / np.where(ref > 0, ref, 1.0), num)
    return out


def assert_close(name, got, want, tol=REL_L2, cos=COS, row_tol=ROW_REL):
    """Whole-tensor rel-L2 and cosine, plus the per-row bound on every row.
    Returns (rel-L2, cosine, worst row error)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    r, c = rel_l2(got, want), cosine(got, want)
    rows = row_errors(got, want)
    worst = float(rows.max()) if rows.size else 0.0
    assert r <= tol and c >= cos, f"{name}: rel-L2 {r:.3e} (<= {tol}), cos {c:.6f} (>= {cos})"
    if worst > row_tol:
        bad = np.argsort(rows)[::-1][:5]
        raise AssertionError(f"{name}: worst row error {worst:.3e} > {row_tol} (rows {bad.tolist()} "
                             f"errors {rows[bad].round(4).tolist()}; {int((rows > row_tol).sum())} rows "
                             f"over the bound of {rows.size})")
    return r, c, worst


# fp32 unit roundoff for directed rounding: a bound that holds whichever rounding
# the matrix cores' accumulation uses
_U32 = 2.0 ** -23


def cancellation_bounds(x, n=512):
    """Per-element absolute bounds on dq (with the positional parts also dq_pe and
    dk_pe) for a problem whose exact dS is zero on every valid slot: one unmasked
    slot per token, no sink and no lse gradient give P = 1, so dS = P (dP - delta)
    vanishes only because dP = <dO, kv_j> and delta = <dO, O> are equal (O is kv_j).
    The library forms the two as fp32 sums of the same bf16 products in different
    orders; each sum differs from its exact value by at most gamma_n = n u / (1 - n u)
    times the sum of its products' magnitudes (recursive summation in any order),
    so |dS| <= gamma_n (sum |dO kv_j| + sum |dO O|).  The outputs are scale times sums
    of dS times |kv|, |k_pe| or |q_pe| (1% on top covers P's own rounding, the bf16
    rounding of dS and of the output, and the fp32 sums over slots).  Masked slots
    contribute nothing, so fully masked rows must come out exactly zero."""
    kv, dO, O, idx = (np.asarray(x[k]) for k in ("kv", "dO", "O", "idx"))
    kv64, dO64, O64 = (orc.bf16_to_f64(a) for a in (kv, dO, O))
    T, H, _ = dO64.shape
    N = kv64.shape[0]
    scale = x.get("scale", SCALE)
    g = n * _U32 / (1.0 - n * _U32)
    valid = (idx >= 0) & (idx < N)
    rows = np.where(valid, idx, 0)
    sum_o = np.abs(dO64 * O64).sum(axis=2)                                   # [T, H]
    out = {"dq": np.zeros((T, H, kv64.shape[1]))}
    pe = "q_pe" in x
    if pe:
        kpe64, qpe64 = orc.bf16_to_f64(np.asarray(x["k_pe"])), orc.bf16_to_f64(np.asarray(x["q_pe"]))
        out["dq_pe"] = np.zeros((T, H, kpe64.shape[1]))
        out["dk_pe"] = np.zeros((N, kpe64.shape[1]))
    for k in range(idx.shape[1]):
        v = valid[:, k]
        kvk = kv64[rows[:, k]]                                               # [T, 512]
        b = g * (np.einsum("thd,td->th", np.abs(dO64), np.abs(kvk)) + sum_o) * v[:, None]
        out["dq"] += b[:, :, None] * np.abs(kvk)[:, None, :]
        if pe:
            out["dq_pe"] += b[:, :, None] * np.abs(kpe64[rows[:, k]])[:, None, :]
            np.add.at(out["dk_pe"], rows[v, k], np.einsum("th,thd->td", b[v], np.abs(qpe64[v])))
    return {name: 1.01 * scale * a for name, a in out.items()}


def assert_cancellation_zero(name, got, bound):
    """A result whose exact value is zero through cancellation: every element
    within its rounding bound (exactly zero where the bound is zero)."""
    got = np.asarray(got, dtype=np.float64)
    over = np.abs(got) > bound
    assert not over.any(), (f"{name}: {int(over.sum())} elements over the rounding bound, "
                            f"worst |got| {np.abs(got).max():.3e}")
    return float(np.abs(got).max(initial=0.0))


# a whole reference tensor below this is no gradient of these inputs but a
# cancellation: it is checked against the rounding bound instead of relatively
_CANCEL_MAX = 1e-9


def assert_close_or_cancelled(name, got, want, x, key):
    """assert_close, unless the whole reference is zero through cancellation:
    then the reference must itself sit at the fp64 level of the same bound
    (2^-29 of the fp32 one), and the result within the fp32 bound of it."""
    want = np.asarray(want, dtype=np.float64)
    if np.abs(want).max(initial=0.0) > _CANCEL_MAX:
        return assert_close(name, got, want)
    b = cancellation_bounds(x)[key]
    assert np.all(np.abs(want) <= b * 2.0 ** -29), f"{name}: tiny reference is no cancellation"
    assert_cancellation_zero(name, got, b + np.abs(want))
    return None


def single_slot_problem(T, H, N, pe, seed):
    """One valid slot per token (token 3 fully masked, token T//2 out of range,
    rows drawn with replacement), no sink: P = 1 on every valid slot, so dq (and
    dq_pe, dk_pe) are zero through cancellation.  With the oracle forward's O, lse."""
    rng = np.random.default_rng([seed, T, H, N])
    idx = rng.integers(0, N, size=(T, 1)).astype(np.int32)
    idx[min(3, T - 1)] = -1
    idx[T // 2] = N + 4
    x = {"q": inputs.normal_bf16((T, H, 512), seed, 1), "kv": inputs.normal_bf16((N, 512), seed, 2),
         "dO": inputs.normal_bf16((T, H, 512), seed, 3), "idx": idx, "sink": None, "scale": SCALE}
    if pe:
        x["q_pe"], x["k_pe"] = inputs.normal_bf16((T, H, 64), seed, 5), inputs.normal_bf16((N, 64), seed, 6)
        x["scale"] = SCALE_PE
    return _with_forward(x)


def oracle_backward_chunked(x, dlse=None, chunk=32, workers=None):
    """The oracle backward over all tokens, evaluated on token chunks in parallel
    threads (each chunk is one plain orc.backward call on a token slice; the
    chunks' dkv and d_sink contributions are added in float64).  Returns the
    same keys as orc.backward."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    T, H, Dh = x["q"].shape
    N = x["kv"].shape[0]
    workers = workers or min(16, len(os.sched_getaffinity(0)))
    dq = np.empty((T, H, Dh))
    delta = np.empty((T, H))
    dkv = np.zeros((N, Dh))
    dsink = np.zeros(H)

    pe = x.get("q_pe") is not None
    scale = x.get("scale", SCALE)
    if pe:
        dq_pe = np.empty((T, H, x["q_pe"].shape[2]))
        dk_pe = np.zeros((N, x["k_pe"].shape[1]))

    def run(t0):
        t1 = min(T, t0 + chunk)
        r = orc.backward(x["q"][t0:t1], x["kv"], x["dO"][t0:t1], x["O"][t0:t1], x["lse"][t0:t1],
                         x["idx"][t0:t1], x["sink"], scale, dlse=None if dlse is None else dlse[t0:t1],
                         q_pe=x["q_pe"][t0:t1] if pe else None, k_pe=x["k_pe"] if pe else None)
        return t0, t1, r

    starts = list(range(0, T, chunk))
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        for i in range(0, len(starts), 4 * workers):      # bounded number of partial dkv in flight
            for t0, t1, r in ex.map(run, starts[i:i + 4 * workers]):
                dq[t0:t1] = r["dq"]
                delta[t0:t1] = r["delta"]
                dkv += r["dkv"]
                if r["d_sink"] is not None:
                    dsink += r["d_sink"]
                if pe:
                    dq_pe[t0:t1] = r["dq_pe"]
                    dk_pe += r["dk_pe"]
    out = {"dq": dq, "dkv": dkv, "d_sink": dsink if x["sink"] is not None else None, "delta": delta}
    if pe:
        out.update(dq_pe=dq_pe, dk_pe=dk_pe)
    return out


def oracle_forward_chunked(x, chunk=32, workers=None):
    """orc.forward over all tokens, on token chunks in parallel threads (each
    chunk one plain orc.forward call on a token slice).  Returns (O, lse) in
    float64, exactly as one orc.forward call would."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    T, H, Dh = x["q"].shape
    workers = workers or min(16, len(os.sched_getaffinity(0)))
    O = np.empty((T, H, Dh))
    lse = np.empty((T, H))

    pe = x.get("q_pe") is not None

    def run(t0):
        t1 = min(T, t0 + chunk)
        O[t0:t1], lse[t0:t1] = orc.forward(x["q"][t0:t1], x["kv"], x["idx"][t0:t1], x["sink"],
                                           x.get("scale", SCALE), q_pe=x["q_pe"][t0:t1] if pe else None,
                                           k_pe=x["k_pe"] if pe else None)

    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        list(ex.map(run, range(0, T, chunk)))
    return O, lse


def _with_forward(x):
    O64, lse64 = oracle_forward_chunked(x)
    x = dict(x)
    x["O"], x["lse"] = orc.emit_forward_outputs(O64, lse64)
    x["O64"] = O64                                      # for the forward's own checks
    return x


@functools.lru_cache(maxsize=3)
def workload(name: str):
    """Seeded inputs plus the oracle forward's rounded O (bf16 bits) and lse (fp32)."""
    return _with_forward(inputs.make(name, sink=True))


@functools.lru_cache(maxsize=2)
def workload_nosink(name: str):
    return _with_forward(inputs.make(name, sink=False))


SCALE_PE = 1.0 / math.sqrt(512 + 64)   # the has_pe=True workloads' scale


@functools.lru_cache(maxsize=2)
def workload_pe(name: str, sink: bool = True):
    """A seeded workload with the positional parts q_pe, k_pe (scale 1/sqrt(576)),
    plus the oracle forward's rounded O and lse."""
    x = dict(inputs.make(name, sink=sink))
    x["q_pe"], x["k_pe"] = inputs.make_pe(name)
    x["scale"] = SCALE_PE
    return _with_forward(x)


@functools.lru_cache(maxsize=2)
def full_reference(name: str, with_dlse: bool = False):
    """The oracle backward of a whole seeded workload (all tokens, all kv rows)."""
    x = workload(name)
    return oracle_backward_chunked(x, dlse=inputs.make_dlse(name) if with_dlse else None)


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
