"""Plain float64 CPU oracle of DSv4-style sparse MLA attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or calls this
module; only the test suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP path.

Source: ROCm/aiter PR 4766, "[DSV4] Sparse MLA training backward".
  * Contract section -- shared-KV GQA (K == V == one dense kv tensor of width
    512), scale 1/sqrt(512), index -1 masked, a per-head attention sink that
    enters the softmax denominator only; the forward's lse already includes the
    sink (lse = running max + log of the running sum, natural log).
  * Contract section -- num_kv may exceed T (kv rows past T form a compressed
    pool).
  * Structure table -- the backward's phases: delta = rowsum(O*dO); dQ (which
    also yields dS and P); the dKV intermediate contracted over all heads; the
    inverted top-k (CSR) build; the per-kv-row gather; the sink gradient.

Everything is the plain definition evaluated in float64; there is no tiling,
fusion or reordering.  Readings where the page is silent (each listed with the
design notes):
  * an index outside [0, num_kv) is masked exactly like -1;
  * the sink is a raw per-head logit (not multiplied by the scale) with a zero
    value vector; "no sink" means sink = -inf;
  * a row with no valid slot and no sink has lse = -inf and contributes zero
    everywhere (exp(-inf - (-inf)) is never evaluated);
  * duplicate indices within a row are independent slots;
  * an optional upstream gradient of lse, dlse [T,H], is the one input the
    page does not name.  Since d lse / d S_k = P_k and d lse / d sink = P_sink,
    it adds P * dlse to dS and P_sink * dlse to d_sink; both terms are what
    replacing delta by delta - dlse gives.  Without it, dlse = 0;
  * d_sink[h] = -sum_t P_sink[t,h] * (delta[t,h] - dlse[t,h])
    (dO/dsink = -P_sink * O, dlse/dsink = P_sink);
  * the CSR lists valid slots s = t*topk + k ordered by (index, s);
  * the has_pe=True variant, which the Contract section names (as the
    forward's other path) without describing: q carries an extra positional
    part q_pe [T,H,Dp] and the keys an extra part k_pe [N,Dp] shared by all
    heads (DeepSeek's decoupled RoPE, Dp = 64), the logit is
    scale * (<q, kv> + <q_pe, k_pe>), the values are kv alone.  Its extra
    gradients are dq_pe = scale * sum_k dS k_pe and, per kv row,
    dk_pe = sum over slots of sum_h scale * dS q_pe; everything else keeps its
    has_pe=False form.  The scale is whatever the caller passes (the natural
    choice is 1/sqrt(512 + Dp)).
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# bf16 / fp32 codecs (exact)
# --------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bfloat16 -> float64: the bf16 pattern is the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 directly to bfloat16, nearest with ties to even (one rounding).

    bf16 keeps 8 significant bits and float32's exponent range.  For |x| with
    frexp exponent e (x = m * 2**e, 0.5 <= |m| < 1) the spacing of bf16 values is
    2**(e-8) in the normal range and 2**-133 below it; np.rint rounds half to
    even.  The rounded value is exactly representable in float32, whose top 16
    bits are the bf16 pattern.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    fin = np.isfinite(x)
    _, e = np.frexp(np.where(fin, x, 0.0))
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(np.where(fin, x, 0.0) / quantum) * quantum
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)  # exact unless it overflows to +-inf
    out[...] = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[np.isnan(x)] = 0x7FC0
    out[np.isposinf(x)] = 0x7F80
    out[np.isneginf(x)] = 0xFF80
    return out


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> float32, IEEE round to nearest even."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------


def _valid(idx_row: np.ndarray, num_kv: int) -> np.ndarray:
    """Slots whose index addresses a kv row; anything else is masked."""
    return (idx_row >= 0) & (idx_row < num_kv)


def _sink64(sink, H: int) -> np.ndarray:
    if sink is None:
        return np.full(H, -np.inf)
    return np.asarray(sink, dtype=np.float64).reshape(H)


def _as64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


def _probs(s: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """P = exp(s - lse) per row; rows with lse = -inf give P = 0."""
    out = np.zeros_like(s)
    live = np.isfinite(lse)
    if np.any(live):
        out[live] = np.exp(s[live] - lse[live, None])
    return out


def _sink_prob(sink: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """P_sink = exp(sink - lse); zero when there is no sink or lse = -inf."""
    out = np.zeros_like(lse)
    live = np.isfinite(lse) & np.isfinite(sink)
    out[live] = np.exp(sink[live] - lse[live])
    return out


# --------------------------------------------------------------------------
# forward (produces the backward's O and lse inputs)
# --------------------------------------------------------------------------


def _logits(q_t, G, scale, qpe_t=None, Gpe=None):
    """scale * (q kv^T [+ q_pe k_pe^T]) for the gathered rows G (and Gpe)."""
    s = q_t @ G.T
    if qpe_t is not None:
        s = s + qpe_t @ Gpe.T
    return scale * s


def forward_token(q_t, kv64, idx_row, sink64, scale, qpe_t=None, kpe64=None):
    """One query token, all heads.  q_t: [H,D] float64.  Returns (O_t [H,D], lse_t [H]).

    S_k = scale * <q, kv[idx_k]> (+ scale * <q_pe, k_pe[idx_k]>) over valid k;
    m = max(S, sink); Z = sum_k exp(S_k - m) + exp(sink - m); lse = m + ln Z;
    O = sum_k exp(S_k - lse) kv[idx_k]   (the sink's value vector is zero).
    """
    H, Dh = q_t.shape
    v = _valid(idx_row, kv64.shape[0])
    G = kv64[idx_row[v]]                       # [nv, D]
    Gpe = None if kpe64 is None else kpe64[idx_row[v]]
    s = _logits(q_t, G, scale, qpe_t, Gpe)     # [H, nv]
    m = np.maximum(s.max(axis=1) if G.shape[0] else np.full(H, -np.inf), sink64)
    lse = np.full(H, -np.inf)
    live = np.isfinite(m)
    if np.any(live):
        z = np.exp(s[live] - m[live, None]).sum(axis=1)
        has_sink = np.isfinite(sink64[live])
        z = z + np.where(has_sink, np.exp(np.where(has_sink, sink64[live] - m[live], 0.0)), 0.0)
        lse[live] = m[live] + np.log(z)
    P = _probs(s, lse)
    O = P @ G if G.shape[0] else np.zeros((H, Dh))
    return O, lse


def forward(q, kv, idx, sink, scale, q_pe=None, k_pe=None):
    """Sparse MLA forward in float64.  q [T,H,D], kv [N,D] (bf16 bits or floats),
    idx [T,K] int, sink [H] or None; with has_pe also q_pe [T,H,Dp], k_pe [N,Dp].
    Returns (O [T,H,D] f64, lse [T,H] f64)."""
    kv64 = _as64(kv)
    kpe64 = None if k_pe is None else _as64(k_pe)
    T, H, Dh = np.shape(q)
    s64 = _sink64(sink, H)
    O = np.empty((T, H, Dh))
    lse = np.empty((T, H))
    for t in range(T):
        O[t], lse[t] = forward_token(_as64(q[t]), kv64, np.asarray(idx[t]), s64, scale,
                                     None if q_pe is None else _as64(q_pe[t]), kpe64)
    return O, lse


def emit_forward_outputs(O, lse):
    """Round the forward outputs the way the backward consumes them:
    O -> bf16 (one rounding from float64, ties to even), lse -> float32."""
    return f64_to_bf16_rne(O), f64_to_f32(lse)


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------


def backward_token(q_t, kv64, dO_t, O_t, lse_t, idx_row, sink64, scale, dlse_t=None, qpe_t=None,
                   kpe64=None):
    """Backward of one query token, all heads, following the phase definitions.

    delta = rowsum(O * dO)
    P     = exp(S - lse)        S = scale * q kv^T (+ scale * q_pe k_pe^T)   (0 on masked slots)
    dP    = dO kv^T
    dS    = P * (dP - delta + dlse)        (dlse = 0 when not given)
    dq    = scale * dS kv                  dq_pe = scale * dS k_pe
    interm[k] = sum_h (scale * dS[h,k] q[h] + P[h,k] dO[h])   (0 on masked slots)
    interm_pe[k] = sum_h scale * dS[h,k] q_pe[h]
    d_sink contribution = -P_sink * (delta - dlse)

    Returns a dict of per-token arrays; P, dS are [H, K], interm is [K, D]
    (with has_pe also dq_pe [H, Dp] and interm_pe [K, Dp]).
    """
    H, Dh = q_t.shape
    K = idx_row.shape[0]
    v = _valid(idx_row, kv64.shape[0])
    G = kv64[idx_row[v]]
    Gpe = None if kpe64 is None else kpe64[idx_row[v]]
    delta = np.sum(O_t * dO_t, axis=1)
    dl = np.zeros(H) if dlse_t is None else np.asarray(dlse_t, dtype=np.float64)
    s = _logits(q_t, G, scale, qpe_t, Gpe)
    Pv = _probs(s, lse_t)
    dPv = dO_t @ G.T
    dSv = Pv * (dPv - delta[:, None] + dl[:, None])
    dq = scale * (dSv @ G) if G.shape[0] else np.zeros((H, Dh))
    P = np.zeros((H, K))
    dS = np.zeros((H, K))
    P[:, v] = Pv
    dS[:, v] = dSv
    interm = np.zeros((K, Dh))
    interm[v] = scale * (dSv.T @ q_t) + Pv.T @ dO_t
    p_sink = _sink_prob(sink64, lse_t)
    out = {"dq": dq, "delta": delta, "P": P, "dS": dS, "interm": interm,
           "dsink": -p_sink * (delta - dl), "valid": v}
    if qpe_t is not None:
        Dp = qpe_t.shape[1]
        out["dq_pe"] = scale * (dSv @ Gpe) if G.shape[0] else np.zeros((H, Dp))
        interm_pe = np.zeros((K, Dp))
        interm_pe[v] = scale * (dSv.T @ qpe_t)
        out["interm_pe"] = interm_pe
    return out


def backward(q, kv, dO, O, lse, idx, sink, scale, stages=False, dlse=None, q_pe=None, k_pe=None):
    """Full backward in float64.  Inputs as consumed by the op: q, kv, dO, O as
    bf16 bits (or floats), lse float, idx int, sink [H] or None, dlse [T,H] or
    None; with has_pe also q_pe [T,H,Dp] and k_pe [N,Dp].

    Returns dict with dq [T,H,D], dkv [N,D], d_sink [H] (None without a sink),
    delta [T,H]; with has_pe also dq_pe [T,H,Dp] and dk_pe [N,Dp]; with
    stages=True also P, dS [T,H,K] and interm [T,K,D] (and interm_pe).
    """
    kv64 = _as64(kv)
    kpe64 = None if k_pe is None else _as64(k_pe)
    N, Dh = kv64.shape
    T, H, _ = np.shape(q)
    K = np.shape(idx)[1]
    lse64 = np.asarray(lse, dtype=np.float64)
    s64 = _sink64(sink, H)
    dq = np.empty((T, H, Dh))
    dkv = np.zeros((N, Dh))
    delta = np.empty((T, H))
    dsink = np.zeros(H)
    pe = kpe64 is not None
    if pe:
        Dp = kpe64.shape[1]
        dq_pe = np.empty((T, H, Dp))
        dk_pe = np.zeros((N, Dp))
    if stages:
        P = np.zeros((T, H, K))
        dS = np.zeros((T, H, K))
        interm = np.zeros((T, K, Dh))
        if pe:
            interm_pe = np.zeros((T, K, Dp))
    for t in range(T):
        row = np.asarray(idx[t])
        r = backward_token(_as64(q[t]), kv64, _as64(dO[t]), _as64(O[t]), lse64[t], row, s64, scale,
                           None if dlse is None else dlse[t],
                           _as64(q_pe[t]) if pe else None, kpe64)
        dq[t] = r["dq"]
        delta[t] = r["delta"]
        dsink += r["dsink"]
        v = r["valid"]
        np.add.at(dkv, row[v], r["interm"][v])
        if pe:
            dq_pe[t] = r["dq_pe"]
            np.add.at(dk_pe, row[v], r["interm_pe"][v])
        if stages:
            P[t], dS[t], interm[t] = r["P"], r["dS"], r["interm"]
            if pe:
                interm_pe[t] = r["interm_pe"]
    out = {"dq": dq, "dkv": dkv, "d_sink": dsink if sink is not None else None, "delta": delta}
    if pe:
        out.update(dq_pe=dq_pe, dk_pe=dk_pe)
    if stages:
        out.update(P=P, dS=dS, interm=interm)
        if pe:
            out["interm_pe"] = interm_pe
    return out


def backward_tokens(q, kv, dO, O, lse, idx, sink, scale, tokens, dlse=None, q_pe=None, k_pe=None):
    """dq, delta, P, dS and interm (with has_pe also dq_pe, interm_pe) for a
    subset of query tokens only."""
    kv64 = _as64(kv)
    kpe64 = None if k_pe is None else _as64(k_pe)
    H = np.shape(q)[1]
    s64 = _sink64(sink, H)
    lse64 = np.asarray(lse, dtype=np.float64)
    res = [backward_token(_as64(q[t]), kv64, _as64(dO[t]), _as64(O[t]), lse64[t],
                          np.asarray(idx[t]), s64, scale, None if dlse is None else dlse[t],
                          None if q_pe is None else _as64(q_pe[t]), kpe64)
           for t in tokens]
    keys = ("dq", "delta", "P", "dS", "interm") + (("dq_pe", "interm_pe") if kpe64 is not None else ())
    return {k: np.stack([r[k] for r in res]) for k in keys}


def dkv_rows(q, kv, dO, O, lse, idx, sink, scale, rows, dlse=None):
    """dkv for selected kv rows only: the sum of interm over every valid slot
    (t, k) with idx[t, k] == j, each slot's interm evaluated from its definition."""
    kv64 = _as64(kv)
    N, Dh = kv64.shape
    idx = np.asarray(idx)
    lse64 = np.asarray(lse, dtype=np.float64)
    out = np.zeros((len(rows), Dh))
    for r, j in enumerate(rows):
        ts, ks = np.nonzero(idx == j)
        for t in np.unique(ts):
            q_t, dO_t = _as64(q[t]), _as64(dO[t])
            delta = np.sum(_as64(O[t]) * dO_t, axis=1)
            dl = 0.0 if dlse is None else np.asarray(dlse[t], dtype=np.float64)
            g = kv64[j]
            s = scale * (q_t @ g)
            P = _probs(s[:, None], lse64[t])[:, 0]
            dS = P * (dO_t @ g - delta + dl)
            contrib = scale * (dS @ q_t) + P @ dO_t
            out[r] += contrib * np.count_nonzero(ts == t)
    return out


def d_sink(dO, O, lse, sink, dlse=None):
    """d_sink[h] = -sum_t exp(sink[h] - lse[t,h]) * (rowsum(O * dO)[t,h] - dlse[t,h])."""
    T, H, _ = np.shape(O)
    s64 = _sink64(sink, H)
    lse64 = np.asarray(lse, dtype=np.float64)
    acc = np.zeros(H)
    for t in range(T):
        delta = np.sum(_as64(O[t]) * _as64(dO[t]), axis=1)
        if dlse is not None:
            delta = delta - np.asarray(dlse[t], dtype=np.float64)
        acc -= _sink_prob(s64, lse64[t]) * delta
    return acc


def delta(dO, O):
    """delta[t,h] = sum_d O[t,h,d] * dO[t,h,d]."""
    T = np.shape(O)[0]
    return np.stack([np.sum(_as64(O[t]) * _as64(dO[t]), axis=1) for t in range(T)])


def dkv_from_interm(interm, idx, num_kv):
    """dkv[j] = sum of interm[t, k] over valid slots (t, k) with idx[t, k] == j
    (the gather phase).  interm: [T, K, D] (bf16 bits or floats)."""
    it = _as64(interm)
    T, K, Dh = it.shape
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    v = (flat >= 0) & (flat < num_kv)
    dkv = np.zeros((num_kv, Dh))
    np.add.at(dkv, flat[v], it.reshape(T * K, Dh)[v])
    return dkv


# --------------------------------------------------------------------------
# inverted top-k (CSR)
# --------------------------------------------------------------------------


def csr(idx, num_kv):
    """Inverted index: valid slots s = t*K + k grouped by kv row, ascending in s.

    Returns (row_ptr int32 [num_kv+1], slots int32 [nnz]): row_ptr is the
    exclusive running total of per-row counts, and slots[row_ptr[j]:row_ptr[j+1]]
    lists the slots that address row j, in increasing order.
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    s = np.nonzero((flat >= 0) & (flat < num_kv))[0]
    keys = flat[s]
    order = np.argsort(keys, kind="stable")        # s is already ascending
    counts = np.bincount(keys, minlength=num_kv)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return row_ptr, s[order].astype(np.int32)


def count_invalid(idx, num_kv):
    """Number of index values that are neither -1 nor a kv row."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    return int(np.count_nonzero((flat != -1) & ((flat < 0) | (flat >= num_kv))))
