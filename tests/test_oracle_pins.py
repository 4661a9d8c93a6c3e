"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test checks the oracle against something its own code does not restate:
central finite differences of the forward, torch's dense attention with
autograd (a library routine) in the special case where the sparse op is dense
causal attention, closed forms, invariants the mathematics fixes, brute force
on tiny inputs, and numbers the page prints.  A plausible mistake in the oracle
(a dropped term, a wrong sign or index, a transposed operand, a missing scale,
the sink treated as a value-carrying key or scaled) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import smla_oracle as orc
from sparse_mla_attention_smla_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# bf16 / fp32 codecs
# --------------------------------------------------------------------------

def test_bf16_codec_known_patterns():
    # IEEE bfloat16 encodings: sign | 8-bit exponent | 7-bit fraction
    vals = np.array([1.0, -2.0, 0.5, 3.0, 0.0, -0.0, 65280.0, 2.0 ** -126, 2.0 ** -133])
    want = np.array([0x3F80, 0xC000, 0x3F00, 0x4040, 0x0000, 0x8000, 0x477F, 0x0080, 0x0001],
                    dtype=np.uint16)
    assert np.array_equal(orc.f64_to_bf16_rne(vals), want)
    assert np.array_equal(orc.bf16_to_f64(want), vals)


def test_bf16_rounding_ties_and_double_rounding():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even pattern 0x3F80.
    # 1 + 3*2^-8 is halfway between 1+2^-7 (0x3F81) and 1+2^-6 (0x3F82): even is 0x3F82.
    # 1 + 2^-8 + 2^-40 lies above the halfway point: a single rounding from float64
    # gives 0x3F81, while rounding through float32 first would give 0x3F80.
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -40, -(1 + 2 ** -8 + 2 ** -40)])
    assert list(orc.f64_to_bf16_rne(x)) == [0x3F80, 0x3F82, 0x3F81, 0xBF81]


def test_bf16_matches_torch_on_float32_values():
    # torch's float32 -> bfloat16 cast is round-to-nearest-even: a library routine.
    rng = np.random.default_rng(7)
    x32 = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f64_to_bf16_rne(x32.astype(np.float64)), want)
    back = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.bf16_to_f64(want), back)


# --------------------------------------------------------------------------
# finite differences of L = <dO, O(q, kv, sink)>
# --------------------------------------------------------------------------

def _fd_case(D, with_sink, seed):
    rng = np.random.default_rng(seed)
    T, H, P = 6, 3, 3
    N = T + P
    K = 4
    idx = np.array([
        [0, -1, -1, -1],          # one valid slot
        [1, 0, -1, 7],            # pool row 7 and padding
        [2, 2, 6, -1],            # duplicate index
        [-1, -1, -1, -1],         # all masked
        [4, 3, N + 2, -5],        # out-of-range values are masked
        [5, 8, 1, 6],
    ], dtype=np.int64)
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((N, D))
    dO = rng.standard_normal((T, H, D))
    sink = rng.standard_normal(H) if with_sink else None
    return q, kv, dO, idx, sink, 0.37


def _loss(q, kv, sink, dO, idx, scale):
    O, _ = orc.forward(q, kv, idx, sink, scale)
    return float(np.sum(O * dO))


@pytest.mark.parametrize("D", [8, 16])
@pytest.mark.parametrize("with_sink", [True, False])
def test_backward_matches_central_differences(D, with_sink):
    q, kv, dO, idx, sink, scale = _fd_case(D, with_sink, seed=11 + D + with_sink)
    O, lse = orc.forward(q, kv, idx, sink, scale)
    g = orc.backward(q, kv, dO, O, lse, idx, sink, scale)

    def fd(arr, setter):
        out = np.empty(arr.shape)
        for i in np.ndindex(arr.shape):
            x0 = arr[i]
            eps = 1e-6 * max(1.0, abs(x0))
            arr[i] = x0 + eps
            lp = setter()
            arr[i] = x0 - eps
            lm = setter()
            arr[i] = x0
            out[i] = (lp - lm) / (2 * eps)
        return out

    L = lambda: _loss(q, kv, sink, dO, idx, scale)
    np.testing.assert_allclose(g["dq"], fd(q, L), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(g["dkv"], fd(kv, L), rtol=1e-6, atol=1e-8)
    if with_sink:
        np.testing.assert_allclose(g["d_sink"], fd(sink, L), rtol=1e-6, atol=1e-8)
    # the all-masked row gets an exactly zero dq
    assert np.all(g["dq"][3] == 0.0)


def test_random_direction_derivative_at_full_width():
    # directional derivative check at D=512 with the tiny workload's index structure
    w = inputs.WORKLOADS["tiny"]
    rng = np.random.default_rng(5)
    T, H, N, K, D = 12, 2, 12, 6, 512
    idx = inputs.make_indices(inputs.Workload("t", 0, T, H, N, K, "causal"), rng)
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((N, D))
    dO = rng.standard_normal((T, H, D))
    sink = rng.standard_normal(H)
    scale = 1 / math.sqrt(D)
    O, lse = orc.forward(q, kv, idx, sink, scale)
    g = orc.backward(q, kv, dO, O, lse, idx, sink, scale)
    dq_dir, dkv_dir, ds_dir = (rng.standard_normal(q.shape), rng.standard_normal(kv.shape),
                               rng.standard_normal(H))
    eps = 1e-5
    lp = _loss(q + eps * dq_dir, kv + eps * dkv_dir, sink + eps * ds_dir, dO, idx, scale)
    lm = _loss(q - eps * dq_dir, kv - eps * dkv_dir, sink - eps * ds_dir, dO, idx, scale)
    fd = (lp - lm) / (2 * eps)
    an = np.sum(g["dq"] * dq_dir) + np.sum(g["dkv"] * dkv_dir) + np.sum(g["d_sink"] * ds_dir)
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))
    assert w.topk == 16


# --------------------------------------------------------------------------
# with an upstream gradient of lse: L = <dO, O> + <dlse, lse>
# --------------------------------------------------------------------------

def _loss_lse(q, kv, sink, dO, dlse, idx, scale):
    O, lse = orc.forward(q, kv, idx, sink, scale)
    live = np.isfinite(lse)      # a row with no slot and no sink has lse = -inf, constant
    return float(np.sum(O * dO) + np.sum(dlse[live] * lse[live]))


@pytest.mark.parametrize("with_sink", [True, False])
def test_dlse_backward_matches_central_differences(with_sink):
    q, kv, dO, idx, sink, scale = _fd_case(8, with_sink, seed=31 + with_sink)
    dlse = np.random.default_rng(41).standard_normal((q.shape[0], q.shape[1]))
    O, lse = orc.forward(q, kv, idx, sink, scale)
    g = orc.backward(q, kv, dO, O, lse, idx, sink, scale, dlse=dlse)

    def fd(arr):
        out = np.empty(arr.shape)
        for i in np.ndindex(arr.shape):
            x0 = arr[i]
            eps = 1e-6 * max(1.0, abs(x0))
            arr[i] = x0 + eps
            lp = _loss_lse(q, kv, sink, dO, dlse, idx, scale)
            arr[i] = x0 - eps
            lm = _loss_lse(q, kv, sink, dO, dlse, idx, scale)
            arr[i] = x0
            out[i] = (lp - lm) / (2 * eps)
        return out

    np.testing.assert_allclose(g["dq"], fd(q), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(g["dkv"], fd(kv), rtol=1e-6, atol=1e-8)
    if with_sink:
        np.testing.assert_allclose(g["d_sink"], fd(sink), rtol=1e-6, atol=1e-8)
    assert np.all(g["dq"][3] == 0.0)


def test_dlse_alone_closed_forms():
    # dO = 0 and dlse = 1: the gradient of sum(lse).  d lse / d q = scale * sum_k P_k kv_k
    # = scale * O (the forward's output), and d lse / d sink = P_sink.
    q, kv, dO, idx, sink, scale = _random_case(7)
    O, lse = orc.forward(q, kv, idx, sink, scale)
    g = orc.backward(q, kv, np.zeros_like(dO), O, lse, idx, sink, scale, dlse=np.ones(lse.shape))
    np.testing.assert_allclose(g["dq"], scale * O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["d_sink"], np.exp(sink[None, :] - lse).sum(0), rtol=1e-12)


def test_linearity_in_dO_and_dlse():
    q, kv, dO, idx, sink, scale = _random_case(8)
    rng = np.random.default_rng(98)
    dO2 = rng.standard_normal(dO.shape)
    O, lse = orc.forward(q, kv, idx, sink, scale)
    d1, d2 = rng.standard_normal(lse.shape), rng.standard_normal(lse.shape)
    a, b = 1.3, -0.6
    g1 = orc.backward(q, kv, dO, O, lse, idx, sink, scale, dlse=d1)
    g2 = orc.backward(q, kv, dO2, O, lse, idx, sink, scale, dlse=d2)
    g12 = orc.backward(q, kv, a * dO + b * dO2, O, lse, idx, sink, scale, dlse=a * d1 + b * d2)
    for k in ("dq", "dkv", "d_sink"):
        np.testing.assert_allclose(g12[k], a * g1[k] + b * g2[k], rtol=1e-11, atol=1e-12)
    toks = [1, 9]
    s = orc.backward_tokens(q, kv, dO, O, lse, idx, sink, scale, toks, dlse=d1)
    np.testing.assert_allclose(s["dq"], g1["dq"][toks], rtol=1e-14)
    np.testing.assert_allclose(orc.dkv_rows(q, kv, dO, O, lse, idx, sink, scale, [0, 4], dlse=d1),
                               g1["dkv"][[0, 4]], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(orc.d_sink(dO, O, lse, sink, dlse=d1), g1["d_sink"], rtol=1e-13)


# --------------------------------------------------------------------------
# dense special case == causal attention with a sink logit (torch, autograd)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("with_dlse", [False, True])
@pytest.mark.parametrize("with_sink", [True, False])
def test_dense_causal_case_matches_torch_sdpa(with_sink, with_dlse):
    from torch.nn.attention import SDPBackend, sdpa_kernel
    rng = np.random.default_rng(3)
    T, H, D = 12, 4, 32
    scale = 1 / math.sqrt(D)
    idx = np.full((T, T), -1, dtype=np.int64)
    for t in range(T):
        idx[t, : t + 1] = np.arange(t + 1)
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    dO = rng.standard_normal((T, H, D))
    sink = rng.standard_normal(H)

    dlse = rng.standard_normal((T, H)) if with_dlse else None
    O, lse = orc.forward(q, kv, idx, sink if with_sink else None, scale)
    g = orc.backward(q, kv, dO, O, lse, idx, sink if with_sink else None, scale, dlse=dlse)

    tq = torch.tensor(q, requires_grad=True)
    tkv = torch.tensor(kv, requires_grad=True)
    tsink = torch.tensor(sink, requires_grad=True)
    # keys/values = kv rows plus one extra key whose logit is the sink and whose value is 0
    kext = torch.cat([tkv, torch.zeros(1, D, dtype=torch.float64)], 0)
    causal = torch.full((T, T + 1), float("-inf"), dtype=torch.float64)
    causal[:, :T] = torch.triu(torch.full((T, T), float("-inf"), dtype=torch.float64), 1)
    mask = causal[None].repeat(H, 1, 1)
    if with_sink:
        mask[:, :, T] = 0.0
        # last key column carries the per-head sink logit
        mask = mask + torch.nn.functional.pad(tsink[:, None, None].expand(H, T, 1), (T, 0))
    qh = tq.permute(1, 0, 2)[None]                       # [1,H,T,D]
    kh = kext[None, None].expand(1, H, T + 1, D)
    with sdpa_kernel(SDPBackend.MATH):
        out = torch.nn.functional.scaled_dot_product_attention(qh, kh, kh, attn_mask=mask[None], scale=scale)
    ref_O = out[0].permute(1, 0, 2)
    ref_lse = torch.logsumexp(scale * (qh @ kh.transpose(-1, -2)) + mask[None], dim=-1)[0].T
    np.testing.assert_allclose(O, ref_O.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse.detach().numpy(), rtol=1e-12, atol=1e-13)
    loss = torch.sum(ref_O * torch.tensor(dO))
    if with_dlse:
        loss = loss + torch.sum(ref_lse * torch.tensor(dlse))
    loss.backward()
    np.testing.assert_allclose(g["dq"], tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dkv"], tkv.grad.numpy(), rtol=1e-10, atol=1e-12)
    if with_sink:
        np.testing.assert_allclose(g["d_sink"], tsink.grad.numpy(), rtol=1e-10, atol=1e-12)
    else:
        assert g["d_sink"] is None


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_single_slot_closed_forms():
    rng = np.random.default_rng(9)
    H, D, N = 3, 16, 5
    scale = 0.25
    q = rng.standard_normal((2, H, D))
    kv = rng.standard_normal((N, D))
    dO = rng.standard_normal((2, H, D))
    sink = rng.standard_normal(H)
    idx = np.array([[3, -1, -1], [3, -1, -1]])
    # token 0 without sink: P = 1, O = kv[3], dS = 0, interm = sum_h dO
    O, lse = orc.forward(q[:1], kv, idx[:1], None, scale)
    np.testing.assert_allclose(O[0], np.tile(kv[3], (H, 1)), rtol=1e-15)
    np.testing.assert_allclose(lse[0], scale * q[0] @ kv[3], rtol=1e-15)
    r = orc.backward_token(q[0], kv, dO[0], O[0], lse[0], idx[0], np.full(H, -np.inf), scale)
    np.testing.assert_allclose(r["dq"], 0.0, atol=1e-13)
    np.testing.assert_allclose(r["interm"][0], dO[0].sum(0), rtol=1e-12, atol=1e-13)
    assert np.all(r["interm"][1:] == 0.0)
    # with a sink: P = logistic(s - sink), dq = scale P(1-P) dP kv, d_sink = -(1-P) P dP
    O, lse = orc.forward(q[1:], kv, idx[1:], sink, scale)
    s = scale * q[1] @ kv[3]
    p = expit(s - sink)
    np.testing.assert_allclose(O[0], p[:, None] * kv[3], rtol=1e-13)
    np.testing.assert_allclose(lse[0], np.logaddexp(s, sink), rtol=1e-13)
    r = orc.backward_token(q[1], kv, dO[1], O[0], lse[0], idx[1], sink, scale)
    dP = dO[1] @ kv[3]
    np.testing.assert_allclose(r["dq"], (scale * p * (1 - p) * dP)[:, None] * kv[3], rtol=1e-11)
    np.testing.assert_allclose(r["dsink"], -(1 - p) * p * dP, rtol=1e-11)
    np.testing.assert_allclose(r["interm"][0], (scale * p * (1 - p) * dP) @ q[1] + p @ dO[1],
                               rtol=1e-11)


def test_identical_rows_give_uniform_probabilities():
    rng = np.random.default_rng(4)
    H, D, N, K = 2, 8, 6, 4
    kv = np.tile(rng.standard_normal(D), (N, 1))
    q = rng.standard_normal((1, H, D))
    idx = np.array([[0, 2, 5, -1]])
    O, lse = orc.forward(q, kv, idx, None, 0.5)
    np.testing.assert_allclose(O[0], np.tile(kv[0], (H, 1)), rtol=1e-14)
    np.testing.assert_allclose(lse[0], 0.5 * q[0] @ kv[0] + np.log(3.0), rtol=1e-14)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def _random_case(seed, T=16, H=4, D=16, P=6, K=8, with_sink=True):
    rng = np.random.default_rng(seed)
    N = T + P
    idx = np.full((T, K), -1, dtype=np.int64)
    for t in range(T):
        n = rng.integers(1, K + 1)
        idx[t, :n] = rng.choice(N - 2, n, replace=False)   # last two kv rows stay unused
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((N, D))
    dO = rng.standard_normal((T, H, D))
    sink = rng.standard_normal(H) if with_sink else None
    return q, kv, dO, idx, sink, 1 / math.sqrt(D)


def test_probabilities_sum_to_one_with_sink_and_delta_identity():
    q, kv, dO, idx, sink, scale = _random_case(1)
    O, lse = orc.forward(q, kv, idx, sink, scale)
    g = orc.backward(q, kv, dO, O, lse, idx, sink, scale, stages=True)
    p_sink = np.exp(sink[None, :] - lse)
    np.testing.assert_allclose(g["P"].sum(-1) + p_sink, 1.0, rtol=1e-14)
    # delta = rowsum(O dO) equals sum_k P_k dP_k when O is the exact forward
    kv_g = kv[np.where(idx >= 0, idx, 0)]                       # [T,K,D]
    dP = np.einsum("thd,tkd->thk", dO, kv_g)
    np.testing.assert_allclose(g["delta"], np.sum(g["P"] * dP, -1), rtol=1e-12, atol=1e-13)
    # shift invariance of the logits: sum_k dS = P_sink * delta, so
    # d_sink = -sum_{t,k} dS
    np.testing.assert_allclose(g["d_sink"], -g["dS"].sum(axis=(0, 2)), rtol=1e-11, atol=1e-13)


def test_masking_invariants():
    q, kv, dO, idx, sink, scale = _random_case(2)
    O, lse = orc.forward(q, kv, idx, sink, scale)
    g = orc.backward(q, kv, dO, O, lse, idx, sink, scale)
    # appending -1 (and out-of-range) columns leaves every output identical
    pad = np.concatenate([idx, np.full((idx.shape[0], 3), -1), np.full((idx.shape[0], 1), 10 ** 6)], 1)
    O2, lse2 = orc.forward(q, kv, pad, sink, scale)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)
    g2 = orc.backward(q, kv, dO, O, lse, pad, sink, scale)
    for k in ("dq", "dkv", "d_sink"):
        assert np.array_equal(g[k], g2[k])
    # kv rows that no valid slot addresses get exactly zero gradient
    unused = np.setdiff1d(np.arange(kv.shape[0]), idx[idx >= 0])
    assert unused.size > 0
    assert np.all(g["dkv"][unused] == 0.0)
    # an all-masked row: dq exactly zero; without a sink lse = -inf and O = 0
    idx3 = idx.copy()
    idx3[5] = -1
    O3, lse3 = orc.forward(q, kv, idx3, None, scale)
    assert np.all(O3[5] == 0.0) and np.all(np.isneginf(lse3[5]))
    g3 = orc.backward(q, kv, dO, O3, lse3, idx3, None, scale)
    assert np.all(g3["dq"][5] == 0.0) and np.all(np.isfinite(g3["dkv"]))
    O4, lse4 = orc.forward(q, kv, idx3, sink, scale)
    np.testing.assert_array_equal(lse4[5], sink)
    g4 = orc.backward(q, kv, dO, O4, lse4, idx3, sink, scale)
    assert np.all(g4["dq"][5] == 0.0)


def test_linearity_in_dO():
    q, kv, dO, idx, sink, scale = _random_case(3)
    dO2 = np.random.default_rng(99).standard_normal(dO.shape)
    O, lse = orc.forward(q, kv, idx, sink, scale)
    a, b = 0.7, -1.9
    g1 = orc.backward(q, kv, dO, O, lse, idx, sink, scale)
    g2 = orc.backward(q, kv, dO2, O, lse, idx, sink, scale)
    g12 = orc.backward(q, kv, a * dO + b * dO2, O, lse, idx, sink, scale)
    for k in ("dq", "dkv", "d_sink"):
        np.testing.assert_allclose(g12[k], a * g1[k] + b * g2[k], rtol=1e-11, atol=1e-12)


def test_slot_permutation_invariance():
    q, kv, dO, idx, sink, scale = _random_case(4)
    O, lse = orc.forward(q, kv, idx, sink, scale)
    g = orc.backward(q, kv, dO, O, lse, idx, sink, scale)
    rng = np.random.default_rng(0)
    T, K = idx.shape
    perms = np.stack([rng.permutation(K) for _ in range(T)])
    idxp = np.take_along_axis(idx, perms, 1)
    Op, lsep = orc.forward(q, kv, idxp, sink, scale)
    np.testing.assert_allclose(Op, O, rtol=1e-13, atol=1e-14)
    gp = orc.backward(q, kv, dO, O, lse, idxp, sink, scale)
    for k in ("dq", "dkv", "d_sink"):
        np.testing.assert_allclose(gp[k], g[k], rtol=1e-12, atol=1e-13)
    # the CSR lists the same (row, slot) pairs, slots renamed through the permutation
    rp, sl = orc.csr(idx, kv.shape[0])
    rpp, slp = orc.csr(idxp, kv.shape[0])
    assert np.array_equal(rp, rpp)
    t_of, k_of = slp // K, slp % K
    orig = t_of * K + perms[t_of, k_of]
    for j in range(kv.shape[0]):
        assert sorted(orig[rpp[j]:rpp[j + 1]]) == list(sl[rp[j]:rp[j + 1]])


def test_sampled_helpers_agree_with_full_backward():
    q, kv, dO, idx, sink, scale = _random_case(6)
    O, lse = orc.forward(q, kv, idx, sink, scale)
    g = orc.backward(q, kv, dO, O, lse, idx, sink, scale, stages=True)
    toks = [0, 5, 15]
    s = orc.backward_tokens(q, kv, dO, O, lse, idx, sink, scale, toks)
    np.testing.assert_allclose(s["dq"], g["dq"][toks], rtol=1e-14)
    np.testing.assert_allclose(s["interm"], g["interm"][toks], rtol=1e-14)
    rows = [0, 3, kv.shape[0] - 1]
    np.testing.assert_allclose(orc.dkv_rows(q, kv, dO, O, lse, idx, sink, scale, rows),
                               g["dkv"][rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(orc.d_sink(dO, O, lse, sink), g["d_sink"], rtol=1e-13)
    np.testing.assert_allclose(orc.delta(dO, O), g["delta"], rtol=1e-14)


# --------------------------------------------------------------------------
# the gather phase on its own: dkv from a given intermediate
# --------------------------------------------------------------------------

@pytest.mark.parametrize("D", [8, 16])
def test_dkv_from_interm_equals_the_finite_difference_pinned_dkv(D):
    """Gathering the oracle's own per-slot intermediate must give the dkv that
    central finite differences pin (test_backward_matches_central_differences):
    the index set there has a duplicate index within a row, -1 padding, an
    all-masked row and out-of-range values."""
    for with_sink in (True, False):
        q, kv, dO, idx, sink, scale = _fd_case(D, with_sink, seed=11 + D + with_sink)
        O, lse = orc.forward(q, kv, idx, sink, scale)
        g = orc.backward(q, kv, dO, O, lse, idx, sink, scale, stages=True)
        got = orc.dkv_from_interm(g["interm"], idx, kv.shape[0])
        np.testing.assert_allclose(got, g["dkv"], rtol=1e-13, atol=1e-15)


def test_dkv_from_interm_brute_force():
    """Against a plain loop over slots, on arbitrary values: duplicate indices add
    both rows, -1 and out-of-range indices are dropped, rows nobody addresses are
    exactly zero.  Also through the bf16 bit-pattern input the GPU tests pass."""
    rng = np.random.default_rng(41)
    idx = np.array([[3, -1, 0, 3], [6, 0, 9, -1], [-7, 2, 2, 6], [1, 1, 1, 1], [-1, -1, -1, -1]])
    N, Dh = 8, 5
    T, K = idx.shape
    interm = rng.standard_normal((T, K, Dh))
    want = np.zeros((N, Dh))
    for t in range(T):
        for k in range(K):
            j = idx[t, k]
            if 0 <= j < N:
                want[j] += interm[t, k]
    got = orc.dkv_from_interm(interm, idx, N)
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)
    assert np.all(got[[4, 5, 7]] == 0.0)                   # never addressed
    np.testing.assert_allclose(got[1], interm[3].sum(axis=0), rtol=1e-15)   # four duplicates
    # a row's slot order does not matter; masked slots carry arbitrary values
    perm = rng.permutation(K)
    np.testing.assert_allclose(orc.dkv_from_interm(interm[:, perm], idx[:, perm], N), want, rtol=1e-14)
    # bf16 bit patterns are decoded exactly before summing
    bits = orc.f64_to_bf16_rne(interm)
    dec = orc.bf16_to_f64(bits)
    want_b = np.zeros((N, Dh))
    for t in range(T):
        for k in range(K):
            if 0 <= idx[t, k] < N:
                want_b[idx[t, k]] += dec[t, k]
    np.testing.assert_allclose(orc.dkv_from_interm(bits, idx, N), want_b, rtol=1e-15, atol=0)


# --------------------------------------------------------------------------
# CSR
# --------------------------------------------------------------------------

def test_csr_brute_force_and_structure():
    idx = np.array([[3, -1, 0, 3], [6, 0, 9, -1], [-7, 2, 2, 6], [1, 1, 1, 1], [-1, -1, -1, -1]])
    N = 7
    row_ptr, slots = orc.csr(idx, N)
    flat = idx.reshape(-1)
    want_ptr, want = [0], []
    for j in range(N):
        for s in range(flat.size):
            if flat[s] == j:
                want.append(s)
        want_ptr.append(len(want))
    assert list(row_ptr) == want_ptr and list(slots) == want
    assert orc.count_invalid(idx, N) == 2   # 9 and -7


def test_csr_invariants_on_headline_indices():
    w = inputs.WORKLOADS["headline"]
    idx = inputs.make_indices(w, np.random.default_rng(1000 + w.index))
    row_ptr, slots = orc.csr(idx, w.num_kv)
    assert row_ptr[0] == 0 and row_ptr[-1] == slots.size == 1_793_728
    assert np.all(np.diff(row_ptr) >= 0)
    flat = idx.reshape(-1)
    rows = np.repeat(np.arange(w.num_kv), np.diff(row_ptr))
    assert np.array_equal(flat[slots], rows)
    same = rows[1:] == rows[:-1]
    assert np.all(slots[1:][same] > slots[:-1][same])


# --------------------------------------------------------------------------
# numbers the page prints
# --------------------------------------------------------------------------

def test_page_flop_convention_and_interm_size():
    g = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))
    w = inputs.WORKLOADS["headline"]
    assert (w.T, w.H, w.topk) == (g["T"], g["H"], g["topk"])
    for row in g["rows"]:
        assert round(w.flops() / (row["ms"] * 1e-3) / 1e12) == row["tflops"], row
    assert w.T * w.topk * g["D"] * 2 / 2 ** 30 == g["interm_gib"]


# --------------------------------------------------------------------------
# generator recipe
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name,nnz", [("tiny", 904), ("small", 122_944), ("headline", 1_793_728),
                                      ("skewed", 1_793_728), ("long", 3_890_880),
                                      ("headline_h64", 1_793_728)])
def test_generator_index_structure(name, nnz):
    w = inputs.WORKLOADS[name]
    idx = inputs.make_indices(w, np.random.default_rng(1000 + w.index))
    assert idx.shape == (w.T, w.topk) and idx.dtype == np.int32
    valid = idx >= 0
    assert int(valid.sum()) == nnz
    for t in (0, 1, w.T // 2, w.T - 1):
        row = idx[t][valid[t]]
        assert np.all(np.diff(row) > 0) and np.all(idx[t][row.size:] == -1)
        if w.selection == "causal":
            assert row.size == min(w.topk, t + 1) and row.max() <= t
        else:
            win = row[row < w.T]
            assert np.array_equal(win, np.arange(max(0, t - 127), t + 1))
            pool = row[row >= w.T] - w.T
            assert np.all(4 * pool + 3 <= t)
    if name == "skewed":
        counts = np.bincount(idx[valid], minlength=w.num_kv)
        assert counts[w.T] > 3000     # pool row 0 collects thousands of contributors


# --------------------------------------------------------------------------
# the has_pe=True variant: a positional part on q and on the keys only
# --------------------------------------------------------------------------

def _pe_parts(T, H, N, Dp, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, H, Dp)), rng.standard_normal((N, Dp))


@pytest.mark.parametrize("with_sink", [True, False])
def test_pe_backward_matches_central_differences(with_sink):
    """L = <dO, O(q, q_pe, kv, k_pe, sink)>: every gradient, the two positional
    ones included, against central differences (duplicate, -1, out-of-range and
    all-masked slots as in the plain case)."""
    D, Dp = 8, 4
    q, kv, dO, idx, sink, scale = _fd_case(D, with_sink, seed=61 + with_sink)
    q_pe, k_pe = _pe_parts(q.shape[0], q.shape[1], kv.shape[0], Dp, seed=62)
    O, lse = orc.forward(q, kv, idx, sink, scale, q_pe=q_pe, k_pe=k_pe)
    g = orc.backward(q, kv, dO, O, lse, idx, sink, scale, q_pe=q_pe, k_pe=k_pe)

    def loss():
        return float(np.sum(orc.forward(q, kv, idx, sink, scale, q_pe=q_pe, k_pe=k_pe)[0] * dO))

    def fd(arr):
        out = np.empty(arr.shape)
        for i in np.ndindex(arr.shape):
            x0 = arr[i]
            eps = 1e-6 * max(1.0, abs(x0))
            arr[i] = x0 + eps
            lp = loss()
            arr[i] = x0 - eps
            lm = loss()
            arr[i] = x0
            out[i] = (lp - lm) / (2 * eps)
        return out

    for name, arr in (("dq", q), ("dq_pe", q_pe), ("dkv", kv), ("dk_pe", k_pe)):
        np.testing.assert_allclose(g[name], fd(arr), rtol=1e-6, atol=1e-8, err_msg=name)
    if with_sink:
        np.testing.assert_allclose(g["d_sink"], fd(sink), rtol=1e-6, atol=1e-8)
    assert np.all(g["dq_pe"][3] == 0.0)           # the all-masked row
    # the gather phase on the positional intermediate gives dk_pe
    st = orc.backward(q, kv, dO, O, lse, idx, sink, scale, stages=True, q_pe=q_pe, k_pe=k_pe)
    np.testing.assert_allclose(orc.dkv_from_interm(st["interm_pe"], idx, kv.shape[0]), g["dk_pe"],
                               rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("with_sink", [True, False])
def test_pe_dense_causal_case_matches_torch_sdpa(with_sink):
    """Dense causal case: SDPA with 576-wide queries/keys ([q, q_pe], [kv, k_pe]) and
    512-wide values (kv) -- torch's attention allows the value width to differ."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    rng = np.random.default_rng(13)
    T, H, D, Dp = 10, 3, 24, 8
    scale = 1 / math.sqrt(D + Dp)
    idx = np.full((T, T), -1, dtype=np.int64)
    for t in range(T):
        idx[t, : t + 1] = np.arange(t + 1)
    q, kv, dO = rng.standard_normal((T, H, D)), rng.standard_normal((T, D)), rng.standard_normal((T, H, D))
    q_pe, k_pe = rng.standard_normal((T, H, Dp)), rng.standard_normal((T, Dp))
    sink = rng.standard_normal(H)
    sk = sink if with_sink else None
    O, lse = orc.forward(q, kv, idx, sk, scale, q_pe=q_pe, k_pe=k_pe)
    g = orc.backward(q, kv, dO, O, lse, idx, sk, scale, q_pe=q_pe, k_pe=k_pe)

    tq, tqp = torch.tensor(q, requires_grad=True), torch.tensor(q_pe, requires_grad=True)
    tkv, tkp = torch.tensor(kv, requires_grad=True), torch.tensor(k_pe, requires_grad=True)
    tsink = torch.tensor(sink, requires_grad=True)
    z = lambda w: torch.zeros(1, w, dtype=torch.float64)
    keys = torch.cat([torch.cat([tkv, tkp], 1), z(D + Dp)], 0)          # + the sink's key (logit via mask)
    vals = torch.cat([tkv, z(D)], 0)                                     # the sink carries no value
    mask = torch.full((H, T, T + 1), float("-inf"), dtype=torch.float64)
    mask[:, :, :T] = torch.triu(torch.full((T, T), float("-inf"), dtype=torch.float64), 1)
    if with_sink:
        mask[:, :, T] = 0.0
        mask = mask + torch.nn.functional.pad(tsink[:, None, None].expand(H, T, 1), (T, 0))
    qh = torch.cat([tq, tqp], 2).permute(1, 0, 2)[None]
    kh = keys[None, None].expand(1, H, T + 1, D + Dp)
    vh = vals[None, None].expand(1, H, T + 1, D)
    with sdpa_kernel(SDPBackend.MATH):
        out = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask[None], scale=scale)
    ref_O = out[0].permute(1, 0, 2)
    np.testing.assert_allclose(O, ref_O.detach().numpy(), rtol=1e-12, atol=1e-13)
    torch.sum(ref_O * torch.tensor(dO)).backward()
    for name, t_ in (("dq", tq), ("dq_pe", tqp), ("dkv", tkv), ("dk_pe", tkp)):
        np.testing.assert_allclose(g[name], t_.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)
    if with_sink:
        np.testing.assert_allclose(g["d_sink"], tsink.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_pe_zero_parts_reduce_to_the_plain_op():
    """q_pe = 0 leaves every logit unchanged: O, lse, dq, dkv, d_sink equal the plain
    op's and dk_pe = 0 exactly; k_pe = 0 likewise, with dq_pe = 0 exactly."""
    q, kv, dO, idx, sink, scale = _random_case(21)
    T, H, _ = q.shape
    N = kv.shape[0]
    q_pe, k_pe = _pe_parts(T, H, N, 6, seed=22)
    O, lse = orc.forward(q, kv, idx, sink, scale)
    g = orc.backward(q, kv, dO, O, lse, idx, sink, scale)
    for qp, kp, zero in ((np.zeros_like(q_pe), k_pe, "dk_pe"), (q_pe, np.zeros_like(k_pe), "dq_pe")):
        O2, lse2 = orc.forward(q, kv, idx, sink, scale, q_pe=qp, k_pe=kp)
        np.testing.assert_array_equal(O2, O)
        np.testing.assert_array_equal(lse2, lse)
        g2 = orc.backward(q, kv, dO, O, lse, idx, sink, scale, q_pe=qp, k_pe=kp)
        for k in ("dq", "dkv", "d_sink"):
            np.testing.assert_allclose(g2[k], g[k], rtol=1e-13, atol=1e-15, err_msg=k)
        assert np.all(g2[zero] == 0.0)
    # a positional part that matches the content part doubles the logits: same as q scaled by 2
    q_pe2, k_pe2 = q.copy(), kv.copy()
    O3, lse3 = orc.forward(q, kv, idx, sink, scale, q_pe=q_pe2, k_pe=k_pe2)
    O4, lse4 = orc.forward(2 * q, kv, idx, sink, scale)
    np.testing.assert_allclose(O3, O4, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse3, lse4, rtol=1e-13)
