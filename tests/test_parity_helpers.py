"""CPU checks of the parity machinery the GPU tests rely on.

* The per-row bound rejects an output with one dropped (zeroed) or garbled row
  even when the whole-tensor rel-L2 and cosine bars still pass, and accepts
  bf16-level noise.
* The chunked oracle helpers (token slices evaluated in parallel threads) give
  what one plain oracle call over all tokens gives.
"""
import math

import numpy as np
import pytest

from oracle import smla_oracle as orc
from sparse_mla_attention_smla_amd import inputs
from tests import _helpers as hp


def _bf16_noise(a, rel, seed):
    rng = np.random.default_rng(seed)
    return a * (1.0 + rel * rng.standard_normal(a.shape))


def test_row_bound_catches_one_zeroed_row_that_the_global_bars_miss():
    rng = np.random.default_rng(3)
    want = rng.standard_normal((1024, 64, 512))            # 65,536 rows, the small workload's dq shape
    got = _bf16_noise(want, 2.3e-3, 4)
    hp.assert_close("noisy", got, want)                    # bf16-level noise passes
    norms = np.linalg.norm(want.reshape(-1, 512), axis=1)
    r = int(np.argsort(norms)[norms.size // 2])            # a median-norm row
    bad = got.reshape(-1, 512).copy()
    bad[r] = 0.0
    bad = bad.reshape(got.shape)
    assert hp.rel_l2(bad, want) <= hp.REL_L2 and hp.cosine(bad, want) >= hp.COS
    with pytest.raises(AssertionError, match="worst row error"):
        hp.assert_close("zeroed row", bad, want)
    garbled = got.reshape(-1, 512).copy()
    garbled[r] = garbled[r][::-1]
    with pytest.raises(AssertionError):
        hp.assert_close("garbled row", garbled.reshape(got.shape), want)


def test_row_bound_floor_for_near_zero_rows():
    rng = np.random.default_rng(5)
    want = rng.standard_normal((200, 512))
    want[7] *= 1e-6                                        # a near-zero row
    got = _bf16_noise(want, 2e-3, 6)
    got[7] += 1e-4 * rng.standard_normal(512)             # large relative, tiny absolute error
    hp.assert_close("near-zero row", got, want)
    errs = hp.row_errors(got, want)
    assert errs[7] < 1e-2 and errs.size == 200
    # a 1-D array: every element is its own row
    assert hp.row_errors(np.array([1.0, 2.0]), np.array([1.0, 2.1])).shape == (2,)


def test_chunked_oracle_equals_one_plain_call():
    w = inputs.Workload("chk", 9, T=45, H=16, num_kv=60, topk=24, selection="swa_pool", window=8,
                        pool_stride=2, pool_picks=16)
    x = inputs.make(w, sink=True)
    scale = 1.0 / math.sqrt(512)
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], scale)
    O64c, lse64c = hp.oracle_forward_chunked(x, chunk=7, workers=3)
    assert np.array_equal(O64, O64c) and np.array_equal(lse64, lse64c)
    x = dict(x)
    x["O"], x["lse"] = orc.emit_forward_outputs(O64, lse64)
    dlse = np.random.default_rng(1).standard_normal((w.T, w.H)).astype(np.float32)
    for dl in (None, dlse):
        ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], scale, dlse=dl)
        got = hp.oracle_backward_chunked(x, dlse=dl, chunk=7, workers=3)
        assert np.array_equal(got["dq"], ref["dq"])
        assert np.array_equal(got["delta"], ref["delta"])
        np.testing.assert_allclose(got["dkv"], ref["dkv"], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(got["d_sink"], ref["d_sink"], rtol=1e-12)


def test_chunked_oracle_with_positional_parts():
    w = inputs.Workload("chkpe", 10, T=30, H=16, num_kv=40, topk=16, selection="swa_pool", window=6,
                        pool_stride=2, pool_picks=10)
    x = dict(inputs.make(w, sink=True))
    x["q_pe"], x["k_pe"] = inputs.make_pe(w)
    x["scale"] = hp.SCALE_PE
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], x["scale"], q_pe=x["q_pe"], k_pe=x["k_pe"])
    O64c, lse64c = hp.oracle_forward_chunked(x, chunk=7, workers=3)
    assert np.array_equal(O64, O64c) and np.array_equal(lse64, lse64c)
    x["O"], x["lse"] = orc.emit_forward_outputs(O64, lse64)
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], x["scale"],
                       q_pe=x["q_pe"], k_pe=x["k_pe"])
    got = hp.oracle_backward_chunked(x, chunk=7, workers=3)
    assert np.array_equal(got["dq"], ref["dq"]) and np.array_equal(got["dq_pe"], ref["dq_pe"])
    for k in ("dkv", "dk_pe", "d_sink"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-13, err_msg=k)


@pytest.mark.parametrize("pe", [False, True])
def test_cancellation_bound_admits_fp32_reorderings_and_catches_a_dropped_delta(pe):
    """The bound for results that are zero only through cancellation: dq from an
    fp32 emulation in which dP and delta are summed in two different orders
    stays within it (exactly zero on masked tokens), the oracle's own result sits
    at its fp64 level, and a dS that drops delta, or takes it from a wrong row,
    lands far outside."""
    x = hp.single_slot_problem(24, 16, 40, pe, seed=71)
    ref = hp.oracle_backward_chunked(x, chunk=8, workers=2)
    b = hp.cancellation_bounds(x)
    keys = ("dq", "dq_pe", "dk_pe") if pe else ("dq",)
    for k in keys:
        assert np.all(np.abs(ref[k]) <= b[k] * 2.0 ** -29), k
    assert np.all(b["dq"][[3, 12]] == 0.0)
    kv = orc.bf16_to_f64(x["kv"]).astype(np.float32)
    dO = orc.bf16_to_f64(x["dO"]).astype(np.float32)
    O = orc.bf16_to_f64(x["O"]).astype(np.float32)
    j = np.clip(x["idx"][:, 0], 0, kv.shape[0] - 1)
    valid = (x["idx"][:, 0] >= 0) & (x["idx"][:, 0] < kv.shape[0])
    dP = np.einsum("thd,td->th", dO, kv[j]).astype(np.float32)              # one summation order
    delta = np.zeros(dO.shape[:2], dtype=np.float32)
    for d in range(511, -1, -1):                                             # another: sequential, reversed
        delta = (delta + dO[:, :, d] * O[:, :, d]).astype(np.float32)
    scale = np.float32(x["scale"])

    def dq_of(ds):
        ds = np.where(valid[:, None], ds, 0.0).astype(np.float32)
        return (scale * ds[:, :, None] * kv[j][:, None, :]).astype(np.float64)

    emul = dq_of(dP - delta)
    assert np.abs(emul).max() > 0.0                                          # the orders do differ
    hp.assert_cancellation_zero("fp32 emulation", emul, b["dq"])
    hp.assert_close_or_cancelled("fp32 emulation", emul, ref["dq"], x, "dq")
    assert b["dq"].max() < 1e-2
    for wrong in (dP, dP - np.roll(delta, 1, axis=0)):
        with pytest.raises(AssertionError, match="over the rounding bound"):
            hp.assert_cancellation_zero("planted", dq_of(wrong), b["dq"])
