"""GPU parity of the has_pe=True variant (positional parts q_pe, k_pe) against
the fp64 oracle, through the C ABI (smla_fwd_pe, smla_bwd_pe).

Bars as for the plain op: every row of dq, dq_pe, dkv, dk_pe and every head
of d_sink within the per-row bound, the whole tensors within rel-L2 5e-3 and
cosine 0.9999; lse within 1e-4.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import smla_oracle as orc
from sparse_mla_attention_smla_amd import inputs
from tests._helpers import (SCALE_PE, _with_forward, assert_close, assert_close_or_cancelled, dev, dev_bf16,
                            host_bf16, oracle_backward_chunked, single_slot_problem, workload_pe)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU only with -m gpu
    pytest.skip("no GPU", allow_module_level=True)

from sparse_mla_attention_smla_amd import binding as B  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x):
    d = {k: dev_bf16(x[k]) for k in ("q", "q_pe", "kv", "k_pe", "dO", "O")}
    d["idx"] = dev(x["idx"])
    d["lse"] = dev(x["lse"])
    d["sink"] = dev(x["sink"]) if x["sink"] is not None else None
    return d


def _bwd(d, x, dlse=None, **kw):
    out = B.smla_bwd_pe(d["q"], d["q_pe"], d["kv"], d["k_pe"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"],
                        x["scale"], dlse=None if dlse is None else dev(dlse), **kw)
    torch.cuda.synchronize()
    return out


def _check(label, x, ref, got):
    dq, dq_pe, dkv, dk_pe, ds = got[:5]
    for name, g, r in (("dq", dq, ref["dq"]), ("dq_pe", dq_pe, ref["dq_pe"]), ("dkv", dkv, ref["dkv"]),
                       ("dk_pe", dk_pe, ref["dk_pe"])):
        gh = host_bf16(g)
        if name == "dkv":
            if np.linalg.norm(r) == 0.0:                 # every token fully masked
                assert np.all(gh == 0.0), f"{label} {name}"
                continue
            res = assert_close(f"{label} {name}", gh, r)
        else:                                            # zero by cancellation with one slot per token
            res = assert_close_or_cancelled(f"{label} {name}", gh, r, x, name)
        if res is None:
            _say(f"[pe] {label}: {name} zero by cancellation, max |got| {np.abs(gh).max():.1e}")
        else:
            _say(f"[pe] {label}: {name} rel-L2 {res[0]:.2e} worst row {res[2]:.2e}")
    unused = np.linalg.norm(ref["dkv"], axis=1) == 0.0
    assert np.all(host_bf16(dkv)[unused] == 0.0) and np.all(host_bf16(dk_pe)[unused] == 0.0)
    if x["sink"] is not None:
        assert_close(f"{label} d_sink", ds.cpu().numpy(), ref["d_sink"])
    else:
        assert ds is None


@pytest.mark.parametrize("name,sink", [("tiny", True), ("small", True), ("small", False), ("mid", True),
                                       ("headline", True)])
def test_pe_backward_all_rows(name, sink):
    _say(f"[pe] {name} sink={sink}: inputs and the oracle forward")
    x = workload_pe(name, sink)
    d = _dev(x)
    got = _bwd(d, x, count_invalid=True)
    assert int(got[5].item()) == 0
    _say(f"[pe] {name}: oracle backward")
    ref = oracle_backward_chunked(x)
    _check(name, x, ref, got)
    # the positional term matters: without it the logits (and so dq) move far
    if name == "small":
        plain = orc.backward_tokens(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"],
                                    x["scale"], range(8, 16))
        assert np.linalg.norm(plain["dq"] - ref["dq"][8:16]) > 0.1 * np.linalg.norm(ref["dq"][8:16])
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["tiny", "small", "mid", "headline"])
def test_pe_forward_all_rows(name):
    x = workload_pe(name, True)
    o, lse = B.smla_fwd_pe(dev_bf16(x["q"]), dev_bf16(x["q_pe"]), dev_bf16(x["kv"]), dev_bf16(x["k_pe"]),
                           dev(x["idx"]), dev(x["sink"]), x["scale"])
    torch.cuda.synchronize()
    rl, c, worst = assert_close(f"{name} O (pe)", host_bf16(o), x["O64"])
    _say(f"[pe fwd] {name}: O rel-L2 {rl:.2e} worst row {worst:.2e}")
    got = lse.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - x["lse"].astype(np.float64))) < 1e-4


def _custom_pe(T, H, N, K, seed, sink=True, dup=False):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, N, size=(T, K)).astype(np.int32)
    if not dup:
        for t in range(T):
            n = int(rng.integers(0, min(K, N) + 1))
            row = np.full(K, -1, np.int32)
            row[:n] = np.sort(rng.choice(N, n, replace=False))
            idx[t] = row
    else:
        idx = np.where(rng.random((T, K)) < 0.25, -1, idx)
        bad = rng.random((T, K)) < 0.03
        idx = np.where(bad, np.where(rng.random((T, K)) < 0.5, -4, N + 7), idx).astype(np.int32)
    idx[min(2, T - 1)] = -1                         # an all-masked token
    s = 7000 + seed
    x = {"q": inputs.normal_bf16((T, H, 512), s, 1), "kv": inputs.normal_bf16((N, 512), s, 2),
         "dO": inputs.normal_bf16((T, H, 512), s, 3), "idx": idx,
         "q_pe": inputs.normal_bf16((T, H, 64), s, 5), "k_pe": inputs.normal_bf16((N, 64), s, 6),
         "sink": rng.standard_normal(H).astype(np.float32) if sink else None, "scale": SCALE_PE}
    return _with_forward(x)


@pytest.mark.parametrize("T,H,N,K,sink,dup,with_dlse", [
    (37, 48, 53, 40, True, False, False),    # a padded 48-head group, ragged tail tile
    (21, 32, 45, 64, False, True, True),     # slot-split 32 heads, duplicates / out of range, dlse
    (12, 64, 80, 600, True, True, False),    # topk beyond one index chunk
    (9, 128, 300, 96, True, False, True),    # most kv rows unused, dlse
    (17, 112, 30, 33, True, True, False),    # 7 head blocks of 16, 4 reduction steps with a half
    (13, 96, 70, 100, False, True, True),    # 96 heads: fused intermediate with 3 positional steps
])
def test_pe_ragged(T, H, N, K, sink, dup, with_dlse):
    _say(f"[pe ragged] T={T} H={H} N={N} K={K} sink={sink} dup={dup} dlse={with_dlse}")
    x = _custom_pe(T, H, N, K, seed=T * 100 + H, sink=sink, dup=dup)
    dlse = np.random.default_rng(T + K).standard_normal((T, H)).astype(np.float32) if with_dlse else None
    d = _dev(x)
    got = _bwd(d, x, dlse=dlse, count_invalid=True)
    assert int(got[5].item()) == orc.count_invalid(x["idx"], N)
    ref = oracle_backward_chunked(x, dlse=dlse, chunk=8)
    _check(f"ragged T={T} H={H} K={K}", x, ref, got)
    assert np.all(host_bf16(got[0])[min(2, T - 1)] == 0.0) and np.all(host_bf16(got[1])[min(2, T - 1)] == 0.0)
    o, lse = B.smla_fwd_pe(d["q"], d["q_pe"], d["kv"], d["k_pe"], d["idx"], d["sink"], x["scale"])
    torch.cuda.synchronize()
    assert_close("O (pe ragged)", host_bf16(o), x["O64"])
    got_l = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(x["lse"])
    assert np.array_equal(np.isfinite(got_l), fin)
    assert np.max(np.abs(got_l[fin] - x["lse"][fin].astype(np.float64)), initial=0.0) < 1e-4


def _fuzz_pe(seed):
    """A random has_pe=True problem: any H the library takes, topk up to two index
    chunks, slots drawn with replacement, -1 and out-of-range values anywhere;
    the odd seeds have hundreds of tokens, so persistent workgroups take several
    items and stream across them."""
    rng = np.random.default_rng([91, seed])
    T = int(rng.integers(300, 601)) if seed % 2 else int(rng.integers(1, 41))
    H = int(rng.choice([16, 32, 48, 64, 80, 96, 112, 128]))
    N = T + int(rng.integers(0, 160))
    K = int(rng.choice([1, 16, 33, 64, 200, 512, 513, 600] if seed % 2 == 0 else [64, 200, 512]))
    idx = rng.integers(0, N, size=(T, K)).astype(np.int32)
    idx = np.where(rng.random((T, K)) < 0.25, -1, idx)
    bad = rng.random((T, K)) < 0.02
    idx = np.where(bad, np.where(rng.random((T, K)) < 0.5, -3, N + 9), idx).astype(np.int32)
    s = 9000 + seed
    x = {"q": inputs.normal_bf16((T, H, 512), s, 1), "kv": inputs.normal_bf16((N, 512), s, 2),
         "dO": inputs.normal_bf16((T, H, 512), s, 3), "idx": idx,
         "q_pe": inputs.normal_bf16((T, H, 64), s, 5), "k_pe": inputs.normal_bf16((N, 64), s, 6),
         "sink": rng.standard_normal(H).astype(np.float32) if rng.integers(0, 2) else None,
         "scale": SCALE_PE}
    dlse = rng.standard_normal((T, H)).astype(np.float32) if rng.integers(0, 2) else None
    return _with_forward(x), dlse


@pytest.mark.parametrize("seed", range(8))
def test_pe_random_problems(seed):
    x, dlse = _fuzz_pe(seed)
    T, H, _ = x["q"].shape
    N, K = x["kv"].shape[0], x["idx"].shape[1]
    _say(f"[pe fuzz {seed}] T={T} H={H} N={N} K={K} sink={x['sink'] is not None} dlse={dlse is not None}")
    d = _dev(x)
    o, lse = B.smla_fwd_pe(d["q"], d["q_pe"], d["kv"], d["k_pe"], d["idx"], d["sink"], x["scale"])
    torch.cuda.synchronize()
    assert_close("O (pe fuzz)", host_bf16(o), x["O64"])
    got_l = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(x["lse"])
    assert np.array_equal(np.isfinite(got_l), fin)
    assert np.max(np.abs(got_l[fin] - x["lse"][fin].astype(np.float64)), initial=0.0) < 1e-4
    got = _bwd(d, x, dlse=dlse, count_invalid=True)
    assert int(got[5].item()) == orc.count_invalid(x["idx"], N)
    ref = oracle_backward_chunked(x, dlse=dlse, chunk=16)
    _check(f"pe fuzz {seed}", x, ref, got)
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("H", [16, 32, 64, 128])
def test_pe_single_slot_tokens_cancel(H):
    """One valid slot per token, no sink, no lse gradient: P = 1, so dq, dq_pe and
    dk_pe are zero only through cancellation of dP and delta (fp32 sums in
    different orders); each within its rounding bound, exactly zero on the masked
    tokens and unused rows; dkv (the value part) within the usual bars."""
    x = single_slot_problem(40, H, 50, True, seed=37)
    _say(f"[pe single slot] H={H}")
    got = _bwd(_dev(x), x)
    ref = oracle_backward_chunked(x, chunk=16)
    for i, name in ((0, "dq"), (1, "dq_pe"), (3, "dk_pe")):
        g = host_bf16(got[i])
        assert assert_close_or_cancelled(name, g, ref[name], x, name) is None
        _say(f"[pe single slot] H={H}: max |{name}| {np.abs(g).max():.1e}")
    assert np.all(host_bf16(got[0])[[3, 20]] == 0.0) and np.all(host_bf16(got[1])[[3, 20]] == 0.0)
    assert_close("dkv", host_bf16(got[2]), ref["dkv"])
    assert got[4] is None


def test_pe_autograd_function():
    """sparse_mla_pe under torch autograd: the loss <O, W> + <lse, V> gives the
    gradients of q, q_pe, kv, k_pe and sink matching the oracle backward with
    dO = W and dlse = V, on the O and lse the forward returned."""
    from tests._helpers import host_bits
    T, H, N, K = 29, 64, 50, 40
    rng = np.random.default_rng(17)
    idx = rng.integers(0, N, size=(T, K)).astype(np.int32)
    idx = np.where(rng.random((T, K)) < 0.3, -1, idx).astype(np.int32)
    s = 7100
    x = {"q": inputs.normal_bf16((T, H, 512), s, 1), "kv": inputs.normal_bf16((N, 512), s, 2),
         "q_pe": inputs.normal_bf16((T, H, 64), s, 5), "k_pe": inputs.normal_bf16((N, 64), s, 6),
         "idx": idx, "sink": rng.standard_normal(H).astype(np.float32)}
    W = inputs.normal_bf16((T, H, 512), s, 7)
    V = rng.standard_normal((T, H)).astype(np.float32)
    q, q_pe, kv, k_pe = (dev_bf16(x[k]).requires_grad_() for k in ("q", "q_pe", "kv", "k_pe"))
    sink = dev(x["sink"]).requires_grad_()
    o, lse = B.sparse_mla_pe(q, q_pe, kv, k_pe, dev(idx), sink, SCALE_PE)
    ((o.float() * dev_bf16(W).float()).sum() + (lse * dev(V)).sum()).backward()
    torch.cuda.synchronize()
    ref = orc.backward(x["q"], x["kv"], W, host_bits(o.detach()), lse.detach().cpu().numpy(), idx, x["sink"],
                       SCALE_PE, dlse=V, q_pe=x["q_pe"], k_pe=x["k_pe"])
    for name, g in (("dq", q.grad), ("dq_pe", q_pe.grad), ("dkv", kv.grad), ("dk_pe", k_pe.grad)):
        rl, _, worst = assert_close(f"autograd {name}", host_bf16(g), ref[name])
        _say(f"[pe autograd] {name}: rel-L2 {rl:.2e} worst row {worst:.2e}")
    assert_close("autograd d_sink", sink.grad.cpu().numpy(), ref["d_sink"])


@pytest.mark.parametrize("H", [16, 32, 48, 80])
def test_pe_full_rows_other_head_counts(H):
    """has_pe=True at 16 and 32 heads (slot-split producers), 48 and 80 (a padded
    last group; with 16 and 48 the intermediate's last positional step is half
    dS rows, half zeros), 700 tokens, so persistent workgroups stream across
    items: every row of dq, dq_pe, dkv, dk_pe and d_sink, and the forward's O
    and lse."""
    w = inputs.Workload(f"pe_h{H}", 60 + H // 16, T=700, H=H, num_kv=875, topk=512, selection="swa_pool",
                        window=128, pool_stride=4, pool_picks=384)
    x = dict(inputs.make(w, sink=True))
    x["q_pe"], x["k_pe"] = inputs.make_pe(w)
    x["scale"] = SCALE_PE
    x = _with_forward(x)
    _say(f"[pe rows] H={H}: T={w.T}")
    d = _dev(x)
    got = _bwd(d, x)
    ref = oracle_backward_chunked(x)
    _check(f"H={H} T={w.T}", x, ref, got)
    o, lse = B.smla_fwd_pe(d["q"], d["q_pe"], d["kv"], d["k_pe"], d["idx"], d["sink"], x["scale"])
    torch.cuda.synchronize()
    assert_close("O", host_bf16(o), x["O64"])
    fin = np.isfinite(x["lse"])
    assert np.max(np.abs(lse.cpu().numpy().astype(np.float64)[fin] - x["lse"][fin].astype(np.float64))) < 1e-4


@pytest.mark.parametrize("H", [128, 48, 32])
def test_pe_topk_beyond_one_chunk_many_items(H):
    """has_pe=True with topk 1100 on 600 tokens (duplicates, -1 and out-of-range
    slots in every index chunk): each persistent workgroup takes several items
    of three segments, in the dQ stream and in the multi-chunk forward (48
    heads: a padded group; 32: the slot-split dQ).  Every row of O, lse, dq, dq_pe, dkv, dk_pe and
    d_sink against the oracle."""
    T, N, K = 600, 900, 1100
    x = _custom_pe(T, H, N, K, seed=11 * H, sink=True, dup=True)
    _say(f"[pe topk>512 many] T={T} H={H} N={N} K={K}")
    d = _dev(x)
    o, lse = B.smla_fwd_pe(d["q"], d["q_pe"], d["kv"], d["k_pe"], d["idx"], d["sink"], x["scale"])
    torch.cuda.synchronize()
    r, _, worst = assert_close("O (pe topk>512)", host_bf16(o), x["O64"])
    _say(f"[pe topk>512 many] H={H}: O rel-L2 {r:.2e} worst row {worst:.2e}")
    got_l = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(x["lse"])
    assert np.array_equal(np.isfinite(got_l), fin)
    assert np.max(np.abs(got_l[fin] - x["lse"][fin].astype(np.float64)), initial=0.0) < 1e-4
    got = _bwd(d, x)
    ref = oracle_backward_chunked(x, chunk=16)
    _check(f"topk>512 T={T} H={H}", x, ref, got)
    del d
    torch.cuda.empty_cache()


def test_pe_full_rows_past_4gib_of_intermediate():
    """has_pe=True on 16384 tokens of 16 heads: the intermediate holds 8 GiB, so
    the later tokens' intermediate rows, dS/P blocks and slot ids sit past 2^32
    bytes (as in the plain test of that shape), and the positional intermediate
    (1 GiB), dq_pe and the positional gather address those tokens too: every row
    of dq, dq_pe, dkv, dk_pe and d_sink against the oracle."""
    w = inputs.Workload("pe_t16384_h16", 70, T=16384, H=16, num_kv=20480, topk=512, selection="swa_pool",
                        window=128, pool_stride=4, pool_picks=384)
    x = dict(inputs.make(w, sink=True))
    x["q_pe"], x["k_pe"] = inputs.make_pe(w)
    x["scale"] = SCALE_PE
    x = _with_forward(x)
    _say(f"[pe rows] T={w.T} H={w.H}")
    got = _bwd(_dev(x), x)
    _say(f"[pe rows] T={w.T}: oracle backward over all tokens")
    ref = oracle_backward_chunked(x)
    _check(f"T={w.T} H={w.H}", x, ref, got)
    torch.cuda.empty_cache()


def test_pe_zero_positional_parts_equal_the_plain_backward():
    """q_pe = 0: every logit is the plain one, so smla_bwd_pe must give smla_bwd's
    dq, dkv and d_sink (the plain call may take another dQ kernel, so up to
    rounding) and an exactly zero dk_pe."""
    x = dict(workload_pe("small", True))
    T, H, _ = x["q"].shape
    d = _dev(x)
    d["q_pe"] = torch.zeros_like(d["q_pe"])
    got = _bwd(d, x)
    want = B.smla_bwd(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"], x["scale"])
    torch.cuda.synchronize()
    for a, b, name in ((got[0], want[0], "dq"), (got[2], want[1], "dkv")):
        rl, _, _ = assert_close(f"{name} (q_pe = 0 vs plain)", host_bf16(a), host_bf16(b), tol=1e-3)
        same = float((a.view(torch.int16) == b.view(torch.int16)).float().mean())
        _say(f"[pe zero] {name}: rel-L2 {rl:.1e} vs the plain backward, {100 * same:.2f}% bit-equal")
    assert_close("d_sink (q_pe = 0 vs plain)", got[4].cpu().numpy(), want[2].cpu().numpy(), tol=1e-6)
    assert torch.all(got[3].float() == 0)


def test_pe_deterministic_and_graph_replays_match_eager():
    """smla_bwd_pe twice gives the same bits; captured in a HIP graph (with its
    helper-stream work folded onto the capturing stream), three replays with
    eager work in between equal the eager call bit for bit."""
    x = workload_pe("small", True)
    d = _dev(x)
    T, H, _ = x["q"].shape
    N, K = x["kv"].shape[0], x["idx"].shape[1]
    ws = torch.empty((B.bwd_pe_workspace_bytes(T, H, N, K),), dtype=torch.uint8, device="cuda")
    first = _bwd(d, x, workspace=ws)
    second = _bwd(d, x, workspace=ws)
    for a, b, name in zip(first[:4], second[:4], ("dq", "dq_pe", "dkv", "dk_pe")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs between runs"
    assert torch.equal(first[4], second[4])
    outs = (torch.empty_like(d["q"]), torch.empty_like(d["q_pe"]), torch.empty_like(d["kv"]),
            torch.empty_like(d["k_pe"]), torch.empty_like(d["sink"]))

    def call():
        B.smla_bwd_pe(d["q"], d["q_pe"], d["kv"], d["k_pe"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"],
                      x["scale"], workspace=ws, out=outs)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up call on the capture stream, outside capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(0)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b, name in zip(outs[:4], first[:4], ("dq", "dq_pe", "dkv", "dk_pe")):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}: {name}"
        assert torch.equal(outs[4], first[4]), f"replay {rep}: d_sink"
