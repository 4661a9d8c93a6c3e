"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Every call goes through the C ABI (libsmla.so via the ctypes binding).  Inputs
are the seeded workloads; O and lse come from the oracle forward, rounded the
way the backward consumes them.  Bars: the CSR is bit-exact; dq, dkv, d_sink
(and the bf16 stage tensors) within rel-L2 5e-3 and cosine 0.9999 of the oracle.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

from oracle import smla_oracle as orc
from sparse_mla_attention_smla_amd import inputs
from tests._helpers import (SCALE, _with_forward, assert_close, assert_close_or_cancelled, dev, dev_bf16,
                            dsp_from_logical, dsp_map, dsp_to_logical, full_reference, host_bf16, host_bits,
                            oracle_backward_chunked, rel_l2, single_slot_problem, workload, workload_nosink)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU only with -m gpu
    pytest.skip("no GPU", allow_module_level=True)

from sparse_mla_attention_smla_amd import binding as B  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _to_dev(x):
    d = {k: dev_bf16(x[k]) for k in ("q", "kv", "dO", "O")}
    d["idx"] = dev(x["idx"])
    d["lse"] = dev(x["lse"])
    d["sink"] = dev(x["sink"]) if x["sink"] is not None else None
    return d


def _run_bwd(d, **kw):
    out = B.smla_bwd(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"], SCALE, **kw)
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------------------
# small workloads: full oracle, stage by stage
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module", params=["tiny", "small", "small_nosink"])
def small_case(request):
    name = request.param
    x = workload_nosink("small") if name == "small_nosink" else workload(name)
    _say(f"[case] {name}: T={x['q'].shape[0]} H={x['q'].shape[1]} topk={x['idx'].shape[1]}")
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE,
                       stages=True)
    return name, x, ref, _to_dev(x)


def test_end_to_end(small_case):
    name, x, ref, d = small_case
    dq, dkv, ds = _run_bwd(d)
    assert_close(f"{name} dq", host_bf16(dq), ref["dq"])
    assert_close(f"{name} dkv", host_bf16(dkv), ref["dkv"])
    if x["sink"] is not None:
        assert_close(f"{name} d_sink", ds.cpu().numpy(), ref["d_sink"])
    else:
        assert ds is None


def test_stage_delta(small_case):
    name, x, ref, d = small_case
    delta = B.smla_delta(d["O"], d["dO"])
    torch.cuda.synchronize()
    assert rel_l2(delta.cpu().numpy(), ref["delta"]) < 1e-5
    dlse = inputs.make_dlse(name.replace("_nosink", ""))
    shifted = B.smla_delta(d["O"], d["dO"], dlse=dev(dlse))
    torch.cuda.synchronize()
    assert rel_l2(shifted.cpu().numpy(), ref["delta"] - dlse) < 1e-5


def test_end_to_end_with_dlse(small_case):
    """An upstream gradient of lse: dS gains P*dlse, d_sink gains P_sink*dlse."""
    name, x, ref, d = small_case
    dlse = inputs.make_dlse(name.replace("_nosink", ""))
    want = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE,
                        dlse=dlse)
    dq, dkv, ds = _run_bwd(d, dlse=dev(dlse))
    assert_close(f"{name} dq (dlse)", host_bf16(dq), want["dq"])
    assert_close(f"{name} dkv (dlse)", host_bf16(dkv), want["dkv"])
    if x["sink"] is not None:
        assert_close(f"{name} d_sink (dlse)", ds.cpu().numpy(), want["d_sink"])
    # the term is not negligible: it moves dq by several times the tolerance
    assert rel_l2(want["dq"], ref["dq"]) > 4 * 5e-3


def test_stage_dq_and_dsp(small_case):
    name, x, ref, d = small_case
    delta = dev(ref["delta"].astype(np.float32))
    T, K = x["idx"].shape
    H = x["q"].shape[1]
    # blocks past a token's last tile are never written: fill the buffer with 1.0
    # first, so they hold finite values and an unwritten tail column would show
    dsp_buf = torch.full((B.dsp_numel(T, H, K),), 1.0, dtype=torch.bfloat16, device="cuda")
    dq, dsp = B.smla_dq(d["q"], d["kv"], d["dO"], d["lse"], delta, d["idx"], SCALE, dsp=dsp_buf)
    torch.cuda.synchronize()
    assert_close(f"{name} dq stage", host_bf16(dq), ref["dq"])
    ntk = (K + 31) // 32
    got = dsp_to_logical(host_bf16(dsp), H).reshape(T, ntk, 2 * H, 32)
    t, b, c, k = dsp_map(x["idx"], x["kv"].shape[0])
    got_ds = got[t, b, :H, c]                              # [nnz, H]
    got_p = got[t, b, H:, c]
    assert_close(f"{name} scale*dS", got_ds, SCALE * ref["dS"][t, :, k])
    assert_close(f"{name} P", got_p, ref["P"][t, :, k])
    # tail columns of each token's last block of a run are exact zeros
    filled = np.zeros((T, ntk, 32), bool)
    filled[t, b, c] = True
    used = np.zeros((T, ntk), bool)
    used[t, b] = True
    tail = used[:, :, None] & ~filled
    assert np.all(got.transpose(0, 1, 3, 2)[tail] == 0.0)


def test_stage_interm(small_case):
    name, x, ref, d = small_case
    H = x["q"].shape[1]
    T, K = x["idx"].shape
    N = x["kv"].shape[0]
    # dS/P blocks built from the oracle's P and dS (rounded to bf16 as consumed)
    ntk = (K + 31) // 32
    t, b, c, k = dsp_map(x["idx"], N)
    blocks = np.zeros((T, ntk, 2 * H, 32))
    blocks[t, b, :H, c] = SCALE * ref["dS"][t, :, k]
    blocks[t, b, H:, c] = ref["P"][t, :, k]
    bits = orc.f64_to_bf16_rne(blocks)
    interm = B.smla_interm(d["q"], d["dO"], dev_bf16(dsp_from_logical(bits, H)), d["idx"], N)
    torch.cuda.synchronize()
    got = host_bf16(interm).reshape(T, K, 512)
    blk64 = orc.bf16_to_f64(bits)
    dsk = blk64[t, b, :H, c]                               # [nnz, H]
    pk = blk64[t, b, H:, c]
    q64, dO64 = orc.bf16_to_f64(x["q"]), orc.bf16_to_f64(x["dO"])
    want = np.einsum("nh,nhd->nd", dsk, q64[t]) + np.einsum("nh,nhd->nd", pk, dO64[t])
    assert_close(f"{name} interm", got[t, k], want)
    # and against the oracle's own interm (through the rounded blocks)
    assert_close(f"{name} interm vs oracle", got[t, k], ref["interm"][t, k])


def test_stage_csr_bit_exact(small_case):
    name, x, ref, d = small_case
    N = x["kv"].shape[0]
    row_ptr, slots, n_inv = B.smla_build_csr(d["idx"], N, count_invalid=True)
    torch.cuda.synchronize()
    rp, sl = orc.csr(x["idx"], N)
    assert np.array_equal(row_ptr.cpu().numpy(), rp)
    assert np.array_equal(slots.cpu().numpy()[: rp[-1]], sl)
    assert int(n_inv.item()) == orc.count_invalid(x["idx"], N)


def test_stage_gather(small_case):
    name, x, ref, d = small_case
    T, K = x["idx"].shape
    N = x["kv"].shape[0]
    interm_bits = orc.f64_to_bf16_rne(ref["interm"])          # oracle interm, rounded
    rp, sl = orc.csr(x["idx"], N)
    dkv = B.smla_gather(dev_bf16(interm_bits.reshape(T * K, 512)), dev(rp), dev(sl), T, K, N)
    torch.cuda.synchronize()
    want = orc.dkv_from_interm(interm_bits, x["idx"], N)
    assert_close(f"{name} gather", host_bf16(dkv), want, tol=3e-3)
    unused = np.setdiff1d(np.arange(N), x["idx"][x["idx"] >= 0])
    assert np.all(host_bf16(dkv)[unused] == 0.0)


def test_stage_dsink(small_case):
    name, x, ref, d = small_case
    if x["sink"] is None:
        pytest.skip("no sink in this case")
    ds = B.smla_dsink(d["lse"], dev(ref["delta"].astype(np.float32)), d["sink"])
    torch.cuda.synchronize()
    assert rel_l2(ds.cpu().numpy(), ref["d_sink"]) < 1e-4


def host_bits_t(t):
    return t.view(torch.int16)


def test_deterministic_and_poisoned_workspace(small_case):
    name, x, ref, d = small_case
    T, H, _ = x["q"].shape
    N, K = x["kv"].shape[0], x["idx"].shape[1]
    ws = torch.full((B.bwd_workspace_bytes(T, H, N, K),), 0xFF, dtype=torch.uint8, device="cuda")
    a = _run_bwd(d, workspace=ws)
    ws.fill_(0x00)
    b = _run_bwd(d, workspace=ws)
    ws.fill_(0x7F)
    c = _run_bwd(d, workspace=ws)
    for i in range(2):
        assert torch.equal(host_bits_t(a[i]), host_bits_t(b[i])) and torch.equal(host_bits_t(a[i]), host_bits_t(c[i]))
    if a[2] is not None:
        assert torch.equal(a[2], b[2]) and torch.equal(a[2], c[2])


def test_timed_call_equals_plain_call(small_case):
    """smla_bwd_timed does the same work as smla_bwd (bit for bit) and records its
    five stage events in order on the call's stream."""
    name, x, ref, d = small_case
    a = _run_bwd(d)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    b = _run_bwd(d, events=evs)
    for i in range(2):
        assert torch.equal(host_bits_t(a[i]), host_bits_t(b[i]))
    if a[2] is not None:
        assert torch.equal(a[2], b[2])
    spans = [evs[k].elapsed_time(evs[k + 1]) for k in range(4)]
    assert all(t >= 0.0 for t in spans), spans
    assert spans[1] > 0.0                                   # dQ ran between events 1 and 2


def test_concurrent_calls_from_two_threads(small_case):
    """Two host threads, each on its own stream, call smla_bwd at the same time
    (the enqueues share the library's helper stream); both results must equal
    the single-threaded ones bit for bit."""
    import threading
    name, x, ref, d = small_case
    want = _run_bwd(d)
    d2 = dict(d)
    d2["dO"] = (d["dO"].float() * -0.5).bfloat16()
    want2 = _run_bwd(d2)
    out = {}

    def work(key, dd):
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            for _ in range(3):
                r = B.smla_bwd(dd["q"], dd["kv"], dd["dO"], dd["O"], dd["lse"], dd["idx"], dd["sink"], SCALE)
            st.synchronize()
        out[key] = r

    th = [threading.Thread(target=work, args=(k, dd)) for k, dd in (("a", d), ("b", d2))]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    for key, w in (("a", want), ("b", want2)):
        for i in range(2):
            assert torch.equal(host_bits_t(out[key][i]), host_bits_t(w[i])), (key, i)
        if w[2] is not None:
            assert torch.equal(out[key][2], w[2]), key


def test_graph_capture_replays_match_eager(small_case):
    """smla_bwd (including its fork to the helper stream and the join back) is
    captured into a graph; every replay, with eager work and synchronisations in
    between, must equal the eager call bit for bit (the results are
    deterministic, so equality is the right bar)."""
    name, x, ref, d = small_case
    T, H, _ = x["q"].shape
    N, K = x["kv"].shape[0], x["idx"].shape[1]
    ws = torch.empty((B.bwd_workspace_bytes(T, H, N, K),), dtype=torch.uint8, device="cuda")
    eager = _run_bwd(d, workspace=ws)
    dq = torch.empty_like(d["q"])
    dkv = torch.empty_like(d["kv"])
    ds = torch.empty_like(d["sink"]) if d["sink"] is not None else None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up call on the capture stream, outside capture
        B.smla_bwd(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"], SCALE,
                   workspace=ws, out=(dq, dkv, ds))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.smla_bwd(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"], SCALE,
                   workspace=ws, out=(dq, dkv, ds))
    torch.cuda.synchronize()
    for rep in range(3):
        dq.fill_(0); dkv.fill_(0)       # eager work between replays
        if ds is not None:
            ds.fill_(0)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(host_bits_t(dq), host_bits_t(eager[0])), f"replay {rep}: dq"
        assert torch.equal(host_bits_t(dkv), host_bits_t(eager[1])), f"replay {rep}: dkv"
        if ds is not None:
            assert torch.equal(ds, eager[2]), f"replay {rep}: d_sink"


def test_capture_on_one_thread_while_another_calls_eagerly(small_case):
    """Thread A captures smla_bwd into a graph (the call then stays on the capture
    stream); while that capture is open, thread B makes eager calls on its own
    stream (which use the library's helper stream).  B's results and every
    replay of A's graph must equal the single-threaded eager results bit for bit."""
    import threading
    name, x, ref, d = small_case
    T, H, _ = x["q"].shape
    N, K = x["kv"].shape[0], x["idx"].shape[1]
    want = _run_bwd(d)
    d2 = dict(d)
    d2["dO"] = (d["dO"].float() * 0.75).bfloat16()
    want2 = _run_bwd(d2)
    nbytes = B.bwd_workspace_bytes(T, H, N, K)
    ws_a = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    out_a = (torch.empty_like(d["q"]), torch.empty_like(d["kv"]),
             torch.empty_like(d["sink"]) if d["sink"] is not None else None)
    out_b = (torch.empty_like(d["q"]), torch.empty_like(d["kv"]),
             torch.empty_like(d["sink"]) if d["sink"] is not None else None)
    stream_b = torch.cuda.Stream()
    torch.cuda.synchronize()
    in_capture, b_done = threading.Event(), threading.Event()
    errors = []

    def thread_b():
        try:
            assert in_capture.wait(60)
            with torch.cuda.stream(stream_b):
                for _ in range(3):
                    B.smla_bwd(d2["q"], d2["kv"], d2["dO"], d2["O"], d2["lse"], d2["idx"], d2["sink"], SCALE,
                               workspace=ws_b, out=out_b)
            stream_b.synchronize()
        except BaseException as e:     # reported by the main thread
            errors.append(e)
        finally:
            b_done.set()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):     # warm-up outside capture
        B.smla_bwd(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"], SCALE,
                   workspace=ws_a, out=out_a)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    tb = threading.Thread(target=thread_b)
    tb.start()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        B.smla_bwd(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"], SCALE,
                   workspace=ws_a, out=out_a)
        in_capture.set()
        assert b_done.wait(120), "thread B did not finish"
    tb.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.equal(host_bits_t(out_b[i]), host_bits_t(want2[i])), ("B", i)
    if want2[2] is not None:
        assert torch.equal(out_b[2], want2[2])
    for rep in range(3):
        out_a[0].fill_(0); out_a[1].fill_(0)
        ws_a.fill_(0x11)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(host_bits_t(out_a[i]), host_bits_t(want[i])), (rep, i)
        if want[2] is not None:
            assert torch.equal(out_a[2], want[2]), rep


def test_two_captures_open_at_once_and_two_calls_in_one_capture(small_case):
    """Two threads each capture smla_bwd into their own graph while the other's
    capture is open (each capture gets its own helper stream); thread A's graph
    holds two calls (the second reuses the helper its capture already joined).
    Every replay equals the eager results bit for bit."""
    import threading
    name, x, ref, d = small_case
    T, H, _ = x["q"].shape
    N, K = x["kv"].shape[0], x["idx"].shape[1]
    d2 = dict(d)
    d2["dO"] = (d["dO"].float() * 0.75).bfloat16()
    want = (_run_bwd(d), _run_bwd(d2))
    nbytes = B.bwd_workspace_bytes(T, H, N, K)
    ws = [torch.empty((nbytes,), dtype=torch.uint8, device="cuda") for _ in range(3)]

    def outs():
        return (torch.empty_like(d["q"]), torch.empty_like(d["kv"]),
                torch.empty_like(d["sink"]) if d["sink"] is not None else None)
    out = [outs() for _ in range(3)]         # A: calls 0 (inputs d) and 1 (d2); B: call 2 (d2)
    args = [d, d2, d2]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for i in range(3):                        # warm-up outside capture
        with torch.cuda.stream(streams[0]):
            a = args[i]
            B.smla_bwd(a["q"], a["kv"], a["dO"], a["O"], a["lse"], a["idx"], a["sink"], SCALE,
                       workspace=ws[i], out=out[i])
    torch.cuda.synchronize()
    graphs = [torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()]
    barrier = threading.Barrier(2, timeout=120)
    errors = []

    def capture(k, calls):
        # capture_begin/capture_end directly: the torch.cuda.graph context manager
        # synchronises the device on entry, which another thread's open capture forbids
        try:
            with torch.cuda.stream(streams[k]):
                graphs[k].capture_begin(capture_error_mode="thread_local")
                try:
                    barrier.wait()           # both captures are open from here
                    for i in calls:
                        a = args[i]
                        B.smla_bwd(a["q"], a["kv"], a["dO"], a["O"], a["lse"], a["idx"], a["sink"], SCALE,
                                   workspace=ws[i], out=out[i])
                    barrier.wait()           # ... until both have enqueued their calls
                finally:
                    graphs[k].capture_end()
        except BaseException as e:
            errors.append(e)
            barrier.abort()

    ta = threading.Thread(target=capture, args=(0, (0, 1)))
    tb = threading.Thread(target=capture, args=(1, (2,)))
    ta.start(); tb.start()
    ta.join(180); tb.join(180)
    assert not ta.is_alive() and not tb.is_alive(), "capture threads did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for rep in range(3):
        for o in out:
            o[0].fill_(0); o[1].fill_(0)
        for w in ws:
            w.fill_(0x3C)
        torch.cuda.synchronize()
        graphs[rep % 2].replay()
        graphs[(rep + 1) % 2].replay()
        torch.cuda.synchronize()
        for i, wi in ((0, 0), (1, 1), (2, 1)):
            for k in range(2):
                assert torch.equal(host_bits_t(out[i][k]), host_bits_t(want[wi][k])), (rep, i, k)
            if want[wi][2] is not None:
                assert torch.equal(out[i][2], want[wi][2]), (rep, i)


def test_binding_rejects_bad_outputs_and_workspaces():
    """Wrongly shaped, typed or placed outputs and workspaces raise before anything
    is enqueued; a workspace smaller than needed is reported by the library itself
    (the binding passes the buffer's real size)."""
    x = _to_dev(_oracle_inputs(_custom(8, 16, 8, 16, seed=2)))
    args = (x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE)
    dq, dkv, ds = torch.empty_like(x["q"]), torch.empty_like(x["kv"]), torch.empty_like(x["sink"])
    with pytest.raises(ValueError, match="dq must have shape"):
        B.smla_bwd(*args, out=(dq[:4], dkv, ds))
    with pytest.raises(TypeError, match="dkv must be"):
        B.smla_bwd(*args, out=(dq, dkv.float(), ds))
    with pytest.raises(ValueError, match="contiguous"):
        B.smla_bwd(*args, out=(dq, torch.empty(512, 8, dtype=torch.bfloat16, device="cuda").t(), ds))
    with pytest.raises(ValueError, match="d_sink must be given"):
        B.smla_bwd(*args, out=(dq, dkv, None))
    with pytest.raises(ValueError, match="dq must have shape"):
        B.smla_bwd_phased(*args, phase_tokens=4, out=(dq[:4], dkv, ds))
    with pytest.raises(TypeError, match="workspace must be"):
        B.smla_bwd(*args, workspace=torch.empty(1 << 20, dtype=torch.float32, device="cuda"))
    small_ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    for call in (lambda: B.smla_bwd(*args, workspace=small_ws),
                 lambda: B.smla_bwd_phased(*args, phase_tokens=4, workspace=small_ws),
                 lambda: B.smla_build_csr(x["idx"], 8, workspace=small_ws),
                 lambda: B.smla_dsink(x["lse"], torch.zeros_like(x["lse"]), x["sink"],
                                      workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))):
        with pytest.raises(B.SmlaError) as e:
            call()
        assert e.value.status == 4
    rp, sl = B.smla_build_csr(x["idx"], 8)
    interm = torch.zeros((8 * 16, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.SmlaError) as e:
        B.smla_gather(interm, rp, sl, 8, 16, 8, workspace=small_ws[:1])
    assert e.value.status == 4
    with pytest.raises(ValueError, match="slots holds"):
        B.smla_build_csr(x["idx"], 8, out=(torch.empty(9, dtype=torch.int32, device="cuda"),
                                           torch.empty(5, dtype=torch.int32, device="cuda")))
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# forward (test-input producer)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,sink", [("tiny", True), ("small", True), ("small", False)])
def test_forward_matches_oracle(name, sink):
    x = inputs.make(name, sink=sink)
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], SCALE)
    s = dev(x["sink"]) if sink else None
    o, lse = B.smla_fwd(dev_bf16(x["q"]), dev_bf16(x["kv"]), dev(x["idx"]), s, SCALE)
    torch.cuda.synchronize()
    assert_close(f"{name} O", host_bf16(o), O64)
    got = lse.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - lse64)) < 1e-4


@pytest.mark.parametrize("T,H,N,K,sink", [
    (40, 64, 70, 512, True),    # one full 512-slot chunk, ragged last tile, empty rows
    (23, 128, 60, 33, False),   # two 64-head groups, 2 tiles per token, no sink
    (50, 64, 50, 1, True),      # topk = 1: every token has at most one tile
    (9, 64, 300, 96, True),     # most kv rows unused
    (19, 32, 19, 16, True),     # 32 heads: a padded group of two 16-head blocks
    (21, 96, 45, 64, False),    # 96 heads: a full group and a padded one, no sink
    (25, 48, 33, 40, True),     # 48 heads: a padded group of three blocks
    (12, 64, 80, 600, True),    # topk beyond one index chunk: the multi-segment persistent forward
])
def test_forward_ragged(T, H, N, K, sink):
    x = _custom(T, H, N, K, seed=7 * T + H, sink=sink, pool_frac=0.5)
    if K > 512:
        x["idx"] = inputs.shuffle_slots(x["idx"], seed=T + K)   # valid slots in both chunks
    x["idx"][2] = -1                                    # an all-masked token
    _say(f"[fwd ragged] T={T} H={H} N={N} K={K} sink={sink}")
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], SCALE)
    s = dev(x["sink"]) if sink else None
    o, lse = B.smla_fwd(dev_bf16(x["q"]), dev_bf16(x["kv"]), dev(x["idx"]), s, SCALE)
    torch.cuda.synchronize()
    got_o = host_bf16(o)
    assert_close("O", got_o, O64)
    got = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse64)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.max(np.abs(got[fin] - lse64[fin])) < 1e-4
    assert np.all(got_o[2] == 0.0)
    if sink:
        # no valid slot: lse is the sink (to fp32 rounding of the log2-domain round trip)
        np.testing.assert_allclose(got[2], x["sink"].astype(np.float64), rtol=1e-6, atol=1e-7)


def test_forward_rising_logits_rescale_path():
    """Logits that grow along the slot order by far more than the lazy-rescale
    threshold for some heads (every tile moves the reference max), stay flat or
    fall for others: both the rescaled and the untouched accumulators must
    match the oracle."""
    T, H, N, K = 6, 64, 520, 512
    rng = np.random.default_rng(17)
    u = rng.standard_normal(512)
    a = np.linspace(-1.0, 1.5, H)                      # per-head slope of the logits
    q = np.stack([a[:, None] * u[None, :]] * T)        # [T,H,512]
    kv = (np.arange(N)[:, None] / 64.0) * u[None, :] + 0.05 * rng.standard_normal((N, 512))
    idx = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    idx[1, 300:] = -1
    idx[3] = np.sort(rng.choice(N, K, replace=False)).astype(np.int32)
    qb, kvb = orc.f64_to_bf16_rne(q), orc.f64_to_bf16_rne(kv)
    sink = rng.standard_normal(H).astype(np.float32)
    O64, lse64 = orc.forward(qb, kvb, idx, sink, SCALE)
    o, lse = B.smla_fwd(dev_bf16(qb), dev_bf16(kvb), dev(idx), dev(sink), SCALE)
    torch.cuda.synchronize()
    assert_close("O (rising logits)", host_bf16(o), O64)
    got = lse.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - lse64) / np.maximum(1.0, np.abs(lse64))) < 1e-5


@pytest.mark.parametrize("name", ["headline", "mid"])
def test_forward_full_size_all_rows(name):
    """The forward in the benchmark's launch configuration, every (t, h) row of O
    and every lse against the oracle forward."""
    x = workload(name)
    _say(f"[fwd full] {name}")
    o, lse = B.smla_fwd(dev_bf16(x["q"]), dev_bf16(x["kv"]), dev(x["idx"]), dev(x["sink"]), SCALE)
    torch.cuda.synchronize()
    r, c, worst = assert_close(f"{name} O", host_bf16(o), x["O64"])
    _say(f"[fwd full] {name}: O rel-L2 {r:.2e}, worst row {worst:.2e}")
    got = lse.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - x["lse"].astype(np.float64))) < 1e-4


# ---------------------------------------------------------------------------
# edge cases: ragged shapes, masks, empty inputs
# ---------------------------------------------------------------------------

def _custom(T, H, N, K, seed, sink=True, pool_frac=0.0):
    rng = np.random.default_rng(seed)
    idx = np.full((T, K), -1, dtype=np.int32)
    for t in range(T):
        n = int(rng.integers(0, K + 1))
        cand = np.arange(min(N, max(1, t + 1 + int(pool_frac * (N - T)))))
        n = min(n, cand.size)
        idx[t, :n] = np.sort(rng.choice(cand, n, replace=False))
    x = {"q": inputs.normal_bf16((T, H, 512), seed, 1), "kv": inputs.normal_bf16((N, 512), seed, 2),
         "dO": inputs.normal_bf16((T, H, 512), seed, 3), "idx": idx,
         "sink": rng.standard_normal(H).astype(np.float32) if sink else None}
    return x


def _oracle_inputs(x):
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], SCALE)
    x["O"], x["lse"] = orc.emit_forward_outputs(O64, lse64)
    return x


@pytest.mark.parametrize("T,H,N,K,sink,with_dlse", [
    (37, 48, 53, 40, True, False),    # 3-wave head groups, ragged 32-slot tail, pool rows
    (20, 32, 20, 1, True, False),     # topk = 1
    (33, 80, 40, 70, False, False),   # 1-wave head groups, no sink
    (17, 112, 30, 33, True, False),
    (9, 128, 300, 96, True, False),   # most kv rows unused
    (21, 96, 45, 64, True, False),    # 6 reduction steps in the intermediate, 2-wave dQ blocks
    (37, 48, 53, 40, True, True),     # with dlse: the all-masked row gets P_sink = 1
    (33, 80, 40, 70, False, True),    # with dlse, no sink: the all-masked row stays zero
])
def test_ragged_shapes(T, H, N, K, sink, with_dlse):
    x = _custom(T, H, N, K, seed=T * 1000 + H, sink=sink, pool_frac=0.5)
    x["idx"][3] = -1                                    # one all-masked row
    x = _oracle_inputs(x)
    _say(f"[ragged] T={T} H={H} N={N} K={K} sink={sink} dlse={with_dlse}")
    dlse = (np.random.default_rng(T + H).standard_normal((T, H)).astype(np.float32)
            if with_dlse else None)
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE,
                       dlse=dlse)
    dq, dkv, ds = _run_bwd(_to_dev(x), dlse=None if dlse is None else dev(dlse))
    assert_close("dq", host_bf16(dq), ref["dq"])
    assert_close("dkv", host_bf16(dkv), ref["dkv"])
    assert np.all(host_bf16(dq)[3] == 0.0)
    unused = np.setdiff1d(np.arange(N), x["idx"][x["idx"] >= 0])
    assert np.all(host_bf16(dkv)[unused] == 0.0)
    if sink:
        assert_close("d_sink", ds.cpu().numpy(), ref["d_sink"])


@pytest.mark.parametrize("N", [300_000, (1 << 20) - 1])
def test_many_kv_rows_mostly_unused(N):
    """num_kv in the hundreds of thousands, up to the largest the library takes,
    with a few tokens: the CSR scans, the gather plan and the row sums must cover
    every row (all but a few hundred of them empty, so zero) and the used ones,
    the first and the last row among them, must match the oracle."""
    T, H, K = 12, 16, 32
    rng = np.random.default_rng(4242)
    idx = rng.integers(0, N, size=(T, K)).astype(np.int32)
    idx = np.where(rng.random((T, K)) < 0.2, -1, idx).astype(np.int32)
    idx[0, 0], idx[1, 0], idx[2, 5] = N - 1, 0, N - 1
    x = {"q": inputs.normal_bf16((T, H, 512), 4242, 1), "kv": inputs.normal_bf16((N, 512), 4242, 2),
         "dO": inputs.normal_bf16((T, H, 512), 4242, 3), "idx": idx,
         "sink": rng.standard_normal(H).astype(np.float32)}
    _say(f"[many kv] T={T} H={H} N={N} K={K}")
    x = _oracle_inputs(x)
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE)
    d = _to_dev(x)
    dq, dkv, ds = _run_bwd(d)
    assert_close("dq", host_bf16(dq), ref["dq"])
    got = host_bf16(dkv)
    used = np.unique(idx[idx >= 0])
    assert_close("dkv (used rows)", got[used], ref["dkv"][used])
    mask = np.ones(N, dtype=bool)
    mask[used] = False
    assert not np.any(got[mask]), "an unused kv row is not zero"
    assert_close("d_sink", ds.cpu().numpy(), ref["d_sink"])
    row_ptr, slots = B.smla_build_csr(d["idx"], N)
    rp, sl = orc.csr(idx, N)
    assert np.array_equal(row_ptr.cpu().numpy(), rp)
    assert np.array_equal(slots.cpu().numpy()[: rp[-1]], sl)
    del d, dq, dkv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("H", [64, 16])
def test_very_large_topk(H):
    """topk = 65536: 128 index chunks per token, so a dQ item streams through 128
    segments and the forward through as many chunks; slots drawn with
    replacement from 70,000 rows, a quarter masked, one token with only three
    valid slots.  Backward against the oracle (dkv on the used rows, the rest
    exactly zero), the CSR bit-exact, the forward's O and lse."""
    T, N, K = 3, 70_000, 1 << 16
    rng = np.random.default_rng(6500 + H)
    idx = rng.integers(0, N, size=(T, K)).astype(np.int32)
    idx = np.where(rng.random((T, K)) < 0.25, -1, idx).astype(np.int32)
    idx[1] = -1
    idx[1, [7, 40000, K - 1]] = [5, N - 1, 5]
    x = {"q": inputs.normal_bf16((T, H, 512), 6500 + H, 1), "kv": inputs.normal_bf16((N, 512), 6500 + H, 2),
         "dO": inputs.normal_bf16((T, H, 512), 6500 + H, 3), "idx": idx,
         "sink": rng.standard_normal(H).astype(np.float32)}
    _say(f"[large topk] T={T} H={H} N={N} K={K}")
    x = _oracle_inputs(x)
    d = _to_dev(x)
    dq, dkv, ds = _run_bwd(d)
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE)
    assert_close("dq", host_bf16(dq), ref["dq"])
    got = host_bf16(dkv)
    used = np.unique(idx[idx >= 0])
    assert_close("dkv (used rows)", got[used], ref["dkv"][used])
    mask = np.ones(N, dtype=bool)
    mask[used] = False
    assert not np.any(got[mask]), "an unused kv row is not zero"
    assert_close("d_sink", ds.cpu().numpy(), ref["d_sink"])
    row_ptr, slots = B.smla_build_csr(d["idx"], N)
    rp, sl = orc.csr(idx, N)
    assert np.array_equal(row_ptr.cpu().numpy(), rp)
    assert np.array_equal(slots.cpu().numpy()[: rp[-1]], sl)
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], SCALE)
    o, lse = B.smla_fwd(d["q"], d["kv"], d["idx"], d["sink"], SCALE)
    torch.cuda.synchronize()
    assert_close("O", host_bf16(o), O64)
    assert np.max(np.abs(lse.cpu().numpy().astype(np.float64) - lse64)) < 1e-4
    del d, dq, dkv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("scale,H", [(0.07, 64), (1.0 / 16, 16), (0.02, 128), (2.0, 64)])
def test_non_default_scale(scale, H):
    """Any finite scale, not only 1/sqrt(512): forward and backward against the
    oracle at the same scale, with dlse (so every use of the scale is exercised:
    the logits, dS, the dq and dkv terms and the lse); scale 2 gives logits of
    about +-90, a nearly one-hot softmax."""
    T, N, K = 21, 40, 70
    x = _custom(T, H, N, K, seed=int(scale * 1000) % 997 + H, sink=True, pool_frac=0.5)
    x["idx"][5] = -1
    _say(f"[scale] {scale} H={H}")
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], scale)
    x["O"], x["lse"] = orc.emit_forward_outputs(O64, lse64)
    d = _to_dev(x)
    o, lse = B.smla_fwd(d["q"], d["kv"], d["idx"], d["sink"], scale)
    dlse = np.random.default_rng(H).standard_normal((T, H)).astype(np.float32)
    dq, dkv, ds = B.smla_bwd(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"], scale,
                             dlse=dev(dlse))
    torch.cuda.synchronize()
    assert_close("O", host_bf16(o), O64)
    fin = np.isfinite(lse64)
    assert np.max(np.abs(lse.cpu().numpy().astype(np.float64)[fin] - lse64[fin])) < 1e-4
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], scale, dlse=dlse)
    assert_close("dq", host_bf16(dq), ref["dq"])
    assert_close("dkv", host_bf16(dkv), ref["dkv"])
    assert_close("d_sink", ds.cpu().numpy(), ref["d_sink"])


def test_extreme_sink_values():
    """Sinks of +30 (the sink takes nearly all the probability: P of about e^-30,
    dq and the dS terms tiny but still relative-accurate), -30 (no effect) and
    0 across the heads: forward, backward and d_sink against the oracle, per head."""
    T, H, N, K = 19, 64, 30, 40
    x = _custom(T, H, N, K, seed=4321, sink=True, pool_frac=0.5)
    x["sink"] = np.tile(np.array([30.0, -30.0, 0.0, 12.0], dtype=np.float32), H // 4)
    x = _oracle_inputs(x)
    d = _to_dev(x)
    o, lse = B.smla_fwd(d["q"], d["kv"], d["idx"], d["sink"], SCALE)
    dq, dkv, ds = _run_bwd(d)
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], SCALE)
    assert np.max(np.abs(lse.cpu().numpy().astype(np.float64) - lse64)) < 1e-4
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE)
    got_o, got_dq = host_bf16(o), host_bf16(dq)
    for h0 in range(4):   # each sink value on its own: the +30 heads are ~e^-30 smaller
        sl = slice(h0, None, 4)
        assert_close(f"O (sink {x['sink'][h0]})", got_o[:, sl], O64[:, sl])
        assert_close(f"dq (sink {x['sink'][h0]})", got_dq[:, sl], ref["dq"][:, sl])
        assert_close(f"d_sink (sink {x['sink'][h0]})", ds.cpu().numpy()[sl], ref["d_sink"][sl])
    assert_close("dkv", host_bf16(dkv), ref["dkv"])


@pytest.mark.parametrize("H", [64, 48])
def test_forward_chunks_with_empty_ones(H):
    """Forward with topk 1600 (four index chunks, the last of 64 slots): a token
    whose middle chunk is all masked, one whose trailing chunks are, one with a
    single valid slot in its last chunk, an all-masked token, and random ones.
    O and lse against the oracle; the all-masked token gets O = 0, lse = sink."""
    T, N, K = 10, 900, 1600
    rng = np.random.default_rng(1600 + H)
    idx = rng.integers(0, N, size=(T, K)).astype(np.int32)
    idx = np.where(rng.random((T, K)) < 0.3, -1, idx).astype(np.int32)
    idx[0, 512:1024] = -1            # an empty middle chunk
    idx[1, 1024:] = -1               # empty trailing chunks
    idx[2, :] = -1
    idx[2, K - 1] = 17               # one valid slot, in the last chunk
    idx[3, :] = -1                   # no valid slot
    idx[4, 1:] = -1                  # one valid slot, in the first chunk
    x = {"q": inputs.normal_bf16((T, H, 512), 1600 + H, 1), "kv": inputs.normal_bf16((N, 512), 1600 + H, 2),
         "idx": idx, "sink": rng.standard_normal(H).astype(np.float32)}
    _say(f"[fwd chunks] H={H} K={K}")
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], SCALE)
    o, lse = B.smla_fwd(dev_bf16(x["q"]), dev_bf16(x["kv"]), dev(x["idx"]), dev(x["sink"]), SCALE)
    torch.cuda.synchronize()
    got_o = host_bf16(o)
    got_l = lse.cpu().numpy().astype(np.float64)
    assert_close("O", got_o, O64)
    assert np.max(np.abs(got_l - lse64)) < 1e-4
    assert np.all(got_o[3] == 0.0)
    np.testing.assert_allclose(got_l[3], x["sink"].astype(np.float64), rtol=1e-6, atol=1e-6)


def _fuzz_case(seed):
    """A random small problem: any H the library takes, topk up to two index chunks,
    slots drawn with replacement (duplicate rows within a token), -1 padding and a
    few out-of-range values mixed in anywhere."""
    rng = np.random.default_rng([77, seed])
    T = int(rng.integers(1, 41))
    H = int(rng.choice([16, 32, 48, 64, 80, 96, 112, 128]))
    N = T + int(rng.integers(0, 120))
    K = int(rng.choice([1, 7, 16, 31, 32, 33, 64, 100, 512, 513, 600]))
    idx = rng.integers(0, N, size=(T, K)).astype(np.int32)
    idx = np.where(rng.random((T, K)) < 0.25, -1, idx)
    bad = rng.random((T, K)) < 0.02
    idx = np.where(bad, np.where(rng.random((T, K)) < 0.5, -5, N + 2), idx).astype(np.int32)
    sink = bool(rng.integers(0, 2))
    x = {"q": inputs.normal_bf16((T, H, 512), 5000 + seed, 1), "kv": inputs.normal_bf16((N, 512), 5000 + seed, 2),
         "dO": inputs.normal_bf16((T, H, 512), 5000 + seed, 3), "idx": idx,
         "sink": rng.standard_normal(H).astype(np.float32) if sink else None}
    dlse = rng.standard_normal((T, H)).astype(np.float32) if rng.integers(0, 2) else None
    return x, dlse


@pytest.mark.parametrize("seed", range(24))
def test_random_problems(seed):
    x, dlse = _fuzz_case(seed)
    T, H, _ = x["q"].shape
    N, K = x["kv"].shape[0], x["idx"].shape[1]
    dups = sum(int(np.unique(r[r >= 0]).size < (r >= 0).sum()) for r in x["idx"])
    _say(f"[fuzz {seed}] T={T} H={H} N={N} K={K} sink={x['sink'] is not None} "
         f"dlse={dlse is not None} rows with duplicates={dups}")
    x = _oracle_inputs(x)
    d = _to_dev(x)
    # forward
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], SCALE)
    o, lse = B.smla_fwd(d["q"], d["kv"], d["idx"], d["sink"], SCALE)
    torch.cuda.synchronize()
    assert_close("O", host_bf16(o), O64)
    got = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse64)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.max(np.abs(got[fin] - lse64[fin]), initial=0.0) < 1e-4
    # backward
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE, dlse=dlse)
    dq, dkv, ds, n_inv = _run_bwd(d, dlse=None if dlse is None else dev(dlse), count_invalid=True)
    assert int(n_inv.item()) == orc.count_invalid(x["idx"], N)
    assert_close_or_cancelled("dq", host_bf16(dq), ref["dq"], x, "dq")   # one slot per token: zero by cancellation
    if np.linalg.norm(ref["dkv"]) == 0.0:                                 # every token fully masked
        assert np.all(host_bf16(dkv) == 0.0)
    else:
        assert_close("dkv", host_bf16(dkv), ref["dkv"])
    if x["sink"] is not None:
        assert_close("d_sink", ds.cpu().numpy(), ref["d_sink"])
    unused = np.setdiff1d(np.arange(N), x["idx"][(x["idx"] >= 0) & (x["idx"] < N)])
    assert np.all(host_bf16(dkv)[unused] == 0.0)
    row_ptr, slots = B.smla_build_csr(d["idx"], N)
    rp, sl = orc.csr(x["idx"], N)
    assert np.array_equal(row_ptr.cpu().numpy(), rp)
    assert np.array_equal(slots.cpu().numpy()[: rp[-1]], sl)


@pytest.mark.parametrize("H", [16, 32, 64, 128])
def test_single_slot_tokens_dq_cancels(H):
    """One valid slot per token, no sink, no lse gradient: P = 1, so the exact dq
    is zero only because dP and delta cancel, and the library sums the two in
    fp32 in different orders.  dq within the fp32 rounding bound of that (exactly
    zero on the masked tokens), dkv (then the value part, the sum of dO over the
    tokens that picked the row) within the usual bars; every dQ kernel (16, 32 and
    64 heads per workgroup)."""
    x = single_slot_problem(40, H, 50, False, seed=31)
    _say(f"[single slot] H={H}")
    dq, dkv, ds = _run_bwd(_to_dev(x))
    assert ds is None
    ref = oracle_backward_chunked(x, chunk=16)
    got = host_bf16(dq)
    assert assert_close_or_cancelled("dq", got, ref["dq"], x, "dq") is None
    assert np.all(got[3] == 0.0) and np.all(got[20] == 0.0)
    _say(f"[single slot] H={H}: max |dq| {np.abs(got).max():.1e}")
    assert_close("dkv", host_bf16(dkv), ref["dkv"])


@pytest.mark.parametrize("H,sink", [(64, True), (128, False)])
def test_topk_beyond_one_chunk(H, sink):
    """topk > 512: each token's slots form several 512-slot segments (the last
    one empty for most rows), so the persistent dQ stream continues an item
    across segments, and the forward takes its multi-chunk kernel."""
    T, N, K = 20, 700, 1100
    x = _custom(T, H, N, K, seed=K + H, sink=sink, pool_frac=1.0)
    x["idx"][4] = -1
    x["idx"][5, :] = np.sort(np.random.default_rng(3).choice(N, K, replace=True)).astype(np.int32)
    x = _oracle_inputs(x)
    _say(f"[topk>512] T={T} H={H} N={N} K={K} sink={sink}; valid per row "
         f"{np.sum((x['idx'] >= 0), axis=1).tolist()}")
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE)
    d = _to_dev(x)
    dq, dkv, ds = _run_bwd(d)
    assert_close("dq", host_bf16(dq), ref["dq"])
    assert_close("dkv", host_bf16(dkv), ref["dkv"])
    assert np.all(host_bf16(dq)[4] == 0.0)
    if sink:
        assert_close("d_sink", ds.cpu().numpy(), ref["d_sink"])
    O64, _ = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], SCALE)
    o, _ = B.smla_fwd(d["q"], d["kv"], d["idx"], d["sink"], SCALE)
    torch.cuda.synchronize()
    assert_close("O", host_bf16(o), O64)
    dq2, dkv2, _ = B.smla_bwd_phased(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"],
                                     SCALE, phase_tokens=7)
    torch.cuda.synchronize()
    assert_close("dq (phased)", host_bf16(dq2), ref["dq"])
    assert_close("dkv (phased)", host_bf16(dkv2), ref["dkv"])


def _many_multi_segment_items(T, H, N, K, seed):
    """T tokens whose topk spans several 512-slot index chunks: the even tokens'
    slots shuffled (valid ones in every chunk), one all-masked token, one whose
    valid slots lie only in its last chunk, one with a single valid slot."""
    x = _custom(T, H, N, K, seed=seed, sink=True, pool_frac=1.0)
    x["idx"][::2] = inputs.shuffle_slots(x["idx"][::2], seed=seed)
    x["idx"][7] = -1
    x["idx"][8, : (K - 1) // 512 * 512] = -1
    x["idx"][9, 1:] = -1
    return x


@pytest.mark.parametrize("H", [128, 48, 16])
def test_topk_beyond_one_chunk_many_items(H):
    """topk 1100 on 600 tokens: each persistent workgroup takes several items of
    three segments each, so the dQ stream reloads q/dO and the forward's
    consumers finish a head from the published softmax state while the next
    item's first tiles are already produced (48 heads: with a padded group; 16:
    the slot-split dQ and a padded forward).
    Every dq, dkv, O and lse row against the oracle; the all-masked token exact."""
    T, N, K = 600, 900, 1100
    x = _with_forward(_many_multi_segment_items(T, H, N, K, seed=5 * K + H))
    _say(f"[topk>512 many] T={T} H={H} N={N} K={K}: valid per row min "
         f"{int(np.sum(x['idx'] >= 0, axis=1).min())} max {int(np.sum(x['idx'] >= 0, axis=1).max())}")
    d = _to_dev(x)
    o, lse = B.smla_fwd(d["q"], d["kv"], d["idx"], d["sink"], SCALE)
    dq, dkv, ds = _run_bwd(d)
    r, _, worst = assert_close("O", host_bf16(o), x["O64"])
    _say(f"[topk>512 many] H={H}: O rel-L2 {r:.2e} worst row {worst:.2e}")
    got_l = lse.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got_l - x["lse"].astype(np.float64))) < 1e-4
    assert np.all(host_bf16(o)[7] == 0.0)
    ref = oracle_backward_chunked(x, chunk=16)
    for name, g in (("dq", dq), ("dkv", dkv)):
        r, _, worst = assert_close(name, host_bf16(g), ref[name])
        _say(f"[topk>512 many] H={H}: {name} rel-L2 {r:.2e} worst row {worst:.2e}")
    assert np.all(host_bf16(dq)[7] == 0.0)
    assert_close("d_sink", ds.cpu().numpy(), ref["d_sink"])
    del d
    torch.cuda.empty_cache()


def test_shuffled_slots_invalid_indices_and_padding():
    x = dict(workload("small"))
    idx = inputs.shuffle_slots(x["idx"], seed=5)
    rng = np.random.default_rng(8)
    bad = rng.random(idx.shape) < 0.01
    idx = np.where(bad, np.where(rng.random(idx.shape) < 0.5, -7, x["kv"].shape[0] + 3), idx)
    idx = np.concatenate([idx, np.full((idx.shape[0], 16), -1, np.int32)], axis=1).astype(np.int32)
    x["idx"] = idx
    x = _oracle_inputs(x)
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], idx, x["sink"], SCALE)
    dq, dkv, ds, n_inv = _run_bwd(_to_dev(x), count_invalid=True)
    assert_close("dq", host_bf16(dq), ref["dq"])
    assert_close("dkv", host_bf16(dkv), ref["dkv"])
    assert_close("d_sink", ds.cpu().numpy(), ref["d_sink"])
    assert int(n_inv.item()) == orc.count_invalid(idx, x["kv"].shape[0]) > 0
    row_ptr, slots = B.smla_build_csr(dev(idx), x["kv"].shape[0])
    rp, sl = orc.csr(idx, x["kv"].shape[0])
    assert np.array_equal(row_ptr.cpu().numpy(), rp)
    assert np.array_equal(slots.cpu().numpy()[: rp[-1]], sl)


def test_all_masked_without_sink_gives_zero():
    x = _custom(16, 64, 40, 32, seed=3, sink=False)
    x["idx"][:] = -1
    x = _oracle_inputs(x)
    assert np.all(np.isneginf(x["lse"]))
    dq, dkv, ds = _run_bwd(_to_dev(x))
    assert np.all(host_bf16(dq) == 0.0) and np.all(host_bf16(dkv) == 0.0)
    o, lse = B.smla_fwd(dev_bf16(x["q"]), dev_bf16(x["kv"]), dev(x["idx"]), None, SCALE)
    torch.cuda.synchronize()
    assert np.all(host_bf16(o) == 0.0) and np.all(np.isneginf(lse.cpu().numpy()))


def test_empty_T():
    H, N, K = 64, 8, 16
    z = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    sink = torch.randn(H, device="cuda")
    dq, dkv, ds = B.smla_bwd(z(0, H, 512), torch.randn(N, 512, device="cuda").bfloat16(), z(0, H, 512),
                             z(0, H, 512), torch.empty(0, H, device="cuda"),
                             torch.empty(0, K, dtype=torch.int32, device="cuda"), sink, SCALE)
    torch.cuda.synchronize()
    assert torch.all(dkv.float() == 0) and torch.all(ds == 0)


def test_error_codes_from_device_side_entry():
    x = _to_dev(_oracle_inputs(_custom(8, 16, 8, 16, seed=1)))
    with pytest.raises(B.SmlaError) as e:
        B.smla_bwd(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE,
                   workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 4
    with pytest.raises(B.SmlaError) as e:
        B.smla_bwd(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE,
                   out=(x["q"], torch.empty_like(x["kv"]), torch.empty(16, device="cuda")))
    assert e.value.status == 1   # dq aliases q


def test_c_abi_refuses_memory_not_on_the_device():
    """Host memory (pageable or pinned) handed to the C entry points in place of
    an input, an output or the workspace is refused with SMLA_ERR_INVALID_ARG
    before anything is enqueued (the device outputs keep their sentinel)."""
    x = _to_dev(_oracle_inputs(_custom(8, 16, 8, 16, seed=2)))
    T, H, _ = x["q"].shape
    N, K = x["kv"].shape[0], x["idx"].shape[1]
    lib, p = B.lib(), B._ptr
    s = B._stream(x["q"].device)
    host_q = torch.zeros_like(x["q"], device="cpu")
    pinned = torch.zeros((T, H, 512), dtype=torch.bfloat16).pin_memory()
    o = torch.full_like(x["q"], 7.0)
    lse = torch.full((T, H), 7.0, device="cuda")
    assert lib.smla_fwd(p(host_q), p(x["kv"]), p(x["idx"]), p(x["sink"]), T, H, N, K, SCALE, p(o), p(lse), s) == 1
    assert lib.smla_fwd(p(x["q"]), p(x["kv"]), p(x["idx"]), p(x["sink"]), T, H, N, K, SCALE, p(pinned), p(lse),
                        s) == 1
    nbytes = B.bwd_workspace_bytes(T, H, N, K)
    ws_dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws_host = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    dq = torch.full_like(x["q"], 7.0)
    dkv = torch.full_like(x["kv"], 7.0)
    ds = torch.full((H,), 7.0, device="cuda")

    def bwd(dq_ptr, ws):
        return lib.smla_bwd(p(x["q"]), p(x["kv"]), p(x["dO"]), p(x["O"]), p(x["lse"]), p(x["idx"]), p(x["sink"]),
                            None, T, H, N, K, SCALE, 0, dq_ptr, p(dkv), p(ds), None, p(ws), nbytes, s)

    assert bwd(p(pinned), ws_dev) == 1
    assert bwd(p(dq), ws_host) == 1
    torch.cuda.synchronize()
    assert torch.all(o.float() == 7.0) and torch.all(dq.float() == 7.0) and torch.all(dkv.float() == 7.0)
    assert bwd(p(dq), ws_dev) == 0                      # the same call on device memory runs
    torch.cuda.synchronize()
    assert not torch.all(dq.float() == 7.0)


def test_autograd_function_and_the_pages_call_form():
    """sparse_mla under torch autograd (forward smla_fwd, backward smla_bwd): the
    loss <O, W> + <lse, V> gives q.grad, kv.grad and sink.grad matching the oracle
    backward with dO = W and dlse = V (on the O and lse the forward returned);
    with only O used the gradients are smla_bwd's without dlse, bit for bit;
    sparse_mla_bwd_dsv4 is smla_bwd."""
    T, H, N, K = 37, 64, 60, 48
    x = _custom(T, H, N, K, seed=12, sink=True, pool_frac=0.5)
    x["idx"][4] = -1
    W = inputs.normal_bf16((T, H, 512), 99, 7)
    V = np.random.default_rng(5).standard_normal((T, H)).astype(np.float32)
    idx = dev(x["idx"])

    def leaves():
        return (dev_bf16(x["q"]).requires_grad_(), dev_bf16(x["kv"]).requires_grad_(),
                dev(x["sink"]).requires_grad_())

    q, kv, sink = leaves()
    o, lse = B.sparse_mla(q, kv, idx, sink)
    ((o.float() * dev_bf16(W).float()).sum() + (lse * dev(V)).sum()).backward()
    torch.cuda.synchronize()
    # the backward's own inputs are the forward's outputs: the oracle backward
    # takes those same O and lse (the forward is checked against the oracle too)
    O64, lse64 = orc.forward(x["q"], x["kv"], x["idx"], x["sink"], SCALE)
    assert_close("O", host_bf16(o.detach()), O64)
    ref = orc.backward(x["q"], x["kv"], W, host_bits(o.detach()), lse.detach().cpu().numpy(), x["idx"],
                       x["sink"], SCALE, dlse=V)
    assert_close("q.grad", host_bf16(q.grad), ref["dq"])
    assert_close("kv.grad", host_bf16(kv.grad), ref["dkv"])
    assert_close("sink.grad", sink.grad.cpu().numpy(), ref["d_sink"])
    # only O in the loss: lse's gradient is zero, so the call is smla_bwd without dlse
    q2, kv2, sink2 = leaves()
    o2, lse2 = B.sparse_mla(q2, kv2, idx, sink2)
    (o2.float() * dev_bf16(W).float()).sum().backward()
    want = B.smla_bwd(q2.detach(), kv2.detach(), dev_bf16(W), o2.detach(), lse2.detach(), idx, sink2.detach())
    page = B.sparse_mla_bwd_dsv4(q2.detach(), kv2.detach(), dev_bf16(W), o2.detach(), lse2.detach(), idx,
                                 attn_sink=sink2.detach())
    torch.cuda.synchronize()
    for got, w, pg in ((q2.grad, want[0], page[0]), (kv2.grad, want[1], page[1]), (sink2.grad, want[2], page[2])):
        assert torch.equal(got, w) and torch.equal(pg, w)


# ---------------------------------------------------------------------------
# token-phased backward (bounded workspace)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,phase,with_dlse", [("small", 100, False), ("small_nosink", 300, True),
                                                  ("tiny", 7, True)])
def test_phased_matches_oracle(name, phase, with_dlse):
    x = workload_nosink("small") if name == "small_nosink" else workload(name)
    base = name.replace("_nosink", "")
    dlse = inputs.make_dlse(base) if with_dlse else None
    _say(f"[phased] {name} phase_tokens={phase} dlse={with_dlse}")
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], x["idx"], x["sink"], SCALE, dlse=dlse)
    d = _to_dev(x)
    dq, dkv, ds, n_inv = B.smla_bwd_phased(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"],
                                           SCALE, phase_tokens=phase, count_invalid=True,
                                           dlse=None if dlse is None else dev(dlse))
    torch.cuda.synchronize()
    assert_close(f"{name} dq (phased)", host_bf16(dq), ref["dq"])
    assert_close(f"{name} dkv (phased)", host_bf16(dkv), ref["dkv"])
    if x["sink"] is not None:
        assert_close(f"{name} d_sink (phased)", ds.cpu().numpy(), ref["d_sink"])
    assert int(n_inv.item()) == 0


def test_phased_one_phase_equals_bwd():
    x = workload("small")
    d = _to_dev(x)
    T = x["q"].shape[0]
    a = _run_bwd(d)
    for phase in (T, 10 * T):
        b = B.smla_bwd_phased(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"], SCALE,
                              phase_tokens=phase)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(host_bits_t(a[i]), host_bits_t(b[i])), (phase, i)
        assert torch.equal(a[2], b[2])


def test_phased_graph_capture_replays_match_eager():
    """The phased backward forks to the helper stream once per phase; captured
    into a graph, every replay must equal the eager call bit for bit."""
    x = workload("small")
    d = _to_dev(x)
    T, H, _ = x["q"].shape
    N, K = x["kv"].shape[0], x["idx"].shape[1]
    ws = torch.empty((B.lib().smla_bwd_phased_workspace_bytes(T, H, N, K, 300, 0),), dtype=torch.uint8,
                     device="cuda")
    args = (d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"], SCALE)
    eager = B.smla_bwd_phased(*args, phase_tokens=300, workspace=ws)
    torch.cuda.synchronize()
    dq, dkv, ds = torch.empty_like(d["q"]), torch.empty_like(d["kv"]), torch.empty_like(d["sink"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.smla_bwd_phased(*args, phase_tokens=300, workspace=ws, out=(dq, dkv, ds))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.smla_bwd_phased(*args, phase_tokens=300, workspace=ws, out=(dq, dkv, ds))
    torch.cuda.synchronize()
    for rep in range(3):
        dq.fill_(0); dkv.fill_(0); ds.fill_(0); ws.fill_(0x33)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(host_bits_t(dq), host_bits_t(eager[0])), f"replay {rep}: dq"
        assert torch.equal(host_bits_t(dkv), host_bits_t(eager[1])), f"replay {rep}: dkv"
        assert torch.equal(ds, eager[2]), f"replay {rep}: d_sink"


def test_phased_invalid_indices_are_counted_over_phases():
    x = dict(workload("small"))
    rng = np.random.default_rng(12)
    idx = x["idx"].copy()
    bad = rng.random(idx.shape) < 0.02
    idx = np.where(bad, np.where(rng.random(idx.shape) < 0.5, -9, x["kv"].shape[0] + 1), idx).astype(np.int32)
    x["idx"] = idx
    x = _oracle_inputs(x)
    ref = orc.backward(x["q"], x["kv"], x["dO"], x["O"], x["lse"], idx, x["sink"], SCALE)
    d = _to_dev(x)
    dq, dkv, ds, n_inv = B.smla_bwd_phased(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"],
                                           SCALE, phase_tokens=333, count_invalid=True)
    torch.cuda.synchronize()
    assert_close("dq", host_bf16(dq), ref["dq"])
    assert_close("dkv", host_bf16(dkv), ref["dkv"])
    assert int(n_inv.item()) == orc.count_invalid(idx, x["kv"].shape[0]) > 0


def test_phased_headline_all_rows():
    x = workload("headline")
    d = _to_dev(x)
    _say("[phased] headline, phase_tokens=1000")
    dq, dkv, ds = B.smla_bwd_phased(d["q"], d["kv"], d["dO"], d["O"], d["lse"], d["idx"], d["sink"], SCALE,
                                    phase_tokens=1000)
    torch.cuda.synchronize()
    ref = full_reference("headline")
    assert_close("headline dq (phased)", host_bf16(dq), ref["dq"])
    assert_close("headline dkv (phased)", host_bf16(dkv), ref["dkv"])
    assert_close("headline d_sink (phased)", ds.cpu().numpy(), ref["d_sink"])
    del d
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# full-size workloads (the benchmark's launch configuration): every output row
# ---------------------------------------------------------------------------

def _check_all_rows(name, x, ref, dq, dkv, ds):
    w = x["workload"]
    r, c, worst = assert_close(f"{name} dq", host_bf16(dq), ref["dq"])
    _say(f"[full] {name}: dq rel-L2 {r:.2e} cos {c:.7f} worst (t,h) row {worst:.2e} over {w.T * w.H} rows")
    got_kv = host_bf16(dkv)
    r, c, worst = assert_close(f"{name} dkv", got_kv, ref["dkv"])
    _say(f"[full] {name}: dkv rel-L2 {r:.2e} cos {c:.7f} worst kv row {worst:.2e} over {w.num_kv} rows")
    unused = np.linalg.norm(ref["dkv"], axis=1) == 0.0
    assert np.all(got_kv[unused] == 0.0)
    if x["sink"] is not None:
        r, c, worst = assert_close(f"{name} d_sink", ds.cpu().numpy(), ref["d_sink"])
        _say(f"[full] {name}: d_sink rel-L2 {r:.2e} worst head {worst:.2e}")


# headline-like shapes that divide evenly nowhere: T = 3000 leaves the last round
# of persistent dQ items ragged; 2500 tokens of 64 heads with topk 480 (15 tiles);
# 16384 tokens of 16 heads put 8 GiB in the intermediate, so its rows, the dS/P
# blocks and the CSR slot ids of the later tokens sit past 2^32 bytes
_OTHER_SHAPES = {
    "t16384_h16": inputs.Workload("t16384_h16", 22, T=16384, H=16, num_kv=20480, topk=512, selection="swa_pool",
                                  window=128, pool_stride=4, pool_picks=384),
    # head counts that are not a multiple of 64, with several items per persistent
    # workgroup: 32 heads (slot-split producers), 48 and 112 (a last group of three
    # 16-head blocks), 80 (of one), 96 (of two)
    **{f"t{T}_h{H}": inputs.Workload(f"t{T}_h{H}", 40 + H // 16, T=T, H=H, num_kv=T + T // 4, topk=512,
                                     selection="swa_pool", window=128, pool_stride=4, pool_picks=384)
       for T, H in ((1500, 32), (1200, 48), (600, 80), (700, 96), (600, 112))},
    "t3000": inputs.Workload("t3000", 20, T=3000, H=128, num_kv=3750, topk=512, selection="swa_pool",
                             window=128, pool_stride=4, pool_picks=384),
    "t2500_h64_k480": inputs.Workload("t2500_h64_k480", 21, T=2500, H=64, num_kv=3125, topk=480,
                                      selection="swa_pool_zipf", window=128, pool_stride=4, pool_picks=352),
}


@pytest.mark.parametrize("name", sorted(_OTHER_SHAPES))
def test_full_size_other_shapes_all_rows(name):
    """Every dq row, dkv row and d_sink head against the oracle on seeded
    headline-like workloads of other sizes; the CSR bit-exact."""
    w = _OTHER_SHAPES[name]
    _say(f"[full] {name}: T={w.T} H={w.H} num_kv={w.num_kv} topk={w.topk}")
    x = _with_forward(inputs.make(w, sink=True))
    d = _to_dev(x)
    dq, dkv, ds = _run_bwd(d)
    row_ptr, slots = B.smla_build_csr(d["idx"], w.num_kv)
    rp, sl = orc.csr(x["idx"], w.num_kv)
    assert np.array_equal(row_ptr.cpu().numpy(), rp)
    assert np.array_equal(slots.cpu().numpy()[: rp[-1]], sl)
    _say(f"[full] {name}: oracle backward over all {w.T} tokens")
    ref = oracle_backward_chunked(x)
    _check_all_rows(name, x, ref, dq, dkv, ds)
    o, lse = B.smla_fwd(d["q"], d["kv"], d["idx"], d["sink"], SCALE)
    torch.cuda.synchronize()
    assert_close(f"{name} O", host_bf16(o), x["O64"])
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,with_dlse", [("headline", False), ("skewed", False), ("long", False),
                                            ("headline", True), ("headline_h64", False),
                                            ("mid", False)])
def test_full_size_all_rows(name, with_dlse):
    """smla_bwd on a whole seeded workload: the CSR bit-exact, and every dq row
    (t, h), every dkv row and every head of d_sink against the oracle backward
    evaluated over all tokens."""
    _say(f"[full] {name}: inputs and the oracle forward (dlse={with_dlse})")
    x = workload(name)
    w = x["workload"]
    d = _to_dev(x)
    dlse = inputs.make_dlse(name) if with_dlse else None
    _say(f"[full] {name}: running smla_bwd")
    dq, dkv, ds = _run_bwd(d, dlse=None if dlse is None else dev(dlse))
    row_ptr, slots = B.smla_build_csr(d["idx"], w.num_kv)
    rp, sl = orc.csr(x["idx"], w.num_kv)
    assert np.array_equal(row_ptr.cpu().numpy(), rp)
    assert np.array_equal(slots.cpu().numpy()[: rp[-1]], sl)
    _say(f"[full] {name}: oracle backward over all {w.T} tokens")
    ref = full_reference(name, with_dlse)
    _check_all_rows(name + (" (dlse)" if with_dlse else ""), x, ref, dq, dkv, ds)
    del d
    torch.cuda.empty_cache()
