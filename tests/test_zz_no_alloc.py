"""The backward entry point that allocates nothing (smla_bwd_noalloc).

GPU: two calls in a row, the second on a smaller input, each checked against
smla_bwd on the same inputs -- dq and d_sink bit for bit (the phased path
computes them exactly as the plain one), dkv to the parity bar (only the fp32
summation order across token phases differs).  CPU: argument errors and a
shape too large for the library's scratch come back before any HIP call.
"""
import ctypes
import math

import numpy as np
import pytest

from sparse_mla_attention_smla_amd import binding as B
from sparse_mla_attention_smla_amd import inputs

SCALE = 1.0 / math.sqrt(512)
A = 0x10000000  # fake, aligned device addresses (never dereferenced)


def _call(lib, T=64, H=16, N=64, K=16, flags=0, **ptr):
    p = dict(q=A, kv=2 * A, dO=3 * A, o=4 * A, lse=5 * A, idx=6 * A, sink=7 * A, dlse=None,
             dq=8 * A, dkv=9 * A, d_sink=10 * A, n_inv=None)
    p.update(ptr)
    return lib.smla_bwd_noalloc(p["q"], p["kv"], p["dO"], p["o"], p["lse"], p["idx"], p["sink"], p["dlse"],
                                T, H, N, K, 0.05, flags, p["dq"], p["dkv"], p["d_sink"], p["n_inv"], None)


def test_noalloc_argument_errors_on_the_host():
    import os
    if not os.path.exists(B.LIB_PATH):
        from sparse_mla_attention_smla_amd import build
        build.build()
    lib = B.lib()
    assert _call(lib, H=24) == 2                       # shape
    assert _call(lib, flags=1) == 1                    # reserved flags
    assert _call(lib, q=None) == 1
    assert _call(lib, dq=A) == 1                       # dq aliases q
    assert _call(lib, q=A + 2) == 3                    # alignment
    assert _call(lib, sink=None) == 1                  # d_sink without sink
    # the fp32 running dkv alone (num_kv * 2 KiB) exceeds the 256 MiB scratch
    assert _call(lib, T=64, N=200_000) == 4
    # a valid call gets past validation and then needs a gfx950 device
    assert _call(lib) in (5, 6)


@pytest.mark.gpu
def test_noalloc_two_calls_match_smla_bwd():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests._helpers import assert_close, host_bf16

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    for name, with_dlse in (("headline", True), ("small", False)):   # the second call is smaller
        x = inputs.make(name, sink=True)
        w = x["workload"]
        print(f"[noalloc] {name}: T={w.T} H={w.H} num_kv={w.num_kv} topk={w.topk}", flush=True)
        q, kv, dO = d16(x["q"]), d16(x["kv"]), d16(x["dO"])
        idx = torch.from_numpy(x["idx"]).cuda()
        sink = torch.from_numpy(x["sink"]).cuda()
        dlse = torch.from_numpy(inputs.make_dlse(name)).cuda() if with_dlse else None
        O, lse = B.smla_fwd(q, kv, idx, sink, SCALE)
        want = B.smla_bwd(q, kv, dO, O, lse, idx, sink, SCALE, dlse=dlse, count_invalid=True)
        torch.cuda.synchronize()
        out = (torch.full_like(q, 7.0), torch.full_like(kv, 7.0), torch.full_like(sink, 7.0))
        got = B.smla_bwd_noalloc(q, kv, dO, O, lse, idx, sink, SCALE, out=out, dlse=dlse, count_invalid=True)
        torch.cuda.synchronize()
        assert got[0] is out[0]
        assert torch.equal(got[0].view(torch.int16), want[0].view(torch.int16)), f"{name}: dq"
        assert torch.equal(got[2], want[2]), f"{name}: d_sink"
        assert int(got[3].item()) == int(want[3].item()) == 0
        r, c, worst = assert_close(f"{name} dkv (noalloc vs smla_bwd)", host_bf16(got[1]), host_bf16(want[1]))
        print(f"[noalloc] {name}: dq and d_sink bit-equal; dkv rel-L2 {r:.2e} worst row {worst:.2e}",
              flush=True)
        del q, kv, dO, O, lse, want, got, out
        torch.cuda.empty_cache()
