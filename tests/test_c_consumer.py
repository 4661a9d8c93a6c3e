"""The C ABI used from plain C: tests/c_abi/smla_c_bwd.c includes only
include/smla.h and the HIP runtime's C header, allocates its own device memory
and calls smla_fwd and smla_bwd.  Its outputs are compared with the fp64
oracle (to the parity bars) and with the binding's call on the same inputs
(bit for bit: same library, same kernels)."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import smla_oracle as orc
from tests._helpers import assert_close, full_reference, workload

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "smla_c_bwd")


def _binary():
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is not built (build() compiles it)")
    return BIN


def test_c_consumer_reports_usage_errors():
    """Wrong arguments end with a message and status 1 before any HIP call."""
    r = subprocess.run([_binary()], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1
    assert "usage" in r.stderr


@pytest.mark.gpu
def test_c_consumer_matches_oracle_and_binding(tmp_path):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mla_attention_smla_amd import binding as B

    name = "small"
    x = workload(name)
    T, H, _ = x["q"].shape
    N, K = x["kv"].shape[0], x["idx"].shape[1]
    ind, outd = tmp_path / "in", tmp_path / "out"
    ind.mkdir()
    outd.mkdir()
    files = {"q.bin": x["q"], "kv.bin": x["kv"], "dO.bin": x["dO"], "o.bin": x["O"],
             "lse.bin": x["lse"].astype(np.float32), "idx.bin": x["idx"].astype(np.int32),
             "sink.bin": x["sink"].astype(np.float32)}
    for f, a in files.items():
        np.ascontiguousarray(a).tofile(ind / f)
    print(f"[c-abi] running {BIN} on {name} (T={T} H={H} N={N} K={K})", flush=True)
    sys.stdout.flush()
    r = subprocess.run([_binary(), str(ind), str(outd), str(T), str(H), str(N), str(K)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    dq = np.fromfile(outd / "dq.bin", dtype=np.uint16).reshape(T, H, 512)
    dkv = np.fromfile(outd / "dkv.bin", dtype=np.uint16).reshape(N, 512)
    ds = np.fromfile(outd / "dsink.bin", dtype=np.float32)
    fo = np.fromfile(outd / "fo.bin", dtype=np.uint16).reshape(T, H, 512)
    fl = np.fromfile(outd / "flse.bin", dtype=np.float32).reshape(T, H)

    ref = full_reference(name)
    assert_close("C consumer dq", orc.bf16_to_f64(dq), ref["dq"])
    assert_close("C consumer dkv", orc.bf16_to_f64(dkv), ref["dkv"])
    assert_close("C consumer d_sink", ds.astype(np.float64), ref["d_sink"])
    assert_close("C consumer forward o", orc.bf16_to_f64(fo), x["O64"])
    assert np.max(np.abs(fl.astype(np.float64) - x["lse"].astype(np.float64))) < 1e-4

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    got = B.smla_bwd(d16(x["q"]), d16(x["kv"]), d16(x["dO"]), d16(x["O"]),
                     torch.from_numpy(x["lse"]).cuda(), torch.from_numpy(x["idx"]).cuda(),
                     torch.from_numpy(x["sink"]).cuda(), 1.0 / np.sqrt(512.0))
    torch.cuda.synchronize()
    assert np.array_equal(got[0].view(torch.int16).cpu().numpy().view(np.uint16), dq)
    assert np.array_equal(got[1].view(torch.int16).cpu().numpy().view(np.uint16), dkv)
    assert np.array_equal(got[2].cpu().numpy(), ds)
