"""Host-side checks of the C ABI (no GPU needed).

The library must load and export every entry point include/smla.h declares,
and argument errors must come back as status codes before any HIP call -- so
they can be forced here with fake (never dereferenced) device addresses.
"""
import ctypes
import os
import re

import pytest

from sparse_mla_attention_smla_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")

OK, INVALID, SHAPE, ALIGN, WORKSPACE, ARCH, HIP = range(7)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from sparse_mla_attention_smla_amd import build
        build.build()
    return B.lib()


def test_header_and_binding_agree(lib):
    names = declared_functions()
    assert len(names) == 21
    assert sorted(B.EXPORTED) == names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert getattr(lib, name) is not None
    out = os.popen(f"nm -D --defined-only {B.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_status_strings(lib):
    for code, text in [(0, "ok"), (SHAPE, "unsupported shape"), (ARCH, "device is not gfx950"),
                       (99, "unknown status")]:
        assert B.status_string(code) == text


def test_workspace_sizes(lib):
    # headline shape: delta 2 MiB + dS/P 1 GiB + interm 2 GiB + CSR/gather scratch
    n = lib.smla_bwd_workspace_bytes(4096, 128, 5120, 512, 0)
    assert 3.0 * 2 ** 30 < n < 3.2 * 2 ** 30
    assert lib.smla_bwd_workspace_bytes(64, 24, 64, 16, 0) == 0          # H % 16 != 0
    assert lib.smla_bwd_workspace_bytes(64, 16, 63, 16, 0) == 0          # num_kv < T
    assert lib.smla_csr_workspace_bytes(64, 16, 64) > 0
    assert lib.smla_gather_workspace_bytes(64, 16, 64) > 0
    assert lib.smla_dsink_workspace_bytes(64, 16) == 2 * 16 * 4
    # the reserved flags word: any nonzero value makes the query return 0
    assert lib.smla_bwd_workspace_bytes(4096, 128, 5120, 512, 1) == 0
    assert lib.smla_bwd_workspace_bytes(64, 16, 64, 16, 1 << 31) == 0
    assert lib.smla_bwd_phased_workspace_bytes(64, 16, 64, 16, 16, 4) == 0
    # phased: bounded by the phase, plus an fp32 running dkv (num_kv * 2 KiB)
    full = lib.smla_bwd_phased_workspace_bytes(4096, 128, 5120, 512, 4096, 0)
    part = lib.smla_bwd_phased_workspace_bytes(4096, 128, 5120, 512, 512, 0)
    assert part < full / 6 and full > n
    assert lib.smla_bwd_phased_workspace_bytes(4096, 128, 5120, 512, 10 ** 6, 0) == full
    assert lib.smla_bwd_phased_workspace_bytes(64, 16, 64, 16, 0, 0) == 0


A = 0x10000000  # fake, 256-B aligned device addresses (never dereferenced)


def _bwd(lib, T=64, H=16, N=64, K=16, scale=0.05, sink=True, d_sink=True, ws=1 << 34, flags=0, **ptr):
    p = dict(q=A, kv=2 * A, dO=3 * A, o=4 * A, lse=5 * A, idx=6 * A, sink=7 * A if sink else None,
             dlse=None, dq=8 * A, dkv=9 * A, d_sink=10 * A if d_sink else None, n_inv=None, work=11 * A)
    p.update(ptr)
    return lib.smla_bwd(p["q"], p["kv"], p["dO"], p["o"], p["lse"], p["idx"], p["sink"], p["dlse"],
                        T, H, N, K,
                        scale, flags, p["dq"], p["dkv"], p["d_sink"], p["n_inv"], p["work"], ws, None)


def test_bwd_argument_errors(lib):
    assert _bwd(lib, H=24) == SHAPE
    assert _bwd(lib, H=144) == SHAPE
    assert _bwd(lib, K=0) == SHAPE
    assert _bwd(lib, T=1, N=64, K=(1 << 20) + 16) == SHAPE    # topk past the 32-bit row offsets
    assert lib.smla_bwd_workspace_bytes(1, 16, 64, (1 << 20) + 16, 0) == 0
    assert _bwd(lib, N=63) == SHAPE                       # num_kv < T
    assert _bwd(lib, N=1 << 20) == SHAPE
    assert _bwd(lib, T=1 << 20, N=1 << 20 - 1, K=4096) == SHAPE
    assert _bwd(lib, scale=float("nan")) == INVALID
    assert _bwd(lib, flags=1) == INVALID                  # reserved flags must be 0
    assert _bwd(lib, flags=1 << 31) == INVALID
    assert _bwd(lib, d_sink=False) == INVALID             # sink without d_sink
    assert _bwd(lib, sink=False) == INVALID               # d_sink without sink
    assert _bwd(lib, q=None) == INVALID
    assert _bwd(lib, q=A + 2) == ALIGN
    assert _bwd(lib, lse=5 * A + 2) == ALIGN
    assert _bwd(lib, work=None) == WORKSPACE
    assert _bwd(lib, ws=1024) == WORKSPACE
    assert _bwd(lib, dq=A) == INVALID                     # dq aliases q
    assert _bwd(lib, work=9 * A + 4096) == INVALID        # workspace inside dkv
    assert _bwd(lib, dlse=12 * A + 2) == ALIGN
    assert _bwd(lib, n_inv=8 * A + 64) == INVALID         # n_invalid inside dq
    assert _bwd(lib, dlse=12 * A) in (HIP, ARCH)          # dlse is optional
    # a valid call gets past validation and then needs a gfx950 device
    assert _bwd(lib) in (HIP, ARCH)


def test_timed_bwd_argument_errors(lib):
    import ctypes
    p = [A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A, None, 64, 16, 64, 16, 0.05, 0,
         8 * A, 9 * A, 10 * A, None, 11 * A, 1 << 34, None]
    assert lib.smla_bwd_timed(*p, None) == INVALID                       # no event array
    evs = (ctypes.c_void_p * 5)(1, 2, None, 4, 5)
    assert lib.smla_bwd_timed(*p, evs) == INVALID                        # a NULL event
    full = (ctypes.c_void_p * 5)(1, 2, 3, 4, 5)
    bad = list(p)
    bad[10] = 63                                                         # num_kv < T
    assert lib.smla_bwd_timed(*bad, full) == SHAPE
    bad = list(p)
    bad[13] = 2                                                          # reserved flags
    assert lib.smla_bwd_timed(*bad, full) == INVALID


def test_phased_argument_errors(lib):
    def call(phase=16, ws=1 << 34, flags=0, **kw):
        p = dict(q=A, kv=2 * A, dO=3 * A, o=4 * A, lse=5 * A, idx=6 * A, sink=7 * A, dlse=None,
                 dq=8 * A, dkv=9 * A, d_sink=10 * A, n_inv=None, work=11 * A)
        p.update(kw)
        return lib.smla_bwd_phased(p["q"], p["kv"], p["dO"], p["o"], p["lse"], p["idx"], p["sink"],
                                   p["dlse"], 64, 16, 64, 16, 0.05, flags, phase, p["dq"], p["dkv"],
                                   p["d_sink"], p["n_inv"], p["work"], ws, None)
    assert call(phase=0) == SHAPE
    assert call(flags=8) == INVALID
    assert call(ws=1024) == WORKSPACE
    assert call(d_sink=None) == INVALID
    assert call(dkv=A) == INVALID                          # dkv aliases q
    assert call(dlse=12 * A + 2) == ALIGN
    assert call() in (HIP, ARCH)


def test_stage_argument_errors(lib):
    assert lib.smla_delta(A, 2 * A, None, 4, 16, A, None) == INVALID          # delta aliases o
    assert lib.smla_delta(A, 2 * A, 3 * A, 4, 16, 3 * A, None) == INVALID     # delta aliases dlse
    assert lib.smla_delta(A, 2 * A, None, 4, 20, 3 * A, None) == SHAPE
    assert lib.smla_delta(A + 8, 2 * A, None, 4, 16, 3 * A, None) == ALIGN
    assert lib.smla_delta(A, 2 * A, 4 * A + 2, 4, 16, 3 * A, None) == ALIGN
    assert lib.smla_build_csr(A, 4, 16, 3, 2 * A, 3 * A, None, 4 * A, 1 << 30, None) == SHAPE
    assert lib.smla_build_csr(A, 4, 16, 8, 2 * A, 3 * A, None, 4 * A, 8, None) == WORKSPACE
    assert lib.smla_gather(A, 2 * A, 3 * A, 4, 16, 8, 4 * A, None, 0, None) == WORKSPACE
    assert lib.smla_dsink(A, 2 * A, None, 4, 16, 3 * A, 4 * A, 1024, None) == INVALID
    assert lib.smla_fwd(A, 2 * A, 3 * A, None, 4, 16, 8, 16, float("inf"), 4 * A, 5 * A, None) == INVALID
    assert lib.smla_fwd(A, 2 * A, 3 * A, None, 4, 16, 8, 16, 0.1, A, 5 * A, None) == INVALID


def test_pe_argument_errors(lib):
    T, H, N, K = 64, 16, 64, 16
    p = dict(q=A, q_pe=12 * A, kv=2 * A, k_pe=13 * A, dO=3 * A, o=4 * A, lse=5 * A, idx=6 * A, sink=7 * A,
             dlse=None, dq=8 * A, dq_pe=14 * A, dkv=9 * A, dk_pe=15 * A, d_sink=10 * A, n_inv=None,
             work=11 * A)

    def call(flags=0, ws=1 << 34, T=T, **kw):
        a = dict(p)
        a.update(kw)
        return lib.smla_bwd_pe(a["q"], a["q_pe"], a["kv"], a["k_pe"], a["dO"], a["o"], a["lse"], a["idx"],
                               a["sink"], a["dlse"], T, H, N, K, 0.05, flags, a["dq"], a["dq_pe"], a["dkv"],
                               a["dk_pe"], a["d_sink"], a["n_inv"], a["work"], ws, None)
    assert call(flags=1) == INVALID
    assert call(q_pe=None) == INVALID
    assert call(dk_pe=None) == INVALID
    assert call(q_pe=12 * A + 8) == ALIGN
    assert call(dq_pe=A) == INVALID                          # dq_pe aliases q
    assert call(dk_pe=13 * A) == INVALID                     # dk_pe aliases k_pe
    assert call(ws=1024) == WORKSPACE
    assert call() in (HIP, ARCH)
    n = lib.smla_bwd_pe_workspace_bytes(4096, 128, 5120, 512, 0)
    assert n - lib.smla_bwd_workspace_bytes(4096, 128, 5120, 512, 0) >= 4096 * 512 * 128   # + interm_pe
    assert lib.smla_bwd_pe_workspace_bytes(4096, 128, 5120, 512, 2) == 0
    assert lib.smla_fwd_pe(A, 12 * A, 2 * A, 13 * A, 6 * A, None, T, H, N, K, 0.1, 12 * A, 5 * A, None) == INVALID
    assert lib.smla_fwd_pe(A, None, 2 * A, 13 * A, 6 * A, None, T, H, N, K, 0.1, 4 * A, 5 * A, None) == INVALID
    assert lib.smla_fwd_pe(A, 12 * A, 2 * A, 13 * A, 6 * A, None, T, H, N, K, 0.1, 4 * A, 5 * A, None) in (HIP, ARCH)


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def test_traffic_hash_ignores_comments_only():
    # the stored HBM-traffic figure is keyed to the kernel code without comments
    import bench
    a = "int f(int x) { // add one\n  return x + 1; /* done */ }\n"
    b = "int f(int x) {\n\n  return x + 1;   }  // a different comment\n"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    assert len(bench.kernel_source_hash()) == 16


def test_cpu_baseline_record_on_a_small_sample():
    # the bench's CPU leg: the oracle backward timed on a token sample, with the
    # host it ran on (threads, CPU model, BLAS) recorded beside the rate
    import bench
    from sparse_mla_attention_smla_amd import inputs
    rec = bench.cpu_baseline(inputs.WORKLOADS["tiny"], 8)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOPS" and rec["value"] > 0
    assert rec["cores"] >= 1 and rec["host_cpus"] >= 1
    assert isinstance(rec["cpu_model"], str) and rec["cpu_model"]
    assert isinstance(rec["blas"], str) and rec["blas"]
    assert "8 evenly spaced of 64 tokens" in rec["sample"]


def test_dsp_piece_layout_helpers_match_the_documented_offsets():
    """The test helpers that read and build dS/P blocks follow the offset formula
    documented with smla_dq in include/smla.h (host-side index bookkeeping)."""
    import numpy as np
    from tests._helpers import dsp_from_logical, dsp_to_logical
    for H in (16, 48, 128):
        logical = np.arange(2 * 2 * H * 32).reshape(2, 2 * H, 32)
        flat = dsp_from_logical(logical, H)
        for b in range(2):
            for r in range(2 * H):
                for j in range(32):
                    off = (r // 16) * 512 + ((j % 16) // 4 * 16 + r % 16) * 8 + (j // 16) * 4 + j % 4
                    assert flat[b * 2 * H * 32 + off] == logical[b, r, j]
        assert np.array_equal(dsp_to_logical(flat, H).reshape(logical.shape), logical)
