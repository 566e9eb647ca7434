"""Host-only checks of the libkvpop C ABI: the library loads, exports every
symbol include/kvpop.h declares, sizes workspaces, and rejects invalid
arguments before launching anything (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

import fixed_budget_sparse_amd as kv
from fixed_budget_sparse_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvpop.h")


def _lib():
    if not os.path.exists(kv.library_path()):
        pytest.skip("libkvpop.so not built")
    return kv.lib()


def test_header_symbols_exported():
    L = _lib()
    declared = set(re.findall(r"\b(kvpop_[a-z_]+)\s*\(", open(HEADER).read()))
    assert declared == set(kv.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(L, name), name
    assert kv.abi_version() == 6
    words = re.search(r"#define KVPOP_CACHE_STATE_WORDS (\d+)", open(HEADER).read())
    assert words and int(words.group(1)) == B.CACHE_STATE_WORDS
    assert L.kvpop_status_string(3).decode() == "workspace too small"


def _pr(**over):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, seq_len=16384, head_dim=128, sink=16,
                window=512, topk=1520)
    base.update(over)
    return B.Problem(**base)


def test_workspace_sizes():
    _lib()
    pr = _pr()
    for call in range(4):
        n = kv.workspace_size(call, pr)
        assert (n > 0) == (call != B.CALL_FUTURE_TARGET)
    # invalid problems size to 0
    assert kv.workspace_size(0, _pr(n_q_heads=30)) == 0
    assert kv.workspace_size(1, _pr(head_dim=96)) == 0
    assert kv.workspace_size(1, _pr(window=0)) == 0
    assert kv.workspace_size(9, pr) == 0
    # the threshold workspace scales with batch * heads * S
    assert kv.workspace_size(0, _pr(seq_len=32768)) > kv.workspace_size(0, pr)


def _call_thresholds(pr, prio=1, rank=1, tau=1, ws=None, n=0):
    L = _lib()
    c = pr.c()
    vp = ctypes.c_void_p
    return L.kvpop_thresholds(ctypes.byref(c), vp(prio), vp(rank), vp(tau), vp(ws), n, vp(0))


def test_error_paths_return_before_launch():
    L = _lib()
    vp = ctypes.c_void_p
    # bad shapes
    assert _call_thresholds(_pr(n_q_heads=31)) == 1
    assert _call_thresholds(_pr(seq_len=0)) == 1
    assert _call_thresholds(_pr(sink=-1)) == 1
    assert _call_thresholds(_pr(seq_len=1 << 20)) == 2
    # NULL outputs
    assert _call_thresholds(_pr(), prio=None) == 1
    # short workspace
    pr = _pr()
    n = kv.workspace_size(0, pr)
    assert _call_thresholds(pr, ws=256, n=n - 1) == 3
    assert _call_thresholds(pr, ws=None, n=n) == 3
    # misaligned workspace
    assert _call_thresholds(pr, ws=4096 + 4, n=n) == 1
    # forward: w >= 1, D in {64,128}, G <= 32
    c = _pr(window=0).c()
    assert L.kvpop_masked_attn_fwd(ctypes.byref(c), *[vp(1)] * 7, vp(256), 1 << 40, vp(0)) == 1
    c = _pr(head_dim=80).c()
    assert L.kvpop_masked_attn_fwd(ctypes.byref(c), *[vp(1)] * 7, vp(256), 1 << 40, vp(0)) == 2
    c = _pr(n_q_heads=64, n_kv_heads=1).c()
    assert L.kvpop_future_target(ctypes.byref(c), *[vp(1)] * 4, vp(0), 0, vp(0)) == 2
    c = _pr(qkv_dtype=7).c()
    assert L.kvpop_future_target(ctypes.byref(c), *[vp(1)] * 4, vp(0), 0, vp(0)) == 1
    # decode: NULL cache, missing pointers, short workspace
    c = _pr().c()
    assert L.kvpop_decode_step(ctypes.byref(c), None, *[vp(1)] * 7, vp(256), 1 << 40, vp(0)) == 1
    cache = B._Cache(1, 1, 1, 1, 1)
    assert L.kvpop_decode_step(ctypes.byref(c), ctypes.byref(cache), *[vp(1)] * 5, vp(0), vp(1),
                               vp(256), 1 << 40, vp(0)) == 1
    assert L.kvpop_decode_step(ctypes.byref(c), ctypes.byref(cache), *[vp(1)] * 7, vp(256), 16,
                               vp(0)) == 3


def test_decode_noalloc_error_paths():
    """The no-allocation decode refuses, before touching the device, problems
    whose split-K scratch exceeds its fixed array, and invalid arguments."""
    L = _lib()
    vp = ctypes.c_void_p
    cache = B._Cache(1, 1, 1, 1, 1)
    # 32 (sequence, KV head) pairs with 32-head query groups and a 2^16-token
    # budget: 16 splits x 1024 query rows x 130 floats > 8 MiB
    big = _pr(batch=4, n_q_heads=256, n_kv_heads=8, topk=1 << 16)
    assert kv.workspace_size(B.CALL_DECODE, big) > 8 << 20
    c = big.c()
    assert L.kvpop_decode_step_noalloc(ctypes.byref(c), ctypes.byref(cache), *[vp(1)] * 7,
                                       vp(0)) == 5
    assert L.kvpop_status_string(5).decode().startswith("problem exceeds the fixed scratch")
    # the benchmark's long-context decode fits (8 sequences, B = 4096)
    long8 = _pr(batch=8, window=1024, topk=3056)
    assert 0 < kv.workspace_size(B.CALL_DECODE, long8) <= 8 << 20
    c = _pr().c()
    assert L.kvpop_decode_step_noalloc(ctypes.byref(c), None, *[vp(1)] * 7, vp(0)) == 1
    assert L.kvpop_decode_step_noalloc(ctypes.byref(c), ctypes.byref(cache), *[vp(1)] * 5, vp(0),
                                       vp(1), vp(0)) == 1
    c = _pr(window=0).c()
    assert L.kvpop_decode_step_noalloc(ctypes.byref(c), ctypes.byref(cache), *[vp(1)] * 7,
                                       vp(0)) == 1


def test_cache_state_alignment_refused():
    """A cache state array not aligned to 16 bytes (its records are read 16
    bytes at a time) is refused by every call that takes a cache, before any
    launch; NULL is accepted (every full step then scans the slots)."""
    L = _lib()
    vp = ctypes.c_void_p
    bad = B._Cache(1, 1, 1, 1, 1, 8)
    c = _pr().c()
    assert L.kvpop_decode_step(ctypes.byref(c), ctypes.byref(bad), *[vp(1)] * 8, 1 << 20,
                               vp(0)) == 1
    assert L.kvpop_decode_step_noalloc(ctypes.byref(c), ctypes.byref(bad), *[vp(1)] * 7,
                                       vp(0)) == 1
    cp = _pr(n_q_heads=8).c()
    assert L.kvpop_cache_from_prefill(ctypes.byref(cp), ctypes.byref(bad), *[vp(1)] * 5,
                                      vp(0)) == 1
    # a NULL state passes the cache checks: the no-alloc call then refuses
    # the oversized problem for its scratch, not for the cache
    big = _pr(batch=4, n_q_heads=256, n_kv_heads=8, topk=1 << 16).c()
    assert L.kvpop_decode_step_noalloc(ctypes.byref(big), ctypes.byref(B._Cache(1, 1, 1, 1, 1)),
                                       *[vp(1)] * 7, vp(0)) == 5


def test_label_error_paths():
    L = _lib()
    vp = ctypes.c_void_p
    c = _pr().c()
    assert L.kvpop_boundary_labels(ctypes.byref(c), vp(1), vp(1), 0, vp(1), vp(1), vp(0)) == 1
    assert L.kvpop_boundary_labels(ctypes.byref(c), vp(1), None, 4, vp(1), vp(1), vp(0)) == 1
    c = _pr(seq_len=32769).c()
    assert L.kvpop_boundary_labels(ctypes.byref(c), vp(1), vp(1), 4, vp(1), vp(1), vp(0)) == 2
    c = _pr(seq_len=0).c()
    assert L.kvpop_boundary_labels(ctypes.byref(c), vp(1), vp(1), 4, vp(1), vp(1), vp(0)) == 1


def test_backward_error_paths():
    L = _lib()
    vp = ctypes.c_void_p
    args = [vp(1)] * 11
    c = _pr(qkv_dtype=1).c()          # float32 inputs: not implemented
    assert L.kvpop_masked_attn_bwd(ctypes.byref(c), *args, vp(256), 1 << 40, vp(0)) == 2
    c = _pr(window=0).c()
    assert L.kvpop_masked_attn_bwd(ctypes.byref(c), *args, vp(256), 1 << 40, vp(0)) == 1
    c = _pr().c()
    assert L.kvpop_masked_attn_bwd(ctypes.byref(c), *args, vp(256), 16, vp(0)) == 3
    assert L.kvpop_masked_attn_bwd(ctypes.byref(c), *args[:10], None, vp(256), 1 << 40,
                                   vp(0)) == 1
    assert kv.workspace_size(B.CALL_MASKED_BWD, _pr()) > kv.workspace_size(1, _pr())


def test_binding_refuses_cpu_tensors():
    import torch
    _lib()
    with pytest.raises(kv.KvpopError):
        kv.thresholds(torch.zeros(1, 1, 8), 0, 1, 2)


def test_abi_validation_under_sanitizers(tmp_path):
    """The library's host code built with AddressSanitizer and
    UndefinedBehaviorSanitizer, driven through every error path by
    tests/abi_check.c (no GPU: every call returns before a launch)."""
    import shutil
    import subprocess
    from fixed_budget_sparse_amd import build as Bd
    try:
        rt = Bd.asan_runtime_dir()
        clang = Bd._llvm_bin("clang")
    except RuntimeError:
        pytest.skip("ROCm toolchain not found")
    if not rt or not os.path.exists(clang):
        pytest.skip("clang sanitizer runtime not found")
    lib = Bd.build_sanitized(str(tmp_path))
    exe = str(tmp_path / "abi_check")
    rocm = os.path.join(os.path.dirname(os.path.realpath(Bd._hipcc())), "..")
    cmd = [clang, "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-shared-libsan", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(rocm, "include"), os.path.join(ROOT, "tests", "abi_check.c"),
           lib, "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + rt, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    env["LD_LIBRARY_PATH"] = rt + ":" + os.path.join(rocm, "lib") + ":" + env.get("LD_LIBRARY_PATH", "")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "abi_check ok" in r.stdout, r.stdout + r.stderr
