"""Host-side checks of the C ABI that need no GPU: the library loads, exports every
function include/pion_prefix.h declares, and rejects bad arguments (and unknown
sessions) before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_prefix_amd as kp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "pion_prefix.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pion_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kp.LIB_PATH):
        from kv_cache_prefix_amd.build import build
        build()
    return kp.lib()


def test_library_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) == 19, names
    assert set(names) == set(kp.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_last_plan_and_stream_read_without_a_gpu(lib):
    # a call rejected before any launch leaves an empty plan; the measurement aid
    # validates its arguments on the host
    assert lib.pion_kv_quantize_mlx4g32(None, 4, 33, None, None, None, None) == kp.PION_ERR_INVALID
    assert kp.pion_prefix_last_plan() == ""
    assert lib.pion_bench_stream_read(None, 17, None, None) == kp.PION_ERR_INVALID
    assert lib.pion_bench_stream_read(None, 0, None, None) == kp.PION_OK
    assert kp.pion_prefix_last_plan() == ""
    flops = ctypes.c_double(-1.0)
    assert lib.pion_bench_mfma_peak(0, ctypes.byref(flops), None, None) == kp.PION_ERR_INVALID
    assert lib.pion_bench_mfma_peak(8, None, None, None) == kp.PION_ERR_INVALID
    assert flops.value == -1.0 and kp.pion_prefix_last_plan() == ""


def test_noalloc_query_argument_validation(lib):
    # the same host checks as pion_prefix_query, before the scratch area is touched
    q = lib.pion_prefix_query_noalloc
    assert q(None, 0, 8, 128, 1, None, None, None, None, None) == kp.PION_ERR_INVALID
    assert q(b"x", 0, 8, 100, 1, None, None, None, None, None) == kp.PION_ERR_INVALID
    assert kp.status_str(kp.PION_ERR_SCRATCH) == "exceeds the fixed scratch area"


def test_status_strings(lib):
    assert kp.status_str(0) == "ok"
    assert kp.status_str(kp.PION_ERR_NOT_FOUND) == "session not found"
    assert kp.status_str(12345) == "unknown status"


def test_lookup_and_drop_of_absent_session(lib):
    assert lib.pion_prefix_lookup(b"nope", 0) == 0
    assert lib.pion_prefix_drop(b"nope", 3) == 0
    assert lib.pion_prefix_drop(b"nope", -1) == 0
    assert lib.pion_prefix_lookup(None, 0) == kp.PION_ERR_INVALID
    assert lib.pion_prefix_lookup(b"", 0) == kp.PION_ERR_INVALID
    assert lib.pion_prefix_lookup(b"x" * 256, 0) == kp.PION_ERR_INVALID
    H = ctypes.c_int()
    assert lib.pion_prefix_info(b"nope", 0, ctypes.byref(H), None, None, None) == kp.PION_ERR_NOT_FOUND


def test_capacity_and_stats_without_slots(lib):
    assert lib.pion_prefix_stats(None) == kp.PION_ERR_INVALID
    set_cap = lib.pion_prefix_set_capacity
    assert set_cap(0, 0, 0) == kp.PION_ERR_INVALID          # at least one slot
    assert set_cap(5, -1, 0) == kp.PION_ERR_INVALID
    assert set_cap(5, 0, -1) == kp.PION_ERR_INVALID
    before = kp.pion_prefix_stats()
    assert set_cap(5, 1 << 20, 3) == kp.PION_OK
    s = kp.pion_prefix_stats()
    assert (s["max_slots"], s["max_bytes"], s["cold_capacity"]) == (5, 1 << 20, 3)
    assert s["warm_slots"] == s["cold_slots"] == s["resident_bytes"] == 0
    assert s["demotions"] == before["demotions"] and s["rehydrates"] == before["rehydrates"]
    assert set_cap(before["max_slots"], before["max_bytes"], before["cold_capacity"]) == kp.PION_OK
    assert kp.status_str(kp.PION_ERR_COLDMISS) == "cold miss"


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def test_store_argument_validation(lib):
    st = lib.pion_prefix_store
    assert st(None, 0, 2, 8, 64, FAKE, FAKE, 0, None) == kp.PION_ERR_INVALID
    assert st(b"s", 0, 0, 8, 64, FAKE, FAKE, 0, None) == kp.PION_ERR_INVALID
    assert st(b"s", 0, 256, 8, 64, FAKE, FAKE, 0, None) == kp.PION_ERR_INVALID
    assert st(b"s", 0, 2, 0, 64, FAKE, FAKE, 0, None) == kp.PION_ERR_INVALID
    assert st(b"s", 0, 2, 8, 0, FAKE, FAKE, 0, None) == kp.PION_ERR_INVALID
    assert st(b"s", 0, 2, 8, 64, None, FAKE, 0, None) == kp.PION_ERR_INVALID
    assert st(b"s", 0, 2, 8, 64, FAKE, FAKE, 7, None) == kp.PION_ERR_INVALID
    assert st(b"s", 0, 2, 8, 48, FAKE, FAKE, 1, None) == kp.PION_ERR_INVALID    # D % 32
    assert st(b"s", 0, 2, 8, 48, FAKE, FAKE, 0, None) == kp.PION_ERR_UNSUPPORTED  # D set
    for D in (32, 96, 160, 192, 512):  # supported: fails later, on the fake pointers
        assert st(b"s", 0, 2, 8, D, FAKE, FAKE, 0, None) == kp.PION_ERR_INVALID
    # mlx4g32 codes of one kv-head past a 32-bit buffer range
    assert st(b"s", 0, 1, 1 << 24, 512, FAKE, FAKE, 1, None) == kp.PION_ERR_UNSUPPORTED
    # a host pointer is not device memory
    buf = np.zeros(2 * 8 * 64, np.float16)
    hp = ctypes.c_void_p(buf.ctypes.data)
    assert st(b"s", 0, 2, 8, 64, hp, hp, 0, None) == kp.PION_ERR_INVALID
    assert lib.pion_prefix_lookup(b"s", 0) == 0


def test_query_argument_validation(lib):
    q = lib.pion_prefix_query
    assert q(None, 0, 2, 64, 1, FAKE, None, FAKE, None, None) == kp.PION_ERR_INVALID
    assert q(b"s", 0, 0, 64, 1, FAKE, None, FAKE, None, None) == kp.PION_ERR_INVALID
    assert q(b"s", 0, 129, 64, 1, FAKE, None, FAKE, None, None) == kp.PION_ERR_INVALID
    assert q(b"s", 0, 2, 64, 0, FAKE, None, FAKE, None, None) == kp.PION_ERR_INVALID
    assert q(b"s", 0, 2, 64, 1, None, None, FAKE, None, None) == kp.PION_ERR_INVALID
    assert q(b"s", 0, 2, 64, 1, FAKE, None, None, None, None) == kp.PION_ERR_INVALID
    assert q(b"s", 0, 2, 80, 1, FAKE, None, FAKE, None, None) == kp.PION_ERR_UNSUPPORTED
    assert q(b"s", 0, 2, 64, 1, FAKE, None, FAKE, None, None) == kp.PION_ERR_NOT_FOUND


def test_layers_argument_validation(lib):
    ql = lib.pion_prefix_query_layers
    assert ql(b"s", 0, 0, 8, 128, 1, FAKE, None, FAKE, None, None) == kp.PION_ERR_INVALID
    assert ql(b"s", 0, 65, 8, 128, 1, FAKE, None, FAKE, None, None) == kp.PION_ERR_INVALID
    assert ql(b"s", 0, 32, 8, 100, 1, FAKE, None, FAKE, None, None) == kp.PION_ERR_UNSUPPORTED
    assert ql(b"s", 0, 32, 8, 128, 1, FAKE, None, FAKE, None, None) == kp.PION_ERR_NOT_FOUND


def test_fused_argument_validation(lib):
    f = lib.pion_prefix_query_fused
    hm_bad = (ctypes.c_int32 * 4)(0, 1, 2, 9)
    hm_ok = (ctypes.c_int32 * 4)(0, 1, 1, 0)
    # M > S_suf
    assert f(b"s", 0, 4, 64, 5, 4, 2, FAKE, FAKE, FAKE, None, FAKE, None, None) == kp.PION_ERR_INVALID
    # null suffix with S_suf > 0
    assert f(b"s", 0, 4, 64, 1, 4, 2, FAKE, None, FAKE, None, FAKE, None, None) == kp.PION_ERR_INVALID
    # head_map entry out of range
    assert f(b"s", 0, 4, 64, 1, 4, 2, FAKE, FAKE, FAKE, hm_bad, FAKE, None, None) == kp.PION_ERR_INVALID
    # H_kv not dividing H_q without a map
    assert f(b"s", 0, 4, 64, 1, 4, 3, FAKE, FAKE, FAKE, None, FAKE, None, None) == kp.PION_ERR_INVALID
    assert f(b"s", 0, 4, 64, 1, -1, 2, FAKE, FAKE, FAKE, None, FAKE, None, None) == kp.PION_ERR_INVALID
    # everything valid but no such session
    assert f(b"s", 0, 4, 64, 1, 4, 2, FAKE, FAKE, FAKE, hm_ok, FAKE, None, None) == kp.PION_ERR_NOT_FOUND
    assert f(b"s", 0, 4, 64, 3, 0, 2, FAKE, None, None, None, FAKE, None, None) == kp.PION_ERR_NOT_FOUND


def test_sparse_auto_argument_validation(lib):
    s = lib.pion_prefix_query_sparse_auto
    args = lambda B, K, S, H_kv=1: (b"s", 0, 8, 256, B, K, H_kv, S, FAKE, FAKE, FAKE, None, FAKE,
                                    None, None, None)
    assert s(*args(0, 8, 0)) == kp.PION_ERR_INVALID
    assert s(*args(64, 0, 0)) == kp.PION_ERR_INVALID
    assert s(*args(64, 1025, 0)) == kp.PION_ERR_INVALID
    assert s(*args(64, 8, -1)) == kp.PION_ERR_INVALID
    assert s(*args(64, 8, 0, 3)) == kp.PION_ERR_INVALID         # 3 does not divide 8
    assert s(*args(64, 8, 64)) == kp.PION_ERR_NOT_FOUND
    assert s(*args(64, 8, 0)) == kp.PION_ERR_NOT_FOUND


def test_quantize_argument_validation(lib):
    qz = lib.pion_kv_quantize_mlx4g32
    assert qz(FAKE, 4, 48, FAKE, FAKE, FAKE, None) == kp.PION_ERR_INVALID
    assert qz(FAKE, -1, 64, FAKE, FAKE, FAKE, None) == kp.PION_ERR_INVALID
    assert qz(None, 4, 64, FAKE, FAKE, FAKE, None) == kp.PION_ERR_INVALID
    assert qz(None, 0, 64, None, None, None, None) == kp.PION_OK       # empty is a no-op


def test_binding_rejects_cpu_tensors():
    import torch
    K = torch.zeros(2, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        kp.pion_prefix_store("s", 0, K, K)


def test_vstore_argument_validation(lib):
    f = lib.pion_vstore_fetch_f32
    assert f(None, 0, 10, 64, 0, 1, FAKE, None) == kp.PION_ERR_INVALID
    assert f(FAKE, 7, 10, 64, 0, 1, FAKE, None) == kp.PION_ERR_INVALID        # format
    assert f(FAKE, 1, 10, 48, 0, 1, FAKE, None) == kp.PION_ERR_INVALID        # mlx4g32: kv % 32
    assert f(FAKE, 0, 10, 48, 0, 1, FAKE, None) == kp.PION_ERR_INVALID        # fp16: kv % 32
    assert f(FAKE, 0, 10, 64, 5, 11, FAKE, None) == kp.PION_ERR_INVALID       # past n_rows
    assert f(FAKE, 0, 10, 64, 5, 4, FAKE, None) == kp.PION_ERR_INVALID        # end < start
    assert f(FAKE, 0, 10, 64, 3, 3, FAKE, None) == kp.PION_OK                 # empty range
    assert f(ctypes.c_void_p(0x1004), 0, 10, 64, 0, 1, FAKE, None) == kp.PION_ERR_INVALID
    w = lib.pion_prefix_warm
    assert w(b"s", 0, 2, 8, 64, 7, FAKE, FAKE, 0, None) == kp.PION_ERR_INVALID  # src format
    assert w(b"s", 0, 2, 8, 64, 0, FAKE, FAKE, 5, None) == kp.PION_ERR_INVALID  # slot format
    assert w(b"s", 0, 2, 8, 48, 0, FAKE, FAKE, 0, None) == kp.PION_ERR_UNSUPPORTED
    assert w(b"s", 0, 2, 8, 64, 0, None, FAKE, 0, None) == kp.PION_ERR_INVALID
    assert w(b"s", 0, 2, 8, 64, 0, FAKE, FAKE, 0, None) == kp.PION_ERR_INVALID  # not device memory
    assert lib.pion_prefix_lookup(b"s", 0) == 0


def test_binding_rejects_bad_tensors_before_calling_the_library(lib):
    # the Python binding checks device, dtype, contiguity and shapes itself; on a CPU
    # tensor it raises before any library call
    import torch
    cpu = torch.zeros((2, 8, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensor"):
        kp.pion_prefix_store("s", 0, cpu, cpu)
    with pytest.raises(ValueError, match=r"\[H, N, D\]"):
        kp.pion_prefix_store("s", 0, cpu, cpu[:1])
    with pytest.raises(ValueError, match="GPU tensor"):
        kp.pion_prefix_query("s", 0, torch.zeros((2, 1, 64), dtype=torch.float16),
                             torch.zeros((2, 1, 64)))
    with pytest.raises(ValueError, match="one query row"):
        kp.pion_prefix_query_sparse("s", 0, torch.zeros((2, 3, 64), dtype=torch.float16),
                                    torch.zeros((2, 4), dtype=torch.int32),
                                    torch.zeros(2, dtype=torch.int32), torch.zeros((2, 64)))
    with pytest.raises(ValueError, match="H_kv is required"):
        kp.pion_prefix_query_fused("s", 0, torch.zeros((2, 1, 64), dtype=torch.float16), None, None,
                                   torch.zeros((2, 1, 64)))
    rec = torch.zeros((10, 39), dtype=torch.uint8)  # not 5 * 64 / 8 = 40 bytes a row
    with pytest.raises(ValueError, match=r"\[n, 40\]"):
        kp.pion_vstore_fetch_f32(rec, kp.PION_KV_MLX4G32, 64, 0, 10, torch.zeros((10, 64)))
    with pytest.raises(ValueError, match="one int32 per q-head"):
        kp._head_map([0, 1, 2], 2)
    assert lib.pion_prefix_lookup(b"s", 0) == 0
