"""GPU check of pion_prefix_query_noalloc, the variant of pion_prefix_query whose split
partials and ticket counters live in the library's fixed per-GPU scratch area instead of
allocated device memory: called through the C ABI, its output must equal
pion_prefix_query's on the same inputs, for two calls in a row (the second smaller), and
a plan larger than the area must be refused before any launch."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kp():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_prefix_amd as kp
    kp.lib()
    yield kp
    kp.pion_prefix_drop("na", -1)


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _call(kp, fn, sid, layer, Q):
    """One query through the C ABI (raw pointers, current stream); returns (rc, out, lse)."""
    import torch
    H_q, M, D = Q.shape
    out = torch.full((H_q, M, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((H_q, M), float("nan"), dtype=torch.float32, device="cuda")
    rc = getattr(kp.lib(), fn)(sid.encode(), layer, H_q, D, M, Q.data_ptr(), None,
                               out.data_ptr(), lse.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return rc, out.cpu().numpy(), lse.cpu().numpy()


def test_noalloc_matches_query_two_calls_second_smaller(kp):
    # first: the batched-Q shape (24 q-heads over 8 kv-heads, N = 4096, M = 512: the MFMA
    # kernel with key splits, 32 MB of partials in the scratch); then a smaller M = 1
    # decode layer (split-KV kernel, ticket counters, in-kernel merge)
    big = synth.generate(synth.PREFILL, 40, S_suf=0)
    small = synth.generate(synth.DECODE, 41, N=1000)
    kp.pion_prefix_store("na", 0, _dev(big.K), _dev(big.V))
    kp.pion_prefix_store("na", 1, _dev(small.K), _dev(small.V))
    for layer, inp in ((0, big), (1, small)):
        Q = _dev(inp.Q)
        rc_a, a, la = _call(kp, "pion_prefix_query_noalloc", "na", layer, Q)
        rc_b, b, lb = _call(kp, "pion_prefix_query", "na", layer, Q)
        assert rc_a == 0 and rc_b == 0
        assert np.all(np.isfinite(a)) and np.all(np.isfinite(la))
        assert np.max(np.abs(a.astype(np.float64) - b)) <= 2e-3
        assert np.max(np.abs(la.astype(np.float64) - lb)) <= 1e-4
        np.testing.assert_array_equal(a, b)      # the same kernels and plan: same bits
        np.testing.assert_array_equal(la, lb)
    ref, ref_lse = oracle.prefix_query(small.Q, small.K, small.V)
    assert np.max(np.abs(a - ref)) <= 2e-3 and np.max(np.abs(la - ref_lse)) <= 1e-4


def test_noalloc_refuses_a_plan_larger_than_the_scratch(kp):
    # D = 512 batched-Q runs on the split kernel: 64 q-heads x 512 rows x 512 dims of fp32
    # partials (67 MB) exceed the area; nothing is launched, out stays untouched
    inp = synth.generate(synth.DECODE, 42, N=64, M=512, H_q=64, H_kv=8, D=512)
    kp.pion_prefix_store("na", 2, _dev(inp.K), _dev(inp.V))
    rc, out, lse = _call(kp, "pion_prefix_query_noalloc", "na", 2, _dev(inp.Q))
    assert rc == kp.PION_ERR_SCRATCH
    assert np.all(np.isnan(out)) and np.all(np.isnan(lse))
    assert kp.pion_prefix_last_plan() == ""
    # after the refusal the area still serves a call that fits
    small = synth.generate(synth.DECODE, 43, N=300, H_q=4, H_kv=2, D=64)
    kp.pion_prefix_store("na", 3, _dev(small.K), _dev(small.V))
    rc, a, la = _call(kp, "pion_prefix_query_noalloc", "na", 3, _dev(small.Q))
    assert rc == 0
    ref, ref_lse = oracle.prefix_query(small.Q, small.K, small.V)
    assert np.max(np.abs(a - ref)) <= 2e-3 and np.max(np.abs(la - ref_lse)) <= 1e-4
