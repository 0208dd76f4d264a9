"""GPU parity of fp32-resident slots (PION_KV_FP32: the pages' sdpa_*_fp32 kernels,
"Shared KV Cache Serving", native SDPA paragraph): every query form on fp32 K/V, Q and
suffix against the fp64 oracle on the same seeded fp32 inputs, and the WARM rehydrate
into an fp32 slot (the pages' own dequantize-to-fp32 path) against a slot stored from
the device fetch, and both against the oracle. With fp32 operands no fp16 rounding is allowed anywhere, so the
bound is tighter than the fp16 one: 1e-4 on out, 2e-5 on lse."""
import numpy as np
import pytest

import oracle
import synth
from oracle import vstore as ovs
from test_gpu_parity import check, check_selection, check_sparse, dev, empty, host, kp  # noqa: F401
from test_gpu_parity import sparse_indices

pytestmark = pytest.mark.gpu

F32_OUT, F32_LSE = 1e-4, 2e-5


@pytest.fixture(scope="module", autouse=True)
def _drop_sessions(kp):
    yield
    kp.pion_prefix_drop("f32", -1)


ALL_D = [32, 64, 96, 128, 160, 192, 256, 512]


def check32(out, lse, ref, ref_lse):
    assert np.all(np.isfinite(out))
    err = np.max(np.abs(np.asarray(out, np.float64) - ref))
    assert err <= F32_OUT, f"out max-abs {err}"
    if lse is not None:
        lerr = np.max(np.abs(np.asarray(lse, np.float64) - ref_lse))
        assert lerr <= F32_LSE, f"lse max-abs {lerr}"


def gen(case, layer, **kw):
    return synth.generate(case, layer, dtype="float32", **kw)


def store32(kp, sid, layer, inp):
    kp.pion_prefix_store(sid, layer, dev(inp.K), dev(inp.V), kp.PION_KV_FP32)


def q32(kp, sid, layer, Q, head_map=None):
    H_q, M, D = Q.shape
    out, lse = empty((H_q, M, D)), empty((H_q, M))
    kp.pion_prefix_query(sid, layer, dev(Q), out, lse, head_map=head_map)
    return host(out), host(lse)


@pytest.mark.parametrize("D", ALL_D)
@pytest.mark.parametrize("N", [1, 1000, 5000])
@pytest.mark.parametrize("H_q,H_kv", [(4, 4), (8, 1), (12, 4)])
def test_decode(kp, D, N, H_q, H_kv):
    inp = gen(synth.DECODE, 70, N=N, D=D, H_q=H_q, H_kv=H_kv)
    store32(kp, "f32", 0, inp)
    assert kp.pion_prefix_info("f32", 0) == (H_kv, N, D, kp.PION_KV_FP32)
    check32(*q32(kp, "f32", 0, inp.Q), *oracle.prefix_query(inp.Q, inp.K, inp.V))


def test_decode_arbitrary_head_map(kp):
    inp = gen(synth.DECODE, 71, N=900, H_q=7, H_kv=3)
    hm = synth.random_head_map(7, 3, 4)
    store32(kp, "f32", 1, inp)
    check32(*q32(kp, "f32", 1, inp.Q, hm), *oracle.prefix_query(inp.Q, inp.K, inp.V, hm))


@pytest.mark.parametrize("D", [64, 128, 512])
@pytest.mark.parametrize("M,S_suf", [(1, 40), (5, 70), (40, 40), (70, 100)])
def test_fused_suffix(kp, D, M, S_suf):
    inp = gen(synth.PREFILL, 72, N=300, M=M, S_suf=S_suf, D=D, H_q=6, H_kv=2)
    store32(kp, "f32", 2, inp)
    out, lse = empty((6, M, D)), empty((6, M))
    kp.pion_prefix_query_fused("f32", 2, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    check32(host(out), host(lse), *oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf))


def test_query_layers(kp):
    inputs = [gen(synth.DECODE, 73 + l, N=N, H_q=8, H_kv=2) for l, N in enumerate([1, 700, 3000])]
    for l, inp in enumerate(inputs):
        store32(kp, "f32", 10 + l, inp)
    out, lse = empty((3, 8, 1, 128)), empty((3, 8, 1))
    kp.pion_prefix_query_layers("f32", 10, dev(np.stack([i.Q for i in inputs])), out, lse)
    out, lse = host(out), host(lse)
    for l, inp in enumerate(inputs):
        check32(out[l], lse[l], *oracle.prefix_query(inp.Q, inp.K, inp.V))


@pytest.mark.parametrize("D", [96, 256])
def test_sparse_auto(kp, D):
    import torch
    inp = gen(synth.SPARSE, 74, N=64 * 40, D=D, H_q=4, H_kv=2, S_suf=20, n_needles=3)
    store32(kp, "f32", 3, inp)
    out, lse = empty((4, D)), empty((4,))
    blocks = torch.full((2, 3), -7, dtype=torch.int32, device="cuda")
    kp.pion_prefix_query_sparse_auto("f32", 3, dev(inp.Q), 64, 3, out, lse, blocks,
                                     dev(inp.K_suf), dev(inp.V_suf))
    blocks = host(blocks)
    check_selection(blocks, inp.Q, inp.K, 64, 3, inp.head_map)
    np.testing.assert_array_equal(blocks, inp.needles)
    ref, ref_lse = oracle.prefix_query_blocks(inp.Q, inp.K, inp.V, 64, blocks, inp.head_map,
                                              inp.K_suf, inp.V_suf)
    check32(host(out), host(lse), ref, ref_lse)


@pytest.mark.parametrize("K_sparse_max", [63, 3000])
def test_query_sparse(kp, K_sparse_max):
    rng = np.random.default_rng(K_sparse_max)
    inp = gen(synth.DECODE, 75, N=4000, H_q=4, H_kv=4)
    store32(kp, "f32", 4, inp)
    idx, counts = sparse_indices(rng, 4, 4000, K_sparse_max)
    out, lse = empty((4, 128)), empty((4,))
    kp.pion_prefix_query_sparse("f32", 4, dev(inp.Q), dev(idx), dev(counts), out, lse)
    ref, ref_lse = oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, counts)
    out, lse = host(out), host(lse)
    empty_rows = np.isneginf(ref_lse)
    assert (out[empty_rows] == 0).all() and np.isneginf(lse[empty_rows]).all()
    check32(out[~empty_rows], lse[~empty_rows], ref[~empty_rows], ref_lse[~empty_rows])


@pytest.mark.parametrize("src", [ovs.FP16, ovs.MLX4G32])
@pytest.mark.parametrize("H,N,D", [(3, 257, 96), (8, 1000, 128)])
def test_warm_into_fp32_slot(kp, src, H, N, D):
    inp = synth.generate(synth.DECODE, 76, N=N, D=D, H_q=H, H_kv=H)
    rows = [np.ascontiguousarray(x.transpose(1, 0, 2).reshape(N, H * D)) for x in (inp.K, inp.V)]
    if src == ovs.MLX4G32:
        rows = [synth.mlx4_records(N, H * D, 760 + i) for i in range(2)]
    kp.pion_prefix_warm("f32", 5, H, D, dev(rows[0]), dev(rows[1]), src, kp.PION_KV_FP32)
    assert kp.pion_prefix_info("f32", 5)[3] == kp.PION_KV_FP32
    Kw, Vw = [np.ascontiguousarray(ovs.fetch_f32(r, src, H * D, 0, N).reshape(N, H, D)
                                   .transpose(1, 0, 2)) for r in rows]
    # the slot a WARM must produce, made on the device by the fetch kernel (bit-exact
    # with the oracle's fetch in test_gpu_vstore) and torch's relayout
    import torch
    from test_gpu_vstore import fetched_slot
    kp.pion_prefix_store("f32", 6, *(fetched_slot(kp, r, src, H, D, torch.float32) for r in rows),
                         kp.PION_KV_FP32)
    Q = inp.Q.astype(np.float32)
    a, la = q32(kp, "f32", 5, Q)
    b, lb = q32(kp, "f32", 6, Q)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)
    check32(a, la, *oracle.prefix_query(Q, Kw, Vw))


def test_dtype_follows_the_slot(kp):
    inp = gen(synth.DECODE, 77, N=100, H_q=2, H_kv=2, D=64)
    store32(kp, "f32", 7, inp)
    with pytest.raises(ValueError):
        q32(kp, "f32", 7, inp.Q.astype(np.float16))        # fp16 Q on an fp32 slot
    with pytest.raises(ValueError):
        kp.pion_prefix_store("f32", 8, dev(inp.K.astype(np.float16)), dev(inp.V.astype(np.float16)),
                             kp.PION_KV_FP32)
    kp.pion_prefix_drop("f32", -1)
