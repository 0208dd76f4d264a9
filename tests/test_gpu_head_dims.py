"""GPU parity at every head dim of the pages' native SDPA set, D in {32, 64, 96, 128,
160, 192, 256, 512} ("Shared KV Cache Serving", native Metal SDPA paragraph): each
query form through the C ABI against the fp64 oracle on the same seeded fp16 inputs.
D = 96, 160 and 192 leave lanes of the vector kernels without dims; D = 32 and 512 are
the narrowest and widest rows. Tolerances as in test_gpu_parity."""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import (LSE_TOL, OUT_TOL, check, check_selection, check_sparse,  # noqa: F401
                             dev, empty, host, kp, mlx4_ref, query, sparse_call,
                             sparse_indices, _assert_same_encoding, _quantize_gpu)

pytestmark = pytest.mark.gpu

ALL_D = [32, 64, 96, 128, 160, 192, 256, 512]
NEW_D = [32, 96, 160, 192, 512]


@pytest.mark.parametrize("D", ALL_D)
def test_quantize_every_head_dim(kp, D):
    rng = np.random.default_rng(D)
    x = (rng.standard_normal((333, D)) * rng.lognormal(0, 0.5, (1, D))).astype(np.float16)
    _assert_same_encoding(_quantize_gpu(kp, x), oracle.quantize(x))


@pytest.mark.parametrize("D", NEW_D)
@pytest.mark.parametrize("N", [1, 65, 1000, 5000])
@pytest.mark.parametrize("H_q,H_kv", [(3, 3), (8, 1), (12, 4)])
def test_decode_fp16(kp, D, N, H_q, H_kv):
    inp = synth.generate(synth.DECODE, 20, N=N, D=D, H_q=H_q, H_kv=H_kv)
    kp.pion_prefix_store("t", 700, dev(inp.K), dev(inp.V))
    out, lse = query(kp, "t", 700, inp.Q)
    check(out, lse, *oracle.prefix_query(inp.Q, inp.K, inp.V))


@pytest.mark.parametrize("D", NEW_D)
def test_decode_fp16_arbitrary_head_map(kp, D):
    inp = synth.generate(synth.DECODE, 21, N=700, D=D, H_q=7, H_kv=3)
    hm = synth.random_head_map(7, 3, D)
    kp.pion_prefix_store("t", 701, dev(inp.K), dev(inp.V))
    out, lse = query(kp, "t", 701, inp.Q, head_map=hm)
    check(out, lse, *oracle.prefix_query(inp.Q, inp.K, inp.V, hm))


@pytest.mark.parametrize("D", NEW_D)
@pytest.mark.parametrize("M,S_suf", [(1, 40), (5, 70), (40, 40), (70, 100)])
def test_fused_suffix(kp, D, M, S_suf):
    # M >= 32 runs the MFMA kernel (D = 512: the vector split kernel with M query indices)
    inp = synth.generate(synth.PREFILL, 22, N=300, M=M, S_suf=S_suf, D=D, H_q=6, H_kv=2)
    kp.pion_prefix_store("t", 702, dev(inp.K), dev(inp.V))
    out, lse = empty((6, M, D)), empty((6, M))
    kp.pion_prefix_query_fused("t", 702, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    check(host(out), host(lse), *oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf))


@pytest.mark.parametrize("D", NEW_D)
@pytest.mark.parametrize("H_q,H_kv", [(2, 2), (6, 2), (8, 2), (5, 1)])
def test_mlx4g32_decode(kp, D, H_q, H_kv):
    # rows per group 1, 3, 4 and 4 + 1 on the mlx4g32 kernel
    inp = synth.generate(synth.MLX4_DECODE, 23, N=777, D=D, H_q=H_q, H_kv=H_kv)
    kp.pion_prefix_store("t", 703, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = query(kp, "t", 703, inp.Q)
    check(out, lse, *oracle.prefix_query(inp.Q, *mlx4_ref(inp.K, inp.V)))


@pytest.mark.parametrize("D", NEW_D)
def test_mlx4g32_fused_suffix(kp, D):
    inp = synth.generate(synth.MLX4_DECODE, 24, N=500, D=D, H_q=6, H_kv=2, M=3, S_suf=40)
    kp.pion_prefix_store("t", 704, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = empty((6, 3, D)), empty((6, 3))
    kp.pion_prefix_query_fused("t", 704, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    Kh, Vh = mlx4_ref(inp.K, inp.V)
    check(host(out), host(lse), *oracle.prefix_query_fused(inp.Q, Kh, Vh, inp.K_suf, inp.V_suf))


@pytest.mark.parametrize("D", NEW_D)
def test_sparse_auto(kp, D):
    # needles planted per 64-token block are picked; fused suffix
    inp = synth.generate(synth.SPARSE, 25, N=64 * 40, D=D, H_q=4, H_kv=2, S_suf=20, n_needles=3)
    kp.pion_prefix_store("t", 705, dev(inp.K), dev(inp.V))
    out, lse, blocks = sparse_call(kp, "t", 705, inp, 64, 3, 2)
    check_selection(blocks, inp.Q, inp.K, 64, 3, inp.head_map)
    np.testing.assert_array_equal(blocks, inp.needles)
    ref, ref_lse = oracle.prefix_query_blocks(inp.Q, inp.K, inp.V, 64, blocks, inp.head_map,
                                              inp.K_suf, inp.V_suf)
    check(out, lse, ref, ref_lse)


@pytest.mark.parametrize("D", [96, 512])
def test_sparse_auto_mlx4g32(kp, D):
    inp = synth.generate(synth.SPARSE, 26, N=64 * 30, D=D, H_q=4, H_kv=1, S_suf=8, n_needles=3)
    kp.pion_prefix_store("t", 706, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse, blocks = sparse_call(kp, "t", 706, inp, 64, 3, 1)
    Kh, Vh = mlx4_ref(inp.K, inp.V)
    np.testing.assert_array_equal(blocks[0], inp.needles[0])
    ref, ref_lse = oracle.prefix_query_blocks(inp.Q, Kh, Vh, 64, blocks, inp.head_map,
                                              inp.K_suf, inp.V_suf)
    check(out, lse, ref, ref_lse)


@pytest.mark.parametrize("D", NEW_D)
@pytest.mark.parametrize("K_sparse_max", [63, 3000])
def test_query_sparse(kp, D, K_sparse_max):
    rng = np.random.default_rng(D * K_sparse_max)
    H, N = 4, 4000
    inp = synth.generate(synth.DECODE, 27, N=N, D=D, H_q=H, H_kv=H)
    kp.pion_prefix_store("t", 707, dev(inp.K), dev(inp.V))
    idx, counts = sparse_indices(rng, H, N, K_sparse_max)
    out, lse = empty((H, D)), empty((H,))
    kp.pion_prefix_query_sparse("t", 707, dev(inp.Q), dev(idx), dev(counts), out, lse)
    check_sparse(host(out), host(lse), *oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, counts))


@pytest.mark.parametrize("D", [32, 160, 512])
def test_query_layers(kp, D):
    Ns = [1, 300, 2049]
    inputs = [synth.generate(synth.DECODE, 28 + l, N=N, D=D, H_q=8, H_kv=2) for l, N in enumerate(Ns)]
    for l, inp in enumerate(inputs):
        kp.pion_prefix_store("t", 710 + l, dev(inp.K), dev(inp.V))
    Q = dev(np.stack([inp.Q for inp in inputs]))
    out, lse = empty((3, 8, 1, D)), empty((3, 8, 1))
    kp.pion_prefix_query_layers("t", 710, Q, out, lse)
    out, lse = host(out), host(lse)
    for l, inp in enumerate(inputs):
        check(out[l], lse[l], *oracle.prefix_query(inp.Q, inp.K, inp.V))


def test_unsupported_head_dim(kp):
    import kv_cache_prefix_amd as k
    x = dev(np.zeros((1, 4, 48), np.float16))
    with pytest.raises(k.PionError) as e:
        kp.pion_prefix_store("t", 720, x, x)
    assert e.value.status == k.PION_ERR_UNSUPPORTED


@pytest.mark.parametrize("D", [32, 96, 160, 192])
@pytest.mark.parametrize("N,M,S_suf", [(1000, 130, 200), (777, 257, 0), (64, 32, 0), (300, 40, 40)])
def test_mfma_prefill(kp, D, N, M, S_suf):
    # M >= 32 runs the MFMA kernel with rows padded in LDS to a power-of-two layout
    inp = synth.generate(synth.PREFILL, 29, N=N, M=M, S_suf=S_suf, D=D, H_q=6, H_kv=2)
    kp.pion_prefix_store("t", 730, dev(inp.K), dev(inp.V))
    out, lse = empty((6, M, D)), empty((6, M))
    if S_suf:
        kp.pion_prefix_query_fused("t", 730, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    else:
        kp.pion_prefix_query("t", 730, dev(inp.Q), out, lse)
    out, lse = host(out), host(lse)
    rng = np.random.default_rng(N + M + D)
    rows = [(h, i) for h in range(6) for i in (0, M - 1)] + \
        [(int(h), int(i)) for h, i in zip(rng.integers(0, 6, 30), rng.integers(0, M, 30))]
    ref, ref_lse = oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf, rows=rows)
    check(out, lse, ref, ref_lse, rows=rows)
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("D", [32, 96, 160, 192, 512])
def test_mfma_and_valu_prefill_agree(kp, monkeypatch, D):
    inp = synth.generate(synth.PREFILL, 30, N=500, M=64, S_suf=64, D=D, H_q=6, H_kv=2)
    kp.pion_prefix_store("t", 731, dev(inp.K), dev(inp.V))
    outs = []
    for flag in ("0", "1"):
        monkeypatch.setenv("PION_NO_MFMA", flag)
        out, lse = empty((6, 64, D)), empty((6, 64))
        kp.pion_prefix_query_fused("t", 731, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
        outs.append((host(out), host(lse)))
    ref, ref_lse = oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf)
    for o, l in outs:
        check(o, l, ref, ref_lse)
    assert np.max(np.abs(outs[0][0] - outs[1][0])) <= 2 * OUT_TOL
