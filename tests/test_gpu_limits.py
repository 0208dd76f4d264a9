"""GPU parity at the size limits of the C ABI: the most q-heads a call takes (128), a
million-token prefix (the split-KV grid at its span limit), the most layers per
batched launch (64), the largest K_top (1024) over thousands of blocks, a token list of
a million positions, and a 2048-row batched-Q call. Each against the fp64 oracle on
every output row."""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import check, check_selection, check_sparse, dev, empty, host, kp  # noqa: F401
from test_gpu_parity import assert_unique_selection
from test_gpu_parity import query

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _drop_sessions(kp):
    yield
    kp.pion_prefix_drop("lim", -1)


@pytest.mark.parametrize("H_kv", [1, 8, 128])
def test_most_q_heads(kp, H_kv):
    inp = synth.generate(synth.DECODE, 80, N=3000, H_q=128, H_kv=H_kv)
    kp.pion_prefix_store("lim", 0, dev(inp.K), dev(inp.V))
    out, lse = query(kp, "lim", 0, inp.Q)
    check(out, lse, *oracle.prefix_query(inp.Q, inp.K, inp.V))
    kp.pion_prefix_drop("lim", 0)


@pytest.mark.parametrize("fmt", [0, 1])
def test_million_token_prefix(kp, fmt):
    N = 1 << 20
    inp = synth.generate(synth.DECODE, 81, N=N, D=64, H_q=4, H_kv=1)
    kp.pion_prefix_store("lim", 1, dev(inp.K), dev(inp.V), fmt)
    out, lse = query(kp, "lim", 1, inp.Q)
    if fmt == 0:
        ref = oracle.prefix_query(inp.Q, inp.K, inp.V)
    else:
        Kh = oracle.dequantize(*oracle.quantize(inp.K.reshape(-1, 64))).reshape(inp.K.shape)
        Vh = oracle.dequantize(*oracle.quantize(inp.V.reshape(-1, 64))).reshape(inp.V.shape)
        ref = oracle.prefix_query(inp.Q, Kh, Vh)
    check(out, lse, *ref)
    kp.pion_prefix_drop("lim", 1)


def test_most_layers_per_launch(kp):
    L = 64
    inputs = [synth.generate(synth.DECODE, 100 + l, N=65 + 37 * l, H_q=8, H_kv=2, D=64) for l in range(L)]
    for l, inp in enumerate(inputs):
        kp.pion_prefix_store("lim", 200 + l, dev(inp.K), dev(inp.V))
    out, lse = empty((L, 8, 1, 64)), empty((L, 8, 1))
    kp.pion_prefix_query_layers("lim", 200, dev(np.stack([i.Q for i in inputs])), out, lse)
    out, lse = host(out), host(lse)
    for l, inp in enumerate(inputs):
        check(out[l], lse[l], *oracle.prefix_query(inp.Q, inp.K, inp.V))
    kp.pion_prefix_drop("lim", -1)


def test_largest_k_top(kp):
    # K_top = 1024 over 2000 blocks with 1024 planted needle blocks: unique by
    # construction, so the radix select must pick exactly the oracle's blocks
    import torch
    B, K_top = 64, 1024
    inp = synth.generate(synth.SPARSE, 82, N=64 * 2000, D=64, H_q=4, H_kv=2, S_suf=16,
                         n_needles=K_top)
    assert_unique_selection(inp.Q, inp.K, B, K_top, inp.head_map)
    kp.pion_prefix_store("lim", 2, dev(inp.K), dev(inp.V))
    out, lse = empty((4, 64)), empty((4,))
    blocks = torch.full((2, K_top), -7, dtype=torch.int32, device="cuda")
    kp.pion_prefix_query_sparse_auto("lim", 2, dev(inp.Q), B, K_top, out, lse, blocks,
                                     dev(inp.K_suf), dev(inp.V_suf))
    blocks = host(blocks)
    ref, ref_lse, ref_blocks = oracle.prefix_query_sparse_auto(
        inp.Q, inp.K, inp.V, B, K_top, inp.head_map, inp.K_suf, inp.V_suf)
    np.testing.assert_array_equal(blocks, ref_blocks)
    np.testing.assert_array_equal(ref_blocks, inp.needles)
    check_selection(blocks, inp.Q, inp.K, B, K_top, inp.head_map)
    check(host(out), host(lse), ref, ref_lse)
    kp.pion_prefix_drop("lim", 2)


def test_million_position_token_list(kp):
    H, N, KS = 2, 300000, 1 << 20
    inp = synth.generate(synth.DECODE, 83, N=N, D=64, H_q=H, H_kv=H)
    rng = np.random.default_rng(83)
    idx = rng.integers(0, N, size=(H, KS)).astype(np.int32)
    counts = np.array([KS, KS - 12345], np.int32)
    kp.pion_prefix_store("lim", 3, dev(inp.K), dev(inp.V))
    out, lse = empty((H, 64)), empty((H,))
    kp.pion_prefix_query_sparse("lim", 3, dev(inp.Q), dev(idx), dev(counts), out, lse)
    check_sparse(host(out), host(lse), *oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, counts))
    kp.pion_prefix_drop("lim", 3)


def test_2048_query_rows(kp):
    M = 2048
    inp = synth.generate(synth.PREFILL, 84, N=3000, M=M, S_suf=M, H_q=4, H_kv=2)
    kp.pion_prefix_store("lim", 4, dev(inp.K), dev(inp.V))
    out, lse = empty((4, M, 128)), empty((4, M))
    kp.pion_prefix_query_fused("lim", 4, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    out, lse = host(out), host(lse)
    ref, ref_lse = oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf)
    check(out, lse, ref, ref_lse)
    kp.pion_prefix_drop("lim", 4)


def test_token_list_beyond_a_thousand_spans(kp):
    # 2.2 million listed positions in chunks of 2048: 1075 spans of one row, merged in-kernel
    N, KS = 100000, 2200000
    inp = synth.generate(synth.DECODE, 85, N=N, D=32, H_q=1, H_kv=1)
    rng = np.random.default_rng(85)
    idx = rng.integers(0, N, size=(1, KS)).astype(np.int32)
    kp.pion_prefix_store("lim", 5, dev(inp.K), dev(inp.V))
    out, lse = empty((1, 32)), empty((1,))
    kp.pion_prefix_query_sparse("lim", 5, dev(inp.Q), dev(idx), dev(np.array([KS], np.int32)), out, lse)
    check_sparse(host(out), host(lse), *oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx,
                                                                   np.array([KS], np.int32)))
    kp.pion_prefix_drop("lim", 5)
