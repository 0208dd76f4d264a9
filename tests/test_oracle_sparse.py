"""Pins for the sparse-auto oracle: K_top >= nb reduces to dense attention, a library
stable sort gives the same selection, planted needle blocks are found, ties go to the
lower block index, partial last blocks, and the GQA score is linear in the q-heads."""
import numpy as np
import pytest
import torch

import oracle
import synth


def rnd16(rng, shape, s=1.0):
    return (rng.standard_normal(shape) * s).astype(np.float16)


def test_block_means_edge_shapes():
    rng = np.random.default_rng(0)
    K = rnd16(rng, (2, 10, 8))
    Kd = K.astype(np.float64)
    np.testing.assert_allclose(oracle.block_means(K, 10)[:, 0], Kd.mean(1), atol=1e-15)
    np.testing.assert_array_equal(oracle.block_means(K, 1), Kd)
    km = oracle.block_means(K, 4)            # blocks {0-3}, {4-7}, {8,9}
    assert km.shape == (2, 3, 8)
    np.testing.assert_allclose(km[:, 2], (Kd[:, 8] + Kd[:, 9]) / 2, atol=1e-15)
    np.testing.assert_allclose(km[:, 1], Kd[:, 4:8].sum(1) / 4, atol=1e-15)


def test_gqa_block_score_is_linear_in_mapped_heads():
    rng = np.random.default_rng(1)
    Q = rnd16(rng, (6, 32))
    km = rng.standard_normal((2, 5, 32))
    hm = np.array([0, 1, 1, 0, 0, 1])
    sc = oracle.block_scores(Q, km, hm)
    Qd = Q.astype(np.float64)
    for g in range(2):
        qs = Qd[hm == g].sum(0)
        np.testing.assert_allclose(sc[g], km[g] @ qs, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_selection_matches_library_stable_sort(seed):
    rng = np.random.default_rng(seed)
    score = np.round(rng.standard_normal(40), 1)          # rounding forces many ties
    for K_top in (1, 5, 17, 40, 55):
        order = np.argsort(-score, kind="stable")          # stable: lower index first
        ref = np.sort(order[:min(K_top, 40)])
        np.testing.assert_array_equal(oracle.select_blocks(score, K_top), ref)


def test_duplicate_blocks_lower_index_wins():
    rng = np.random.default_rng(3)
    B, nb, D = 4, 6, 16
    K = rnd16(rng, (1, B * nb, D))
    K[0, 4 * B:5 * B] = K[0, 1 * B:2 * B]                  # block 4 duplicates block 1
    Q = np.zeros((1, 1, D), np.float16)
    km = oracle.block_means(K, B)
    best = int(np.argmax(km[0] @ np.ones(D)))
    K[0, best * B:(best + 1) * B] = -4.0                   # make sure neither is dwarfed
    Q[0, 0] = km[0, 1].astype(np.float16)                  # point the query at block 1
    _, _, blocks = oracle.prefix_query_sparse_auto(Q, K, K, B, 1)
    assert blocks[0, 0] == 1


def test_k_top_covering_all_blocks_is_dense():
    inp = synth.generate(synth.SPARSE, N=640, H_q=4, H_kv=2, D=64)
    B = 64
    for K_top in (10, 11, 64):
        out, lse, blocks = oracle.prefix_query_sparse_auto(inp.Q, inp.K, inp.V, B, K_top, inp.head_map)
        ref, ref_lse = oracle.prefix_query(inp.Q, inp.K, inp.V, inp.head_map)
        np.testing.assert_allclose(out, ref[:, 0], atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse[:, 0], atol=1e-12)
        assert np.all(blocks[:, :10] == np.arange(10)) and np.all(blocks[:, 10:] == -1)


def test_k_top_all_with_suffix_is_fused_dense():
    inp = synth.generate(synth.SPARSE, N=300, H_q=4, H_kv=2, D=64, S_suf=16)
    out, lse, _ = oracle.prefix_query_sparse_auto(inp.Q, inp.K, inp.V, 64, 5, inp.head_map,
                                                  inp.K_suf, inp.V_suf)
    ref, ref_lse = oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf, inp.head_map)
    np.testing.assert_allclose(out, ref[:, 0], atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse[:, 0], atol=1e-12)


def test_sparse_output_is_sdpa_over_gathered_tokens():
    inp = synth.generate(synth.SPARSE, N=1024, S_suf=8)
    B, K_top = 64, 3
    out, lse, blocks = oracle.prefix_query_sparse_auto(inp.Q, inp.K, inp.V, B, K_top, inp.head_map,
                                                       inp.K_suf, inp.V_suf)
    idx = np.concatenate([np.arange(b * B, (b + 1) * B) for b in blocks[0]])
    keys = np.concatenate([inp.K[0, idx], inp.K_suf[0]]).astype(np.float64)
    vals = np.concatenate([inp.V[0, idx], inp.V_suf[0]]).astype(np.float64)
    q = torch.from_numpy(inp.Q[:, 0].astype(np.float64))[:, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, torch.from_numpy(keys)[None].expand(8, -1, -1), torch.from_numpy(vals)[None].expand(8, -1, -1))
    np.testing.assert_allclose(out, ref[:, 0].numpy(), atol=1e-12)


def test_planted_needles_are_selected_full_size():
    """The long-context workload: 8 needle blocks out of 1024 must be exactly the
    selection, with a margin far above any fp32 rounding of the scores."""
    case = synth.SPARSE
    inp = synth.generate(case)
    km = oracle.block_means(inp.K, case.B)
    score = oracle.block_scores(inp.Q[:, 0], km, inp.head_map)
    sel = oracle.select_blocks(score[0], case.K_top)
    np.testing.assert_array_equal(sel, inp.needles[0])
    srt = np.sort(score[0])[::-1]
    gap = srt[case.K_top - 1] - srt[case.K_top]
    # fp32 error bound of a D=256 dot of |q|-sum and |K_mean| plus the mean itself
    qs = np.abs(inp.Q[:, 0].astype(np.float64)).sum(0)
    bound = (case.D + case.B + 8) * 2.0 ** -23 * float(qs @ np.abs(km[0]).max(0))
    assert gap > 10 * bound, (gap, bound)
    # the same decision taken in fp32 (the kernel's precision) agrees
    km32 = inp.K.astype(np.float32).reshape(1, -1, case.B, case.D).sum(2) / np.float32(case.B)
    sc32 = (km32[0] @ inp.Q[:, 0].astype(np.float32).sum(0)).astype(np.float32)
    np.testing.assert_array_equal(np.sort(np.argsort(-sc32, kind="stable")[:8]), inp.needles[0])


# ------------------------------------------------------------------ caller-supplied indices
def _sdpa_weighted(q, K, V, w):
    """torch SDPA of one query row where key j carries multiplicity w_j (additive mask
    ln w_j), in fp64; returns (out, lse)."""
    qt = torch.from_numpy(q.astype(np.float64))[None, None, None, :]
    Kt = torch.from_numpy(K.astype(np.float64))[None, None]
    Vt = torch.from_numpy(V.astype(np.float64))[None, None]
    mask = torch.from_numpy(np.log(np.asarray(w, np.float64)))[None, None, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask)
    s = (Kt[0, 0] @ qt[0, 0, 0]) / np.sqrt(q.shape[-1]) + mask[0, 0, 0]
    return out[0, 0, 0].numpy(), float(torch.logsumexp(s, dim=-1))


def test_query_sparse_all_indices_is_dense():
    inp = synth.generate(synth.DECODE, 3, N=70, H_q=3, H_kv=3, D=64)
    idx = np.tile(np.arange(70), (3, 1))
    out, lse = oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, [70, 70, 70])
    ref, ref_lse = oracle.prefix_query(inp.Q, inp.K, inp.V)
    np.testing.assert_allclose(out, ref[:, 0], atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse[:, 0], atol=1e-13)


def test_query_sparse_is_library_sdpa_over_the_listed_tokens():
    rng = np.random.default_rng(5)
    inp = synth.generate(synth.DECODE, 4, N=200, H_q=2, H_kv=2, D=32)
    idx = rng.integers(0, 200, size=(2, 40))
    idx[0, 7] = idx[0, 3]                       # a token listed twice weighs twice
    idx[1, 5] = -1                              # out of range: skipped
    idx[1, 9] = 200
    counts = [40, 25]                           # head 1 uses the first 25 only
    out, lse = oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, counts)
    for h in range(2):
        sel = [int(t) for t in idx[h, :counts[h]] if 0 <= t < 200]
        uniq, mult = np.unique(sel, return_counts=True)
        ref, ref_lse = _sdpa_weighted(inp.Q[h, 0], inp.K[h, uniq], inp.V[h, uniq], mult)
        np.testing.assert_allclose(out[h], ref, atol=1e-12)
        assert abs(lse[h] - ref_lse) < 1e-12


def test_query_sparse_order_of_indices_is_irrelevant():
    rng = np.random.default_rng(6)
    inp = synth.generate(synth.DECODE, 5, N=90, H_q=2, H_kv=2, D=64)
    idx = rng.integers(0, 90, size=(2, 30))
    a = oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, [30, 30])
    b = oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx[:, ::-1], [30, 30])
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13)


def test_query_sparse_counts_clamp_and_empty_head():
    inp = synth.generate(synth.DECODE, 6, N=50, H_q=3, H_kv=3, D=32)
    idx = np.tile(np.arange(10), (3, 1))
    out, lse = oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, [0, -4, 99])
    assert (out[:2] == 0).all() and np.isneginf(lse[:2]).all()
    ref, ref_lse = oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, [0, 0, 10])
    np.testing.assert_array_equal(out[2], ref[2])     # 99 clamps to K_sparse_max = 10
    assert lse[2] == ref_lse[2]
