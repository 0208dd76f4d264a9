"""Oracle for ATTEND.PREFIX.QUERY_SPARSE_AUTO(_FUSED): block-mean top-K selection over
the resident K, then attention over the chosen blocks (plus the dense suffix).

TEST INFRASTRUCTURE ONLY (tests, smoke check, bench CPU baseline).

Source: Shared KV Cache Serving, Stage 2 (Wire forms and the sparse-mask paragraph:
the server picks block-mean top-K from resident K/V with block size B and K_top
blocks, then runs sparse SDPA over the picked indices; the fused variant also merges
a caller-supplied dense suffix) and the ATTEND.* page (QUERY_SPARSE_AUTO rows: K_mean
cached per slot, GQA-aware).

Readings where the pages are silent:
  * a block's mean is over the tokens it holds (the last block may be partial);
  * a kv-head's block score sums q_h . K_mean over the q-heads h mapped to it; the
    softmax scale is left out (it does not change the order);
  * blocks rank by (score descending, block index ascending) - lower index wins ties;
    the first min(K_top, nb) are kept and reported in ascending block order;
  * the chosen tokens of kv-head g serve every q-head mapped to g.
"""
from __future__ import annotations

import numpy as np

from .attention import attend, f64, resolve_head_map, softmax_scale


def n_blocks(N: int, B: int) -> int:
    return -(-N // B)


def block_means(K, B: int) -> np.ndarray:
    """K [H_kv, N, D] -> K_mean [H_kv, nb, D]: mean of K over the tokens of each block."""
    K = f64(K)
    H_kv, N, D = K.shape
    nb = n_blocks(N, B)
    out = np.empty((H_kv, nb, D))
    for b in range(nb):
        out[:, b, :] = K[:, b * B:min((b + 1) * B, N), :].mean(axis=1)
    return out


def block_scores(Q, K_mean, head_map) -> np.ndarray:
    """Q [H_q, D] (the M=1 query rows), K_mean [H_kv, nb, D] ->
    score [H_kv, nb] = sum over q-heads h with head_map[h] == g of q_h . K_mean[g, b]."""
    Q = f64(Q)
    H_kv, nb, _ = K_mean.shape
    hm = np.asarray(head_map)
    score = np.zeros((H_kv, nb))
    for h in range(Q.shape[0]):
        g = hm[h]
        score[g] += K_mean[g] @ Q[h]
    return score


def select_blocks(score_row, K_top: int) -> np.ndarray:
    """Rank blocks by (score desc, index asc), keep the first min(K_top, nb),
    return them in ascending index order."""
    nb = len(score_row)
    order = sorted(range(nb), key=lambda b: (-score_row[b], b))
    return np.array(sorted(order[:min(K_top, nb)]), dtype=np.int64)


def prefix_query_sparse_auto(Q, K, V, B: int, K_top: int, head_map=None,
                             K_suf=None, V_suf=None):
    """M=1 sparse-auto query. Q [H_q, 1, D]; K/V [H_kv, N, D]; optional dense
    suffix K_suf/V_suf [H_kv, S_suf, D], all of which the single query row sees.

    Returns (out [H_q, D], lse [H_q], blocks [H_kv, K_top] int, -1 past nb)."""
    H_q, M, D = Q.shape
    if M != 1:
        raise ValueError("sparse-auto is an M=1 query")
    H_kv, N, _ = K.shape
    hm = resolve_head_map(H_q, H_kv, head_map)
    tau = softmax_scale(D)
    km = block_means(K, B)
    score = block_scores(Q[:, 0, :], km, hm)
    blocks = np.full((H_kv, K_top), -1, dtype=np.int64)
    for g in range(H_kv):
        sel = select_blocks(score[g], K_top)
        blocks[g, :len(sel)] = sel
    out, lse = prefix_query_blocks(Q, K, V, B, blocks, hm, K_suf, V_suf)
    return out, lse, blocks


def prefix_query_blocks(Q, K, V, B: int, blocks, head_map=None, K_suf=None, V_suf=None):
    """M=1 attention of each q-head over the tokens of the given blocks of its kv-head
    (blocks [H_kv, *], entries < 0 ignored) plus the whole suffix, if any: the attention
    step of the sparse-auto query once its blocks are chosen."""
    H_q, _, D = Q.shape
    H_kv, N, _ = K.shape
    hm = resolve_head_map(H_q, H_kv, head_map)
    tau = softmax_scale(D)
    chosen = [np.concatenate([np.arange(b * B, min((b + 1) * B, N)) for b in row if b >= 0]
                            + [np.zeros(0, np.int64)]).astype(np.int64) for row in blocks]
    out = np.empty((H_q, D))
    lse = np.empty(H_q)
    S_suf = 0 if K_suf is None else K_suf.shape[1]
    for h in range(H_q):
        g = hm[h]
        keys = f64(K[g])[chosen[g]]
        vals = f64(V[g])[chosen[g]]
        if S_suf > 0:
            keys = np.concatenate([keys, f64(K_suf[g])])
            vals = np.concatenate([vals, f64(V_suf[g])])
        out[h], lse[h] = attend(Q[h, 0], keys, vals, tau)
    return out, lse


def prefix_query_sparse(Q, K, V, indices, counts, K_sparse_max=None):
    """ATTEND.PREFIX.QUERY_SPARSE: M=1 attention of q-head h over the caller-supplied
    token indices of kv-head h (ATTEND.* page, QUERY_SPARSE row: per-head indices
    [H, K_sparse_max] and counts [H]).

    Readings where the page is silent: head h lists indices[h, :c] with
    c = min(max(counts[h], 0), K_sparse_max); an index outside [0, N) names no token and
    is skipped; an index listed twice is a key twice; a head with no key gets out = 0
    and lse = -inf (the empty softmax)."""
    H, M, D = Q.shape
    N = K.shape[1]
    indices = np.asarray(indices)
    if K_sparse_max is None:
        K_sparse_max = indices.shape[1]
    tau = softmax_scale(D)
    out = np.zeros((H, D))
    lse = np.full(H, -np.inf)
    for h in range(H):
        c = min(max(int(counts[h]), 0), K_sparse_max)
        idx = np.asarray(indices[h][:c], dtype=np.int64)
        idx = idx[(idx >= 0) & (idx < N)]
        if len(idx):
            out[h], lse[h] = attend(Q[h, 0], f64(K[h])[idx], f64(V[h])[idx], tau)
    return out, lse
