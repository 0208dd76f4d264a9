"""fp64 oracle: dense softmax attention over a resident prefix, LSE merge, and the
fused prefix + causal-suffix form.

TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the bench's CPU-baseline
leg may import this module; the library never routes through it.

Every function computes the plain definition, in fp64, with no blocking or
reordering beyond what that definition states. fp16 inputs convert to fp64 exactly.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np


def f64(x) -> np.ndarray:
    """fp16 (or any float) array -> fp64; exact for fp16 and fp32 inputs (an fp64 array
    is returned as it is)."""
    return np.asarray(x, dtype=np.float64)


def softmax_scale(D: int) -> float:
    """tau = 1/sqrt(D). The pages never print the scale; the tiny dense workload states
    1/sqrt(D) and the pages call the operation scaled-dot-product attention (SDPA)
    (Shared KV Cache Serving, Stage 2, Wire forms), whose usual scale this is."""
    return 1.0 / math.sqrt(D)


def attend(q, K, V, scale: float) -> Tuple[np.ndarray, float]:
    """Softmax attention of one query row over one key set, with its log-sum-exp.

    Shared KV Cache Serving, Stage 2 (Wire forms; "Why this matters": agreement is
    judged against CPU softmax(QK^T)V) and the ATTEND.* page (ATTEND.PREFIX.QUERY row):
        s_j = scale * (q . k_j),  m = max_j s_j,  l = sum_j exp(s_j - m),
        o   = sum_j exp(s_j - m) v_j / l,   lse = m + ln l   (natural log, scaled logits).
    The LSE is what the batched-Q reply's trailer carries for the online-softmax merge
    (Shared KV Cache Serving, Wire-protocol details).
    """
    q = f64(q)
    K = f64(K)
    V = f64(V)
    if K.shape[0] == 0:
        raise ValueError("attention over an empty key set is undefined")
    s = scale * (K @ q)
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    o = (e @ V) / l
    return o, float(m + math.log(l))


def merge(a: Tuple[np.ndarray, float], b: Tuple[np.ndarray, float]) -> Tuple[np.ndarray, float]:
    """Online-softmax (LSE) merge of two partial attentions over disjoint key sets.

    Shared KV Cache Serving, Stage 2 consumer (prefix partial merged with locally
    computed suffix attention) and Tests (merging two attention halves matches the
    whole):
        lse = mx + ln(e^{lse_a - mx} + e^{lse_b - mx}),   mx = max(lse_a, lse_b)
        o   = e^{lse_a - lse} o_a + e^{lse_b - lse} o_b
    """
    (oa, la), (ob, lb) = a, b
    mx = max(la, lb)
    lse = mx + math.log(math.exp(la - mx) + math.exp(lb - mx))
    return math.exp(la - lse) * f64(oa) + math.exp(lb - lse) * f64(ob), lse


def combine(parts: Sequence[Tuple[np.ndarray, float]]) -> Tuple[np.ndarray, float]:
    """n-way merge: the split-over-keys combine is repeated two-way merging."""
    parts = list(parts)
    acc = parts[0]
    for p in parts[1:]:
        acc = merge(acc, p)
    return acc


def resolve_head_map(H_q: int, H_kv: int, head_map=None) -> np.ndarray:
    """q-head -> kv-head. The pages pass a GQA head_map blob (ATTEND.* page,
    QUERY_FUSED row); absent a map, q-head h reads kv-head h // (H_q / H_kv)."""
    if head_map is None:
        if H_q % H_kv:
            raise ValueError("H_q must be a multiple of H_kv without a head_map")
        return np.arange(H_q) // (H_q // H_kv)
    m = np.asarray(head_map).astype(np.int64)
    if m.shape != (H_q,) or m.min() < 0 or m.max() >= H_kv:
        raise ValueError("head_map entries must lie in [0, H_kv)")
    return m


def _rows(H_q: int, M: int, rows: Optional[Iterable[Tuple[int, int]]]):
    if rows is None:
        return [(h, i) for h in range(H_q) for i in range(M)]
    return list(rows)


def prefix_query(Q, K, V, head_map=None, rows=None):
    """ATTEND.PREFIX.QUERY, M >= 1 (batched-Q form): row i of q-head h attends all N
    resident prefix keys of kv-head head_map[h] (ATTEND.* page, ATTEND.PREFIX.QUERY;
    Shared KV Cache Serving, Wire-protocol details: Q is (H, M, D), reply is H*M*D fp32
    followed by the H*M LSE trailer).

    Q [H_q, M, D], K/V [H_kv, N, D]. Returns (out [H_q, M, D], lse [H_q, M]) in fp64;
    with ``rows`` (an iterable of (h, i)), only those rows are computed and the rest
    stay NaN.
    """
    H_q, M, D = Q.shape
    H_kv = K.shape[0]
    hm = resolve_head_map(H_q, H_kv, head_map)
    tau = softmax_scale(D)
    out = np.full((H_q, M, D), np.nan)
    lse = np.full((H_q, M), np.nan)
    for h, i in _rows(H_q, M, rows):
        g = hm[h]
        out[h, i], lse[h, i] = attend(Q[h, i], K[g], V[g], tau)
    return out, lse


def suffix_visible(S_suf: int, M: int, i: int) -> int:
    """Number of suffix keys query row i sees. The fused wire form carries no mask
    (ATTEND.* page, QUERY_FUSED row: suffix SDPA merged with the prefix); the suffix is
    causal, aligned bottom-right: row i sees suffix keys j <= S_suf - M + i, so the last
    row sees them all and M == S_suf is the usual lower-triangular mask."""
    return S_suf - M + i + 1


def prefix_query_fused(Q, K, V, K_suf, V_suf, head_map=None, rows=None):
    """ATTEND.PREFIX.QUERY_FUSED: suffix attention and prefix merge in one call
    (ATTEND.* page, QUERY_FUSED row; Shared KV Cache Serving, Stage 2 wire forms).

    Row i of q-head h, g = head_map[h], attends the union of all N prefix keys of g
    and the causally visible suffix keys of g. This is computed directly over the
    concatenated key set - the definition, not the merge the kernel uses.
    Requires 1 <= M <= S_suf when S_suf > 0.
    """
    H_q, M, D = Q.shape
    H_kv = K.shape[0]
    S_suf = 0 if K_suf is None else K_suf.shape[1]
    if S_suf > 0 and M > S_suf:
        raise ValueError("fused query needs M <= S_suf")
    hm = resolve_head_map(H_q, H_kv, head_map)
    tau = softmax_scale(D)
    out = np.full((H_q, M, D), np.nan)
    lse = np.full((H_q, M), np.nan)
    # per kv-head, the concatenated key set [prefix || suffix] in fp64; row i's keys are
    # its first N + suffix_visible(i) entries
    cat = {}
    for h, i in _rows(H_q, M, rows):
        g = hm[h]
        if g not in cat:
            if S_suf > 0:
                cat[g] = (np.concatenate([f64(K[g]), f64(K_suf[g])]),
                          np.concatenate([f64(V[g]), f64(V_suf[g])]))
            else:
                cat[g] = (f64(K[g]), f64(V[g]))
        n = K.shape[1] + (suffix_visible(S_suf, M, i) if S_suf > 0 else 0)
        out[h, i], lse[h, i] = attend(Q[h, i], cat[g][0][:n], cat[g][1][:n], tau)
    return out, lse
