"""Pins for the fp64 attention oracle: closed forms, a library routine (torch CPU fp64
scaled_dot_product_attention, logsumexp), the merge invariant the pages test
(Shared KV Cache Serving, Tests: merging two attention halves matches the whole),
and high-precision brute force on tiny inputs."""
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
import synth


def rnd16(rng, shape, s=1.0):
    return (rng.standard_normal(shape) * s).astype(np.float16)


# ---------------------------------------------------------------- closed forms
def test_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    q, k, v = rnd16(rng, 64), rnd16(rng, (1, 64)), rnd16(rng, (1, 64))
    tau = 1 / 8
    o, lse = oracle.attend(q, k, v, tau)
    np.testing.assert_array_equal(o, v[0].astype(np.float64))
    assert lse == pytest.approx(tau * float(q.astype(np.float64) @ k[0].astype(np.float64)), abs=1e-14)


def test_zero_query_is_mean_of_values_and_lse_is_ln_n():
    rng = np.random.default_rng(2)
    N = 37
    K, V = rnd16(rng, (N, 32)), rnd16(rng, (N, 32))
    o, lse = oracle.attend(np.zeros(32, np.float16), K, V, 0.3)
    np.testing.assert_allclose(o, V.astype(np.float64).mean(0), rtol=0, atol=1e-14)
    assert lse == pytest.approx(math.log(N), abs=1e-14)


def test_equal_keys_average_and_shift_lse():
    rng = np.random.default_rng(3)
    N, D = 19, 16
    k = rnd16(rng, D)
    K = np.tile(k, (N, 1))
    V = rnd16(rng, (N, D))
    q = rnd16(rng, D)
    tau = 1 / 4
    o, lse = oracle.attend(q, K, V, tau)
    np.testing.assert_allclose(o, V.astype(np.float64).mean(0), atol=1e-14)
    s = tau * float(q.astype(np.float64) @ k.astype(np.float64))
    assert lse == pytest.approx(s + math.log(N), abs=1e-13)


def test_constant_values_pass_through():
    rng = np.random.default_rng(4)
    K = rnd16(rng, (50, 64))
    v = rnd16(rng, 64)
    o, _ = oracle.attend(rnd16(rng, 64), K, np.tile(v, (50, 1)), 0.125)
    np.testing.assert_allclose(o, v.astype(np.float64), atol=1e-14)


def test_scale_is_inverse_sqrt_d():
    for D in (32, 64, 128, 256):
        assert oracle.softmax_scale(D) == 1 / math.sqrt(D)


# ---------------------------------------------------------------- library routine
def _torch_sdpa(Q, K, V, mask=None):
    q = torch.from_numpy(Q.astype(np.float64))
    k = torch.from_numpy(K.astype(np.float64))
    v = torch.from_numpy(V.astype(np.float64))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask).numpy()


def _torch_lse(Q, K, mask=None):
    q = torch.from_numpy(Q.astype(np.float64))
    k = torch.from_numpy(K.astype(np.float64))
    s = (q @ k.transpose(-1, -2)) / math.sqrt(Q.shape[-1])
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    return torch.logsumexp(s, dim=-1).numpy()


def test_prefix_query_matches_torch_sdpa_mha():
    inp = synth.generate(synth.TINY)
    out, lse = oracle.prefix_query(inp.Q, inp.K, inp.V)
    ref = _torch_sdpa(inp.Q, inp.K, inp.V)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _torch_lse(inp.Q, inp.K), rtol=0, atol=1e-12)


def test_batched_q_gqa_equals_mha_on_repeated_kv():
    inp = synth.generate(synth.PREFILL, N=96, M=7, S_suf=0, H_q=6, H_kv=2, D=64)
    out, lse = oracle.prefix_query(inp.Q, inp.K, inp.V, inp.head_map)
    Kr = np.repeat(inp.K, 3, axis=0)
    Vr = np.repeat(inp.V, 3, axis=0)
    np.testing.assert_allclose(out, _torch_sdpa(inp.Q, Kr, Vr), atol=1e-12)
    np.testing.assert_allclose(lse, _torch_lse(inp.Q, Kr), atol=1e-12)
    # M = 1 rows agree with the same rows of the batched call
    out1, lse1 = oracle.prefix_query(inp.Q[:, 3:4], inp.K, inp.V, inp.head_map)
    np.testing.assert_array_equal(out1[:, 0], out[:, 3])
    np.testing.assert_array_equal(lse1[:, 0], lse[:, 3])


def test_default_head_map_is_library_gqa_grouping():
    inp = synth.generate(synth.PREFILL, N=48, M=3, S_suf=0, H_q=8, H_kv=2, D=32)
    out, lse = oracle.prefix_query(inp.Q, inp.K, inp.V)          # no head_map
    q = torch.from_numpy(inp.Q.astype(np.float64))
    k = torch.from_numpy(inp.K.astype(np.float64))
    v = torch.from_numpy(inp.V.astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, enable_gqa=True).numpy()
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_arbitrary_head_map_routes_to_the_named_kv_head():
    rng = np.random.default_rng(5)
    Q, K, V = rnd16(rng, (5, 1, 32)), rnd16(rng, (3, 40, 32)), rnd16(rng, (3, 40, 32))
    hm = np.array([2, 0, 2, 1, 0], np.int32)
    out, lse = oracle.prefix_query(Q, K, V, hm)
    ref = _torch_sdpa(Q, K[hm], V[hm])
    np.testing.assert_allclose(out, ref, atol=1e-12)


@pytest.mark.parametrize("M,S", [(8, 8), (3, 8), (1, 5), (16, 16)])
def test_fused_equals_masked_sdpa_over_prefix_and_suffix(M, S):
    inp = synth.generate(synth.PREFILL, N=40, M=M, S_suf=S, H_q=6, H_kv=2, D=32)
    out, lse = oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf, inp.head_map)
    N = 40
    Kc = np.repeat(np.concatenate([inp.K, inp.K_suf], axis=1), 3, axis=0)
    Vc = np.repeat(np.concatenate([inp.V, inp.V_suf], axis=1), 3, axis=0)
    # row i may see all N prefix keys and suffix keys j with j - i <= S - M
    suf = torch.ones(M, S, dtype=torch.bool).tril(diagonal=S - M)
    mask = torch.cat([torch.ones(M, N, dtype=torch.bool), suf], dim=1)
    np.testing.assert_allclose(out, _torch_sdpa(inp.Q, Kc, Vc, mask), atol=1e-12)
    np.testing.assert_allclose(lse, _torch_lse(inp.Q, Kc, mask), atol=1e-12)
    if M == S:
        # the square case is the library's own causal mask on the suffix part
        q = torch.from_numpy(inp.Q.astype(np.float64))
        ks = torch.from_numpy(np.repeat(inp.K_suf, 3, 0).astype(np.float64))
        vs = torch.from_numpy(np.repeat(inp.V_suf, 3, 0).astype(np.float64))
        o_s = torch.nn.functional.scaled_dot_product_attention(q, ks, vs, is_causal=True).numpy()
        lse_s = _torch_lse(inp.Q, np.repeat(inp.K_suf, 3, 0), torch.ones(M, S, dtype=torch.bool).tril())
        o_p, lse_p = oracle.prefix_query(inp.Q, inp.K, inp.V, inp.head_map)
        for h in range(6):
            for i in range(M):
                o, l = oracle.merge((o_p[h, i], lse_p[h, i]), (o_s[h, i], lse_s[h, i]))
                np.testing.assert_allclose(out[h, i], o, atol=1e-12)
                assert lse[h, i] == pytest.approx(l, abs=1e-12)


def test_fused_rejects_more_queries_than_suffix():
    inp = synth.generate(synth.PREFILL, N=8, M=4, S_suf=3, H_q=2, H_kv=2, D=32)
    with pytest.raises(ValueError):
        oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf)


# ---------------------------------------------------------------- merge invariant
@pytest.mark.parametrize("seed", range(6))
def test_merge_of_disjoint_partitions_equals_union(seed):
    rng = np.random.default_rng(100 + seed)
    N, D = 57, 64
    q, K, V = rnd16(rng, D, 2.0), rnd16(rng, (N, D)), rnd16(rng, (N, D))
    tau = 1 / 8
    whole = oracle.attend(q, K, V, tau)
    perm = rng.permutation(N)
    cut = int(rng.integers(1, N))
    a, b = perm[:cut], perm[cut:]
    m = oracle.merge(oracle.attend(q, K[a], V[a], tau), oracle.attend(q, K[b], V[b], tau))
    m_rev = oracle.merge(oracle.attend(q, K[b], V[b], tau), oracle.attend(q, K[a], V[a], tau))
    for o, l in (m, m_rev):
        np.testing.assert_allclose(o, whole[0], atol=1e-13)
        assert l == pytest.approx(whole[1], abs=1e-13)
    # n-way split in arbitrary order, combined two different ways
    cuts = np.sort(rng.choice(np.arange(1, N), 4, replace=False))
    parts = [oracle.attend(q, K[p], V[p], tau) for p in np.split(perm, cuts)]
    left = oracle.combine(parts)
    right = oracle.merge(oracle.combine(parts[:2]), oracle.combine(parts[2:]))
    for o, l in (left, right):
        np.testing.assert_allclose(o, whole[0], atol=1e-13)
        assert l == pytest.approx(whole[1], abs=1e-13)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed", range(5))
def test_tiny_integer_inputs_against_50_digit_brute_force(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 7))
    D = int(rng.integers(1, 5))
    q = rng.integers(-3, 4, D).astype(np.float16)
    K = rng.integers(-3, 4, (N, D)).astype(np.float16)
    V = rng.integers(-3, 4, (N, D)).astype(np.float16)
    tau = 1 / math.sqrt(D)
    o, lse = oracle.attend(q, K, V, tau)
    with mpmath.workdps(50):
        t = 1 / mpmath.sqrt(D)
        s = [t * sum(mpmath.mpf(int(q[d])) * int(K[j, d]) for d in range(D)) for j in range(N)]
        Z = mpmath.fsum(mpmath.exp(x) for x in s)
        ref_o = [mpmath.fsum(mpmath.exp(s[j]) * int(V[j, d]) for j in range(N)) / Z for d in range(D)]
        ref_lse = mpmath.log(Z)
    np.testing.assert_allclose(o, [float(x) for x in ref_o], rtol=0, atol=1e-13)
    assert lse == pytest.approx(float(ref_lse), abs=1e-13)


def test_lse_is_natural_log():
    # two keys with logits 0 and ln 3: lse = ln(1 + 3) = ln 4
    q = np.array([1.0], np.float16)
    K = np.array([[0.0], [1.0]], np.float16)
    V = np.array([[0.0], [1.0]], np.float16)
    o, lse = oracle.attend(q, K, V, math.log(3.0))
    assert lse == pytest.approx(math.log(4.0), abs=1e-15)
    assert o[0] == pytest.approx(0.75, abs=1e-15)


@pytest.mark.parametrize("seed", range(4))
def test_fp16_rounded_split_partials_stay_within_the_stated_bound(seed):
    # The batched-Q kernel keeps each key split's partial as the split's normalized
    # output rounded to fp16, with its log-sum-exp exact, and merges the splits by the
    # LSE rule. Since the merge weights sum to one, the result differs from attention
    # over all keys by at most 2^-11 of the largest partial element (fp16's unit
    # roundoff), and the LSE not at all. Exact partials from the oracle, rounded here.
    rng = np.random.default_rng(900 + seed)
    D, N, S = 64, 3000, 2 + 4 * seed
    q = rng.standard_normal(D).astype(np.float16)
    K = rng.standard_normal((N, D)).astype(np.float16)
    V = (rng.standard_normal((N, D)) * (4.0 if seed % 2 else 1.0)).astype(np.float16)
    scale = oracle.softmax_scale(D)
    cuts = [0, *np.sort(rng.choice(np.arange(1, N), size=S - 1, replace=False)), N]
    parts = [oracle.attend(q, K[a:b], V[a:b], scale) for a, b in zip(cuts[:-1], cuts[1:])]
    rounded = [(o.astype(np.float16).astype(np.float64), l) for o, l in parts]
    want_o, want_l = oracle.attend(q, K, V, scale)
    got_o, got_l = oracle.combine(rounded)
    err = np.abs(got_o - want_o).max()
    bound = 2.0 ** -11 * max(np.abs(o).max() for o, _ in parts)
    assert 0 < err <= bound * (1 + 1e-9) + 1e-12
    assert abs(got_l - want_l) <= 1e-12 * max(1.0, abs(want_l))
