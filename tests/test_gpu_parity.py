"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle on the
same seeded fp16 inputs. Bit-exact for mlx4g32 codes/scales/biases and for the picked
block indices; max-abs 2e-3 on fp32 outputs and 1e-4 on LSE."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
LSE_TOL = 1e-4


@pytest.fixture(scope="module")
def kp():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_prefix_amd as kp
    kp.lib()          # raises if the library is not built: no fallback
    yield kp
    kp.pion_prefix_drop("t", -1)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def empty(shape, dtype="float32"):
    import torch
    return torch.full(shape, float("nan"), dtype=getattr(torch, dtype), device="cuda") \
        if dtype == "float32" else torch.zeros(shape, dtype=getattr(torch, dtype), device="cuda")


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check(out, lse, ref_out, ref_lse, rows=None):
    out = np.asarray(out, np.float64)
    if rows is not None:
        idx = tuple(np.array(rows).T)
        out, ref_out = out[idx], ref_out[idx]
        if lse is not None:
            lse, ref_lse = np.asarray(lse)[idx], ref_lse[idx]
    assert np.all(np.isfinite(out))
    err = np.max(np.abs(out - ref_out))
    assert err <= OUT_TOL, f"out max-abs {err}"
    if lse is not None:
        lerr = np.max(np.abs(np.asarray(lse, np.float64) - ref_lse))
        assert lerr <= LSE_TOL, f"lse max-abs {lerr}"


def query(kp, sid, layer, Q, head_map=None, want_lse=True):
    H_q, M, D = Q.shape
    out = empty((H_q, M, D))
    lse = empty((H_q, M)) if want_lse else None
    kp.pion_prefix_query(sid, layer, dev(Q), out, lse, head_map=head_map)
    return host(out), (host(lse) if want_lse else None)


# ------------------------------------------------------------------ tiny dense case
def test_tiny_dense_fp16(kp):
    inp = synth.generate(synth.TINY)
    kp.pion_prefix_store("t", 0, dev(inp.K), dev(inp.V))
    assert kp.pion_prefix_lookup("t", 0) == 1
    assert kp.pion_prefix_info("t", 0) == (2, 128, 64, 0)
    out, lse = query(kp, "t", 0, inp.Q)
    ref, ref_lse = oracle.prefix_query(inp.Q, inp.K, inp.V)
    check(out, lse, ref, ref_lse)


def _quantize_gpu(kp, x16):
    import torch
    rows, D = x16.shape
    codes = torch.zeros((rows, D // 8), dtype=torch.int32, device="cuda")
    sc = torch.zeros((rows, D // 32), dtype=torch.float16, device="cuda")
    bi = torch.zeros((rows, D // 32), dtype=torch.float16, device="cuda")
    kp.pion_kv_quantize_mlx4g32(dev(x16), codes, sc, bi)
    return host(codes).view(np.uint32), host(sc), host(bi)


def _assert_same_encoding(got, ref):
    np.testing.assert_array_equal(got[0], ref[0])
    np.testing.assert_array_equal(got[1].view(np.uint16), ref[1].view(np.uint16))
    np.testing.assert_array_equal(got[2].view(np.uint16), ref[2].view(np.uint16))


def test_tiny_quantize_bit_exact(kp):
    inp = synth.generate(synth.TINY)
    for x in (inp.K, inp.V):
        rows = x.reshape(-1, 64)
        _assert_same_encoding(_quantize_gpu(kp, rows), oracle.quantize(rows))


def test_tiny_mlx4g32_query(kp):
    inp = synth.generate(synth.TINY)
    kp.pion_prefix_store("t", 1, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = query(kp, "t", 1, inp.Q)
    Kh = oracle.dequantize(*oracle.quantize(inp.K.reshape(-1, 64))).reshape(inp.K.shape)
    Vh = oracle.dequantize(*oracle.quantize(inp.V.reshape(-1, 64))).reshape(inp.V.shape)
    ref, ref_lse = oracle.prefix_query(inp.Q, Kh, Vh)
    check(out, lse, ref, ref_lse)


# ------------------------------------------------------------------ quantizer
def test_quantize_hand_worked_group_and_edges(kp):
    from conftest import read_golden
    g = read_golden("mlx4g32_group.txt")
    x = np.zeros((7, 64), np.float16)
    x[0, :32] = np.array([float(v) for v in g["x"]], np.float16)
    x[0, 32:] = 1.5                                     # constant group
    x[1, 5] = np.float16(2.0 ** -24)                    # scale underflows fp16
    x[2] = np.linspace(-65504, 65504, 64).astype(np.float16)   # extreme range
    x[3] = (np.arange(64) * 2.0 ** -20).astype(np.float16)     # subnormal inputs
    x[4] = np.linspace(0, 1.1, 64).astype(np.float16)
    x[5] = -np.abs(np.random.default_rng(3).standard_normal(64)).astype(np.float16)
    x[6] = np.random.default_rng(4).standard_normal(64).astype(np.float16) * 1000
    got = _quantize_gpu(kp, x)
    _assert_same_encoding(got, oracle.quantize(x))
    assert [int(w) for w in got[0][0, :4]] == [int(w, 16) for w in g["words"]]


def test_quantize_signed_zero_groups(kp):
    # -0 orders below +0: the bias of a zero-minimum group is -0 exactly when it holds a
    # -0, in either order of the zeros and in any lane of the group's four words
    nz, pz = np.float16(-0.0), np.float16(0.0)
    x = np.zeros((8, 64), np.float16)
    x[0, 0], x[0, 1] = pz, nz                      # +0 then -0
    x[0, 32], x[0, 63] = nz, pz                    # -0 first, +0 in the group's last word
    x[1, :32] = nz                                 # all -0
    x[1, 40] = nz                                  # one -0 in the third word, else +0
    x[2, :32] = nz
    x[2, 7] = np.float16(2.5)                      # -0 minimum, positive range
    x[2, 32:] = np.float16(-1.0)
    x[2, 50], x[2, 51] = nz, pz                    # zero maximum, negative minimum
    rng = np.random.default_rng(5)
    x[3:] = np.abs(rng.standard_normal((5, 64))).astype(np.float16)
    x[3:, ::7] = nz                                # -0 minima among positive values
    x[4:, 3] = pz
    got = _quantize_gpu(kp, x)
    ref = oracle.quantize(x)
    _assert_same_encoding(got, ref)
    assert list(got[2].view(np.uint16)[:2].ravel()) == [0x8000, 0x8000, 0x8000, 0x8000]


@pytest.mark.parametrize("rows,D", [(1, 32), (3, 96), (257, 64), (1001, 128), (77, 256)])
def test_quantize_ragged_shapes(kp, rows, D):
    rng = np.random.default_rng(rows * D)
    x = (rng.standard_normal((rows, D)) * rng.lognormal(0, 0.5, (1, D))).astype(np.float16)
    _assert_same_encoding(_quantize_gpu(kp, x), oracle.quantize(x))


def test_quantize_half_integer_quotients(kp):
    # Groups whose elements sit on, and one fp16 step either side of, (k + 0.5) * s for
    # random fp16 scales s: the quotients (x - b) / s land on or next to the rint ties,
    # where rounding the quotient any other way than the correctly rounded fp32 divide
    # would change a code.
    rng = np.random.default_rng(11)
    rows, D = 512, 256
    x = np.zeros((rows * D // 32, 32), np.float32)
    s = (2.0 ** rng.integers(-12, 6, len(x))) * rng.choice([1.0, 1.5, 1.25, 1.75, 1.375, 3.0 / 7], len(x))
    k = rng.integers(0, 15, (len(x), 30)) + 0.5
    x[:, 0] = 0.0
    x[:, 1] = 15.0 * s
    x[:, 2:] = k * s[:, None]
    x16 = x.astype(np.float16)
    step = rng.integers(-1, 2, x16[:, 2:].shape)          # one fp16 step down, none, up
    x16[:, 2:] = np.where(step < 0, np.nextafter(x16[:, 2:], np.float16(-np.inf)),
                          np.where(step > 0, np.nextafter(x16[:, 2:], np.float16(np.inf)), x16[:, 2:]))
    x16 = np.ascontiguousarray(x16.reshape(rows, D))
    _assert_same_encoding(_quantize_gpu(kp, x16), oracle.quantize(x16))


def test_quantize_full_mlx4g32_decode_shape(kp):
    inp = synth.generate(synth.MLX4_DECODE)
    for x in (inp.K, inp.V):
        rows = x.reshape(-1, 128)
        _assert_same_encoding(_quantize_gpu(kp, rows), oracle.quantize(rows))


# ------------------------------------------------------------------ M=1 decode, fp16
def test_decode_shape_all_32_layers(kp):
    case = synth.DECODE
    for layer in range(case.layers):
        inp = synth.generate(case, layer)
        kp.pion_prefix_store("t", 100 + layer, dev(inp.K), dev(inp.V))
        out, lse = query(kp, "t", 100 + layer, inp.Q)
        ref, ref_lse = oracle.prefix_query(inp.Q, inp.K, inp.V)
        check(out, lse, ref, ref_lse)
    assert kp.pion_prefix_drop("t", 131) == 1
    assert kp.pion_prefix_lookup("t", 131) == 0


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 1000, 4097])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_decode_ragged_lengths(kp, N, D):
    inp = synth.generate(synth.DECODE, 7, N=N, D=D, H_q=4, H_kv=4)
    kp.pion_prefix_store("t", 2, dev(inp.K), dev(inp.V))
    out, lse = query(kp, "t", 2, inp.Q)
    ref, ref_lse = oracle.prefix_query(inp.Q, inp.K, inp.V)
    check(out, lse, ref, ref_lse)


@pytest.mark.parametrize("H_q,H_kv", [(8, 1), (12, 4), (32, 2), (5, 3)])
def test_decode_gqa_and_arbitrary_maps(kp, H_q, H_kv):
    inp = synth.generate(synth.DECODE, 9, N=777, H_q=H_q, H_kv=H_kv)
    hm = synth.random_head_map(H_q, H_kv, 5) if H_q % H_kv else None
    kp.pion_prefix_store("t", 3, dev(inp.K), dev(inp.V))
    out, lse = query(kp, "t", 3, inp.Q, head_map=hm)
    ref, ref_lse = oracle.prefix_query(inp.Q, inp.K, inp.V, hm)
    check(out, lse, ref, ref_lse)
    hm2 = synth.random_head_map(H_q, H_kv, 11)
    out, lse = query(kp, "t", 3, inp.Q, head_map=hm2, want_lse=False)
    ref, _ = oracle.prefix_query(inp.Q, inp.K, inp.V, hm2)
    check(out, None, ref, None)


@pytest.mark.parametrize("N", [1, 31, 33, 777, 5000])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("H_q,H_kv", [(8, 2), (16, 2), (24, 3)])
def test_decode_gqa_mfma(kp, monkeypatch, N, D, H_q, H_kv):
    # the MFMA kernel for row groups of 4 to 8 q-heads at M = 1 (forced for every D and
    # group size here): one span for a few sub-tiles, split spans with the merge beyond;
    # with and without a fused suffix
    monkeypatch.setenv("PION_GQA_MFMA", "1")
    inp = synth.generate(synth.PREFILL, 12, N=N, M=1, S_suf=40, D=D, H_q=H_q, H_kv=H_kv)
    kp.pion_prefix_store("t", 6, dev(inp.K), dev(inp.V))
    out, lse = query(kp, "t", 6, inp.Q)
    check(out, lse, *oracle.prefix_query(inp.Q, inp.K, inp.V))
    out, lse = empty((H_q, 1, D)), empty((H_q, 1))
    kp.pion_prefix_query_fused("t", 6, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    check(host(out), host(lse), *oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf))


def test_decode_gqa_mfma_agrees_with_valu_path(kp, monkeypatch):
    inp = synth.generate(synth.DECODE, 13, N=3000, H_q=32, H_kv=4)
    hm = synth.random_head_map(32, 4, 3)
    kp.pion_prefix_store("t", 7, dev(inp.K), dev(inp.V))
    monkeypatch.setenv("PION_GQA_MFMA", "1")
    a, la = query(kp, "t", 7, inp.Q, head_map=hm)
    monkeypatch.delenv("PION_GQA_MFMA")
    monkeypatch.setenv("PION_NO_GQA_MFMA", "1")
    b, lb = query(kp, "t", 7, inp.Q, head_map=hm)
    ref, ref_lse = oracle.prefix_query(inp.Q, inp.K, inp.V, hm)
    check(a, la, ref, ref_lse)
    check(b, lb, ref, ref_lse)
    assert np.max(np.abs(a - b)) <= 2 * OUT_TOL


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("H_q,H_kv", [(16, 4), (20, 4), (24, 4), (32, 4)])
@pytest.mark.parametrize("force", ["PION_GQA_MFMA", "PION_NO_GQA_MFMA", None])
def test_decode_layers_gqa_groups(kp, monkeypatch, D, H_q, H_kv, force):
    # batched layers of 4 to 8 rows per kv-head (padded groups of 5 to 7 included) on
    # each kernel and on the default choice, with ragged prefix lengths per layer
    if force:
        monkeypatch.setenv(force, "1")
    Ns = [1, 33, 700, 2049, 3000, 64, 129, 1500]
    inputs = [synth.generate(synth.DECODE, 40 + l, N=N, D=D, H_q=H_q, H_kv=H_kv) for l, N in enumerate(Ns)]
    for l, inp in enumerate(inputs):
        kp.pion_prefix_store("t", 740 + l, dev(inp.K), dev(inp.V))
    out, lse = empty((len(Ns), H_q, 1, D)), empty((len(Ns), H_q, 1))
    kp.pion_prefix_query_layers("t", 740, dev(np.stack([i.Q for i in inputs])), out, lse)
    out, lse = host(out), host(lse)
    for l, inp in enumerate(inputs):
        check(out[l], lse[l], *oracle.prefix_query(inp.Q, inp.K, inp.V))
    for l in range(len(Ns)):
        kp.pion_prefix_drop("t", 740 + l)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_prefill_splits_without_keys(kp, D):
    # a short prefix under a long causal suffix: the key range is cut into 64-key splits,
    # and the first row blocks see no key in the later splits (their partials carry
    # weight 0 in the merge); the last row block is ragged
    inp = synth.generate(synth.PREFILL, 14, N=64, M=300, S_suf=300, D=D, H_q=6, H_kv=2)
    kp.pion_prefix_store("t", 8, dev(inp.K), dev(inp.V))
    out, lse = empty((6, 300, D)), empty((6, 300))
    kp.pion_prefix_query_fused("t", 8, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    check(host(out), host(lse), *oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf))
    kp.pion_prefix_drop("t", 8)


def test_restore_replaces_and_unknown_session(kp):
    import kv_cache_prefix_amd as k
    a = synth.generate(synth.DECODE, 1, N=100, H_q=2, H_kv=2)
    b = synth.generate(synth.DECODE, 2, N=300, H_q=2, H_kv=2)
    kp.pion_prefix_store("t", 4, dev(a.K), dev(a.V))
    kp.pion_prefix_store("t", 4, dev(b.K), dev(b.V))
    assert kp.pion_prefix_info("t", 4)[1] == 300
    out, lse = query(kp, "t", 4, b.Q)
    check(out, lse, *oracle.prefix_query(b.Q, b.K, b.V))
    with pytest.raises(k.PionError) as e:
        query(kp, "t", 999, b.Q)
    assert e.value.status == k.PION_ERR_NOT_FOUND


# ------------------------------------------------------------------ batched-Q and fused
@pytest.mark.parametrize("M,S_suf", [(1, 0), (5, 0), (1, 64), (7, 7), (3, 70), (70, 70)])
def test_fused_small(kp, M, S_suf):
    inp = synth.generate(synth.PREFILL, N=300, M=M, S_suf=S_suf, H_q=6, H_kv=2)
    kp.pion_prefix_store("t", 5, dev(inp.K), dev(inp.V))
    out = empty((6, M, 128))
    lse = empty((6, M))
    if S_suf:
        kp.pion_prefix_query_fused("t", 5, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    else:
        kp.pion_prefix_query_fused("t", 5, dev(inp.Q), None, None, out, lse, H_kv=2)
    ref, ref_lse = oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf)
    check(host(out), host(lse), ref, ref_lse)


def test_batched_query_matches_m1_rows(kp):
    inp = synth.generate(synth.PREFILL, N=500, M=9, S_suf=0, H_q=6, H_kv=2)
    kp.pion_prefix_store("t", 6, dev(inp.K), dev(inp.V))
    out, lse = query(kp, "t", 6, inp.Q)
    check(out, lse, *oracle.prefix_query(inp.Q, inp.K, inp.V))


def test_fused_prefill_full_size_all_rows(kp):
    # the full batched-Q workload in the launch configuration the bench times (key
    # splits and their merge kernel): every row of every q-head against the oracle
    case = synth.PREFILL
    inp = synth.generate(case)
    kp.pion_prefix_store("t", 7, dev(inp.K), dev(inp.V))
    out = empty((24, 512, 128))
    lse = empty((24, 512))
    kp.pion_prefix_query_fused("t", 7, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    out, lse = host(out), host(lse)
    ref, ref_lse = oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf)
    check(out, lse, ref, ref_lse)


# ------------------------------------------------------------------ mlx4g32 decode
def test_mlx4g32_decode_full_size(kp):
    case = synth.MLX4_DECODE
    inp = synth.generate(case)
    kp.pion_prefix_store("t", 8, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = query(kp, "t", 8, inp.Q, head_map=inp.head_map)
    Kh = oracle.dequantize(*oracle.quantize(inp.K.reshape(-1, 128))).reshape(inp.K.shape)
    Vh = oracle.dequantize(*oracle.quantize(inp.V.reshape(-1, 128))).reshape(inp.V.shape)
    ref, ref_lse = oracle.prefix_query(inp.Q, Kh, Vh, inp.head_map)
    check(out, lse, ref, ref_lse)


@pytest.mark.parametrize("N,D,H_q,H_kv", [(1, 64, 2, 2), (99, 128, 6, 2), (1000, 256, 8, 1)])
def test_mlx4g32_decode_ragged(kp, N, D, H_q, H_kv):
    inp = synth.generate(synth.MLX4_DECODE, 3, N=N, D=D, H_q=H_q, H_kv=H_kv)
    kp.pion_prefix_store("t", 9, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = query(kp, "t", 9, inp.Q)
    Kh = oracle.dequantize(*oracle.quantize(inp.K.reshape(-1, D))).reshape(inp.K.shape)
    Vh = oracle.dequantize(*oracle.quantize(inp.V.reshape(-1, D))).reshape(inp.V.shape)
    check(out, lse, *oracle.prefix_query(inp.Q, Kh, Vh))


def test_mlx4g32_fused_suffix(kp):
    inp = synth.generate(synth.MLX4_DECODE, 4, N=500, H_q=6, H_kv=2, M=3, S_suf=40)
    kp.pion_prefix_store("t", 10, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = empty((6, 3, 128)), empty((6, 3))
    kp.pion_prefix_query_fused("t", 10, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    Kh = oracle.dequantize(*oracle.quantize(inp.K.reshape(-1, 128))).reshape(inp.K.shape)
    Vh = oracle.dequantize(*oracle.quantize(inp.V.reshape(-1, 128))).reshape(inp.V.shape)
    check(host(out), host(lse), *oracle.prefix_query_fused(inp.Q, Kh, Vh, inp.K_suf, inp.V_suf))


def mlx4_ref(inp_K, inp_V):
    D = inp_K.shape[-1]
    Kh = oracle.dequantize(*oracle.quantize(inp_K.reshape(-1, D))).reshape(inp_K.shape)
    Vh = oracle.dequantize(*oracle.quantize(inp_V.reshape(-1, D))).reshape(inp_V.shape)
    return Kh, Vh


# q-heads per kv-head 1..4 fill one row group; 5 and 6 split into 4 + 1 and 4 + 2
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("H_q,H_kv", [(2, 2), (4, 2), (6, 2), (8, 2), (5, 1), (12, 2)])
def test_mlx4g32_every_row_count(kp, D, H_q, H_kv):
    inp = synth.generate(synth.MLX4_DECODE, 5, N=777, D=D, H_q=H_q, H_kv=H_kv)
    kp.pion_prefix_store("t", 11, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = query(kp, "t", 11, inp.Q)
    check(out, lse, *oracle.prefix_query(inp.Q, *mlx4_ref(inp.K, inp.V)))


# head dim 128 runs on the MFMA kernel by default; PION_NO_MLX4_MFMA=1 selects the vector
# kernel: both against the oracle, on several layers of different lengths in one launch
# (per-problem key counts, spans past a short problem's end) and on single M > 1 queries
@pytest.mark.parametrize("vector", [False, True])
def test_mlx4g32_d128_layers_both_kernels(kp, monkeypatch, vector):
    if vector:
        monkeypatch.setenv("PION_NO_MLX4_MFMA", "1")
    Ns = [1, 63, 64, 65, 700, 5000]
    inputs = [synth.generate(synth.MLX4_DECODE, 60 + l, N=N, H_q=6, H_kv=2) for l, N in enumerate(Ns)]
    for l, inp in enumerate(inputs):
        kp.pion_prefix_store("t", 40 + l, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    L = len(Ns)
    out, lse = empty((L, 6, 1, 128)), empty((L, 6, 1))
    kp.pion_prefix_query_layers("t", 40, dev(np.stack([i.Q for i in inputs])), out, lse)
    plan = kp.pion_prefix_last_plan()
    assert ("mlx4_split_kernel" if vector else "mlx4_mfma_kernel") in plan, plan
    out, lse = host(out), host(lse)
    for l, inp in enumerate(inputs):
        check(out[l], lse[l], *oracle.prefix_query(inp.Q, *mlx4_ref(inp.K, inp.V)))
    inp = synth.generate(synth.MLX4_DECODE, 70, N=3001, H_q=8, H_kv=2, M=5)
    kp.pion_prefix_store("t", 50, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = query(kp, "t", 50, inp.Q)
    check(out, lse, *oracle.prefix_query(inp.Q, *mlx4_ref(inp.K, inp.V)))
    kp.pion_prefix_drop("t", -1)


def test_mlx4g32_uneven_head_map(kp):
    # kv-head 0 gets 5 q-heads (groups of 4 and 1), kv-head 1 gets 2, kv-head 2 gets 1
    inp = synth.generate(synth.MLX4_DECODE, 6, N=300, H_q=8, H_kv=3)
    hm = np.array([0, 1, 0, 0, 2, 0, 1, 0], np.int32)
    kp.pion_prefix_store("t", 12, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = query(kp, "t", 12, inp.Q, head_map=hm)
    check(out, lse, *oracle.prefix_query(inp.Q, *mlx4_ref(inp.K, inp.V), hm))


def test_mlx4g32_large_values_stay_finite(kp):
    # values near the fp16 limit: group scales up to ~8.7e3, where a fp16 weight p * s
    # with p > 7.5 would overflow; the result must stay finite and close in relative terms
    inp = synth.generate(synth.MLX4_DECODE, 7, N=1000, H_q=6, H_kv=2)
    V = (inp.V.astype(np.float32) * 2.0e4).clip(-65504, 65504).astype(np.float16)
    kp.pion_prefix_store("t", 13, dev(inp.K), dev(V), kp.PION_KV_MLX4G32)
    out, lse = query(kp, "t", 13, inp.Q)
    ref, ref_lse = oracle.prefix_query(inp.Q, *mlx4_ref(inp.K, V))
    assert np.all(np.isfinite(out))
    scale = float(np.max(np.abs(V.astype(np.float64))))
    assert np.max(np.abs(out - ref)) <= 1e-3 * scale
    assert np.max(np.abs(lse - ref_lse)) <= LSE_TOL


def test_mlx4g32_rising_logits_rescale(kp):
    # logits rise along the sequence, so every key slot's running max keeps moving
    inp = synth.generate(synth.MLX4_DECODE, 8, N=4096, H_q=3, H_kv=1)
    ramp = np.linspace(0.0, 4.0, 4096, dtype=np.float32)[None, :, None]
    qdir = inp.Q[0, 0].astype(np.float32)
    K = (inp.K.astype(np.float32) * 0.5 + ramp * qdir / np.linalg.norm(qdir)).astype(np.float16)
    kp.pion_prefix_store("t", 14, dev(K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = query(kp, "t", 14, inp.Q)
    check(out, lse, *oracle.prefix_query(inp.Q, *mlx4_ref(K, inp.V)))


@pytest.mark.parametrize("D,H_q,H_kv", [(64, 8, 8), (128, 8, 8), (128, 24, 8)])
def test_mlx4g32_store_encoding_single_key(kp, D, H_q, H_kv):
    # One key per kv-head: out is that token's dequantized V row and lse its scaled
    # q . k over the dequantized K, so every code, scale and bias the store's encoder
    # wrote (K and V in one launch) shows up far above the 1e-5 tolerance if it differs
    # from the oracle's encoding (one code step moves a value by a whole scale).
    inp = synth.generate(synth.MLX4_DECODE, 19 + D + H_q, N=1, H_q=H_q, H_kv=H_kv, D=D)
    kp.pion_prefix_store("t", 16, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = query(kp, "t", 16, inp.Q)
    ref, ref_lse = oracle.prefix_query(inp.Q, *mlx4_ref(inp.K, inp.V))
    np.testing.assert_allclose(out, ref.reshape(out.shape), rtol=0, atol=1e-5)
    np.testing.assert_allclose(lse, ref_lse.reshape(lse.shape), rtol=0, atol=1e-5)
    kp.pion_prefix_drop("t", 16)


def test_mlx4g32_dominant_key(kp):
    # one key aligned with every query: its weight is ~1 and the rest ~0
    inp = synth.generate(synth.MLX4_DECODE, 9, N=2048, H_q=4, H_kv=1)
    K = inp.K.copy()
    qsum = inp.Q[:, 0].astype(np.float32).sum(0)
    K[0, 1234] = (40.0 * qsum / np.linalg.norm(qsum)).astype(np.float16)
    kp.pion_prefix_store("t", 15, dev(K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse = query(kp, "t", 15, inp.Q)
    check(out, lse, *oracle.prefix_query(inp.Q, *mlx4_ref(K, inp.V)))


# ------------------------------------------------------------------ sparse-auto
def sparse_call(kp, sid, layer, inp, B, K_top, H_kv, suffix=True, head_map=None):
    import torch
    H_q, _, D = inp.Q.shape
    out, lse = empty((H_q, D)), empty((H_q,))
    blocks = torch.full((H_kv, K_top), -7, dtype=torch.int32, device="cuda")
    ks = dev(inp.K_suf) if (suffix and inp.K_suf is not None) else None
    vs = dev(inp.V_suf) if (suffix and inp.V_suf is not None) else None
    kp.pion_prefix_query_sparse_auto(sid, layer, dev(inp.Q), B, K_top, out, lse, blocks,
                                     ks, vs, head_map=head_map, H_kv=H_kv)
    return host(out), host(lse), host(blocks)


@pytest.mark.parametrize("force", ["PION_GQA_MFMA", "PION_NO_GQA_MFMA", None])
def test_sparse_auto_full_size(kp, monkeypatch, force):
    # the attention over the chosen blocks on the grouped-query MFMA kernel, on the
    # vector kernel, and on the default choice
    if force:
        monkeypatch.setenv(force, "1")
    case = synth.SPARSE
    inp = synth.generate(case)
    kp.pion_prefix_store("t", 11, dev(inp.K), dev(inp.V))
    for fused in (True, False):
        out, lse, blocks = sparse_call(kp, "t", 11, inp, case.B, case.K_top, 1, suffix=fused)
        ref, ref_lse, ref_blocks = oracle.prefix_query_sparse_auto(
            inp.Q, inp.K, inp.V, case.B, case.K_top, inp.head_map,
            inp.K_suf if fused else None, inp.V_suf if fused else None)
        np.testing.assert_array_equal(blocks, ref_blocks)
        np.testing.assert_array_equal(blocks[0], inp.needles[0])
        check(out, lse, ref, ref_lse)


@pytest.mark.parametrize("N,B,K_top", [(1000, 64, 3), (640, 64, 10), (650, 64, 40), (257, 16, 5)])
def test_sparse_auto_edges(kp, N, B, K_top):
    inp = synth.generate(synth.SPARSE, 2, N=N, H_q=4, H_kv=2, D=64, S_suf=12, n_needles=2)
    kp.pion_prefix_store("t", 12, dev(inp.K), dev(inp.V))
    out, lse, blocks = sparse_call(kp, "t", 12, inp, B, K_top, 2)
    ref, ref_lse, ref_blocks = oracle.prefix_query_sparse_auto(
        inp.Q, inp.K, inp.V, B, K_top, inp.head_map, inp.K_suf, inp.V_suf)
    np.testing.assert_array_equal(blocks, ref_blocks)
    check(out, lse, ref, ref_lse)


def check_selection(blocks, Q, K, B, K_top, head_map=None):
    """The chosen blocks are a valid top-K: ascending, distinct, -1 padded, and every
    chosen block scores (oracle, fp64) at least as high as every other block, up to the
    rounding bound of an fp32 score (2^-12 of the sum of |q_h| . |K_mean| per block).
    Blocks whose scores differ by less than that bound may rank either way."""
    H_q, _, D = Q.shape
    H_kv, N, _ = K.shape
    hm = oracle.resolve_head_map(H_q, H_kv, head_map)
    km = oracle.block_means(K, B)
    score = oracle.block_scores(Q[:, 0, :], km, hm)
    bound = 2.0 ** -12 * oracle.block_scores(np.abs(Q[:, 0, :].astype(np.float64)), np.abs(km), hm)
    nb = km.shape[1]
    n = min(K_top, nb)
    for g in range(H_kv):
        row = blocks[g]
        assert (row[n:] == -1).all()
        sel = row[:n]
        assert (np.diff(sel) > 0).all() and sel[0] >= 0 and sel[-1] < nb
        rest = np.setdiff1d(np.arange(nb), sel)
        if len(rest):
            worst = np.argmin(score[g, sel] + bound[g, sel])
            best = np.argmax(score[g, rest] - bound[g, rest])
            assert score[g, sel][worst] + bound[g, sel][worst] >= score[g, rest][best] - bound[g, rest][best]


def assert_unique_selection(Q, K, B, K_top, head_map=None):
    """The oracle's K_top-th and next block scores are separated by more than ten times
    the rounding bound of an fp32 score, so the top-K set is decided the same way in any
    precision the kernel may use: the selection is unique by construction."""
    H_q, _, D = Q.shape
    H_kv = K.shape[0]
    hm = oracle.resolve_head_map(H_q, H_kv, head_map)
    km = oracle.block_means(K, B)
    score = oracle.block_scores(Q[:, 0, :], km, hm)
    bound = 2.0 ** -12 * oracle.block_scores(np.abs(Q[:, 0, :].astype(np.float64)), np.abs(km), hm)
    for g in range(H_kv):
        order = np.argsort(-score[g], kind="stable")
        if K_top < len(order):
            a, b = order[K_top - 1], order[K_top]
            assert score[g, a] - score[g, b] > 10 * (bound[g, a] + bound[g, b])


# K_top above 64, or more per-workgroup candidates than the candidate merge holds: the
# selection runs the radix select. Needle blocks planted (+3 sigma along the query
# direction, per 64-token block, so 64 / B selected blocks each) make the top K_top
# unique by construction; the picked indices must equal the oracle's bit for bit.
@pytest.mark.parametrize("N,B,K_top,needles",
                         [(20000, 16, 100, 25), (70000, 16, 20, 5), (64 * 300, 64, 65, 65),
                          (64 * 1500, 64, 1024, 1024)])
def test_sparse_auto_radix_select(kp, N, B, K_top, needles):
    inp = synth.generate(synth.SPARSE, 6, N=N, H_q=4, H_kv=2, D=64, S_suf=12, n_needles=needles)
    assert needles * (synth.SPARSE.B // B) == K_top
    assert_unique_selection(inp.Q, inp.K, B, K_top, inp.head_map)
    kp.pion_prefix_store("t", 16, dev(inp.K), dev(inp.V))
    out, lse, blocks = sparse_call(kp, "t", 16, inp, B, K_top, 2)
    ref, ref_lse, ref_blocks = oracle.prefix_query_sparse_auto(
        inp.Q, inp.K, inp.V, B, K_top, inp.head_map, inp.K_suf, inp.V_suf)
    np.testing.assert_array_equal(blocks, ref_blocks)
    planted = synth.SPARSE.B // B
    for g in range(2):
        want = sorted(planted * n + i for n in inp.needles[g] for i in range(planted))
        np.testing.assert_array_equal(ref_blocks[g], want)
    check_selection(blocks, inp.Q, inp.K, B, K_top, inp.head_map)
    check(out, lse, ref, ref_lse)


@pytest.mark.parametrize("K_top", [10, 100])
def test_sparse_auto_all_blocks_tied(kp, K_top):
    # identical blocks score identically: the lowest indices win (candidate merge for 10,
    # radix select for 100)
    inp = synth.generate(synth.SPARSE, 7, N=16 * 300, H_q=2, H_kv=1, D=64, S_suf=0, n_needles=0)
    K = np.broadcast_to(inp.K[:, :1, :], inp.K.shape).copy()
    kp.pion_prefix_store("t", 17, dev(K), dev(inp.V))
    inp.K = K
    out, lse, blocks = sparse_call(kp, "t", 17, inp, 16, K_top, 1, suffix=False)
    np.testing.assert_array_equal(blocks[0], np.arange(K_top))
    ref, ref_lse, ref_blocks = oracle.prefix_query_sparse_auto(inp.Q, K, inp.V, 16, K_top)
    np.testing.assert_array_equal(ref_blocks[0], np.arange(K_top))
    check(out, lse, ref, ref_lse)


def test_sparse_auto_tie_goes_to_lower_block(kp):
    inp = synth.generate(synth.SPARSE, 3, N=64 * 20, H_q=2, H_kv=1, D=128, S_suf=0, n_needles=0)
    K = inp.K.copy()
    K[0, 13 * 64:14 * 64] = K[0, 4 * 64:5 * 64]            # block 13 duplicates block 4
    km = oracle.block_means(K, 64)
    Q = inp.Q.copy()
    Q[:, 0, :] = (km[0, 4] * 4).astype(np.float16)            # point both heads at block 4
    inp.Q, inp.K = Q, K
    kp.pion_prefix_store("t", 13, dev(K), dev(inp.V))
    out, lse, blocks = sparse_call(kp, "t", 13, inp, 64, 1, 1, suffix=False)
    ref, ref_lse, ref_blocks = oracle.prefix_query_sparse_auto(Q, K, inp.V, 64, 1)
    assert ref_blocks[0, 0] == 4 and blocks[0, 0] == 4
    check(out, lse, ref, ref_lse)


def test_sparse_auto_mlx4g32_slot(kp):
    inp = synth.generate(synth.SPARSE, 4, N=64 * 30, H_q=4, H_kv=1, D=128, S_suf=8, n_needles=3)
    kp.pion_prefix_store("t", 14, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    out, lse, blocks = sparse_call(kp, "t", 14, inp, 64, 3, 1)
    Kh = oracle.dequantize(*oracle.quantize(inp.K.reshape(-1, 128))).reshape(inp.K.shape)
    Vh = oracle.dequantize(*oracle.quantize(inp.V.reshape(-1, 128))).reshape(inp.V.shape)
    ref, ref_lse, ref_blocks = oracle.prefix_query_sparse_auto(inp.Q, Kh, Vh, 64, 3, None,
                                                               inp.K_suf, inp.V_suf)
    np.testing.assert_array_equal(blocks, ref_blocks)
    np.testing.assert_array_equal(blocks[0], inp.needles[0])
    check(out, lse, ref, ref_lse)


# ------------------------------------------------------------------ caller-supplied indices
def sparse_indices(rng, H, N, K_sparse_max):
    idx = rng.integers(-3, N + 3, size=(H, K_sparse_max)).astype(np.int32)  # a few out of range
    if K_sparse_max > 4:
        idx[:, 1] = idx[:, 0]                                            # a repeated token
    counts = rng.integers(0, K_sparse_max + 1, size=H).astype(np.int32)
    counts[0] = K_sparse_max
    if H > 2:
        counts[1] = 0                                                    # an empty head
        counts[2] = K_sparse_max + 5                                     # clamps
    return idx, counts


def check_sparse(out, lse, ref, ref_lse):
    empty = np.isneginf(ref_lse)
    assert (out[empty] == 0).all() and np.isneginf(lse[empty]).all()
    check(out[~empty], lse[~empty], ref[~empty], ref_lse[~empty])


@pytest.mark.parametrize("K_sparse_max", [1, 63, 700, 3000])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_query_sparse_indices(kp, D, K_sparse_max):
    import torch
    rng = np.random.default_rng(D + K_sparse_max)
    H, N = 4, 5000
    inp = synth.generate(synth.DECODE, 14, N=N, D=D, H_q=H, H_kv=H)
    kp.pion_prefix_store("t", 18, dev(inp.K), dev(inp.V))
    idx, counts = sparse_indices(rng, H, N, K_sparse_max)
    out, lse = empty((H, D)), empty((H,))
    kp.pion_prefix_query_sparse("t", 18, dev(inp.Q), dev(idx), dev(counts), out, lse)
    ref, ref_lse = oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, counts)
    check_sparse(host(out), host(lse), ref, ref_lse)


def test_query_sparse_all_tokens_equals_dense_query(kp):
    inp = synth.generate(synth.DECODE, 15, N=3000, H_q=8, H_kv=8)
    kp.pion_prefix_store("t", 19, dev(inp.K), dev(inp.V))
    idx = np.tile(np.arange(3000, dtype=np.int32), (8, 1))
    out = empty((8, 128))
    kp.pion_prefix_query_sparse("t", 19, dev(inp.Q), dev(idx), dev(np.full(8, 3000, np.int32)), out)
    dense, _ = query(kp, "t", 19, inp.Q, want_lse=False)
    assert np.max(np.abs(host(out) - dense[:, 0])) <= 2e-4
    check(host(out), None, oracle.prefix_query(inp.Q, inp.K, inp.V)[0][:, 0], None)


def test_query_sparse_rejects_bad_arguments(kp):
    import kv_cache_prefix_amd as k
    inp = synth.generate(synth.DECODE, 16, N=100, H_q=2, H_kv=2, D=64)
    kp.pion_prefix_store("t", 20, dev(inp.K), dev(inp.V))
    idx, counts = dev(np.zeros((2, 4), np.int32)), dev(np.ones(2, np.int32))
    out = empty((2, 64))
    with pytest.raises(k.PionError) as e:  # H differs from the stored H
        kp.pion_prefix_query_sparse("t", 20, dev(np.zeros((3, 1, 64), np.float16)),
                                    dev(np.zeros((3, 4), np.int32)), dev(np.ones(3, np.int32)),
                                    empty((3, 64)))
    assert e.value.status == k.PION_ERR_INVALID
    kp.pion_prefix_store("t", 21, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    with pytest.raises(k.PionError) as e:
        kp.pion_prefix_query_sparse("t", 21, dev(inp.Q), idx, counts, out)
    assert e.value.status == k.PION_ERR_UNSUPPORTED


# ------------------------------------------------------------------ streams
def test_store_on_one_stream_query_on_another(kp):
    import torch
    inp = synth.generate(synth.DECODE, 5, N=3000, H_q=8, H_kv=8)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    K, V, Q = dev(inp.K), dev(inp.V), dev(inp.Q)
    torch.cuda.synchronize()
    out, lse = empty((8, 1, 128)), empty((8, 1))
    kp.pion_prefix_store("t", 15, K, V, stream=s1)
    kp.pion_prefix_query("t", 15, Q, out, lse, stream=s2)
    torch.cuda.synchronize()
    check(host(out), host(lse), *oracle.prefix_query(inp.Q, inp.K, inp.V))


# ------------------------------------------------------------------ batched layers
def test_query_layers_decode_shape(kp):
    import torch
    case = synth.DECODE
    inputs = [synth.generate(case, l) for l in range(case.layers)]
    for l, inp in enumerate(inputs):
        kp.pion_prefix_store("t", 200 + l, dev(inp.K), dev(inp.V))
    Q = dev(np.stack([inp.Q for inp in inputs]))
    out, lse = empty((32, 8, 1, 128)), empty((32, 8, 1))
    kp.pion_prefix_query_layers("t", 200, Q, out, lse)
    out, lse = host(out), host(lse)
    for l, inp in enumerate(inputs):
        check(out[l], lse[l], *oracle.prefix_query(inp.Q, inp.K, inp.V))
    # the same numbers as the per-layer call
    o1, l1 = query(kp, "t", 213, inputs[13].Q)
    np.testing.assert_allclose(out[13], o1, atol=1e-6)


def test_query_layers_ragged_lengths_and_gqa(kp):
    Ns = [1, 65, 300, 2049, 77]
    inputs = [synth.generate(synth.MLX4_DECODE, l, N=N, H_q=6, H_kv=2, D=64, M=3)
              for l, N in enumerate(Ns)]
    for l, inp in enumerate(inputs):
        kp.pion_prefix_store("t", 300 + l, dev(inp.K), dev(inp.V))
    hm = np.array([1, 0, 1, 1, 0, 0], np.int32)
    Q = dev(np.stack([inp.Q for inp in inputs]))
    out, lse = empty((5, 6, 3, 64)), empty((5, 6, 3))
    kp.pion_prefix_query_layers("t", 300, Q, out, lse, head_map=hm)
    out, lse = host(out), host(lse)
    for l, inp in enumerate(inputs):
        check(out[l], lse[l], *oracle.prefix_query(inp.Q, inp.K, inp.V, hm))


def test_query_layers_mlx4g32(kp):
    inputs = [synth.generate(synth.MLX4_DECODE, l, N=1000 + 100 * l, H_q=24, H_kv=8)
              for l in range(3)]
    for l, inp in enumerate(inputs):
        kp.pion_prefix_store("t", 400 + l, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
    Q = dev(np.stack([inp.Q for inp in inputs]))
    out, lse = empty((3, 24, 1, 128)), empty((3, 24, 1))
    kp.pion_prefix_query_layers("t", 400, Q, out, lse)
    out, lse = host(out), host(lse)
    for l, inp in enumerate(inputs):
        Kh = oracle.dequantize(*oracle.quantize(inp.K.reshape(-1, 128))).reshape(inp.K.shape)
        Vh = oracle.dequantize(*oracle.quantize(inp.V.reshape(-1, 128))).reshape(inp.V.shape)
        check(out[l], lse[l], *oracle.prefix_query(inp.Q, Kh, Vh))


def test_query_layers_rejects_mixed_slots(kp):
    import kv_cache_prefix_amd as k
    a = synth.generate(synth.DECODE, 1, N=100, H_q=2, H_kv=2)
    kp.pion_prefix_store("t", 500, dev(a.K), dev(a.V))
    kp.pion_prefix_store("t", 501, dev(a.K), dev(a.V), kp.PION_KV_MLX4G32)
    Q = dev(np.stack([a.Q, a.Q]))
    out = empty((2, 2, 1, 128))
    with pytest.raises(k.PionError) as e:
        kp.pion_prefix_query_layers("t", 500, Q, out)
    assert e.value.status == k.PION_ERR_INVALID
    with pytest.raises(k.PionError) as e:
        kp.pion_prefix_query_layers("t", 501, Q, out)   # layer 502 absent
    assert e.value.status == k.PION_ERR_NOT_FOUND
    assert np.all(np.isnan(host(out)))                  # nothing written on error


# ------------------------------------------------------------------ MFMA batched-Q path
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("N,M,S_suf", [(300, 40, 40), (1000, 130, 200), (64, 32, 0), (777, 257, 0)])
def test_mfma_prefill_shapes(kp, D, N, M, S_suf):
    inp = synth.generate(synth.PREFILL, 11, N=N, M=M, S_suf=S_suf, H_q=6, H_kv=2, D=D)
    kp.pion_prefix_store("t", 600, dev(inp.K), dev(inp.V))
    out, lse = empty((6, M, D)), empty((6, M))
    if S_suf:
        kp.pion_prefix_query_fused("t", 600, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    else:
        kp.pion_prefix_query("t", 600, dev(inp.Q), out, lse)
    out, lse = host(out), host(lse)
    rng = np.random.default_rng(N + M)
    rows = [(h, i) for h in range(6) for i in (0, M - 1)] + \
        [(int(h), int(i)) for h, i in zip(rng.integers(0, 6, 30), rng.integers(0, M, 30))]
    ref, ref_lse = oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf, rows=rows)
    check(out, lse, ref, ref_lse, rows=rows)
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_mfma_prefill_single_split(kp, monkeypatch, D):
    # one split per row block: the kernel writes normalized out and lse itself, with no
    # merge kernel (forced here; also the plan for at most 32 keys, the second call)
    monkeypatch.setenv("PION_PREFILL_SPLITS", "1")
    inp = synth.generate(synth.PREFILL, 15, N=1000, M=200, S_suf=250, D=D, H_q=4, H_kv=2)
    kp.pion_prefix_store("t", 605, dev(inp.K), dev(inp.V))
    out, lse = empty((4, 200, D)), empty((4, 200))
    kp.pion_prefix_query_fused("t", 605, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    assert kp.pion_prefix_last_plan() == f"prefill_kernel<{D}>"
    check(host(out), host(lse), *oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf))
    monkeypatch.delenv("PION_PREFILL_SPLITS")
    inp = synth.generate(synth.PREFILL, 16, N=20, M=64, S_suf=0, D=D, H_q=4, H_kv=2)
    kp.pion_prefix_store("t", 606, dev(inp.K), dev(inp.V))
    out, lse = empty((4, 64, D)), empty((4, 64))
    kp.pion_prefix_query("t", 606, dev(inp.Q), out, lse)
    assert kp.pion_prefix_last_plan() == f"prefill_kernel<{D}>"
    check(host(out), host(lse), *oracle.prefix_query(inp.Q, inp.K, inp.V))


def test_mfma_prefill_sixteen_splits_fp16_partials(kp):
    # One 128-row block per q-head and a long prefix: the plan's largest split count (16)
    # per row block, each split stored as an fp16 normalized partial with its fp32
    # log-sum-exp and merged by the LSE rule. V scaled by 4 (exact in fp16) makes the
    # partials' fp16 rounding four times larger; every row against the oracle.
    inp = synth.generate(synth.PREFILL, 17, N=8000, M=100, S_suf=100, D=128, H_q=2, H_kv=1)
    V4, Vs4 = (inp.V * 4).astype(np.float16), (inp.V_suf * 4).astype(np.float16)
    kp.pion_prefix_store("t", 607, dev(inp.K), dev(V4))
    out, lse = empty((2, 100, 128)), empty((2, 100))
    kp.pion_prefix_query_fused("t", 607, dev(inp.Q), dev(inp.K_suf), dev(Vs4), out, lse)
    check(host(out), host(lse), *oracle.prefix_query_fused(inp.Q, inp.K, V4, inp.K_suf, Vs4))
    kp.pion_prefix_drop("t", 607)


@pytest.mark.parametrize("seed", range(12))
def test_mfma_prefill_random_shapes(kp, seed):
    # Seeded random shapes: every head dim (with and without LDS padding) once without a
    # suffix and once with a causal suffix (the M queries and up to 200 keys before
    # them); ragged prefix lengths (tiles and splits ending mid-tile), H_q a multiple of
    # H_kv. Rows: the first and last of every 128-row block, plus random ones.
    rng = np.random.default_rng(1000 + seed)
    D = (64, 96, 128, 160, 192, 256)[seed % 6]
    H_kv = int(rng.integers(1, 4))
    H_q = H_kv * int(rng.integers(1, 4))
    N = int(rng.integers(1, 3000))
    M = int(rng.integers(32, 300))
    S_suf = M + int(rng.integers(0, 200)) if seed >= 6 else 0
    inp = synth.generate(synth.PREFILL, 2000 + seed, N=N, M=M, S_suf=S_suf, H_q=H_q,
                         H_kv=H_kv, D=D)
    kp.pion_prefix_store("t", 604, dev(inp.K), dev(inp.V))
    out, lse = empty((H_q, M, D)), empty((H_q, M))
    if S_suf:
        kp.pion_prefix_query_fused("t", 604, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
    else:
        kp.pion_prefix_query("t", 604, dev(inp.Q), out, lse)
    ends = sorted({i for b in range(0, M, 128) for i in (b, min(b + 127, M - 1))})
    rows = [(h, i) for h in range(H_q) for i in ends] + \
        [(int(h), int(i)) for h, i in zip(rng.integers(0, H_q, 24), rng.integers(0, M, 24))]
    ref, ref_lse = oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf, rows=rows)
    check(host(out), host(lse), ref, ref_lse, rows=rows)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("growth", [12.0, 60.0])
def test_mfma_prefill_running_max_growth(kp, D, growth):
    # Scores that rise along the keys: K gets a ramp in the direction of every query, so a
    # row's max keeps growing tile after tile by `growth` log2 units in all. At 12 the
    # running max never has to move after the first tile (weights up to 2^12 in fp16);
    # at 60 it moves several times mid-stream, rescaling accumulated O and l. All rows.
    N, M, S_suf, H_q, H_kv = 1500, 200, 200, 4, 2
    inp = synth.generate(synth.PREFILL, 14, N=N, M=M, S_suf=S_suf, H_q=H_q, H_kv=H_kv, D=D)
    rng = np.random.default_rng(14)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    c = 8.0                                           # |q| along u
    qscale = np.log2(np.e) / np.sqrt(D)
    r_max = growth / (c * qscale)                     # ramp end: growth log2 units above 0
    ramp = np.linspace(0.0, r_max, N + S_suf)
    Q = (0.25 * inp.Q.astype(np.float64) + c * u).astype(np.float16)
    K = (0.25 * inp.K.astype(np.float64) + ramp[None, :N, None] * u).astype(np.float16)
    K_suf = (0.25 * inp.K_suf.astype(np.float64) + ramp[None, N:, None] * u).astype(np.float16)
    kp.pion_prefix_store("t", 603, dev(K), dev(inp.V))
    out, lse = empty((H_q, M, D)), empty((H_q, M))
    kp.pion_prefix_query_fused("t", 603, dev(Q), dev(K_suf), dev(inp.V_suf), out, lse)
    check(host(out), host(lse), *oracle.prefix_query_fused(Q, K, inp.V, K_suf, inp.V_suf))


def test_mfma_prefill_arbitrary_head_map_all_rows(kp):
    inp = synth.generate(synth.PREFILL, 12, N=200, M=48, S_suf=50, H_q=5, H_kv=3)
    hm = synth.random_head_map(5, 3, 7)
    kp.pion_prefix_store("t", 601, dev(inp.K), dev(inp.V))
    out, lse = empty((5, 48, 128)), empty((5, 48))
    kp.pion_prefix_query_fused("t", 601, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse,
                               head_map=hm)
    check(host(out), host(lse), *oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf,
                                                           inp.V_suf, hm))


def test_mfma_and_valu_paths_agree(kp, monkeypatch):
    inp = synth.generate(synth.PREFILL, 13, N=500, M=64, S_suf=64, H_q=6, H_kv=2)
    kp.pion_prefix_store("t", 602, dev(inp.K), dev(inp.V))
    outs = []
    for flag in ("0", "1"):
        monkeypatch.setenv("PION_NO_MFMA", flag)
        out, lse = empty((6, 64, 128)), empty((6, 64))
        kp.pion_prefix_query_fused("t", 602, dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf), out, lse)
        outs.append((host(out), host(lse)))
    ref, ref_lse = oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf)
    for o, l in outs:
        check(o, l, ref, ref_lse)


# ------------------------------------------------------------------ bench shapes of the NEXT rows
def test_query_sparse_bench_shape(kp):
    # the QUERY_SPARSE bench workload: H = 8, N = 65536, D = 128, 2048 random indices per head
    import torch
    H, N, D, KS = 8, 65536, 128, 2048
    inp = synth.generate(synth.DECODE, 21, N=N, H_q=H, H_kv=H, D=D)
    rng = np.random.default_rng(21)
    idx = rng.integers(0, N, size=(H, KS)).astype(np.int32)
    counts = np.full(H, KS, np.int32)
    kp.pion_prefix_store("t", 900, dev(inp.K), dev(inp.V))
    out, lse = empty((H, D)), empty((H,))
    kp.pion_prefix_query_sparse("t", 900, dev(inp.Q), dev(idx), dev(counts), out, lse)
    check(host(out), host(lse), *oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, counts))
    kp.pion_prefix_drop("t", 900)


def test_vstore_fetch_bench_shape(kp):
    # one layer-side of the V-store bench workload: N = 2048 tokens, kv = 8 x 128, records
    from oracle import vstore as ovs
    rec = synth.mlx4_records(2048, 1024, 31)
    assert rec.shape == (2048, 640)
    out = empty((2048, 1024))
    kp.pion_vstore_fetch_f32(dev(rec), ovs.MLX4G32, 1024, 0, 2048, out)
    want = ovs.fetch_f32(rec, ovs.MLX4G32, 1024, 0, 2048)
    np.testing.assert_array_equal(host(out).view(np.uint32), want.view(np.uint32))


# ------------------------------------------------------------------ HIP graph capture
def test_graph_replays_match_eager_calls(kp):
    # Two decode calls whose keys are split (partial stores, ticket, in-kernel merge) and
    # a fused prefill (split kernel and merge kernel), captured into one HIP graph. Each
    # replay, with eager work and synchronizations between replays, must reproduce the
    # eager calls bit for bit: the ticket counters reset themselves inside the kernels.
    import torch
    s = torch.cuda.Stream()
    dec = [synth.generate(synth.DECODE, l) for l in range(2)]
    for l, inp in enumerate(dec):
        kp.pion_prefix_store("t", 700 + l, dev(inp.K), dev(inp.V))
    pre = synth.generate(synth.PREFILL, 17, N=500, M=64, S_suf=64, H_q=6, H_kv=2)
    kp.pion_prefix_store("t", 702, dev(pre.K), dev(pre.V))
    Qd = [dev(inp.Q) for inp in dec]
    Qp, Ks, Vs = dev(pre.Q), dev(pre.K_suf), dev(pre.V_suf)
    outs = [empty((8, 1, 128)), empty((8, 1)), empty((8, 1, 128)), empty((8, 1)),
            empty((6, 64, 128)), empty((6, 64))]

    def calls():
        kp.pion_prefix_query("t", 700, Qd[0], outs[0], outs[1], stream=s)
        kp.pion_prefix_query("t", 701, Qd[1], outs[2], outs[3], stream=s)
        kp.pion_prefix_query_fused("t", 702, Qp, Ks, Vs, outs[4], outs[5], stream=s)

    with torch.cuda.stream(s):
        calls()                       # eager: also sets up the stream's workspace
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    check(host(ref[0]), host(ref[1]), *oracle.prefix_query(dec[0].Q, dec[0].K, dec[0].V))
    check(host(ref[4]), host(ref[5]), *oracle.prefix_query_fused(pre.Q, pre.K, pre.V,
                                                                 pre.K_suf, pre.V_suf))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    x_out, x_lse = empty((8, 1, 128)), empty((8, 1))
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {rep} differs from the eager call"
        kp.pion_prefix_query("t", 701, Qd[1], x_out, x_lse)   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(x_out, ref[2])
    for l in range(3):
        kp.pion_prefix_drop("t", 700 + l)


def test_concurrent_queries_on_four_streams(kp):
    # split queries (partial stores, tickets, merges) and a fused prefill issued on four
    # streams at once, no synchronization between the streams: each stream has its own
    # workspace and ticket counters, so the launches may overlap freely
    import torch
    streams = [torch.cuda.Stream() for _ in range(4)]
    layers = [synth.generate(synth.DECODE, 20 + l, N=1500 + 300 * l) for l in range(8)]
    for l, inp in enumerate(layers):
        kp.pion_prefix_store("t", 720 + l, dev(inp.K), dev(inp.V))
    pre = synth.generate(synth.PREFILL, 18, N=700, M=96, S_suf=96, H_q=6, H_kv=2)
    kp.pion_prefix_store("t", 730, dev(pre.K), dev(pre.V))
    Qs = [dev(inp.Q) for inp in layers]
    outs = [(empty((8, 1, 128)), empty((8, 1))) for _ in range(16)]
    pout, plse = empty((6, 96, 128)), empty((6, 96))
    torch.cuda.synchronize()
    for k in range(16):                              # two rounds over the eight layers
        l, s = k % 8, streams[k % 4]
        kp.pion_prefix_query("t", 720 + l, Qs[l], outs[k][0], outs[k][1], stream=s)
        if k == 5:
            kp.pion_prefix_query_fused("t", 730, dev(pre.Q), dev(pre.K_suf), dev(pre.V_suf),
                                       pout, plse, stream=s)
    torch.cuda.synchronize()
    for k in range(16):
        inp = layers[k % 8]
        check(host(outs[k][0]), host(outs[k][1]), *oracle.prefix_query(inp.Q, inp.K, inp.V))
    check(host(pout), host(plse), *oracle.prefix_query_fused(pre.Q, pre.K, pre.V, pre.K_suf,
                                                             pre.V_suf))
    for l in range(9):
        kp.pion_prefix_drop("t", 720 + l if l < 8 else 730)


def test_mlx4g32_store_on_one_stream_query_on_another(kp):
    # the store quantizes on its stream; a query on another stream, issued at once, waits
    # for the codes (the slot's ready event)
    import torch
    inp = synth.generate(synth.MLX4_DECODE, 6, N=5000, H_q=6, H_kv=2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    K, V, Q = dev(inp.K), dev(inp.V), dev(inp.Q)
    torch.cuda.synchronize()
    out, lse = empty((6, 1, 128)), empty((6, 1))
    kp.pion_prefix_store("t", 16, K, V, kp.PION_KV_MLX4G32, stream=s1)
    kp.pion_prefix_query("t", 16, Q, out, lse, head_map=inp.head_map, stream=s2)
    torch.cuda.synchronize()
    Kh = oracle.dequantize(*oracle.quantize(inp.K.reshape(-1, 128))).reshape(inp.K.shape)
    Vh = oracle.dequantize(*oracle.quantize(inp.V.reshape(-1, 128))).reshape(inp.V.shape)
    check(host(out), host(lse), *oracle.prefix_query(inp.Q, Kh, Vh, inp.head_map))
    kp.pion_prefix_drop("t", 16)


def test_sparse_auto_block_means_shared_across_streams(kp):
    # the first query builds the slot's block means on its stream; a second query on
    # another stream, issued without waiting, must wait for that build (the cache's
    # ready event) and pick the same blocks
    import torch
    case = synth.SPARSE
    inp = synth.generate(case, 3, N=16384, H_q=8, H_kv=1, D=256, n_needles=8)
    kp.pion_prefix_store("t", 17, dev(inp.K), dev(inp.V))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    Q, Ks, Vs = dev(inp.Q), dev(inp.K_suf), dev(inp.V_suf)
    res = []
    torch.cuda.synchronize()
    for s in (s1, s2):
        out, lse = empty((8, 256)), empty((8,))
        blocks = torch.full((1, case.K_top), -7, dtype=torch.int32, device="cuda")
        kp.pion_prefix_query_sparse_auto("t", 17, Q, case.B, case.K_top, out, lse, blocks, Ks, Vs,
                                         H_kv=1, stream=s)
        res.append((out, lse, blocks))
    torch.cuda.synchronize()
    ref, ref_lse, ref_blocks = oracle.prefix_query_sparse_auto(
        inp.Q, inp.K, inp.V, case.B, case.K_top, None, inp.K_suf, inp.V_suf)
    for out, lse, blocks in res:
        np.testing.assert_array_equal(host(blocks), ref_blocks)
        check(host(out), host(lse), ref, ref_lse)
    kp.pion_prefix_drop("t", 17)


def test_store_replacing_a_slot_while_a_query_reads_it(kp):
    # a query on one stream, then at once a store that replaces the same slot from another
    # stream: the query reads the old K/V to the end (the old memory is released only
    # after the work queued on it), and a query after the store sees the new K/V
    import torch
    old = synth.generate(synth.DECODE, 7, N=30000, H_q=8, H_kv=8)
    new = synth.generate(synth.DECODE, 8, N=30000, H_q=8, H_kv=8)
    kp.pion_prefix_store("t", 18, dev(old.K), dev(old.V))
    Knew, Vnew, Q = dev(new.K), dev(new.V), dev(old.Q)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    out_a, lse_a = empty((8, 1, 128)), empty((8, 1))
    out_b, lse_b = empty((8, 1, 128)), empty((8, 1))
    kp.pion_prefix_query("t", 18, Q, out_a, lse_a, stream=s1)
    kp.pion_prefix_store("t", 18, Knew, Vnew, stream=s2)
    kp.pion_prefix_query("t", 18, Q, out_b, lse_b, stream=s2)
    torch.cuda.synchronize()
    check(host(out_a), host(lse_a), *oracle.prefix_query(old.Q, old.K, old.V))
    check(host(out_b), host(lse_b), *oracle.prefix_query(old.Q, new.K, new.V))
    kp.pion_prefix_drop("t", 18)
