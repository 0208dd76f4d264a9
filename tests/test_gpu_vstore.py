"""GPU parity of the V-store calls (Shared KV Cache Serving, V.FETCH RANGE and
KV.PREFIX.WARM; V-store page, The mlx4g32 tier): the fetch against the oracle bit for
bit, and the rehydrated slot against a slot stored from the device fetch's output (or,
for an mlx4g32 slot, from the original fp16 K/V): the same slot bytes give bit-identical
query results, and both match the attention oracle. Records are drawn by synth (random
fields) or written by the device encoder; no input of the device comes from the oracle."""
import numpy as np
import pytest

import oracle
import synth
from oracle import vstore as ovs
from test_gpu_parity import check, dev, empty, host, kp, query  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _drop_sessions(kp):
    yield
    kp.pion_prefix_drop("vs", -1)


def rows_of(x_hnd):
    """[H, N, D] -> V-store rows [N, H * D]."""
    H, N, D = x_hnd.shape
    return np.ascontiguousarray(x_hnd.transpose(1, 0, 2).reshape(N, H * D))


def fetched_slot(kp, rows, fmt, H, D, dtype):
    """The slot contents a WARM must produce, built on the device from the fetch kernel
    (checked bit for bit against the oracle by test_fetch_bit_exact) and torch's
    relayout and RNE cast: [H, N, D] in `dtype`."""
    N = rows.shape[0]
    out = empty((N, H * D))
    kp.pion_vstore_fetch_f32(dev(rows), fmt, H * D, 0, N, out)
    return out.reshape(N, H, D).transpose(0, 1).contiguous().to(dtype)


@pytest.mark.parametrize("kv", [32, 96, 1024])
@pytest.mark.parametrize("fmt", [ovs.FP16, ovs.MLX4G32])
def test_fetch_bit_exact(kp, fmt, kv):
    rng = np.random.default_rng(kv + fmt)
    x = (rng.standard_normal((300, kv)) * rng.lognormal(0, 1, (1, kv))).astype(np.float16)
    rows = x if fmt == ovs.FP16 else synth.mlx4_records(300, kv, kv)
    d = dev(rows)
    for start, end in [(0, 300), (17, 18), (123, 299), (5, 5)]:
        out = empty((end - start, kv))
        kp.pion_vstore_fetch_f32(d, fmt, kv, start, end, out)
        got = host(out)
        want = ovs.fetch_f32(rows, fmt, kv, start, end)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("H,N,D", [(1, 1, 32), (3, 257, 96), (8, 1000, 128), (2, 300, 512)])
@pytest.mark.parametrize("src", [ovs.FP16, ovs.MLX4G32])
def test_warm_into_fp16_slot(kp, H, N, D, src):
    import torch
    inp = synth.generate(synth.DECODE, 50, N=N, D=D, H_q=H, H_kv=H)
    Kr, Vr = rows_of(inp.K), rows_of(inp.V)
    if src == ovs.MLX4G32:
        Kr, Vr = synth.mlx4_records(N, H * D, 500 + N), synth.mlx4_records(N, H * D, 501 + N)
    kp.pion_prefix_warm("vs", 0, H, D, dev(Kr), dev(Vr), src)
    assert kp.pion_prefix_info("vs", 0) == (H, N, D, 0)
    if src == ovs.FP16:   # a WARM from fp16 rows is the STORE of the original [H, N, D]
        kp.pion_prefix_store("vs", 1, dev(inp.K), dev(inp.V))
    else:
        kp.pion_prefix_store("vs", 1, fetched_slot(kp, Kr, src, H, D, torch.float16),
                             fetched_slot(kp, Vr, src, H, D, torch.float16))
    Kw, Vw = ovs.warm_fp16(Kr, src, H, D), ovs.warm_fp16(Vr, src, H, D)
    a, la = query(kp, "vs", 0, inp.Q)
    b, lb = query(kp, "vs", 1, inp.Q)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)
    check(a, la, *oracle.prefix_query(inp.Q, Kw, Vw))
    kp.pion_prefix_drop("vs", -1)


@pytest.mark.parametrize("H,N,D", [(1, 1, 32), (3, 257, 96), (8, 1000, 128), (2, 300, 512)])
@pytest.mark.parametrize("src", [ovs.FP16, ovs.MLX4G32])
def test_warm_into_mlx4g32_slot(kp, H, N, D, src):
    import torch
    inp = synth.generate(synth.MLX4_DECODE, 51, N=N, D=D, H_q=H, H_kv=H)
    if src == ovs.FP16:
        # encodes as STORE does: the same slot as a STORE of the original fp16 K/V
        Kr, Vr = rows_of(inp.K), rows_of(inp.V)
        kp.pion_prefix_warm("vs", 0, H, D, dev(Kr), dev(Vr), src, kp.PION_KV_MLX4G32)
        kp.pion_prefix_store("vs", 1, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
        a, la = query(kp, "vs", 0, inp.Q)
        b, lb = query(kp, "vs", 1, inp.Q)
        np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(la, lb)
        Kh = oracle.dequantize(*oracle.quantize(inp.K.reshape(-1, D))).reshape(inp.K.shape)
        Vh = oracle.dequantize(*oracle.quantize(inp.V.reshape(-1, D))).reshape(inp.V.shape)
    else:
        # records kept as they are: the slot answers like attention over their
        # dequantized values; and records written by the device encoder from fp16 rows
        # rehydrate the slot a STORE of those rows with MLX4G32 makes
        Kr, Vr = synth.mlx4_records(N, H * D, 510 + N), synth.mlx4_records(N, H * D, 511 + N)
        kp.pion_prefix_warm("vs", 0, H, D, dev(Kr), dev(Vr), src, kp.PION_KV_MLX4G32)
        a, la = query(kp, "vs", 0, inp.Q)
        Kh = np.ascontiguousarray(ovs.fetch_f32(Kr, src, H * D, 0, N).astype(np.float64)
                                  .reshape(N, H, D).transpose(1, 0, 2))
        Vh = np.ascontiguousarray(ovs.fetch_f32(Vr, src, H * D, 0, N).astype(np.float64)
                                  .reshape(N, H, D).transpose(1, 0, 2))
        enc = [device_records(kp, rows_of(x)) for x in (inp.K, inp.V)]
        kp.pion_prefix_warm("vs", 2, H, D, enc[0], enc[1], src, kp.PION_KV_MLX4G32)
        kp.pion_prefix_store("vs", 3, dev(inp.K), dev(inp.V), kp.PION_KV_MLX4G32)
        c, lc = query(kp, "vs", 2, inp.Q)
        d, ld = query(kp, "vs", 3, inp.Q)
        np.testing.assert_array_equal(c, d)
        np.testing.assert_array_equal(lc, ld)
    check(a, la, *oracle.prefix_query(inp.Q, Kh, Vh))
    kp.pion_prefix_drop("vs", -1)


def device_records(kp, rows16):
    """fp16 V-store rows [N, kv] -> mlx4g32 records [N, 5 kv / 8] on the device: the
    library's encoder, its three outputs concatenated per token in the record order."""
    import torch
    N, kv = rows16.shape
    codes = torch.empty((N, kv // 8), dtype=torch.int32, device="cuda")
    sc = torch.empty((N, kv // 32), dtype=torch.float16, device="cuda")
    bi = torch.empty((N, kv // 32), dtype=torch.float16, device="cuda")
    kp.pion_kv_quantize_mlx4g32(dev(rows16), codes, sc, bi)
    return torch.cat([t.view(torch.uint8).reshape(N, -1) for t in (codes, sc, bi)], 1).contiguous()


def test_warm_rehydrates_a_cold_key(kp):
    saved = kp.pion_prefix_stats()
    assert saved["warm_slots"] == 0, "the slot table must start empty"
    try:
        kp.pion_prefix_set_capacity(1, 0, 16)
        a = synth.generate(synth.DECODE, 52, N=200, D=64, H_q=2, H_kv=2)
        b = synth.generate(synth.DECODE, 53, N=100, D=64, H_q=2, H_kv=2)
        kp.pion_prefix_store("vs", 0, dev(a.K), dev(a.V))
        kp.pion_prefix_store("vs", 1, dev(b.K), dev(b.V))       # demotes layer 0
        assert kp.pion_prefix_lookup("vs", 0) == 2
        r0 = kp.pion_prefix_stats()["rehydrates"]
        Kr, Vr = synth.mlx4_records(200, 128, 520), synth.mlx4_records(200, 128, 521)
        kp.pion_prefix_warm("vs", 0, 2, 64, dev(Kr), dev(Vr), ovs.MLX4G32)
        assert kp.pion_prefix_stats()["rehydrates"] == r0 + 1
        assert kp.pion_prefix_lookup("vs", 0) == 1 and kp.pion_prefix_lookup("vs", 1) == 2
        Kw, Vw = ovs.warm_fp16(Kr, ovs.MLX4G32, 2, 64), ovs.warm_fp16(Vr, ovs.MLX4G32, 2, 64)
        check(*query(kp, "vs", 0, a.Q), *oracle.prefix_query(a.Q, Kw, Vw))
    finally:
        kp.pion_prefix_drop("vs", -1)
        kp.pion_prefix_set_capacity(saved["max_slots"], saved["max_bytes"], saved["cold_capacity"])
