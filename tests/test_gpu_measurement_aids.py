"""GPU checks of the two measurement aids the bench times beside the kernels: the plain
streaming read and the fp16 MFMA stream. Neither computes a result; each must run, leave
its sink untouched (it writes only on a match with a value that realistic data never
gives) and, for the MFMA stream, report the flop count of its launch."""
import pytest
import torch

import kv_cache_prefix_amd as kp

pytestmark = pytest.mark.gpu


def test_stream_read_runs_and_leaves_the_sink():
    buf = torch.ones(1 << 22, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    kp.pion_bench_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert kp.pion_prefix_last_plan() == "stream_read_kernel"
    assert int(sink.item()) == 0


@pytest.mark.parametrize("iters", [1, 64])
def test_mfma_peak_flop_count(iters):
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    flops = kp.pion_bench_mfma_peak(iters, sink)
    torch.cuda.synchronize()
    assert kp.pion_prefix_last_plan() == "mfma_peak_kernel"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # four 256-lane workgroups per CU, four products of 32 x 32 x 16 per wave and round
    assert flops == cus * 4 * 4 * 4 * iters * 2 * 32 * 32 * 16
    assert int(sink.item()) == 0


def test_mfma_peak_rejects_no_rounds():
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    with pytest.raises(kp.PionError):
        kp.pion_bench_mfma_peak(0, sink)
