"""The failure path of the cross-workgroup waits, forced from the host.

nvfp4_test_fail_next_wait gives the next launch that waits on other
workgroups an arrival target no launch reaches: each of its waits gives up
at its bound (0.2 s of the real-time clock), records the failure in the
library's pinned error word, and the kernel finishes normally without the
work that depended on the wait.  The next call that would launch a waiting
kernel reports NVFP4_EDEVICE (launching nothing), and the call after it is
bit-exact again.  No kernel faults or hangs: every wait here is bounded.
"""
import time

import pytest
import torch

import nvfp4_block_scaled_bf16_amd as nv
from nvfp4_block_scaled_bf16_amd import workloads as W
from tests.gpu_util import Guarded, cast_spec, compare_cast, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("schedule,shape", [("resident", (4096, 4096)), ("two_pass", (1072, 544))])
def test_wait_gives_up_and_is_reported(oracle, schedule, shape):
    M, K = shape
    print(f"\n[case] forced wait failure, schedule={schedule} shape={shape}", flush=True)
    x = W.row_scaled_with_outliers(M, K, 4242)
    d = to_dev(x)
    out = Guarded(cast_spec(M, K, nv.PER_TOKEN))
    nv.set_schedule(schedule)
    try:
        nv._check(nv.lib().nvfp4_test_fail_next_wait())
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        nv.quantize_into(d, nv.PER_TOKEN, **out.views)   # enqueued: OK, outputs invalid
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        assert 0.15 < dt < 10.0, f"the forced waits took {dt:.3f} s"
        with pytest.raises(nv.NVFP4Error) as err:
            nv.quantize_into(d, nv.PER_TOKEN, **out.views)
        assert err.value.status == 4 and "gave up" in str(err.value)
        nv.quantize_into(d, nv.PER_TOKEN, **out.views)
        torch.cuda.synchronize()
        compare_cast(out, oracle.quantize(x, nv.PER_TOKEN))
    finally:
        nv.set_schedule("auto")


def test_rht_wait_gives_up_and_is_reported(oracle):
    """The Hadamard-transform cast's amax pass waits for the workgroups that
    zero its outputs: forced to give up, it records the failure, the next
    call reports it, and the call after that is bit-exact."""
    M, K, mask = 1072, 544, 0x1234
    print(f"\n[case] forced wait failure, quantize_rht {M}x{K}", flush=True)
    x = W.row_scaled_with_outliers(M, K, 4343)
    d = to_dev(x)
    out = Guarded(cast_spec(M, K, nv.PER_TOKEN, True, True))
    nv._check(nv.lib().nvfp4_test_fail_next_wait())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    nv.quantize_rht_into(d, nv.PER_TOKEN, mask, **out.views)   # enqueued: OK, outputs invalid
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert 0.15 < dt < 10.0, f"the forced waits took {dt:.3f} s"
    with pytest.raises(nv.NVFP4Error) as err:
        nv.quantize_rht_into(d, nv.PER_TOKEN, mask, **out.views)
    assert err.value.status == 4 and "gave up" in str(err.value)
    nv.quantize_rht_into(d, nv.PER_TOKEN, mask, **out.views)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize_rht(x, nv.PER_TOKEN, mask))
