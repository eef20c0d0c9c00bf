"""pa_decode_noalloc (the fixed per-GPU workspace, for callers that cannot
allocate) against pa_decode: two calls in a row, the second with a smaller
batch, each bit for bit pa_decode's output and within tolerance of the
oracle.  The call runs through the C ABI; its workspace is the library's
own array."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_132_amd as pa
from tests._gpu import assert_decode_close, dev16, dev_i32, dev_pool, host_bits, oracle_decode, pool_of
from workloads import make_custom

pytestmark = pytest.mark.gpu

CASES = [
    # (big batch, smaller batch): lens, Hq, Hkv, D, bs, q_dtype, kv_dtype
    (([300, 1000, 17, 2048, 0, 640], 32, 32, 128, 16, "f16", "f16"),
     ([5, 70, 129], 32, 32, 128, 16, "f16", "f16")),
    (([1500, 40, 800, 3000], 32, 8, 128, 16, "bf16", "fp8_e4m3"),
     ([60, 17], 32, 8, 128, 16, "bf16", "fp8_e4m3")),
    (([700, 33, 1200], 64, 8, 128, 32, "bf16", "bf16"),
     ([100, 1], 64, 8, 128, 32, "bf16", "bf16")),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("partition", [0, 64])
def test_noalloc_equals_pa_decode(case, partition):
    assert pa.load().pa_decode_noalloc_max_workspace() == 64 << 20
    for k, (lens, hq, hkv, d, bs, qd, kvd) in enumerate(CASES[case]):
        b = make_custom(f"noalloc{case}_{k}", 500 + 10 * case + k, lens, hq, hkv, d, bs, qd, kvd)
        bt, L = dev_i32(b.block_table_array()), dev_i32(b.context_lens)
        pool = dev_pool(pool_of(b), kvd)
        q = dev16(b.query, qd)
        want = pa.decode(q, pool, bt, L, b.scale, b.k_scale, b.v_scale, partition_size=partition)
        got = torch.full_like(q, float("nan"))
        pa.decode_noalloc(q, pool, bt, L, b.scale, b.k_scale, b.v_scale, out=got, partition_size=partition)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (case, k)
        ref = oracle_decode(b, pool_of(b), b.query, b.block_table_array(), b.context_lens)
        assert_decode_close(oracle.to_f64(host_bits(got), qd), ref, b)


def test_noalloc_rejects_a_batch_beyond_its_workspace():
    """A batch whose workspace exceeds the fixed array is refused before any
    launch (no device memory is touched)."""
    lib = pa.load()
    need = lib.pa_decode_workspace_size(4096, 64, 64, 128, 16, 4096, pa.PA_F16, 16)
    assert need > lib.pa_decode_noalloc_max_workspace()
    fake = 0x10000
    st = lib.pa_decode_noalloc(fake, fake, pa.PA_F16, fake, pa.PA_F16, fake, fake, 4096, 64, 64, 128, 16, 4096,
                               1 << 20, 0.1, 1.0, 1.0, 16, None)
    assert st == 6      # PA_ERR_WORKSPACE_TOO_SMALL
