"""GPU parity of pa_copy_blocks (copy-on-write and swap) against the oracle.

Every comparison is over the whole destination pool, bit for bit: copied
blocks must equal their sources and every other block must be untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_132_amd as pa
from tests._gpu import assert_decode_close, dev16, dev_i32, dev_pool, host_bits, oracle_decode, pool_of
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _random_pool(rng, nb, bs, hkv, d, kv_dtype):
    if kv_dtype == "fp8_e4m3":
        return rng.integers(0, 256, size=(nb, 2, bs, hkv, d), dtype=np.uint8)
    return rng.integers(0, 1 << 16, size=(nb, 2, bs, hkv, d), dtype=np.uint16)


def _independent_pairs(rng, nb, n):
    blocks = rng.permutation(nb)[:2 * n]
    return np.stack([blocks[:n], blocks[n:]], axis=1).astype(np.int32)


@pytest.mark.parametrize("kv_dtype,bs,hkv,d", [("f16", 16, 8, 64), ("bf16", 32, 4, 128),
                                               ("fp8_e4m3", 16, 8, 128)])
def test_copy_on_write_inside_one_pool(kv_dtype, bs, hkv, d):
    rng = np.random.default_rng(40)
    pool = _random_pool(rng, 96, bs, hkv, d, kv_dtype)
    mapping = _independent_pairs(rng, 96, 30)
    want = oracle.copy_blocks(pool, pool, mapping)
    dev = dev_pool(pool, kv_dtype)
    pa.copy_blocks(dev, dev, dev_i32(mapping))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dev), want)


def test_swap_out_to_pinned_host_and_back():
    """Device -> pinned host pool (swap out), then host -> other device blocks
    (swap in); both bit-exact against the oracle."""
    rng = np.random.default_rng(41)
    nb, bs, hkv, d = 80, 16, 8, 128
    pool = _random_pool(rng, nb, bs, hkv, d, "f16")
    dev = dev_pool(pool, "f16")
    out_blocks = rng.permutation(nb)[:20].astype(np.int32)
    host = torch.zeros((24, 2, bs, hkv, d), dtype=torch.float16, pin_memory=True)
    host_np = np.zeros((24, 2, bs, hkv, d), dtype=np.uint16)
    m_out = np.stack([out_blocks, np.arange(20, dtype=np.int32) + 2], axis=1)
    pa.copy_blocks(dev, host, dev_i32(m_out))
    torch.cuda.synchronize()
    want_host = oracle.copy_blocks(pool, host_np, m_out)
    assert np.array_equal(host.view(torch.int16).numpy().view(np.uint16), want_host)

    free = np.setdiff1d(np.arange(nb), out_blocks)[:20].astype(np.int32)
    m_in = np.stack([np.arange(20, dtype=np.int32) + 2, free], axis=1)
    pa.copy_blocks(host, dev, dev_i32(m_in))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dev), oracle.copy_blocks(want_host, pool, m_in))


def test_out_of_range_pairs_are_skipped():
    rng = np.random.default_rng(42)
    pool = _random_pool(rng, 32, 16, 4, 64, "f16")
    good = np.array([[1, 5], [7, 9]], dtype=np.int32)
    mapping = np.concatenate([good, [[0, 32], [-1, 3], [40, 2]]]).astype(np.int32)
    dev = dev_pool(pool, "f16")
    pa.copy_blocks(dev, dev, dev_i32(mapping))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dev), oracle.copy_blocks(pool, pool, good))


def test_pageable_host_pool_is_refused():
    pool = torch.zeros((4, 2, 16, 4, 64), dtype=torch.float16)          # not pinned
    dev = torch.zeros((4, 2, 16, 4, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        pa.copy_blocks(pool, dev, dev_i32([[0, 1]]))


def test_branch_after_copy_on_write_decodes_like_the_oracle():
    """Two sequences share every block of a 37-token prefix; the second
    copies the shared tail block, points its table at the copy and appends a
    token.  Both decodes match the oracle run on the oracle's own pool."""
    b = make_custom("cow", 43, [37, 37], 16, 16, 128, 16, "f16", "f16")
    pool = pool_of(b)
    row = list(b.tables[0])
    tables = [row, list(row)]
    used = set(int(x) for t in b.tables for x in t)
    fresh = next(x for x in range(pool.shape[0]) if x not in used)
    tables[1][2] = fresh
    bt = np.array(tables, dtype=np.int32)
    lens = np.array([37, 38], dtype=np.int32)
    mapping = np.array([[row[2], fresh]], dtype=np.int32)

    dev = dev_pool(pool, "f16")
    pa.copy_blocks(dev, dev, dev_i32(mapping))
    k_new = np.stack([b.new_key[0][1], b.new_key[0][1]])
    v_new = np.stack([b.new_value[0][1], b.new_value[0][1]])
    # only sequence 1 writes: sequence 0 gets length 0 in the write call
    pa.cache_write(dev, dev16(k_new, "f16"), dev16(v_new, "f16"), dev_i32(bt), dev_i32([0, 38]))
    q = dev16(b.query, "f16")
    out = pa.decode(q, dev, dev_i32(bt), dev_i32(lens), b.scale)
    torch.cuda.synchronize()

    ref_pool = oracle.copy_blocks(pool, pool, mapping)
    ref_pool = oracle.cache_write(ref_pool, "f16", k_new, v_new, "f16", bt, np.array([0, 38], dtype=np.int32), 16)
    assert np.array_equal(host_bits(dev), ref_pool)
    ref = oracle_decode(b, ref_pool, b.query, bt, lens)
    assert_decode_close(oracle.to_f64(host_bits(out), "f16"), ref, b)
    # sequence 0 still reads the untouched original tail block
    ref0 = oracle_decode(b, pool, b.query[:1], bt[:1], lens[:1])
    assert np.array_equal(ref[0], ref0[0])


def test_copy_at_7b_block_size():
    """Full-size blocks of the 7B shape (256 KiB) in a 1200-block pool."""
    rng = np.random.default_rng(44)
    nb = 1200
    pool = _random_pool(rng, nb, 16, 32, 128, "f16")
    mapping = _independent_pairs(rng, nb, 500)
    dev = dev_pool(pool, "f16")
    pa.copy_blocks(dev, dev, dev_i32(mapping))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dev), oracle.copy_blocks(pool, pool, mapping))
