"""GPU parity of the shared-run decode (pa_decode_shared,
pa_decode_write_partials_shared): sequences that share prefix blocks in
aligned runs ([nano-vllm blog §3, §4.3]) have their shared partitions
computed once per run.  Outputs must match the oracle within the decode
tolerance whatever the run size, and the fused write must leave the pool bit
for bit as pa_cache_write does.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_132_amd as pa
from tests._gpu import (
    assert_decode_close, dev16, dev_i32, dev_pool, host_bits, oracle_decode, poison_unused, pool_of,
)
from workloads import make_custom, make_prefix_shared

pytestmark = pytest.mark.gpu


def _decode(batch, pool_dev, bt, lens, run_size, partition_size):
    q = dev16(batch.query, batch.q_dtype)
    out = pa.decode(q, pool_dev, dev_i32(bt), dev_i32(lens), batch.scale, batch.k_scale, batch.v_scale,
                    partition_size=partition_size, run_size=run_size)
    torch.cuda.synchronize()
    return oracle.to_f64(host_bits(out), batch.q_dtype)


CASES = {
    # name: (lens, group, prefix tokens, Hq = Hkv, D, bs, q_dtype, kv_dtype)
    "f16_d128_group8": ([300, 420, 257, 700, 512, 390, 301, 640] * 2, 8, 256, 8, 128, 16, "f16", "f16"),
    "bf16_d64_group8_bs32": ([330, 260, 500, 288, 700, 321, 452, 299] * 2, 8, 256, 4, 64, 32, "bf16", "bf16"),
    "fp8_d128_group4": ([200, 300, 150, 400] * 4, 4, 128, 8, 128, 16, "bf16", "fp8_e4m3"),
    "f16_d128_group2_short": ([70, 200, 65, 64, 300, 129, 40, 520], 2, 64, 8, 128, 16, "f16", "f16"),
    # 16-bit, head_dim 128, block 32: the matrix-core run kernel over two 16-token steps per block
    "bf16_d128_group4_bs32": ([260, 400, 129, 610, 300, 288, 97, 450], 4, 128, 8, 128, 32, "bf16", "bf16"),
}


@pytest.mark.parametrize("run_size", [2, 4, 8])
@pytest.mark.parametrize("name", sorted(CASES))
def test_shared_runs_match_oracle(name, run_size):
    """Runs equal to, inside and across the share groups, partitions of 64
    tokens (several shared per run, tails and short sequences not): all within
    tolerance of the oracle, and of the per-sequence decode."""
    lens, group, prefix, h, d, bs, qd, kvd = CASES[name]
    b = make_custom(name, 200 + sorted(CASES).index(name), lens, h, h, d, bs, qd, kvd,
                    share_group=group, shared_prefix_tokens=prefix)
    bt, L = b.block_table_array(), b.context_lens
    pool = poison_unused(pool_of(b), b.tables, L, kvd)
    pool_dev = dev_pool(pool, kvd)
    ref = oracle_decode(b, pool, b.query, bt, L)
    plain = _decode(b, pool_dev, bt, L, 1, 64)
    for ps in (64, 2 * bs if 2 * bs != 64 else 96):
        got = _decode(b, pool_dev, bt, L, run_size, ps)
        assert_decode_close(got, ref, b)
    assert_decode_close(plain, ref, b)


def test_diverged_sequence_leaves_the_run():
    """One sequence of a run gets private copies of two prefix blocks: the
    partitions holding them are computed per sequence, the others once per
    run; the output follows the private copies (their values differ)."""
    lens = [400, 380, 500, 410, 390, 450, 420, 600]
    b = make_custom("diverge", 230, lens, 8, 8, 128, 16, "f16", "f16", share_group=8, shared_prefix_tokens=256,
                    spare=0.5)
    tabs = [list(t) for t in b.tables]
    used = {int(x) for t in tabs for x in t}
    free = [i for i in range(b.num_blocks) if i not in used]
    pool = np.array(pool_of(b), copy=True)
    for j, blk in zip((3, 9), free[:2]):              # sequence 5, logical blocks 3 and 9 (partitions 0 and 2)
        pool[blk] = pool[tabs[5][j]]
        pool[blk, 1] ^= np.uint16(0x0400)             # change the copy's V rows (exponent bit: finite, different)
        tabs[5][j] = blk
    bt = np.full((b.num_seqs, b.max_blocks_per_seq), -1, dtype=np.int32)
    for s, t in enumerate(tabs):
        bt[s, :len(t)] = t
    L = b.context_lens
    pool = poison_unused(pool, tabs, L, "f16")
    pool_dev = dev_pool(pool, "f16")
    ref = oracle_decode(b, pool, b.query, bt, L)
    for run_size in (2, 8):
        assert_decode_close(_decode(b, pool_dev, bt, L, run_size, 64), ref, b)


def test_write_partials_shared_equals_separate_write():
    """pa_decode_write_partials_shared + pa_decode_merge: the pool bit for bit
    as pa_cache_write leaves it, the output within tolerance of the oracle on
    the written pool."""
    lens = [300, 420, 257, 700, 512, 390, 301, 640]
    b = make_custom("shared_write", 240, lens, 8, 8, 128, 16, "f16", "f16", share_group=8,
                    shared_prefix_tokens=256, appends=1)
    L1 = b.context_lens + 1
    for tab, n in zip(b.tables, L1):
        b.manager.grow_to(tab, int(n))
    bt1 = b.block_table_array()
    pool = poison_unused(pool_of(b), b.tables, L1, "f16")
    pool_dev = dev_pool(pool, "f16")
    k, v = dev16(b.new_key[0], "f16"), dev16(b.new_value[0], "f16")
    q = dev16(b.query, "f16")
    ws = pa.Workspace()
    args = (q, pool_dev, dev_i32(bt1), dev_i32(L1), b.scale)
    out = torch.empty_like(q)
    pa.decode(*args, out=out, workspace=ws, partition_size=64, phase="partials", new_key=k, new_value=v,
              run_size=8)
    pa.decode(*args, out=out, workspace=ws, partition_size=64, phase="merge")
    torch.cuda.synchronize()
    want_pool = oracle.cache_write(pool, "f16", b.new_key[0], b.new_value[0], "f16", bt1, L1, 16)
    assert np.array_equal(host_bits(pool_dev), want_pool)
    ref = oracle_decode(b, want_pool, b.query, bt1, L1)
    assert_decode_close(oracle.to_f64(host_bits(out), "f16"), ref, b)


def test_prefix13b_full_size_runs_of_8():
    """The 13B batch (groups of 8 sharing 140 blocks) with runs of 8 at the
    default partition, at 512 tokens and at 640 (the shared prefix is exactly
    7 partitions): every sequence against the oracle, and within tolerance of
    the per-sequence decode."""
    b = make_prefix_shared()
    bt, L = b.block_table_array(), b.context_lens
    pool_dev = dev_pool(b.kv_pool, "f16")
    plain = _decode(b, pool_dev, bt, L, 1, 0)
    ref = oracle_decode(b, b.kv_pool, b.query, bt, L)
    assert_decode_close(plain, ref, b)
    for ps in (0, 512, 640):
        got = _decode(b, pool_dev, bt, L, 8, ps)
        assert np.isfinite(got).all()
        assert np.abs(got - plain).max() <= 2e-3, ps
        assert_decode_close(got, ref, b)


def test_shared_runs_graph_replays_match_eager():
    """The shared-run step (run kernel, per-sequence kernel, merge) captured in a
    HIP graph: every replay, with eager work and synchronisations between
    replays, equals the eager call bit for bit."""
    lens = [300, 420, 257, 700, 512, 390, 301, 640]
    b = make_custom("shared_graph", 250, lens, 8, 8, 128, 16, "bf16", "bf16", share_group=4,
                    shared_prefix_tokens=256)
    bt, L = dev_i32(b.block_table_array()), dev_i32(b.context_lens)
    pool_dev = dev_pool(pool_of(b), "bf16")
    q = dev16(b.query, "bf16")
    ws = pa.Workspace()
    args = (q, pool_dev, bt, L, b.scale)
    eager = torch.empty_like(q)
    pa.decode(*args, out=eager, workspace=ws, partition_size=64, run_size=4)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pa.decode(*args, out=out, workspace=ws, partition_size=64, run_size=4)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(3):
        out.fill_(float("nan"))
        pa.decode(*args, partition_size=64)                # other eager work on the same pool
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
    ref = oracle_decode(b, pool_of(b), b.query, b.block_table_array(), b.context_lens)
    assert_decode_close(oracle.to_f64(host_bits(out), "bf16"), ref, b)
