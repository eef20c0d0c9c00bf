"""Pins of the CPU oracle to what the pages and mathematics fix (CPU only).

Each check ties the oracle to something other than itself: worked examples the
pages print (fixtures under tests/golden/, each with its citation), closed
forms, library routines (torch's scaled-dot-product attention in float64,
torch's float8_e4m3fn conversion), brute force on tiny inputs, and invariants
the pages state.  The mutation tests at the end plant plausible mistakes in
the oracle and check that some pin catches each one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.paged_attention as opa
from tests.conftest import load_golden
from workloads import BlockManager, make_custom, make_tiny, make_prefix_shared
from workloads.block_manager import blocks_for_tokens, full_blocks


# ---------------------------------------------------------------------------
# test-local construction of paged inputs from contiguous K/V
#
# The pool is built from a flat element address written out from the pages'
# formula ([CANN notes §2.2]: block base = block * block_size * kv_per_token,
# plus offset * kv_per_token) refined to the [block, 2, block_size, heads,
# head_dim] layout of [CANN notes §2.1].  The oracle indexes the 5-D array
# instead, so a transposed index on either side shows up as a mismatch.

def flat_address(blk, kv, off, g, d, bs, Hkv, D):
    kv_per_token = 2 * Hkv * D
    half = Hkv * D
    return blk * bs * kv_per_token + kv * bs * half + off * half + g * D + d


def scatter_contiguous(K, V, tables, lens, num_blocks, bs, fill=np.float16(np.nan)):
    """Place contiguous per-sequence K/V [L, Hkv, D] into a fresh fp16 pool."""
    Hkv, D = K[0].shape[1], K[0].shape[2]
    flat = np.full(num_blocks * 2 * bs * Hkv * D, fill, dtype=np.float16)
    for s, L in enumerate(lens):
        for t in range(L):
            blk = tables[s][t // bs]
            off = t % bs
            for g in range(Hkv):
                a_k = flat_address(blk, 0, off, g, 0, bs, Hkv, D)
                a_v = flat_address(blk, 1, off, g, 0, bs, Hkv, D)
                flat[a_k:a_k + D] = K[s][t, g]
                flat[a_v:a_v + D] = V[s][t, g]
    return flat.reshape(num_blocks, 2, bs, Hkv, D)


def random_paged_case(seed, lens, Hq, Hkv, D, bs, spare_blocks=3):
    rng = np.random.default_rng(seed)
    nblk = sum(blocks_for_tokens(L, bs) for L in lens) + spare_blocks
    mgr = BlockManager(nblk, bs, rng)
    tables = []
    for L in lens:
        tab = []
        mgr.grow_to(tab, L)
        tables.append(tab)
    K = [rng.standard_normal((L, Hkv, D)).astype(np.float16) for L in lens]
    V = [rng.standard_normal((L, Hkv, D)).astype(np.float16) for L in lens]
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float16)
    pool = scatter_contiguous(K, V, tables, lens, nblk, bs)
    MB = max(len(t) for t in tables)
    bt = np.full((len(lens), MB), -1, dtype=np.int32)
    for s, tab in enumerate(tables):
        bt[s, :len(tab)] = tab
    return q, K, V, pool.view(np.uint16), bt, np.array(lens, dtype=np.int32)


def sdpa_dense(q16, K, V, scale):
    """Library reference: torch SDPA in float64 on contiguous K/V, GQA by torch's rule."""
    B, Hq, D = q16.shape
    out = np.zeros((B, Hq, D))
    for s in range(B):
        qs = torch.from_numpy(q16[s].astype(np.float64)).reshape(1, Hq, 1, D)
        ks = torch.from_numpy(K[s].astype(np.float64)).permute(1, 0, 2).unsqueeze(0).contiguous()
        vs = torch.from_numpy(V[s].astype(np.float64)).permute(1, 0, 2).unsqueeze(0).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, scale=scale,
                                                             enable_gqa=(ks.shape[1] != Hq))
        out[s] = o.reshape(Hq, D).numpy()
    return out


def naive_loops(q16, K, V, scale):
    """Brute force with Python loops and math.exp (tiny inputs only)."""
    B, Hq, D = q16.shape
    Hkv = K[0].shape[1]
    out = np.zeros((B, Hq, D))
    for s in range(B):
        L = K[s].shape[0]
        for h in range(Hq):
            g = h * Hkv // Hq
            z = []
            for t in range(L):
                acc = 0.0
                for d in range(D):
                    acc += float(q16[s, h, d]) * float(K[s][t, g, d])
                z.append(scale * acc)
            zmax = max(z)
            w = [math.exp(v - zmax) for v in z]
            tot = sum(w)
            for d in range(D):
                out[s, h, d] = sum(w[t] * float(V[s][t, g, d]) for t in range(L)) / tot
    return out


def oracle_decode(q16, pool, bt, lens, bs, scale):
    return oracle.paged_decode(q16.view(np.uint16), "f16", pool, "f16", bt, lens, bs, scale)


DENSE_CASES = [
    # seed, lens, Hq, Hkv, D, bs
    (11, [20, 37, 16, 1], 4, 4, 16, 16),
    (12, [33, 64, 5], 8, 2, 32, 16),       # GQA 4
    (13, [70, 31], 4, 2, 16, 32),          # GQA 2, block 32
    (14, [100], 8, 1, 8, 16),              # MQA
]


def check_dense_equivalence(case):
    seed, lens, Hq, Hkv, D, bs = case
    q, K, V, pool, bt, L = random_paged_case(seed, lens, Hq, Hkv, D, bs)
    scale = 1.0 / math.sqrt(D)
    got = oracle_decode(q, pool, bt, L, bs, scale)
    ref = sdpa_dense(q, K, V, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", DENSE_CASES)
def test_paged_equals_dense_sdpa(case):
    check_dense_equivalence(case)


def test_paged_equals_naive_loops():
    q, K, V, pool, bt, L = random_paged_case(21, [9, 17, 1], 4, 2, 8, 16)
    scale = 1.0 / math.sqrt(8)
    got = oracle_decode(q, pool, bt, L, 16, scale)
    ref = naive_loops(q, K, V, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# worked examples on the pages

def labelled_pool(num_blocks, bs, Hkv=1, D=2):
    """fp16 pool whose K slot (b, o) holds the values (b, o): readable addresses."""
    pool = np.zeros((num_blocks, 2, bs, Hkv, D), dtype=np.float16)
    for b in range(num_blocks):
        for o in range(bs):
            pool[b, :, o, :, 0] = b
            pool[b, :, o, :, 1] = o
    return pool.view(np.uint16)


def test_block_table_example():
    g = load_golden("block_table_example.json")
    bs, row = g["block_size"], g["row"]
    for t, blk, off in g["token_to_slot"]:
        assert oracle.slot_of(row, t, bs) == (blk, off)
    pool = labelled_pool(32, bs)
    K, V = oracle.gather_kv(pool, "f16", row, 32, bs)
    for t, blk, off in g["token_to_slot"]:
        assert K[t, 0, 0] == blk and K[t, 0, 1] == off


@pytest.mark.parametrize("key", ["list_example", "diagram_example"])
def test_logical_to_physical_order(key):
    g = load_golden("logical_to_physical.json")
    row, bs = g[key], g["block_size"]
    pool = labelled_pool(max(row) + 1, bs)
    L = len(row) * bs
    K, _ = oracle.gather_kv(pool, "f16", row, L, bs)
    blocks_in_order = [int(K[j * bs, 0, 0]) for j in range(len(row))]
    assert blocks_in_order == row
    assert [int(K[t, 0, 1]) for t in range(bs)] == list(range(bs))


def test_partial_tail_block():
    g = load_golden("partial_tail.json")
    bs, L = g["block_size"], g["length"]
    assert oracle.num_blocks_of(L, bs) == g["blocks"]
    row = [5, 2]
    pool = labelled_pool(6, bs)
    K, _ = oracle.gather_kv(pool, "f16", row, L, bs)
    assert K.shape[0] == L
    assert int((K[:, 0, 0] == row[-1]).sum()) == g["valid_in_last"]


def test_full_blocks_only():
    g = load_golden("full_blocks.json")
    assert full_blocks(g["prefix_tokens"], g["block_size"]) == g["full_blocks"]
    assert full_blocks(g["prefix_tokens"], g["block_size"]) * g["block_size"] == g["cached_tokens"]
    # The shared prefix of the 13B workload: the largest run of full 32-token
    # blocks inside the 4500 reusable tokens of a 5000-token prompt.
    assert full_blocks(g["reused_prompt_tokens"], 32) * 32 == 4480 == 140 * 32


def test_kv_size_formula():
    g = load_golden("kv_sizes.json")
    for k in ("llama7b", "llama13b"):
        c = g[k]
        assert oracle.kv_bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["bytes"]) == c["per_token"]
    per_tok = g["llama7b"]["per_token"]
    GiB, MiB = 1 << 30, 1 << 20
    assert per_tok * 4096 == g["gib"]["tokens_4096"] * GiB
    assert 8 * per_tok * 4096 == g["gib"]["requests_8_x_4096"] * GiB
    assert per_tok * 2048 == g["gib"]["tokens_2048"] * GiB
    block = 16 * per_tok
    assert block == g["block_16_mib"] * MiB
    assert 60 * GiB // block == g["pool_60_gib_blocks"]
    assert g["pool_60_gib_blocks"] * 16 == g["pool_60_gib_tokens"]
    assert g["pool_60_gib_tokens"] // 2048 == g["pool_60_gib_requests_2048"]
    assert 20 * GiB // block == g["pool_20_gib_blocks"]
    assert 40000 // 16 == g["tokens_40000_blocks"]
    # one layer of the 7B shape, as the decode pool stores it: 16 KiB per token
    assert oracle.kv_bytes_per_token(1, 32, 128, 2) == 16384


def test_mixed_lengths_total():
    g = load_golden("mixed_lengths.json")
    assert len(g["lengths"]) * max(g["lengths"]) == g["padded_total"]
    assert sum(g["lengths"]) == g["sum_of_lengths"] != g["stated_total"]
    assert 1 - g["sum_of_lengths"] / g["padded_total"] > 0.60


# ---------------------------------------------------------------------------
# closed forms and invariants

def test_length_one_returns_first_value():
    q, K, V, pool, bt, L = random_paged_case(31, [1, 1], 4, 4, 16, 16)
    got = oracle_decode(q, pool, bt, L, 16, 0.25)
    for s in range(2):
        for h in range(4):
            assert np.array_equal(got[s, h], V[s][0, h].astype(np.float64))


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(32)
    L, Hkv, D, bs = 45, 2, 16, 16
    k_row = rng.standard_normal((Hkv, D)).astype(np.float16)
    K = [np.broadcast_to(k_row, (L, Hkv, D)).copy()]
    V = [rng.standard_normal((L, Hkv, D)).astype(np.float16)]
    mgr = BlockManager(8, bs, rng)
    tab = []
    mgr.grow_to(tab, L)
    pool = scatter_contiguous(K, V, [tab], [L], 8, bs).view(np.uint16)
    bt = np.array([tab], dtype=np.int32)
    q = rng.standard_normal((1, 4, D)).astype(np.float16)
    got = oracle_decode(q, pool, bt, np.array([L], np.int32), bs, 0.3)
    mean_v = V[0].astype(np.float64).mean(axis=0)
    for h in range(4):
        np.testing.assert_allclose(got[0, h], mean_v[h // 2], rtol=0, atol=1e-14)


def test_zero_length_gives_zero():
    q, K, V, pool, bt, L = random_paged_case(33, [5, 7], 2, 2, 8, 16)
    L = L.copy()
    L[0] = 0
    got = oracle_decode(q, pool, bt, L, 16, 0.5)
    assert np.all(got[0] == 0) and np.all(np.isfinite(got[1]))


def test_permutation_of_physical_blocks_is_invisible():
    """Blocks may come back in any order ([nano-vllm blog §2.2]); relabelling
    physical blocks changes nothing, bit for bit."""
    b = make_custom("perm", 41, [37, 16, 70, 3], 8, 4, 32, 16, "f16", "f16")
    bt = b.block_table_array()
    ref = oracle.paged_decode(b.query, "f16", b.kv_pool, "f16", bt, b.context_lens, 16, b.scale)
    perm = np.random.default_rng(42).permutation(b.num_blocks)
    pool2 = np.empty_like(b.kv_pool)
    pool2[perm] = b.kv_pool                      # old block i now lives at perm[i]
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    got = oracle.paged_decode(b.query, "f16", pool2, "f16", bt2, b.context_lens, 16, b.scale)
    assert np.array_equal(got, ref)


def test_poisoned_unused_slots_are_ignored():
    """Leftover slots of the last block must not count ([nano-vllm blog §2.3])."""
    b = make_custom("poison", 43, [20, 1, 33], 4, 4, 16, 16, "f16", "f16")
    bt = b.block_table_array()
    ref = oracle.paged_decode(b.query, "f16", b.kv_pool, "f16", bt, b.context_lens, 16, b.scale)
    pool = b.kv_pool.copy()
    used = set()
    for s, L in enumerate(b.context_lens):
        for t in range(int(L)):
            used.add((b.tables[s][t // 16], t % 16))
    for blk in range(b.num_blocks):
        for o in range(16):
            if (blk, o) not in used:
                pool[blk, :, o] = 0x7E00                 # fp16 NaN
    got = oracle.paged_decode(b.query, "f16", pool, "f16", bt, b.context_lens, 16, b.scale)
    assert np.isfinite(got).all()
    assert np.array_equal(got, ref)


def test_shared_prefix_equals_private_copies():
    """Sharing physical prefix blocks is transparent ([nano-vllm blog §6.3])."""
    b = make_prefix_shared(seed=44, num_seqs=4, seq_len=150, group=2, prefix_tokens=128)
    assert max(b.manager.ref_count) == 2
    bt = b.block_table_array()
    ref = oracle.paged_decode(b.query, "f16", b.kv_pool, "f16", bt, b.context_lens, 32, b.scale)
    # give every sequence private copies of its blocks
    tabs, pool = [], [b.kv_pool]
    nxt = b.num_blocks
    for s, tab in enumerate(b.tables):
        new = []
        for blk in tab:
            pool.append(b.kv_pool[blk:blk + 1])
            new.append(nxt)
            nxt += 1
        tabs.append(new)
    pool = np.concatenate(pool)
    bt2 = np.array(tabs, dtype=np.int32)
    got = oracle.paged_decode(b.query, "f16", pool, "f16", bt2, b.context_lens, 32, b.scale)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# cache write

def test_cache_write_tiny_slots():
    """Tiny workload: the 16-token sequence's 17th token opens a new block at
    offset 0; the 20-token sequence's 21st token lands at offset 4 of block 1
    ([CANN notes §4.3]: allocate when the tail is full, else write at token_used)."""
    b = make_tiny()
    lens_after = b.context_lens + 1
    added = [b.manager.grow_to(tab, int(L)) for tab, L in zip(b.tables, lens_after)]
    assert [len(a) for a in added] == [0, 0, 1, 0]
    bt = b.block_table_array()
    pool = b.kv_pool
    new = oracle.cache_write(pool, "f16", b.new_key[0], b.new_value[0], "f16", bt, lens_after, 16)
    expect_slots = {0: (b.tables[0][1], 4), 1: (b.tables[1][2], 5), 2: (b.tables[2][1], 0), 3: (b.tables[3][0], 1)}
    diff = np.argwhere((new != pool).any(axis=(3, 4)))
    changed = {(int(bk), int(kv), int(o)) for bk, kv, o in diff}
    want = set()
    for s, (blk, off) in expect_slots.items():
        want |= {(blk, 0, off), (blk, 1, off)}
        assert np.array_equal(new[blk, 0, off], b.new_key[0][s])
        assert np.array_equal(new[blk, 1, off], b.new_value[0][s])
    assert changed <= want
    assert len(want) == 8


def test_cache_write_zero_length_is_noop():
    b = make_tiny()
    lens = np.array([0, -1, 0, 0], dtype=np.int32)
    new = oracle.cache_write(b.kv_pool, "f16", b.new_key[0], b.new_value[0], "f16",
                             b.block_table_array(), lens, 16)
    assert np.array_equal(new, b.kv_pool)


def test_write_then_decode_attends_new_token():
    """After the write the newest token takes part in attention ([CANN notes §4.3])."""
    b = make_custom("wd", 45, [3], 2, 2, 8, 16, "f16", "f16", appends=1)
    lens = b.context_lens + 1
    b.manager.grow_to(b.tables[0], int(lens[0]))
    bt = b.block_table_array()
    pool = oracle.cache_write(b.kv_pool, "f16", b.new_key[0], b.new_value[0], "f16", bt, lens, 16)
    K, V = oracle.gather_kv(pool, "f16", bt[0], int(lens[0]), 16)
    assert np.array_equal(K[-1], oracle.to_f64(b.new_key[0][0], "f16"))
    assert np.array_equal(V[-1], oracle.to_f64(b.new_value[0][0], "f16"))


# ---------------------------------------------------------------------------
# fp8 e4m3 codec

def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = oracle.e4m3_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], ref[~nan])
    assert np.array_equal(np.signbit(tab[~nan]), np.signbit(ref[~nan]))


def test_e4m3_fixture_values():
    g = load_golden("e4m3_values.json")
    for code, val in g["code_to_value"]:
        v = oracle.e4m3_value(int(code, 16))
        assert v == val and math.copysign(1, v) == math.copysign(1, val)
    for code in g["nan_codes"]:
        assert math.isnan(oracle.e4m3_value(int(code, 16)))
    for x, code in g["round_to_nearest_even"] + g["saturate"]:
        x = float(x)
        assert int(oracle.e4m3_encode(np.float32(x))) == int(code, 16), (x, code)


def test_e4m3_encode_decode_roundtrip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    assert oracle.e4m3_encode(np.float32(np.nan)) in (0x7F, 0xFF)


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(51)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(40.0),
        (rng.standard_normal(50000) * 1e-3).astype(np.float32),
        rng.uniform(-464, 464, 50000).astype(np.float32),
    ])
    # every midpoint between neighbouring codes, and just either side of it
    grid = oracle.e4m3_decode_table()[:0x7F]
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    x = x[np.abs(x) <= 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)


def test_e4m3_quantise_divides_in_float32():
    x = np.array([1.0, 3.0, -7.5, 1e-6, 300.0], dtype=np.float32)
    s = 0.1
    y = x / np.float32(s)
    assert np.array_equal(oracle.e4m3_quantise(x, s), oracle.e4m3_encode(y))
    assert int(oracle.e4m3_quantise(np.float32(1000.0), 1.0)) == 0x7E


def test_fp8_decode_uses_scaled_values():
    b = make_custom("fp8", 52, [40, 17], 8, 2, 16, 16, "bf16", "fp8_e4m3")
    pool = oracle.encode_pool(b.kv_source, "bf16", "fp8_e4m3", b.k_scale, b.v_scale)
    bt = b.block_table_array()
    got = oracle.paged_decode(b.query, "bf16", pool, "fp8_e4m3", bt, b.context_lens, 16,
                              b.scale, b.k_scale, b.v_scale)
    K = [oracle.gather_kv(pool, "fp8_e4m3", bt[s], int(L), 16)[0] * b.k_scale for s, L in enumerate(b.context_lens)]
    V = [oracle.gather_kv(pool, "fp8_e4m3", bt[s], int(L), 16)[1] * b.v_scale for s, L in enumerate(b.context_lens)]
    q = oracle.to_f64(b.query, "bf16")
    for s in range(2):
        qs = torch.from_numpy(q[s]).reshape(1, 8, 1, 16)
        ks = torch.from_numpy(K[s]).permute(1, 0, 2).unsqueeze(0).contiguous()
        vs = torch.from_numpy(V[s]).permute(1, 0, 2).unsqueeze(0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, scale=b.scale, enable_gqa=True)
        np.testing.assert_allclose(got[s], ref.reshape(8, 16).numpy(), rtol=0, atol=1e-12)
    # quantisation error stays small against the unquantised source values
    src_pool = b.kv_source.view(np.uint16)
    exact = oracle.paged_decode(b.query, "bf16", src_pool, "bf16", bt, b.context_lens, 16, b.scale)
    assert np.abs(got - exact).max() < 0.1


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above

def _gather_no_tail_mask(kv_pool, kv_dtype, row, L, bs):
    n = -(-L // bs)
    t = np.arange(n * bs)                       # reads every slot of the last block
    blk = np.asarray(row)[t // bs]
    K = opa.to_f64(kv_pool[blk, 0, t % bs], kv_dtype)
    V = opa.to_f64(kv_pool[blk, 1, t % bs], kv_dtype)
    return K, V


def _gather_swapped_index(kv_pool, kv_dtype, row, L, bs):
    t = np.arange(L)
    blk = np.asarray(row)[np.minimum(t % bs, len(row) - 1)]
    K = opa.to_f64(kv_pool[blk, 0, np.minimum(t // bs, bs - 1)], kv_dtype)
    V = opa.to_f64(kv_pool[blk, 1, np.minimum(t // bs, bs - 1)], kv_dtype)
    return K, V


_REAL_GATHER = opa.gather_kv


def _gather_k_for_v(kv_pool, kv_dtype, row, L, bs):
    K, _ = _REAL_GATHER(kv_pool, kv_dtype, row, L, bs)
    return K, K


def _decode_wrong_group(query, q_dtype, kv_pool, kv_dtype, block_tables, context_lens, block_size,
                        scale, k_scale=1.0, v_scale=1.0, seqs=None):
    q = opa.to_f64(query, q_dtype)
    B, Hq, D = q.shape
    Hkv = kv_pool.shape[3]
    out = np.zeros((B, Hq, D))
    for s in range(B):
        K, V = opa.gather_kv(kv_pool, kv_dtype, block_tables[s], int(context_lens[s]), block_size)
        for h in range(Hq):
            g = h % Hkv                                 # wrong head mapping
            z = scale * (K[:, g] @ q[s, h])
            p = np.exp(z - z.max())
            out[s, h] = (p / p.sum()) @ V[:, g]
    return out


@pytest.mark.parametrize("mutant", ["no_tail_mask", "swapped_index", "k_for_v"])
def test_planted_gather_mistakes_are_caught(monkeypatch, mutant):
    bad = {"no_tail_mask": _gather_no_tail_mask, "swapped_index": _gather_swapped_index,
           "k_for_v": _gather_k_for_v}[mutant]
    monkeypatch.setattr(opa, "gather_kv", bad)
    failures = 0
    for case in DENSE_CASES:
        try:
            check_dense_equivalence(case)
        except AssertionError:
            failures += 1
    assert failures > 0


def test_planted_head_mapping_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "paged_decode", _decode_wrong_group)
    with pytest.raises(AssertionError):
        check_dense_equivalence(DENSE_CASES[1])


def test_planted_encoder_mistake_is_caught(monkeypatch):
    import oracle.fp8_e4m3 as f8
    grid = f8._GRID

    def truncating(y):                       # rounds toward zero instead of to nearest
        a = np.abs(np.asarray(y, np.float32).astype(np.float64))
        idx = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 0x7E)
        return (idx.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)

    monkeypatch.setattr(oracle, "e4m3_encode", truncating)
    with pytest.raises(AssertionError):
        test_e4m3_fixture_values()


# ---------------------------------------------------------------------------
# allocator usage counters ([CANN notes §5.4]) and last-block waste
# ([nano-vllm blog §5.1]: about block_size / 2 tokens per sequence)

@pytest.mark.parametrize("bs", [8, 16, 32])
def test_last_block_waste_closed_form(bs):
    """Lengths covering every residue mod block_size equally often waste
    exactly (block_size - 1) / 2 slots per sequence on average, and the
    slot utilisation is tokens / allocated slots."""
    lens = list(range(1, 4 * bs + 1))                   # 4 full periods of residues
    mgr = BlockManager(sum(blocks_for_tokens(L, bs) for L in lens) + 5, bs)
    tables = []
    for L in lens:
        tab = []
        mgr.grow_to(tab, L)
        tables.append(tab)
    u = mgr.usage(tables, lens)
    assert u["waste_tokens_per_seq"] == (bs - 1) / 2
    slots = sum(-(-L // bs) for L in lens) * bs
    assert u["slot_utilisation"] == sum(lens) / slots
    assert u["allocated_blocks"] == u["used_blocks"] == slots // bs
    assert u["pool_blocks"] - u["allocated_blocks"] == 5


def test_usage_counts_shared_blocks_once():
    b = make_prefix_shared(num_seqs=16, seq_len=300, prefix_tokens=256)
    u = b.manager.usage(b.tables, b.context_lens)
    per_table = sum(len(t) for t in b.tables)
    assert u["used_blocks"] < per_table                  # the shared prefix is counted once
    assert u["used_blocks"] == u["allocated_blocks"]
