"""Pins of the packed multi-token write and paged prefill oracle -- CPU only.

Ties: the packed-layout example of [CANN notes §3.1] (golden fixture); torch's
scaled-dot-product attention in float64 with its own causal mask on
contiguous K/V (fresh prompts) and with an explicit mask built from absolute
positions (prompts with a cached prefix); the last prefill row against the
independently pinned decode oracle; a multi-token write against repeated
single-token writes; the 20-token prompt of [CANN notes §4.2]; chunked
prefill against one-shot prefill; no attention across sequence boundaries.
Planted mistakes in the oracle must fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.prefill as opf
from tests.conftest import load_golden
from tests.test_oracle_pins import scatter_contiguous
from workloads import BlockManager
from workloads.block_manager import blocks_for_tokens


def _case(seed, lens, new, Hq, Hkv, D, bs, spare=3):
    """Contiguous K/V per sequence (full length), a pool holding them, packed
    queries for the last `new[s]` positions of each sequence."""
    rng = np.random.default_rng(seed)
    nblk = sum(blocks_for_tokens(L, bs) for L in lens) + spare
    mgr = BlockManager(nblk, bs, rng)
    tables = []
    for L in lens:
        tab = []
        mgr.grow_to(tab, L)
        tables.append(tab)
    K = [rng.standard_normal((L, Hkv, D)).astype(np.float16) for L in lens]
    V = [rng.standard_normal((L, Hkv, D)).astype(np.float16) for L in lens]
    cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    q = rng.standard_normal((int(cu[-1]), Hq, D)).astype(np.float16)
    pool = scatter_contiguous(K, V, tables, lens, nblk, bs).view(np.uint16)
    MB = max(len(t) for t in tables)
    bt = np.full((len(lens), MB), -1, dtype=np.int32)
    for s, tab in enumerate(tables):
        bt[s, :len(tab)] = tab
    return q, K, V, pool, bt, np.array(lens, dtype=np.int32), cu


def _prefill(q, pool, bt, lens, cu, bs, D):
    return oracle.paged_prefill(q.view(np.uint16), "f16", pool, "f16", bt, lens, cu, bs, 1.0 / math.sqrt(D))


def _sdpa_masked(qs, Ks, Vs, positions, scale):
    """torch SDPA float64: queries at absolute `positions` over keys 0..L-1 of
    one sequence, boolean mask key_pos <= query_pos."""
    n, Hq, D = qs.shape
    L, Hkv, _ = Ks.shape
    qt = torch.from_numpy(qs.astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
    kt = torch.from_numpy(Ks.astype(np.float64)).permute(1, 0, 2).unsqueeze(0).contiguous()
    vt = torch.from_numpy(Vs.astype(np.float64)).permute(1, 0, 2).unsqueeze(0).contiguous()
    mask = torch.from_numpy(np.arange(L)[None, :] <= np.asarray(positions)[:, None])
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                                         enable_gqa=(Hkv != Hq))
    return o.squeeze(0).permute(1, 0, 2).numpy()


def test_packed_layout_example():
    g = load_golden("cu_seqlens_example.json")
    cu = np.concatenate([[0], np.cumsum(g["lengths"])])
    assert cu.tolist() == g["cu_seqlens"] and cu[-1] == g["total_tokens"]
    seq, pos = oracle.packed_positions(g["cu_seqlens"], g["lengths"])
    assert seq.tolist() == [0, 0, 0, 1, 1, 1, 1, 1, 2, 2, 3, 3, 3, 3]
    assert pos.tolist() == [0, 1, 2, 0, 1, 2, 3, 4, 0, 1, 0, 1, 2, 3]


PROMPT_CASES = [
    # seed, lens, Hq, Hkv, D, bs
    (51, [3, 5, 2, 4], 4, 4, 16, 16),          # the packed example's lengths
    (52, [20, 37, 16, 1], 8, 2, 16, 16),       # GQA 4, partial tail blocks
    (53, [70, 33], 4, 1, 32, 32),              # MQA, block 32
]


@pytest.mark.parametrize("case", PROMPT_CASES)
def test_fresh_prompts_equal_causal_sdpa(case):
    """No cached prefix (n = L): each sequence is torch's causal attention on
    its own contiguous K/V, and nothing crosses a sequence boundary."""
    seed, lens, Hq, Hkv, D, bs = case
    q, K, V, pool, bt, L, cu = _case(seed, lens, lens, Hq, Hkv, D, bs)
    got = _prefill(q, pool, bt, L, cu, bs, D)
    for s, n in enumerate(lens):
        qs = torch.from_numpy(q[cu[s]:cu[s + 1]].astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
        ks = torch.from_numpy(K[s].astype(np.float64)).permute(1, 0, 2).unsqueeze(0).contiguous()
        vs = torch.from_numpy(V[s].astype(np.float64)).permute(1, 0, 2).unsqueeze(0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, is_causal=True, scale=1.0 / math.sqrt(D),
                                                               enable_gqa=(Hkv != Hq))
        np.testing.assert_allclose(got[cu[s]:cu[s + 1]], ref.squeeze(0).permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_cached_prefix_equals_masked_sdpa_and_decode():
    """Prompts whose first tokens are already cached: queries sit at positions
    L - n .. L - 1 and see the whole prefix; the last row is the decode
    oracle's output for that sequence."""
    lens, new, D = [40, 64, 17], [9, 1, 17], 16
    q, K, V, pool, bt, L, cu = _case(54, lens, new, 8, 4, D, 16)
    got = _prefill(q, pool, bt, L, cu, 16, D)
    for s in range(3):
        pos = np.arange(lens[s] - new[s], lens[s])
        ref = _sdpa_masked(q[cu[s]:cu[s + 1]], K[s], V[s], pos, 1.0 / math.sqrt(D))
        np.testing.assert_allclose(got[cu[s]:cu[s + 1]], ref, rtol=0, atol=1e-12)
    last = cu[1:] - 1
    dec = oracle.paged_decode(q[last].view(np.uint16), "f16", pool, "f16", bt, L, 16, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(got[last], dec, rtol=0, atol=1e-12)


def test_chunked_prefill_equals_one_shot():
    """A 50-token prompt prefilled as 20 + 30 (the second chunk seeing the
    first through the cache) gives the rows of a one-shot prefill."""
    q, K, V, pool, bt, L, cu = _case(55, [50], [50], 4, 2, 16, 16)
    full = _prefill(q, pool, bt, L, cu, 16, 16)
    first = _prefill(q[:20], pool, bt, np.array([20], dtype=np.int32), np.array([0, 20]), 16, 16)
    second = _prefill(q[20:], pool, bt, L, np.array([0, 30]), 16, 16)
    np.testing.assert_allclose(np.concatenate([first, second]), full, rtol=0, atol=1e-13)


def test_sequences_do_not_see_each_other():
    q, K, V, pool, bt, L, cu = _case(56, [30, 30], [30, 30], 4, 4, 16, 16)
    base = _prefill(q, pool, bt, L, cu, 16, 16)
    pool2 = pool.copy()
    for blk in bt[1][bt[1] >= 0]:
        pool2[blk] = np.float16(7.0).view(np.uint16)     # rewrite sequence 1's K/V
    other = _prefill(q, pool2, bt, L, cu, 16, 16)
    np.testing.assert_array_equal(other[:30], base[:30])
    assert np.abs(other[30:] - base[30:]).max() > 1e-3


def test_multi_token_write_equals_single_token_writes():
    """Writing n tokens per sequence in one call is n one-token writes with
    growing lengths (the single-token write is pinned separately)."""
    rng = np.random.default_rng(57)
    bs, Hkv, D = 16, 2, 16
    lens, new = np.array([20, 37, 5], dtype=np.int32), [20, 6, 3]
    nblk = 12
    mgr = BlockManager(nblk, bs, rng)
    bt = np.full((3, 3), -1, dtype=np.int32)
    for s, Ls in enumerate(lens):
        tab = []
        mgr.grow_to(tab, int(Ls))
        bt[s, :len(tab)] = tab
    cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    k = rng.integers(0, 1 << 16, size=(int(cu[-1]), Hkv, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(int(cu[-1]), Hkv, D), dtype=np.uint16)
    pool = np.full((nblk, 2, bs, Hkv, D), 0x7E00, dtype=np.uint16)
    got = oracle.cache_write_tokens(pool, "f16", k, v, "f16", bt, lens, cu, bs)
    want = pool
    for i in range(max(new)):
        sel = [s for s in range(3) if i < new[s]]
        step_lens = np.array([lens[s] - new[s] + i + 1 if i < new[s] else 0 for s in range(3)], dtype=np.int32)
        kk = np.zeros((3, Hkv, D), dtype=np.uint16)
        vv = np.zeros((3, Hkv, D), dtype=np.uint16)
        for s in sel:
            kk[s], vv[s] = k[cu[s] + i], v[cu[s] + i]
        want = oracle.cache_write(want, "f16", kk, vv, "f16", bt, step_lens, bs)
    np.testing.assert_array_equal(got, want)


def test_twenty_token_prompt_fills_four_slots_of_block_two():
    g = load_golden("partial_tail.json")
    bs, L = g["block_size"], g["length"]
    bt = np.array([[3, 1]], dtype=np.int32)
    k = np.arange(L * 2 * 4, dtype=np.uint16).reshape(L, 2, 4)
    pool = np.full((4, 2, bs, 2, 4), 0xFFFF, dtype=np.uint16)
    out = oracle.cache_write_tokens(pool, "f16", k, k, "f16", bt, [L], [0, L], bs)
    written = (out != 0xFFFF).any(axis=(1, 3, 4))            # [block, offset]
    assert written[3].sum() == bs and written[1].sum() == g["valid_in_last"]
    assert written[1][:g["valid_in_last"]].all() and not written[[0, 2]].any()


def test_planted_mask_mistake_is_caught(monkeypatch):
    def strict(query, q_dtype, kv_pool, kv_dtype, block_tables, context_lens, cu_seqlens, block_size, scale,
               k_scale=1.0, v_scale=1.0):
        # keys strictly before the query (drops the diagonal) -- wrong
        total, Hq, D = query.shape
        q = oracle.to_f64(query, q_dtype)
        out = np.zeros((total, Hq, D))
        cu = np.asarray(cu_seqlens)
        for s in range(len(cu) - 1):
            n = int(cu[s + 1] - cu[s]); L = int(context_lens[s])
            Kf, Vf = oracle.gather_kv(kv_pool, kv_dtype, block_tables[s], L, block_size)
            for i in range(n):
                p = L - n + i
                for h in range(Hq):
                    g = h // (Hq // kv_pool.shape[3])
                    z = scale * (Kf[: max(p, 1), g] @ q[cu[s] + i, h])
                    w = np.exp(z - z.max())
                    out[cu[s] + i, h] = (w / w.sum()) @ Vf[: max(p, 1), g]
        return out
    monkeypatch.setattr(oracle, "paged_prefill", strict)
    with pytest.raises(AssertionError):
        test_fresh_prompts_equal_causal_sdpa(PROMPT_CASES[1])


def test_planted_alignment_mistake_is_caught(monkeypatch):
    def top_left(query, q_dtype, kv_pool, kv_dtype, block_tables, context_lens, cu_seqlens, block_size, scale,
                 k_scale=1.0, v_scale=1.0):
        # queries placed at positions 0..n-1 instead of L-n..L-1 -- wrong
        cu = np.asarray(cu_seqlens)
        n = np.diff(cu)
        return opf.paged_prefill(query, q_dtype, kv_pool, kv_dtype, block_tables, n.astype(np.int32), cu,
                                 block_size, scale, k_scale, v_scale)
    monkeypatch.setattr(oracle, "paged_prefill", top_left)
    with pytest.raises(AssertionError):
        test_cached_prefix_equals_masked_sdpa_and_decode()
