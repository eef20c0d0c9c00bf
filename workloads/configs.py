"""The five synthetic paged-decode workloads, built from a seed.

Every value comes from ``numpy.random.default_rng(seed)`` (PCG64) in a fixed
order: lengths -> block-table permutation -> query -> key half of the pool ->
value half of the pool -> new key/value (and query) per decode step.  Values
are N(0, 1) in float32, cast to the storage dtype with round-to-nearest-even.

Nothing here addresses the pool by (block, offset) or encodes fp8: the pool is
filled slot-for-slot with random values (every slot, spare blocks included),
and the block tables are lists of block ids handed out by the allocator.  For
fp8 KV the generator returns the pre-quantisation values (``kv_source``, bf16)
and the per-tensor scales; turning them into e4m3 codes is the cache write's
job, done by whichever side consumes the batch.

Workloads (shapes of the pages' examples; KV layout [num_blocks, 2, block_size,
num_kv_heads, head_dim] from [CANN notes §2.1]):
  tiny        4 seqs, lengths {20, 37, 16, 1}, 8/8 heads, head_dim 64, fp16,
              block_size 16, 64 physical blocks; one new token per sequence.
  llama7b     32 seqs, 32/32 heads, head_dim 128, fp16, block_size 16,
              lengths uniform in [128, 2048], pool = used blocks + 10 %.
  mixed       8 seqs with the lengths of [CANN notes §1.2] (they sum to 5256),
              32/32 heads, head_dim 128, fp16, block_size 16 or 32, a number
              of append+decode steps.
  prefix13b   64 seqs of 5000 tokens, 40/40 heads, head_dim 128, fp16,
              block_size 32; groups of 8 share the physical blocks of the
              first 4480 tokens (140 full blocks, refcount 8).
  gqa_fp8     256 seqs, 32 query heads over 8 KV heads, head_dim 128, bf16
              query, fp8 e4m3 KV with per-tensor fp32 scales, block_size 16,
              lognormal lengths (median 1000, sigma 1, clipped to [16, 8192]).
  gqa_bf16    64 seqs, 64 query heads over 8 KV heads (GQA-8), head_dim 128,
              bf16 query and KV, block_size 16, lengths uniform in
              [512, 4096] (16-bit grouped-query decode, beyond the pages'
              workloads: the matrix-core kernel for 16-bit KV).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .block_manager import BlockManager, blocks_for_tokens, full_blocks

DTYPES = ("f16", "bf16", "fp8_e4m3")

# Element size in bytes of each storage dtype.
ELEM_BYTES = {"f16": 2, "bf16": 2, "fp8_e4m3": 1}


def _f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); finite inputs only."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def _normal_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) float32 values cast to the bit pattern of a 16-bit storage dtype."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f16":
        return _f32_to_f16_bits(x)
    if dtype == "bf16":
        return _f32_to_bf16_bits(x)
    raise ValueError(f"not a 16-bit dtype: {dtype}")


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact: bf16 is the top half of binary32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class PagedBatch:
    name: str
    seed: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str
    kv_dtype: str
    src_dtype: str
    scale: float
    k_scale: float
    v_scale: float
    context_lens: np.ndarray          # int32 [B], lengths the decode attends over
    tables: list                      # per sequence: list of physical block ids
    manager: BlockManager
    max_blocks_per_seq: int           # columns of the padded block-table array
    query: np.ndarray                 # raw bits [B, Hq, D] of q_dtype
    kv_pool: np.ndarray | None        # raw bits [NB, 2, bs, Hkv, D] (16-bit KV)
    kv_source: np.ndarray | None      # bf16 bits [NB, 2, bs, Hkv, D] (fp8 KV, pre-quantisation)
    new_key: np.ndarray               # raw bits [S, B, Hkv, D] of src_dtype
    new_value: np.ndarray             # raw bits [S, B, Hkv, D] of src_dtype
    step_query: np.ndarray            # raw bits [S, B, Hq, D] of q_dtype
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return self.manager.num_blocks

    @property
    def num_steps(self) -> int:
        """Sets of new key/value/query drawn (one per append step, at least one)."""
        return int(self.new_key.shape[0])

    def block_table_array(self, pad: int = -1) -> np.ndarray:
        """Block tables as an int32 [B, max_blocks_per_seq] array padded with ``pad``."""
        out = np.full((self.num_seqs, self.max_blocks_per_seq), pad, dtype=np.int32)
        for s, tab in enumerate(self.tables):
            if len(tab) > self.max_blocks_per_seq:
                raise ValueError("block table longer than max_blocks_per_seq")
            out[s, : len(tab)] = tab
        return out

    def kv_bytes_per_token(self) -> int:
        """Bytes of K and V for one token of one layer: 2 * Hkv * D * elem_bytes."""
        return 2 * self.num_kv_heads * self.head_dim * ELEM_BYTES[self.kv_dtype]

    def unique_blocks_in_use(self) -> int:
        return int(len({b for tab in self.tables for b in tab}))

    def unique_tokens_in_use(self) -> int:
        """Distinct (block, offset) slots some sequence reads: the tokens a
        batch that shares prefix blocks stores once."""
        slots = set()
        for tab, L in zip(self.tables, self.context_lens):
            for t in range(int(L)):
                slots.add((int(tab[t // self.block_size]), t % self.block_size))
        return len(slots)


def _build(
    name: str,
    seed: int,
    lens_fn,
    num_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    q_dtype: str,
    kv_dtype: str,
    *,
    num_blocks: int | None = None,
    spare: float = 0.10,
    appends: int = 0,
    share_group: int = 1,
    shared_prefix_tokens: int = 0,
    max_blocks_per_seq: int | None = None,
) -> PagedBatch:
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens_fn(rng), dtype=np.int64)
    B = int(lens.shape[0])
    bs = int(block_size)
    final_lens = lens + appends              # lengths after the append+decode steps
    steps = max(int(appends), 1)             # sets of new K/V (and Q) to draw
    if shared_prefix_tokens:
        if B % share_group:
            raise ValueError("number of sequences must be a multiple of the share group")
        prefix_blocks = full_blocks(shared_prefix_tokens, bs)
        if prefix_blocks * bs != shared_prefix_tokens:
            raise ValueError("a shared prefix must consist of full blocks")
        groups = B // share_group
        used = groups * prefix_blocks + sum(
            blocks_for_tokens(int(L), bs) - prefix_blocks for L in final_lens
        )
    else:
        prefix_blocks = 0
        used = sum(blocks_for_tokens(int(L), bs) for L in final_lens)
    if num_blocks is None:
        num_blocks = int(np.ceil(used * (1.0 + spare)))
    if used > num_blocks:
        raise ValueError("pool too small for the workload")

    manager = BlockManager(num_blocks, bs, rng)      # free list = seeded permutation
    tables: list[list[int]] = []
    prefix_of_group: dict[int, list[int]] = {}
    for s in range(B):                                # sequence order, then logical order
        L = int(lens[s])
        if prefix_blocks:
            g = s // share_group
            if g not in prefix_of_group:
                prefix_of_group[g] = manager.allocate(prefix_blocks)
                tab = list(prefix_of_group[g])
            else:
                tab = manager.share(prefix_of_group[g])
        else:
            tab = []
        manager.grow_to(tab, L)
        tables.append(tab)

    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(blocks_for_tokens(int(L), bs) for L in final_lens)

    Hq, Hkv, D = num_heads, num_kv_heads, head_dim
    src_dtype = "bf16" if kv_dtype == "fp8_e4m3" else kv_dtype
    query = _normal_bits(rng, (B, Hq, D), q_dtype)
    pool_shape = (num_blocks, 2, bs, Hkv, D)
    half = (num_blocks, bs, Hkv, D)
    pool = np.empty(pool_shape, dtype=np.uint16)
    pool[:, 0] = _normal_bits(rng, half, src_dtype)   # key half
    pool[:, 1] = _normal_bits(rng, half, src_dtype)   # value half
    new_key = np.empty((steps, B, Hkv, D), dtype=np.uint16)
    new_value = np.empty((steps, B, Hkv, D), dtype=np.uint16)
    step_query = np.empty((steps, B, Hq, D), dtype=np.uint16)
    for t in range(steps):
        new_key[t] = _normal_bits(rng, (B, Hkv, D), src_dtype)
        new_value[t] = _normal_bits(rng, (B, Hkv, D), src_dtype)
        step_query[t] = _normal_bits(rng, (B, Hq, D), q_dtype)

    scale = float(np.float32(1.0 / np.sqrt(D)))
    k_scale = v_scale = 1.0
    kv_pool, kv_source = pool, None
    if kv_dtype == "fp8_e4m3":
        # Per-tensor scales: max |x| / 448 over the generated values, so the
        # largest value maps onto the largest finite e4m3 magnitude.
        k_abs = max(float(np.abs(bf16_bits_to_f32(pool[:, 0])).max()),
                    float(np.abs(bf16_bits_to_f32(new_key)).max()))
        v_abs = max(float(np.abs(bf16_bits_to_f32(pool[:, 1])).max()),
                    float(np.abs(bf16_bits_to_f32(new_value)).max()))
        k_scale = float(np.float32(k_abs / 448.0))
        v_scale = float(np.float32(v_abs / 448.0))
        kv_pool, kv_source = None, pool

    return PagedBatch(
        name=name, seed=seed, num_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        block_size=bs, q_dtype=q_dtype, kv_dtype=kv_dtype, src_dtype=src_dtype,
        scale=scale, k_scale=k_scale, v_scale=v_scale,
        context_lens=lens.astype(np.int32), tables=tables, manager=manager,
        max_blocks_per_seq=int(max_blocks_per_seq), query=query,
        kv_pool=kv_pool, kv_source=kv_source, new_key=new_key,
        new_value=new_value, step_query=step_query,
        notes={"used_blocks": int(used), "prefix_blocks": int(prefix_blocks),
               "prefix_tokens": int(prefix_blocks * bs), "share_group": int(share_group)},
    )


# --------------------------------------------------------------------------
# The five workloads.  Seeds 1..5 by default.

TINY_LENS = (20, 37, 16, 1)
MIXED_LENS = (128, 200, 512, 1024, 2048, 256, 64, 1024)


def make_tiny(seed: int = 1) -> PagedBatch:
    """4 seqs {20,37,16,1}, 8/8 heads, D 64, fp16, bs 16, 64 blocks, one new token each.

    The table has room for the appended token (the 16-token sequence needs a
    second block once it grows to 17)."""
    return _build("tiny", seed, lambda rng: TINY_LENS, 8, 8, 64, 16, "f16", "f16",
                  num_blocks=64, appends=1)


def make_llama7b(seed: int = 2, num_seqs: int = 32, min_len: int = 128, max_len: int = 2048,
                 block_size: int = 16) -> PagedBatch:
    """LLaMA-2-7B single-layer decode: 32/32 heads, D 128, fp16, bs 16, U[128, 2048] lengths.

    Other block sizes (the [nano-vllm blog §5.1] sweep) keep the same lengths."""
    name = "llama7b" if block_size == 16 else f"llama7b_bs{block_size}"
    return _build(name, seed,
                  lambda rng: rng.integers(min_len, max_len, size=num_seqs, endpoint=True),
                  32, 32, 128, block_size, "f16", "f16",
                  max_blocks_per_seq=blocks_for_tokens(max_len, block_size))


def make_mixed(seed: int = 3, block_size: int = 16, steps: int = 33) -> PagedBatch:
    """The mixed-length batch of [CANN notes §1.2]: 8 seqs, 32/32 heads, D 128, fp16."""
    return _build(f"mixed_bs{block_size}", seed, lambda rng: MIXED_LENS, 32, 32, 128,
                  block_size, "f16", "f16", appends=steps)


def make_prefix_shared(seed: int = 4, num_seqs: int = 64, seq_len: int = 5000,
                       group: int = 8, prefix_tokens: int = 4480) -> PagedBatch:
    """13B shape, 40/40 heads, D 128, fp16, bs 32; groups of 8 share 140 prefix blocks."""
    return _build("prefix13b", seed, lambda rng: np.full(num_seqs, seq_len), 40, 40, 128, 32,
                  "f16", "f16", share_group=group, shared_prefix_tokens=prefix_tokens)


def lognormal_lens(rng: np.random.Generator, n: int, median: float = 1000.0, sigma: float = 1.0,
                   lo: int = 16, hi: int = 8192) -> np.ndarray:
    return np.clip(np.rint(np.exp(rng.normal(np.log(median), sigma, size=n))), lo, hi).astype(np.int64)


def make_gqa_fp8(seed: int = 5, num_seqs: int = 256, max_len: int = 8192) -> PagedBatch:
    """GQA-4 with fp8 KV: 32 query heads over 8 KV heads, D 128, bf16 Q, e4m3 KV, bs 16."""
    return _build("gqa_fp8", seed, lambda rng: lognormal_lens(rng, num_seqs, hi=max_len),
                  32, 8, 128, 16, "bf16", "fp8_e4m3",
                  max_blocks_per_seq=blocks_for_tokens(max_len, 16))


def make_gqa_bf16(seed: int = 6, num_seqs: int = 64, min_len: int = 512, max_len: int = 4096) -> PagedBatch:
    """GQA-8 with bf16 KV: 64 query heads over 8 KV heads, D 128, bs 16, U[512, 4096] lengths."""
    return _build("gqa_bf16", seed, lambda rng: rng.integers(min_len, max_len, size=num_seqs, endpoint=True),
                  64, 8, 128, 16, "bf16", "bf16")


def make_custom(name: str, seed: int, lens, num_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, q_dtype: str, kv_dtype: str, **kw) -> PagedBatch:
    """Any other shape (scaled-down parity cases, edge cases)."""
    lens = tuple(int(x) for x in lens)
    return _build(name, seed, lambda rng: lens, num_heads, num_kv_heads, head_dim, block_size,
                  q_dtype, kv_dtype, **kw)


CONFIG_MAKERS = {
    "tiny": make_tiny,
    "llama7b": make_llama7b,
    "mixed_bs16": lambda seed=3: make_mixed(seed, 16),
    "mixed_bs32": lambda seed=3: make_mixed(seed, 32),
    "prefix13b": make_prefix_shared,
    "gqa_fp8": make_gqa_fp8,
    "gqa_bf16": make_gqa_bf16,
}
