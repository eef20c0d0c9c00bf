"""CPU oracle for paged decode attention and the KV cache write.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline may import this package.  The GPU library never calls it and shares
no code with it (no kernels, headers, helpers, tables or constant generators);
the two meet only at the seeded input generators in ``workloads``.

Plain, slow, float64 numpy.  Pins that tie it to the pages and to mathematics
rather than to itself live in ``tests/test_oracle_pins.py``.

Sources, cited in the modules by these short names:
  [nano-vllm blog]  2kiu.com/news/6344849 -- PagedAttention and prefix caching,
                    reproduced with nano-vllm (sections 1-7)
  [vLLM notes]      "vLLM: PagedAttention 与前缀缓存" (personal-site-7tw.pages.dev)
  [CANN notes]      discosf.com/news/6244710 -- Paged KV Cache and Packed
                    Sequence in cann-recipes-infer (sections 1-6)
  [OCP FP8]         OCP 8-bit Floating Point Specification (OFP8), E4M3
"""
from .fp8_e4m3 import (
    e4m3_value,
    e4m3_decode_table,
    e4m3_decode,
    e4m3_encode,
    e4m3_quantise,
    MAX_FINITE,
)
from .block_manager_model import BlockManagerModel, ModelPoolExhausted
from .block_ops import check_block_mapping, copy_blocks
from .prefill import cache_write_tokens, packed_positions, paged_prefill
from .paged_attention import (
    to_f64,
    kv_bytes_per_token,
    slot_of,
    num_blocks_of,
    gather_kv,
    paged_decode,
    encode_for_cache,
    cache_write,
    encode_pool,
)

__all__ = [
    "BlockManagerModel", "ModelPoolExhausted", "check_block_mapping", "copy_blocks", "cache_write_tokens", "packed_positions", "paged_prefill",
    "e4m3_value", "e4m3_decode_table", "e4m3_decode", "e4m3_encode", "e4m3_quantise",
    "MAX_FINITE", "to_f64", "kv_bytes_per_token", "slot_of", "num_blocks_of", "gather_kv",
    "paged_decode", "encode_for_cache", "cache_write", "encode_pool",
]
