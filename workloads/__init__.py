"""Seeded synthetic inputs for paged decode.

This package only *makes inputs*: sequence lengths, block tables handed out by
a host-side free-list allocator, and query / key / value values drawn from a
seeded normal distribution.  It holds none of the attention arithmetic, none
of the cache-write addressing and no fp8 codec, so both the GPU path and the
CPU oracle can be fed from it without sharing any of the method.

Sources (the three web pages on paged KV caches), cited by these short names:
  [nano-vllm blog]  2kiu.com/news/6344849 -- PagedAttention and prefix caching,
                    reproduced with nano-vllm (sections 1-7)
  [vLLM notes]      "vLLM: PagedAttention 与前缀缓存" (personal-site-7tw.pages.dev)
  [CANN notes]      discosf.com/news/6244710 -- Paged KV Cache and Packed
                    Sequence in cann-recipes-infer (sections 1-6)
"""
from .block_manager import BlockManager, PoolExhausted
from .configs import (
    PagedBatch,
    DTYPES,
    make_tiny,
    make_llama7b,
    make_mixed,
    make_prefix_shared,
    make_gqa_fp8,
    make_gqa_bf16,
    make_custom,
    CONFIG_MAKERS,
)
from .prefill import PrefillBatch, make_prefill, make_prefill_mixed

__all__ = [
    "BlockManager",
    "PoolExhausted",
    "PagedBatch",
    "DTYPES",
    "make_tiny",
    "make_llama7b",
    "make_mixed",
    "make_prefix_shared",
    "make_gqa_fp8",
    "make_gqa_bf16",
    "make_custom",
    "CONFIG_MAKERS",
    "PrefillBatch",
    "make_prefill",
    "make_prefill_mixed",
]
