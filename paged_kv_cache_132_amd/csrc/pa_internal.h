// Internal interfaces of the paged-attention library: launch plans, kernel
// argument blocks and launcher entry points shared by the host API and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Threads per workgroup of the decode kernel: four wave64 waves.
constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = kDecodeThreads / 64;

// Geometry of the decode kernel for one (head_dim, kv dtype): a K or V row of
// one KV head (head_dim elements) is read by `row_lanes` lanes with one
// 16-byte load each, so one wave-wide load covers `rows` = 64 / row_lanes
// consecutive KV heads of one token.  A workgroup owns such a group of heads.
//
// Grouped-query attention with head_dim 128 runs instead on the matrix cores
// (decode_gqa_mfma.hip for fp8 KV, decode_gqa16_mfma.hip for fp16 / bf16
// KV): one wave per KV head, 4 KV heads per workgroup.
struct DecodeGeometry {
    bool mfma;       // grouped-query kernel on the matrix cores
    int kv_bytes;    // bytes per KV element
    int row_lanes;   // lanes per KV-head row (vector kernel)
    int rows;        // KV heads per workgroup
    int elems;       // KV elements per lane per token (vector kernel)
    // most workgroups of the attention kernel one compute unit holds: 2 for
    // the matrix-core kernels (registers or LDS allow no more), 8 (the
    // hardware's wave limit) for the vector kernel.  It bounds the token
    // chunks the workspace has room for; a launch never makes more chunks.
    int max_per_cu;
};

bool gqa_mfma_supported(pa_dtype q_dtype, pa_dtype kv_dtype, int head_dim, int group_size);
bool gqa16_mfma_supported(pa_dtype q_dtype, pa_dtype kv_dtype, int head_dim, int group_size);
DecodeGeometry decode_geometry(int head_dim, pa_dtype kv_dtype, int group_size, int block_size);

// Host-side launch plan of one pa_decode call.
//
// Fixed partitions (partition > 0): every sequence is cut into pieces of
// `partition` tokens; a workgroup owns one piece of one sequence.  Token
// chunks (partition == 0, the library's choice): the batch's tokens, laid end
// to end, are cut on the device into as many equal chunks as the GPU holds
// workgroups at once (at least part_min tokens each); a workgroup owns one
// chunk, which may span several sequences.
struct DecodePlan {
    DecodeGeometry geo;
    int groups;          // ceil(num_kv_heads / rows)
    int partition;       // tokens per split-K partition (multiple of block_size); 0: token chunks
    int part_min;        // token chunks: shortest chunk
    int max_partitions;  // fixed partitions: ceil(max tokens / partition)
    int max_chunks;      // token chunks: most chunks a launch can have
    int run_partition;   // partition the shared-run form uses when the caller leaves it to the library
    int64_t grid;        // workgroups launched (token chunks: an upper bound, refined at launch)
    size_t off_n, off_ml, off_o, bytes;   // workspace layout
};

// Pure argument checks (no HIP calls): shared by the API and the CPU tests.
pa_status check_decode_args(const void* out, const void* query, pa_dtype q_dtype,
                            const void* kv_pool, pa_dtype kv_dtype,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                            int32_t num_blocks, float scale, float k_scale, float v_scale,
                            int32_t partition_size);
bool plan_decode(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                 int32_t block_size, int32_t max_blocks_per_seq, pa_dtype kv_dtype,
                 int32_t partition_size, DecodePlan* plan);

struct DecodeArgs {
    void* out;
    const void* query;
    const void* kv_pool;
    const int32_t* block_tables;
    const int32_t* context_lens;
    // Split-K partial results, one slot per segment that is not its
    // sequence's whole range: fixed partitions, slot s * max_partitions + p;
    // token chunks, slot 2c or 2c + 1 of chunk c.
    int32_t* part_n;        // token chunks: [num_seqs, 4] where each sequence's partials lie
    float* part_ml;         // [slots, num_heads, 2] (max, sum) in the log2 domain
    float* part_o;          // [slots, num_heads, head_dim]
    int32_t num_seqs, num_heads, num_kv_heads;
    int32_t block_size, block_shift, max_blocks_per_seq, num_blocks;
    int32_t groups, partition, max_partitions;
    // token chunks (partition == 0): shortest chunk, most chunks, and the
    // workgroups the attention kernel keeps resident on the whole GPU
    int32_t part_min, max_chunks, target_items;
    // partition 0 with a batch that shares prefix blocks, or shared runs:
    // the fixed partition taken instead
    int32_t fallback_partition;
    // token chunks: tokens of layout laid ahead of every sequence (a whole
    // number of blocks, no work), standing for what starting a segment costs
    int32_t seg_head;
    float score_scale;      // scale * k_scale * log2(e): scores in the exp2 domain
    float v_scale;
    // Fused cache write (null: none): the newest token's K/V rows
    // [num_seqs, num_kv_heads, head_dim] in the query dtype, stored into the
    // pool (fp8: divided by write_k_scale / write_v_scale, e4m3-encoded) by
    // the wave that reads that token, before it reads it.
    const void* new_key;
    const void* new_value;
    float write_k_scale, write_v_scale;
    // Shared runs (0 or 1: none): sequences share_run*k .. share_run*k +
    // share_run - 1 form run k.  A partition that every sequence of a run
    // holds whole (with tokens after it) and maps to the same physical blocks
    // is computed once for the run by the run kernel; the per-sequence
    // kernel skips it.
    int32_t share_run;
};

struct WriteArgs {
    void* kv_pool;
    const void* key;            // [num_rows, num_kv_heads, head_dim]
    const void* value;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* cu_seqlens;  // packed runs of new tokens; null: one token per sequence
    int32_t num_seqs, num_rows;
    int32_t num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks;
    float k_scale, v_scale;
};

struct PrefillArgs {
    void* out;                  // [num_tokens, num_heads, head_dim], query dtype
    const void* query;          // [num_tokens, num_heads, head_dim]
    const void* kv_pool;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* cu_seqlens;  // [num_seqs + 1]
    int32_t num_seqs, num_tokens, num_heads, num_kv_heads;
    int32_t block_size, block_shift, max_blocks_per_seq, num_blocks;
    int32_t max_new_tokens;     // a sequence with more new tokens is skipped
    float score_scale;          // scale * k_scale * log2(e)
    float v_scale;
    // Fused prompt-stage write (null: none): the new tokens' K/V rows
    // [num_tokens, num_kv_heads, head_dim] in the (16-bit) pool dtype, stored
    // into their slots and read from here by the attention.
    const void* new_key;
    const void* new_value;
};

struct CopyArgs {
    const uint8_t* src;      // device address of the source pool
    uint8_t* dst;            // device address of the destination pool
    const int32_t* mapping;  // [num_pairs, 2]: (source block, destination block)
    int64_t num_pairs, block_bytes;
    int32_t src_num_blocks, dst_num_blocks;
};

// Workgroups of kDecodeThreads threads (and `dyn_lds` bytes of dynamic LDS)
// of `kernel` the current device holds at once: compute units x resident
// workgroups per unit (at most 8 per unit).  Cached per (device, kernel).
int resident_workgroups(const void* kernel, size_t dyn_lds);
// Compute units of the current device; 256 (MI355X) when the device cannot
// be asked.
int device_cus();
// Workgroups a decode launch needs for the plan; with token chunks it also
// sets a->target_items for `kernel`.
int64_t decode_grid(DecodeArgs* a, const DecodePlan& plan, const void* kernel, size_t dyn_lds);

// pa_decode and its variants: argument checks, plan and launches of the
// given phases (kPhasePartials, kPhaseMerge) with the given workspace.
pa_status decode_phases(int phases, void* out, const void* query, pa_dtype q_dtype, const void* kv_pool,
                        pa_dtype kv_dtype, const int32_t* block_tables, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                        float scale, float k_scale, float v_scale, int32_t partition_size,
                        void* workspace, size_t workspace_bytes, void* stream,
                        const void* new_key, const void* new_value, int32_t run_size);

// Launchers (defined next to their kernels).  Return the hipError_t as int.
// phase bit 1: attention pass (partials), bit 2: split-K merge.
constexpr int kPhasePartials = 1;
constexpr int kPhaseMerge = 2;
int launch_decode(const DecodeArgs& a, const DecodePlan& plan, pa_dtype q_dtype, pa_dtype kv_dtype,
                  int head_dim, int group_size, int phases, void* stream);
int launch_decode_gqa_mfma(const DecodeArgs& a, const DecodePlan& plan, int group_size, void* stream);
int launch_decode_gqa16_mfma(const DecodeArgs& a, const DecodePlan& plan, pa_dtype kv_dtype, int group_size,
                             void* stream);
// the shared-run form on the matrix cores (16-bit KV, head_dim 128, block size >= 16)
int launch_run_gqa16_mfma(const DecodeArgs& a, pa_dtype kv_dtype, void* stream);
int launch_cache_write(const WriteArgs& a, pa_dtype src_dtype, pa_dtype kv_dtype, void* stream);
int launch_copy_blocks(const CopyArgs& a, void* stream);
int64_t prefill_grid(int num_seqs, int num_kv_heads, int group_size, int max_new_tokens, int num_tokens);
int launch_prefill(const PrefillArgs& a, pa_dtype kv_dtype, int head_dim, int group_size, int max_new_tokens,
                   void* stream);

}  // namespace pa
