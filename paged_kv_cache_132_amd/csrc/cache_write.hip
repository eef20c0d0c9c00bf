// pa_cache_write / pa_cache_write_tokens kernels: put new K/V rows into their
// paged slots -- each sequence's newest token in the decode step
// ([nano-vllm blog §4.1 step 3], [CANN notes §4.3 steps 1-3]), or a packed
// run of new tokens per sequence in the prompt stage ([CANN notes §3.1,
// §4.2]: token i of sequence s's run sits at position L_s - n_s + i, so the
// last block is written only as far as the tokens it holds).
//
// Workgroup = (source row, K or V, piece of up to 16 KiB of that half-row).
// The row's slot -- sequence, position, physical block -- is found once per
// workgroup from wave-uniform values (a packed row by binary search over
// cu_seqlens).  A half-row (all KV heads of one token) is contiguous both in
// the source [rows, num_kv_heads, head_dim] and in its pool slot, so thread
// chunks of 16 source bytes map to the same element offsets on both sides
// and every workgroup reads and writes one contiguous segment.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "kv_encode.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWriteThreads = 256;
constexpr int kElemsPerThread = 8;                   // one 16-byte chunk of a 16-bit source
constexpr int kChunksPerThread = 4;
constexpr int kChunksPerGroup = kWriteThreads * kChunksPerThread;

template <int SRC, int KVT>
__global__ __launch_bounds__(kWriteThreads) void cache_write_kernel(WriteArgs a) {
    const int row = blockIdx.x;
    const int kv = blockIdx.y & 1;
    const int piece = blockIdx.y >> 1;

    int s, t;
    if (a.cu_seqlens == nullptr) {
        s = row;
        t = a.context_lens[s] - 1;
    } else {
        // the sequence whose run holds this row: largest s with cu[s] <= row
        if (row >= a.cu_seqlens[a.num_seqs]) return;
        int lo = 0, hi = a.num_seqs;                 // cu[lo] <= row < cu[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.cu_seqlens[mid] <= row) lo = mid;
            else hi = mid;
        }
        s = lo;
        const int first = a.cu_seqlens[s];
        const int n = a.cu_seqlens[s + 1] - first;
        t = a.context_lens[s] - n + (row - first);
    }
    if (t < 0) return;
    const int lb = t / a.block_size;
    if (lb >= a.max_blocks_per_seq) return;
    const int blk = a.block_tables[(int64_t)s * a.max_blocks_per_seq + lb];
    if (blk < 0 || blk >= a.num_blocks) return;
    const int off = t - lb * a.block_size;

    const int64_t half = (int64_t)a.num_kv_heads * a.head_dim;        // elements of one token's K (or V)
    const int n_chunks = (int)(half / kElemsPerThread);
    const uint16_t* src = static_cast<const uint16_t*>(kv ? a.value : a.key) + (int64_t)row * half;
    const int64_t dst_elem = (((int64_t)blk * 2 + kv) * a.block_size + off) * half;
    const float scale = kv ? a.v_scale : a.k_scale;
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
        const int j = piece * kChunksPerGroup + u * kWriteThreads + threadIdx.x;
        if (j >= n_chunks) break;
        const uint4 w = *reinterpret_cast<const uint4*>(src + (int64_t)j * kElemsPerThread);
        if constexpr (KVT != PA_FP8_E4M3) {
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.kv_pool) + dst_elem + (int64_t)j * kElemsPerThread) = w;
        } else {
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < kElemsPerThread; ++e) {
                const uint32_t h = (ws[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
                const float y = __fdiv_rn(widen<SRC>(h), scale);
                packed[e >> 2] |= e4m3_from_float(y) << ((e & 3) * 8);
            }
            *reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.kv_pool) + dst_elem + (int64_t)j * kElemsPerThread) =
                make_uint2(packed[0], packed[1]);
        }
    }
}

template <int SRC, int KVT>
int launch_typed(const WriteArgs& a, hipStream_t stream) {
    if (a.num_rows <= 0) return 0;
    const int64_t n_chunks = (int64_t)a.num_kv_heads * a.head_dim / kElemsPerThread;
    const int64_t pieces = (n_chunks + kChunksPerGroup - 1) / kChunksPerGroup;
    const dim3 grid((unsigned)a.num_rows, (unsigned)(2 * pieces));
    hipLaunchKernelGGL((cache_write_kernel<SRC, KVT>), grid, dim3(kWriteThreads), 0, stream, a);
    return (int)hipGetLastError();
}

}  // namespace

int launch_cache_write(const WriteArgs& a, pa_dtype src_dtype, pa_dtype kv_dtype, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (kv_dtype == PA_F16) return launch_typed<PA_F16, PA_F16>(a, st);
    if (kv_dtype == PA_BF16) return launch_typed<PA_BF16, PA_BF16>(a, st);
    if (src_dtype == PA_BF16) return launch_typed<PA_BF16, PA_FP8_E4M3>(a, st);
    return launch_typed<PA_F16, PA_FP8_E4M3>(a, st);
}

}  // namespace pa
