// pa_copy_blocks kernel: whole-block copies between two pools of one block
// geometry -- the copy-on-write of a shared block before a branch writes into
// it ([nano-vllm blog §4.3]) and the swap of a preempted request's blocks to
// CPU memory and back ([nano-vllm blog §2.2]).
//
// A block is 2 * block_size * num_kv_heads * head_dim elements, contiguous in
// both pools.  Workgroup w copies a 16 KiB piece of one pair's block: 256
// threads x 16 bytes x 4, all loads issued before the stores, so each
// wave moves 4 KiB of contiguous bytes per instruction group.  Pieces of one
// block go to consecutive workgroups.  Pairs whose block ids fall outside
// their pool are skipped.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyPiece = (int64_t)kCopyThreads * 16 * kCopyUnroll;   // bytes per workgroup

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyArgs a) {
    const int64_t pieces = (a.block_bytes + kCopyPiece - 1) / kCopyPiece;
    const int64_t pair = blockIdx.x / pieces;
    const int64_t piece = blockIdx.x % pieces;
    if (pair >= a.num_pairs) return;
    const int src = a.mapping[2 * pair];
    const int dst = a.mapping[2 * pair + 1];
    if (src < 0 || src >= a.src_num_blocks || dst < 0 || dst >= a.dst_num_blocks) return;
    const uint8_t* s = a.src + (int64_t)src * a.block_bytes;
    uint8_t* d = a.dst + (int64_t)dst * a.block_bytes;
    const int64_t base = piece * kCopyPiece + (int64_t)threadIdx.x * 16;
    u32x4 v[kCopyUnroll];
    if ((piece + 1) * kCopyPiece <= a.block_bytes) {
        // a whole piece (every piece when blocks are multiples of 16 KiB):
        // all loads in flight together, then all stores
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s + base + u * kCopyThreads * 16));
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(d + base + u * kCopyThreads * 16));
        return;
    }
    // the block's last, partial piece: offsets past the end re-read its last
    // 16 bytes and store nothing
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t off = min(base + (int64_t)u * kCopyThreads * 16, a.block_bytes - 16);
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s + off));
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t off = base + (int64_t)u * kCopyThreads * 16;
        if (off < a.block_bytes) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(d + off));
    }
}

}  // namespace

int launch_copy_blocks(const CopyArgs& a, void* stream) {
    const int64_t pieces = (a.block_bytes + kCopyPiece - 1) / kCopyPiece;
    const int64_t grid = pieces * a.num_pairs;
    if (grid == 0) return 0;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0,
                       static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

}  // namespace pa
