// pa_decode_noalloc: pa_decode with its split-K workspace in a fixed device
// array of this library instead of caller memory, for callers that cannot
// allocate (code under graph capture, serving loops, harnesses that forbid
// allocation).  Nothing here allocates: the array is part of the library's
// code object, one copy per GPU, kept until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

// The workspace of every pa_decode_noalloc call on a GPU.  In host code this
// name is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress below, once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchAddress {
    std::mutex mu;
    void* ptr[kMaxDevices] = {};
};

ScratchAddress& addresses() {
    static ScratchAddress a;
    return a;
}

// Device address of the current device's copy of `scratch`; null (with the
// HIP error cleared) if the runtime cannot give it.
void* scratch_address(int dev) {
    ScratchAddress& a = addresses();
    std::lock_guard<std::mutex> lock(a.mu);
    if (!a.ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        a.ptr[dev] = p;
    }
    return a.ptr[dev];
}

}  // namespace
}  // namespace pa

extern "C" {

size_t pa_decode_noalloc_max_workspace(void) { return pa::kScratchBytes; }

pa_status pa_decode_noalloc(void* out, const void* query, pa_dtype q_dtype, const void* kv_pool,
                            pa_dtype kv_dtype, const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                            float k_scale, float v_scale, int32_t partition_size, void* stream) {
    // the plain argument checks first: a call that would be rejected needs no device
    pa_status st = pa::check_decode_args(out, query, q_dtype, kv_pool, kv_dtype, block_tables, context_lens,
                                         num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                         max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, partition_size);
    if (st != PA_OK || num_seqs == 0) return st;
    const size_t need = pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                                 max_blocks_per_seq, kv_dtype, partition_size);
    if (need == 0) return PA_ERR_BAD_SHAPE;
    if (need > pa::kScratchBytes) return PA_ERR_WORKSPACE_TOO_SMALL;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return PA_ERR_HIP;
    }
    if (dev < 0 || dev >= pa::kMaxDevices) return PA_ERR_UNSUPPORTED;
    void* ws = pa::scratch_address(dev);
    if (!ws) return PA_ERR_HIP;
    return pa::decode_phases(pa::kPhasePartials | pa::kPhaseMerge, out, query, q_dtype, kv_pool, kv_dtype,
                             block_tables, context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, partition_size, ws,
                             pa::kScratchBytes, stream, nullptr, nullptr, 1);
}

}  // extern "C"
