// Host side of the C ABI: argument checks, the split-K launch plan, workspace
// layout and kernel launches.  No device memory is allocated here and no call
// waits for the device.
#include <hip/hip_runtime_api.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <unordered_map>

#include "pa.h"
#include "pa_internal.h"

namespace pa {

namespace {

bool known_dtype(pa_dtype d) { return d == PA_F16 || d == PA_BF16 || d == PA_FP8_E4M3; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int elem_bytes(pa_dtype d) { return d == PA_FP8_E4M3 ? 1 : 2; }

int log2_exact(int x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return (1 << s) == x ? s : -1;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kMaxPartition = 1 << 20;

}  // namespace

DecodeGeometry decode_geometry(int head_dim, pa_dtype kv_dtype, int group_size, int block_size) {
    DecodeGeometry g;
    // fp8 KV is only paired with a bf16 query, 16-bit KV with a query of its
    // own dtype (checked with the arguments); the matrix-core kernels walk
    // 16-token steps that must not cross a block
    g.mfma = block_size >= 16 && (gqa_mfma_supported(PA_BF16, kv_dtype, head_dim, group_size) ||
                                  gqa16_mfma_supported(kv_dtype, kv_dtype, head_dim, group_size));
    g.kv_bytes = kv_dtype == PA_FP8_E4M3 ? 1 : 2;
    g.row_lanes = head_dim * g.kv_bytes / 16;
    g.rows = g.mfma ? kDecodeWaves : 64 / g.row_lanes;
    g.elems = 16 / g.kv_bytes;
    g.max_per_cu = g.mfma ? 2 : 8;
    return g;
}

pa_status check_decode_args(const void* out, const void* query, pa_dtype q_dtype,
                            const void* kv_pool, pa_dtype kv_dtype,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                            int32_t num_blocks, float scale, float k_scale, float v_scale,
                            int32_t partition_size) {
    if (!known_dtype(q_dtype) || !known_dtype(kv_dtype)) return PA_ERR_BAD_DTYPE;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || partition_size < 0)
        return PA_ERR_BAD_SHAPE;
    if (num_heads % num_kv_heads != 0) return PA_ERR_BAD_SHAPE;
    const int group = num_heads / num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
    const bool combo = (q_dtype == PA_F16 && kv_dtype == PA_F16) ||
                       (q_dtype == PA_BF16 && kv_dtype == PA_BF16) ||
                       (q_dtype == PA_BF16 && kv_dtype == PA_FP8_E4M3);
    if (!combo) return PA_ERR_UNSUPPORTED;
    if (partition_size != 0 && (partition_size % block_size != 0 || partition_size > kMaxPartition))
        return PA_ERR_BAD_SHAPE;
    if ((int64_t)max_blocks_per_seq * block_size > (int64_t)INT32_MAX / 2) return PA_ERR_BAD_SHAPE;
    // the kernels step from a block's K half to its V half with a 32-bit offset
    if ((int64_t)block_size * num_kv_heads * head_dim * elem_bytes(kv_dtype) > (int64_t)UINT32_MAX)
        return PA_ERR_BAD_SHAPE;
    if (!isfinite(scale)) return PA_ERR_BAD_SHAPE;
    if (kv_dtype == PA_FP8_E4M3 &&
        !(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f))
        return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0) return PA_OK;
    if (!out || !query || !kv_pool || !block_tables || !context_lens) return PA_ERR_NULL_POINTER;
    if (!aligned16(out) || !aligned16(query) || !aligned16(kv_pool) || !aligned16(block_tables) ||
        !aligned16(context_lens))
        return PA_ERR_MISALIGNED;
    return PA_OK;
}

bool plan_decode(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                 int32_t block_size, int32_t max_blocks_per_seq, pa_dtype kv_dtype,
                 int32_t partition_size, DecodePlan* plan) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
        block_size <= 0 || partition_size < 0 || num_heads % num_kv_heads != 0)
        return false;
    if (head_dim != 64 && head_dim != 128) return false;
    if (!known_dtype(kv_dtype)) return false;
    if (partition_size != 0 && (partition_size % block_size != 0 || partition_size > kMaxPartition))
        return false;
    DecodePlan p;
    p.geo = decode_geometry(head_dim, kv_dtype, num_heads / num_kv_heads, block_size);
    p.groups = (num_kv_heads + p.geo.rows - 1) / p.geo.rows;
    const int64_t max_tokens = (int64_t)max_blocks_per_seq * block_size;
    // The partition the shared-run form takes when the caller leaves it to
    // the library: the largest (fewest partials, least per-workgroup
    // start-up) that still gives at least 2048 workgroups -- 256 CUs several
    // times over -- when every sequence is at its longest.
    {
        const int64_t heads_x_seqs = (int64_t)p.groups * num_seqs;
        int part = 1024;
        while (part > 64 && heads_x_seqs * ((max_tokens + part - 1) / part) < 2048) part /= 2;
        if (part < block_size) part = block_size;
        p.run_partition = (part + block_size - 1) / block_size * block_size;
    }
    // token chunks: at least 128 tokens (whole blocks) each, never more chunks
    // than the GPU holds workgroups at once, nor than the batch's tokens fill
    // (a batch too small to fill the GPU then leaves fewer partials for the
    // merge; 64-token chunks were slower there, 256 too few for the 7B batch)
    p.part_min = (128 + block_size - 1) / block_size * block_size;
    {
        const int64_t by_slots = std::max<int64_t>(1, (int64_t)device_cus() * p.geo.max_per_cu / p.groups);
        const int64_t by_tokens = std::max<int64_t>(1, ((int64_t)num_seqs * max_tokens + p.part_min - 1) / p.part_min);
        p.max_chunks = (int)std::min(by_slots, by_tokens);
    }
    int64_t slots;                                   // partial-result slots the workspace holds
    if (partition_size > 0) {
        p.partition = partition_size;
        p.max_partitions = (int)((max_tokens + partition_size - 1) / partition_size);
        p.grid = (int64_t)p.groups * num_seqs * p.max_partitions;
        slots = (int64_t)num_seqs * p.max_partitions;
    } else {
        p.partition = 0;
        p.max_partitions = (int)((max_tokens + p.run_partition - 1) / p.run_partition);
        p.grid = (int64_t)p.groups * p.max_chunks;
        // room for the chunks' partials, or for the shared-run form's
        slots = std::max<int64_t>(2 * (int64_t)p.max_chunks, (int64_t)num_seqs * p.max_partitions);
    }
    if (p.grid > INT32_MAX || (int64_t)p.groups * num_seqs * p.max_partitions > INT32_MAX) return false;
    const size_t n_part = (size_t)slots * num_heads;
    p.off_n = 0;
    p.off_ml = align_up((size_t)num_seqs * 4 * sizeof(int32_t), 256);
    p.off_o = p.off_ml + align_up(n_part * 2 * sizeof(float), 256);
    p.bytes = p.off_o + align_up(n_part * (size_t)head_dim * sizeof(float), 256);
    if (p.bytes == 0) p.bytes = 256;
    *plan = p;
    return true;
}

namespace {

struct DeviceCache {
    std::mutex mu;
    std::unordered_map<int, int> cus;                                     // device -> compute units
    std::map<std::tuple<int, const void*, size_t>, int> resident;        // (device, kernel, lds) -> workgroups
};

DeviceCache& device_cache() {
    static DeviceCache c;
    return c;
}

int current_cus(int* dev_out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    *dev_out = dev;
    DeviceCache& c = device_cache();
    std::lock_guard<std::mutex> lock(c.mu);
    auto it = c.cus.find(dev);
    if (it != c.cus.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        cus = 0;
    }
    c.cus[dev] = cus;
    return cus;
}

}  // namespace

int device_cus() {
    int dev = 0;
    const int cus = current_cus(&dev);
    return cus > 0 ? cus : 256;
}

int resident_workgroups(const void* kernel, size_t dyn_lds) {
    int dev = 0;
    const int cus = current_cus(&dev);
    if (cus <= 0) return 0;
    DeviceCache& c = device_cache();
    std::lock_guard<std::mutex> lock(c.mu);
    const auto key = std::make_tuple(dev, kernel, dyn_lds);
    auto it = c.resident.find(key);
    if (it != c.resident.end()) return it->second;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kDecodeThreads, dyn_lds) != hipSuccess) {
        (void)hipGetLastError();
        per_cu = 0;
    }
    const int n = std::min(std::max(per_cu, 0) * cus, 8 * cus);
    c.resident[key] = n;
    return n;
}

int64_t decode_grid(DecodeArgs* a, const DecodePlan& plan, const void* kernel, size_t dyn_lds) {
    if (a->partition > 0) return plan.grid;
    // token chunks: one per resident workgroup slot (split among the groups)
    int slots = resident_workgroups(kernel, dyn_lds);
    if (slots <= 0) slots = plan.max_chunks * plan.groups;
    slots = std::min(slots, plan.max_chunks * plan.groups);
    a->target_items = slots;
    // enough workgroups for the chunks, or for the fixed partitions a batch
    // that shares prefix blocks takes instead (those past the layout's items
    // leave at once, in slots the others have freed)
    const int64_t fixed = (int64_t)plan.groups * a->num_seqs * plan.max_partitions;
    return std::max<int64_t>((int64_t)std::max(slots / plan.groups, 1) * plan.groups, fixed);
}

}  // namespace pa

using namespace pa;

extern "C" {

const char* pa_status_string(pa_status status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_NULL_POINTER: return "PA_ERR_NULL_POINTER";
        case PA_ERR_BAD_SHAPE: return "PA_ERR_BAD_SHAPE";
        case PA_ERR_BAD_DTYPE: return "PA_ERR_BAD_DTYPE";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
        case PA_ERR_MISALIGNED: return "PA_ERR_MISALIGNED";
        case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
        case PA_ERR_HIP: return "PA_ERR_HIP";
        case PA_ERR_POOL_EXHAUSTED: return "PA_ERR_POOL_EXHAUSTED";
        case PA_ERR_UNKNOWN_SEQUENCE: return "PA_ERR_UNKNOWN_SEQUENCE";
    }
    return "PA_ERR_UNKNOWN";
}

static pa_status cache_write_rows(void* kv_pool, pa_dtype kv_dtype, const void* key, const void* value,
                                  pa_dtype src_dtype, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* cu_seqlens, int32_t num_seqs,
                                  int32_t num_rows, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                  float k_scale, float v_scale, void* stream) {
    if (!known_dtype(kv_dtype) || !known_dtype(src_dtype)) return PA_ERR_BAD_DTYPE;
    if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks_per_seq <= 0 || num_blocks <= 0)
        return PA_ERR_BAD_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
    const bool combo = (src_dtype == kv_dtype && src_dtype != PA_FP8_E4M3) ||
                       (kv_dtype == PA_FP8_E4M3 && (src_dtype == PA_BF16 || src_dtype == PA_F16));
    if (!combo) return PA_ERR_UNSUPPORTED;
    if (kv_dtype == PA_FP8_E4M3 &&
        !(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f))
        return PA_ERR_BAD_SHAPE;
    if (num_rows < 0) return PA_ERR_BAD_SHAPE;
    if ((int64_t)num_rows * num_kv_heads * head_dim * 2 > (int64_t)INT32_MAX) return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0 || num_rows == 0) return PA_OK;
    if (!kv_pool || !key || !value || !block_tables || !context_lens) return PA_ERR_NULL_POINTER;
    if (!aligned16(kv_pool) || !aligned16(key) || !aligned16(value) || !aligned16(block_tables) ||
        !aligned16(context_lens))
        return PA_ERR_MISALIGNED;

    WriteArgs a;
    a.kv_pool = kv_pool;
    a.key = key;
    a.value = value;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.cu_seqlens = cu_seqlens;
    a.num_seqs = num_seqs;
    a.num_rows = num_rows;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    return launch_cache_write(a, src_dtype, kv_dtype, stream) == 0 ? PA_OK : PA_ERR_HIP;
}

pa_status pa_cache_write(void* kv_pool, pa_dtype kv_dtype, const void* key, const void* value,
                         pa_dtype src_dtype, const int32_t* block_tables,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                         int32_t num_blocks, float k_scale, float v_scale, void* stream) {
    return cache_write_rows(kv_pool, kv_dtype, key, value, src_dtype, block_tables, context_lens, nullptr,
                            num_seqs, num_seqs, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                            num_blocks, k_scale, v_scale, stream);
}

pa_status pa_cache_write_tokens(void* kv_pool, pa_dtype kv_dtype, const void* key, const void* value,
                                pa_dtype src_dtype, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* cu_seqlens, int32_t num_seqs,
                                int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                float k_scale, float v_scale, void* stream) {
    if (num_seqs > 0 && num_tokens > 0) {
        if (!cu_seqlens) return PA_ERR_NULL_POINTER;
        if (!aligned16(cu_seqlens)) return PA_ERR_MISALIGNED;
    }
    return cache_write_rows(kv_pool, kv_dtype, key, value, src_dtype, block_tables, context_lens, cu_seqlens,
                            num_seqs, num_tokens, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                            num_blocks, k_scale, v_scale, stream);
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                 pa_dtype kv_dtype, int32_t requested) {
    DecodePlan p;
    if (!plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     kv_dtype, requested, &p))
        return 0;
    return requested > 0 ? p.partition : p.part_min;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                pa_dtype kv_dtype, int32_t partition_size) {
    DecodePlan p;
    if (!plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     kv_dtype, partition_size, &p))
        return 0;
    return p.bytes;
}

// Argument checks of pa_prefill; *work is set when there is anything to launch.
static pa_status check_prefill_args(const void* out, const void* query, pa_dtype q_dtype, const void* kv_pool,
                                    pa_dtype kv_dtype, const int32_t* block_tables, const int32_t* context_lens,
                                    const int32_t* cu_seqlens, int32_t num_seqs, int32_t num_tokens,
                                    int32_t max_new_tokens, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                    int32_t num_blocks, float scale, float k_scale, float v_scale, bool* work) {
    *work = false;
    // the per-call checks are those of pa_decode, with no split-K partition
    pa_status st = check_decode_args(out, query, q_dtype, kv_pool, kv_dtype, block_tables, context_lens,
                                     num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                     max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, 0);
    if (st != PA_OK) return st;
    if (num_tokens < 0 || max_new_tokens < 0) return PA_ERR_BAD_SHAPE;
    if ((int64_t)num_tokens * num_heads * head_dim > (int64_t)INT32_MAX * 8) return PA_ERR_BAD_SHAPE;
    // the prompt kernel addresses within a block in 32 bits
    if ((int64_t)2 * block_size * num_kv_heads * head_dim * elem_bytes(kv_dtype) > (int64_t)UINT32_MAX)
        return PA_ERR_BAD_SHAPE;
    const int group = num_heads / num_kv_heads;
    if (prefill_grid(num_seqs, num_kv_heads, group, max_new_tokens, num_tokens) > (int64_t)INT32_MAX)
        return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0 || num_tokens == 0 || max_new_tokens == 0) return PA_OK;
    if (!cu_seqlens) return PA_ERR_NULL_POINTER;
    if (!aligned16(cu_seqlens)) return PA_ERR_MISALIGNED;
    *work = true;
    return PA_OK;
}

static pa_status prefill_impl(void* out, const void* query, pa_dtype q_dtype, const void* kv_pool,
                              pa_dtype kv_dtype, const int32_t* block_tables, const int32_t* context_lens,
                              const int32_t* cu_seqlens, int32_t num_seqs, int32_t num_tokens,
                              int32_t max_new_tokens, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                              float k_scale, float v_scale, void* stream, const void* new_key,
                              const void* new_value) {
    bool work = false;
    const pa_status st = check_prefill_args(out, query, q_dtype, kv_pool, kv_dtype, block_tables, context_lens,
                                            cu_seqlens, num_seqs, num_tokens, max_new_tokens, num_heads,
                                            num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                                            scale, k_scale, v_scale, &work);
    if (st != PA_OK || !work) return st;
    const int group = num_heads / num_kv_heads;
    const bool fp8 = kv_dtype == PA_FP8_E4M3;
    PrefillArgs a;
    a.out = out;
    a.query = query;
    a.kv_pool = kv_pool;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.cu_seqlens = cu_seqlens;
    a.num_seqs = num_seqs;
    a.num_tokens = num_tokens;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.block_shift = log2_exact(block_size);
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.max_new_tokens = max_new_tokens;
    a.score_scale = scale * (fp8 ? k_scale : 1.0f) * 1.4426950408889634f;
    a.v_scale = fp8 ? v_scale : 1.0f;
    a.new_key = new_key;
    a.new_value = new_value;
    return launch_prefill(a, kv_dtype, head_dim, group, max_new_tokens, stream) == 0 ? PA_OK : PA_ERR_HIP;
}

pa_status pa_prefill(void* out, const void* query, pa_dtype q_dtype, const void* kv_pool, pa_dtype kv_dtype,
                     const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_seqlens,
                     int32_t num_seqs, int32_t num_tokens, int32_t max_new_tokens, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                     int32_t num_blocks, float scale, float k_scale, float v_scale, void* stream) {
    return prefill_impl(out, query, q_dtype, kv_pool, kv_dtype, block_tables, context_lens, cu_seqlens, num_seqs,
                        num_tokens, max_new_tokens, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, stream, nullptr, nullptr);
}

pa_status pa_prefill_write(void* out, const void* query, pa_dtype q_dtype, void* kv_pool, pa_dtype kv_dtype,
                           const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_seqlens,
                           int32_t num_seqs, int32_t num_tokens, int32_t max_new_tokens, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int32_t num_blocks, float scale, float k_scale,
                           float v_scale, void* stream, const void* key, const void* value,
                           pa_dtype src_dtype) {
    bool work = false;
    pa_status st = check_prefill_args(out, query, q_dtype, kv_pool, kv_dtype, block_tables, context_lens,
                                      cu_seqlens, num_seqs, num_tokens, max_new_tokens, num_heads, num_kv_heads,
                                      head_dim, block_size, max_blocks_per_seq, num_blocks, scale, k_scale,
                                      v_scale, &work);
    if (st != PA_OK) return st;
    if (kv_dtype == PA_FP8_E4M3) {
        // the attention reads the encoded codes: write first, then attend
        // (both calls' checks pass before anything is launched)
        if (src_dtype != PA_BF16 && src_dtype != PA_F16) return known_dtype(src_dtype) ? PA_ERR_UNSUPPORTED
                                                                                       : PA_ERR_BAD_DTYPE;
        if (!work) return PA_OK;
        if (!key || !value) return PA_ERR_NULL_POINTER;
        if (!aligned16(key) || !aligned16(value)) return PA_ERR_MISALIGNED;
        st = pa_cache_write_tokens(kv_pool, kv_dtype, key, value, src_dtype, block_tables, context_lens,
                                   cu_seqlens, num_seqs, num_tokens, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, num_blocks, k_scale, v_scale, stream);
        if (st != PA_OK) return st;
        return pa_prefill(out, query, q_dtype, kv_pool, kv_dtype, block_tables, context_lens, cu_seqlens,
                          num_seqs, num_tokens, max_new_tokens, num_heads, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, stream);
    }
    if (!known_dtype(src_dtype)) return PA_ERR_BAD_DTYPE;
    if (src_dtype != kv_dtype) return PA_ERR_UNSUPPORTED;
    if (!work) return PA_OK;
    if (!key || !value) return PA_ERR_NULL_POINTER;
    if (!aligned16(key) || !aligned16(value)) return PA_ERR_MISALIGNED;
    return prefill_impl(out, query, q_dtype, kv_pool, kv_dtype, block_tables, context_lens, cu_seqlens, num_seqs,
                        num_tokens, max_new_tokens, num_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, stream, key, value);
}

// Device address of a pool: device memory of the current device, or host
// memory allocated pinned (hipHostMalloc), which kernels reach through the
// same virtual address.  Anything else (pageable host memory, another
// device's memory) is refused rather than handed to a kernel.
static bool pool_device_address(const void* p, const void** out) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();                       // do not leave the error for a later check
        return false;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (attr.type == hipMemoryTypeDevice && attr.device == dev) {
        *out = p;
        return true;
    }
    if (attr.type == hipMemoryTypeHost && attr.devicePointer == p) {
        *out = p;
        return true;
    }
    return false;
}

pa_status pa_copy_blocks(const void* src_pool, int32_t src_num_blocks, void* dst_pool,
                         int32_t dst_num_blocks, pa_dtype kv_dtype, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim, const int32_t* block_mapping,
                         int32_t num_pairs, void* stream) {
    if (!known_dtype(kv_dtype)) return PA_ERR_BAD_DTYPE;
    if (src_num_blocks <= 0 || dst_num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || num_pairs < 0)
        return PA_ERR_BAD_SHAPE;
    const int64_t block_bytes = (int64_t)2 * block_size * num_kv_heads * head_dim * elem_bytes(kv_dtype);
    if (block_bytes % 16 != 0) return PA_ERR_BAD_SHAPE;
    if (num_pairs == 0) return PA_OK;
    if (!src_pool || !dst_pool || !block_mapping) return PA_ERR_NULL_POINTER;
    if (!aligned16(src_pool) || !aligned16(dst_pool) || !aligned16(block_mapping)) return PA_ERR_MISALIGNED;
    const void* src_dev = nullptr;
    const void* dst_dev = nullptr;
    if (!pool_device_address(src_pool, &src_dev) || !pool_device_address(dst_pool, &dst_dev))
        return PA_ERR_UNSUPPORTED;
    CopyArgs a;
    a.src = static_cast<const uint8_t*>(src_dev);
    a.dst = static_cast<uint8_t*>(const_cast<void*>(dst_dev));
    a.mapping = block_mapping;
    a.num_pairs = num_pairs;
    a.block_bytes = block_bytes;
    a.src_num_blocks = src_num_blocks;
    a.dst_num_blocks = dst_num_blocks;
    return launch_copy_blocks(a, stream) == 0 ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"

namespace pa {
// Token chunks: the head laid ahead of each sequence in the layout, in
// tokens (rounded up to whole blocks): about what a workgroup streams in the
// time a fresh segment start costs it, per kernel.
constexpr int kSegHeadVector = 64;
constexpr int kSegHeadMfma16 = 64;
constexpr int kSegHeadFp8 = 160;

int seg_head_tokens(const DecodePlan& p, pa_dtype kv_dtype, int block_size) {
    const int t = !p.geo.mfma ? kSegHeadVector : kv_dtype == PA_FP8_E4M3 ? kSegHeadFp8 : kSegHeadMfma16;
    return (t + block_size - 1) / block_size * block_size;
}

pa_status decode_phases(int phases, void* out, const void* query, pa_dtype q_dtype, const void* kv_pool,
                        pa_dtype kv_dtype, const int32_t* block_tables, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                        float scale, float k_scale, float v_scale, int32_t partition_size,
                        void* workspace, size_t workspace_bytes, void* stream,
                        const void* new_key, const void* new_value, int32_t run_size) {
    pa_status st = check_decode_args(out, query, q_dtype, kv_pool, kv_dtype, block_tables,
                                     context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                                     block_size, max_blocks_per_seq, num_blocks, scale, k_scale,
                                     v_scale, partition_size);
    if (st != PA_OK) return st;
    if (run_size < 1) return PA_ERR_BAD_SHAPE;
    if (run_size != 1 && run_size != 2 && run_size != 4 && run_size != 8) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    DecodePlan plan;
    if (!plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     kv_dtype, partition_size, &plan))
        return PA_ERR_BAD_SHAPE;
    if (!workspace) return PA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return PA_ERR_MISALIGNED;
    if (workspace_bytes < plan.bytes) return PA_ERR_WORKSPACE_TOO_SMALL;

    const bool fp8 = kv_dtype == PA_FP8_E4M3;
    DecodeArgs a;
    a.out = out;
    a.query = query;
    a.kv_pool = kv_pool;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    char* ws = static_cast<char*>(workspace);
    a.part_n = reinterpret_cast<int32_t*>(ws + plan.off_n);
    a.part_ml = reinterpret_cast<float*>(ws + plan.off_ml);
    a.part_o = reinterpret_cast<float*>(ws + plan.off_o);
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.block_shift = log2_exact(block_size);
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.groups = plan.groups;
    a.partition = plan.partition;
    a.max_partitions = plan.max_partitions;
    a.part_min = plan.part_min;
    a.max_chunks = plan.max_chunks;
    a.target_items = plan.max_chunks * plan.groups;    // the launcher sets it from the kernel's occupancy
    a.fallback_partition = plan.run_partition;
    a.seg_head = seg_head_tokens(plan, kv_dtype, block_size);
    a.score_scale = scale * (fp8 ? k_scale : 1.0f) * 1.4426950408889634f;
    a.v_scale = fp8 ? v_scale : 1.0f;
    a.new_key = new_key;
    a.new_value = new_value;
    a.write_k_scale = k_scale;
    a.write_v_scale = v_scale;
    // shared runs go to the vector kernel's run form: one query head per KV head
    a.share_run = (run_size > 1 && !plan.geo.mfma && num_heads == num_kv_heads) ? run_size : 0;
    if (a.share_run > 1 && plan.partition == 0) {
        // the run form walks fixed partitions (the workspace has room for them)
        plan.partition = plan.run_partition;
        plan.grid = (int64_t)plan.groups * num_seqs * plan.max_partitions;
        a.partition = plan.partition;
    }
    const int err = launch_decode(a, plan, q_dtype, kv_dtype, head_dim, num_heads / num_kv_heads,
                                  phases, stream);
    return err == 0 ? PA_OK : PA_ERR_HIP;
}
}  // namespace pa

extern "C" {

#define PA_DECODE_PARAMS                                                                          \
    void *out, const void *query, pa_dtype q_dtype, const void *kv_pool, pa_dtype kv_dtype,       \
        const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,               \
        int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,            \
        int32_t max_blocks_per_seq, int32_t num_blocks, float scale, float k_scale, float v_scale, \
        int32_t partition_size, void *workspace, size_t workspace_bytes, void *stream
#define PA_DECODE_ARGS                                                                              \
    out, query, q_dtype, kv_pool, kv_dtype, block_tables, context_lens, num_seqs, num_heads,        \
        num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, \
        partition_size, workspace, workspace_bytes, stream

pa_status pa_decode(PA_DECODE_PARAMS) {
    return decode_phases(kPhasePartials | kPhaseMerge, PA_DECODE_ARGS, nullptr, nullptr, 1);
}
pa_status pa_decode_partials(PA_DECODE_PARAMS) {
    return decode_phases(kPhasePartials, PA_DECODE_ARGS, nullptr, nullptr, 1);
}
pa_status pa_decode_merge(PA_DECODE_PARAMS) {
    return decode_phases(kPhaseMerge, PA_DECODE_ARGS, nullptr, nullptr, 1);
}

// pa_decode with the newest tokens' K/V written by the attention pass itself
static pa_status check_write_source(int32_t num_seqs, pa_dtype q_dtype, const void* key, const void* value,
                                    pa_dtype src_dtype) {
    if (!known_dtype(src_dtype)) return PA_ERR_BAD_DTYPE;
    if (src_dtype != q_dtype) return PA_ERR_UNSUPPORTED;         // the fused write takes query-dtype rows
    if (num_seqs > 0) {
        if (!key || !value) return PA_ERR_NULL_POINTER;
        if (!aligned16(key) || !aligned16(value)) return PA_ERR_MISALIGNED;
    }
    return PA_OK;
}

static pa_status decode_write_phases(int phases, PA_DECODE_PARAMS, const void* key, const void* value,
                                     pa_dtype src_dtype, int32_t run_size = 1) {
    const pa_status st = check_write_source(num_seqs, q_dtype, key, value, src_dtype);
    if (st != PA_OK) return st;
    return decode_phases(phases, PA_DECODE_ARGS, key, value, run_size);
}

pa_status pa_decode_write(PA_DECODE_PARAMS, const void* key, const void* value, pa_dtype src_dtype) {
    return decode_write_phases(kPhasePartials | kPhaseMerge, PA_DECODE_ARGS, key, value, src_dtype);
}
pa_status pa_decode_write_partials(PA_DECODE_PARAMS, const void* key, const void* value, pa_dtype src_dtype) {
    return decode_write_phases(kPhasePartials, PA_DECODE_ARGS, key, value, src_dtype);
}

pa_status pa_decode_shared(PA_DECODE_PARAMS, int32_t run_size) {
    return decode_phases(kPhasePartials | kPhaseMerge, PA_DECODE_ARGS, nullptr, nullptr, run_size);
}
pa_status pa_decode_write_partials_shared(PA_DECODE_PARAMS, const void* key, const void* value, pa_dtype src_dtype,
                                          int32_t run_size) {
    return decode_write_phases(kPhasePartials, PA_DECODE_ARGS, key, value, src_dtype, run_size);
}

}  // extern "C"
