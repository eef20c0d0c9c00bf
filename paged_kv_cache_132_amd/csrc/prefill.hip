// pa_prefill: causal attention of packed new queries over the paged KV pool
// on the matrix cores ([CANN notes §3.1-3.3]: packed sequences bounded by
// cu_seqlens, a block-diagonal causal mask, K/V found through the block
// table; [nano-vllm blog §4.3]: a prompt with a cached prefix computes only
// its tail, which still attends to the whole prefix).
//
// Query row (i, h) of sequence s -- new token i (position L - n + i), query
// head h -- attends to keys 0 .. L - n + i of its own sequence.
//
// Work decomposition
//   Workgroup = (sequence, KV head g, tile of 64 rows); rows are the
//   (new token, query head) pairs of the G query heads that read KV head g,
//   token-major, so one K/V tile in LDS serves G heads.  Wave w owns rows
//   16w .. 16w+15 of the tile.  Tiles are dispatched last tile first: the
//   latest queries see the most keys.
//
// Per 32-key tile (lane l: c = l % 16, q = l / 16):
//   load  the 256 threads read the tile's K and V rows through the block
//         table (16 bytes each) and stage them in LDS: K row-major, V
//         transposed (head_dim-major); fp8 is widened to bf16 exactly.
//         The next tile's loads are in flight while this one is computed.
//   S^T = K Q^T on v_mfma_f32_16x16x32_{f16,bf16}: A = K rows (lane: key c,
//         head_dim 8q..8q+7 of each 32-wide step), B = the queries (lane:
//         row c, the same head_dim positions, held in registers).  Two
//         16-key tiles give lane (c, q) the scores of keys 4q+i and 16+4q+i
//         for row c.
//   soft  online softmax in the exp2 domain: masked keys (after the row's
//         position) get weight 0; probabilities are rounded to the MFMA
//         input type once and the running sum uses the rounded values.
//         With bf16 K/V the probability is split into a bf16 part and a bf16
//         remainder and PV runs on both: one bf16 rounding (2^-9 relative)
//         of a peaked softmax would otherwise move an output by up to
//         2^-9 x the spread of the V values it weights.
//   PV    A = P is the lane's own 8 probabilities (k-slot j = key 4q+j for
//         j < 4, 16+4q+j-4 otherwise); B = V^T read back from LDS at the
//         same key order; head_dim/16 MFMAs accumulate O[row][d] in fp32.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;           // 4 waves
constexpr int kRows = 64;               // (token, head) rows per workgroup
constexpr int kKeys = 32;               // keys per tile

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float shfl_xor(float x, int m) {
    const int lane = __lane_id();
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float from_lane(float x, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
    const uint32_t b = __float_as_uint(x);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// The matrix-core input type: fp16 queries run on fp16 MFMAs, bf16 queries
// (bf16 or fp8 KV) on bf16 MFMAs.
template <int QT>
struct Mma;

template <>
struct Mma<PA_F16> {
    typedef f16x8 Vec;
    static __device__ __forceinline__ f32x4 run(Vec a, Vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t round(float x) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
    static __device__ __forceinline__ float widen(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
};

template <>
struct Mma<PA_BF16> {
    typedef bf16x8 Vec;
    static __device__ __forceinline__ f32x4 run(Vec a, Vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t round(float x) { return bf16_rne(x); }
    static __device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
};

// 16 fp8 codes -> 16 bf16 bit patterns (exact), as two 16-byte words.
__device__ __forceinline__ void widen16_fp8(uint4 w, uint4& lo, uint4& hi) {
    const uint32_t src[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[k], 1.0f, false);
        const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[k], 1.0f, true);
        o[2 * k] = __builtin_bit_cast(uint32_t, a);
        o[2 * k + 1] = __builtin_bit_cast(uint32_t, b);
    }
    lo = make_uint4(o[0], o[1], o[2], o[3]);
    hi = make_uint4(o[4], o[5], o[6], o[7]);
}

template <int QT, int KVT, int D, int G>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
    using M = Mma<QT>;
    using Vec = typename M::Vec;
    constexpr int KB = KVT == PA_FP8_E4M3 ? 1 : 2;      // pool bytes per element
    constexpr int EPC = 16 / KB;                        // elements per 16-byte chunk
    constexpr int CPK = D / EPC;                        // chunks per key row
    constexpr int CHUNKS = kKeys * CPK;                 // chunks per K (or V) tile
    constexpr int U = (CHUNKS + kThreads - 1) / kThreads;
    constexpr int KS = D + 8;                           // LDS K row stride (elements)
    constexpr int VS = kKeys + 4;                       // LDS V^T row stride (elements)
    constexpr int KSTEPS = D / 32;
    constexpr int DT = D / 16;
    constexpr bool SPLIT = QT == PA_BF16 && KVT == PA_BF16;   // P = bf16 part + bf16 remainder

    __shared__ __attribute__((aligned(16))) uint16_t s_k[kKeys * KS];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[D * VS];

    // ---- work item ----------------------------------------------------------
    const int Hkv = a.num_kv_heads;
    int x = blockIdx.x;
    const int g = x % Hkv;
    x /= Hkv;
    const int s = x % a.num_seqs;
    const int tile_rev = x / a.num_seqs;
    const int first = a.cu_seqlens[s];
    const int n = a.cu_seqlens[s + 1] - first;
    const int L = min(a.context_lens[s], a.max_blocks_per_seq << a.block_shift);
    if (n <= 0 || n > L || first < 0 || first + n > a.num_tokens) return;   // nothing new, or an impossible run
    const int rows = n * G;
    const int tile = (rows + kRows - 1) / kRows - 1 - tile_rev;
    if (tile < 0) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane & 15;
    const int q = lane >> 4;
    const int Hq = a.num_heads;
    const int row0 = tile * kRows;

    // this lane's row (as the B-operand column and for the softmax state)
    const int r = min(row0 + 16 * wave + c, rows - 1);
    const int pos = L - n + r / G;                       // query position
    Vec qop[KSTEPS];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.query) +
                             ((int64_t)(first + r / G) * Hq + g * G + r % G) * D + 8 * q;
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k) qop[k] = __builtin_bit_cast(Vec, *reinterpret_cast<const uint4*>(qp + 32 * k));
    }
    const int last_row = min(row0 + kRows, rows) - 1;
    const int p_max = L - n + last_row / G;              // the latest query of the tile
    const int n_tiles = p_max / kKeys + 1;

    // ---- K/V tile loads ---------------------------------------------------------
    const int shift = a.block_shift;
    const int64_t row_bytes = (int64_t)Hkv * D * KB;
    const uint8_t* pool = static_cast<const uint8_t*>(a.kv_pool);
    const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;

    auto load_tile = [&](int kt, uint4 (&kr)[U], uint4 (&vr)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ci = tid + kThreads * u;
            if (ci < CHUNKS) {
                const int key = ci / CPK;
                const int ch = ci % CPK;
                const int t = min(kt * kKeys + key, L - 1);   // keys past the last position are masked
                int blk = bt_row[t >> shift];
                blk = (blk >= 0 && blk < a.num_blocks) ? blk : 0;
                const int64_t krow = ((int64_t)blk * 2 << shift) + (t & (a.block_size - 1));
                const uint8_t* kp = pool + krow * row_bytes + (int64_t)(g * D + ch * EPC) * KB;
                kr[u] = *reinterpret_cast<const uint4*>(kp);
                vr[u] = *reinterpret_cast<const uint4*>(kp + (row_bytes << shift));
            }
        }
    };

    auto store_tile = [&](const uint4 (&kr)[U], const uint4 (&vr)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ci = tid + kThreads * u;
            if (ci < CHUNKS) {
                const int key = ci / CPK;
                const int d0 = (ci % CPK) * EPC;
                uint4 k16[2], v16[2];
                if constexpr (KVT == PA_FP8_E4M3) {
                    widen16_fp8(kr[u], k16[0], k16[1]);
                    widen16_fp8(vr[u], v16[0], v16[1]);
                } else {
                    k16[0] = kr[u];
                    v16[0] = vr[u];
                }
#pragma unroll
                for (int h = 0; h < EPC / 8; ++h) {
                    *reinterpret_cast<uint4*>(&s_k[key * KS + d0 + 8 * h]) = k16[h];
                    const uint32_t w[4] = {v16[h].x, v16[h].y, v16[h].z, v16[h].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        s_vt[(d0 + 8 * h + e) * VS + key] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
                }
            }
        }
    };

    // ---- main loop --------------------------------------------------------------
    float m_run = -INFINITY;   // running max of row c (same in the 4 lanes of the row)
    float l_lane = 0.f;        // this lane's share of row c's running sum
    f32x4 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 kr[U], vr[U];
    load_tile(0, kr, vr);
    for (int kt = 0; kt < n_tiles; ++kt) {
        store_tile(kr, vr);
        __syncthreads();
        if (kt + 1 < n_tiles) load_tile(kt + 1, kr, vr);

        // S^T = K Q^T for the tile's two 16-key halves
        f32x4 sacc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k) {
                const Vec kf = __builtin_bit_cast(Vec, *reinterpret_cast<const uint4*>(&s_k[(16 * u + c) * KS + 32 * k + 8 * q]));
                acc = M::run(kf, qop[k], acc);
            }
            sacc[u] = acc;
        }
        // online softmax (lane: keys 4q+i and 16+4q+i of row c)
        float sc[8];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kt * kKeys + 16 * u + 4 * q + i;
                const float v = key <= pos ? sacc[u][i] * a.score_scale : -INFINITY;
                sc[4 * u + i] = v;
                mx = fmaxf(mx, v);
            }
        }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);              // finite: key 0 precedes every query
        const float alpha = fast_exp2(m_run - m_new);
        uint16_t pb[8], pl[8];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pe = sc[e] == -INFINITY ? 0.f : fast_exp2(sc[e] - m_new);
            pb[e] = M::round(pe);
            psum += M::widen(pb[e]);
            if constexpr (SPLIT) {
                pl[e] = M::round(pe - M::widen(pb[e]));        // the difference is exact in fp32
                psum += M::widen(pl[e]);
            }
        }
        l_lane = l_lane * alpha + psum;
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
            float ar[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ar[i] = from_lane(alpha, 4 * q + i);
#pragma unroll
            for (int t = 0; t < DT; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[t][i] *= ar[i];
            }
        }
        // O += P V
        auto pack8 = [](const uint16_t (&v)[8]) {
            return __builtin_bit_cast(Vec, make_uint4((uint32_t)v[0] | ((uint32_t)v[1] << 16),
                                                      (uint32_t)v[2] | ((uint32_t)v[3] << 16),
                                                      (uint32_t)v[4] | ((uint32_t)v[5] << 16),
                                                      (uint32_t)v[6] | ((uint32_t)v[7] << 16)));
        };
        const Vec pop = pack8(pb);
        Vec pop_lo;
        if constexpr (SPLIT) pop_lo = pack8(pl);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const uint16_t* vrow = &s_vt[(16 * t + c) * VS + 4 * q];
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
            const Vec vf = __builtin_bit_cast(Vec, make_uint4(lo[0], lo[1], hi[0], hi[1]));
            oacc[t] = M::run(pop, vf, oacc[t]);
            if constexpr (SPLIT) oacc[t] = M::run(pop_lo, vf, oacc[t]);
        }
        __syncthreads();
    }

    // ---- finish: row sums, normalise, store ----------------------------------
    l_lane += shfl_xor(l_lane, 16);
    l_lane += shfl_xor(l_lane, 32);
    float lr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lr[i] = from_lane(l_lane, 4 * q + i);
    uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int R = row0 + 16 * wave + 4 * q + i;
        if (R >= rows) continue;
        const float inv = a.v_scale / lr[i];
        uint16_t* dst = out + ((int64_t)(first + R / G) * Hq + g * G + R % G) * D + c;
#pragma unroll
        for (int t = 0; t < DT; ++t) dst[16 * t] = M::round(oacc[t][i] * inv);
    }
}

template <int QT, int KVT, int D>
int launch_g(const PrefillArgs& a, int group_size, int64_t grid, hipStream_t st) {
    const dim3 g3((unsigned)grid), block(kThreads);
    switch (group_size) {
        case 1: hipLaunchKernelGGL((prefill_kernel<QT, KVT, D, 1>), g3, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<QT, KVT, D, 2>), g3, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<QT, KVT, D, 4>), g3, block, 0, st, a); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<QT, KVT, D, 8>), g3, block, 0, st, a); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

template <int QT, int KVT>
int launch_d(const PrefillArgs& a, int head_dim, int group_size, int64_t grid, hipStream_t st) {
    if (head_dim == 64) return launch_g<QT, KVT, 64>(a, group_size, grid, st);
    return launch_g<QT, KVT, 128>(a, group_size, grid, st);
}

}  // namespace

int64_t prefill_grid(int num_seqs, int num_kv_heads, int group_size, int max_new_tokens) {
    const int64_t tiles = ((int64_t)max_new_tokens * group_size + kRows - 1) / kRows;
    return tiles * num_seqs * num_kv_heads;
}

int launch_prefill(const PrefillArgs& a, pa_dtype kv_dtype, int head_dim, int group_size, int max_new_tokens,
                   void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t grid = prefill_grid(a.num_seqs, a.num_kv_heads, group_size, max_new_tokens);
    if (grid == 0) return 0;
    if (kv_dtype == PA_F16) return launch_d<PA_F16, PA_F16>(a, head_dim, group_size, grid, st);
    if (kv_dtype == PA_BF16) return launch_d<PA_BF16, PA_BF16>(a, head_dim, group_size, grid, st);
    return launch_d<PA_BF16, PA_FP8_E4M3>(a, head_dim, group_size, grid, st);
}

}  // namespace pa
