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
//   Workgroup = (sequence, KV head g, tile of 128 rows); rows are the
//   (new token, query head) pairs of the G query heads that read KV head g,
//   token-major, so one K/V tile in LDS serves G heads.  Wave w owns rows
//   32w .. 32w+31 of the tile as two 16-row MFMA blocks, so every K and V
//   operand read from LDS feeds two MFMAs.  Tiles are dispatched last tile
//   first: the latest queries see the most keys.  The sequence's block table
//   is staged in LDS once (tables of up to 2048 blocks).
//
// Per 32-key tile (lane l: c = l % 16, q = l / 16):
//   load  the 256 threads read the tile's K and V rows through the block
//         table (16 bytes each) and store them row-major into one of two LDS
//         buffers (fp8 widened to bf16 exactly).  Tile kt + 1 is stored
//         while tile kt is computed and the loads of tile kt + 2 go out
//         right after: one barrier per tile.
//   S^T = K Q^T on v_mfma_f32_16x16x32_{f16,bf16}: A = K rows (lane: key c,
//         head_dim 8q..8q+7 of each 32-wide step), B = the queries (lane:
//         row c, the same head_dim positions, held in registers).  Two
//         16-key tiles give lane (c, q) the scores of keys 4q+i and 16+4q+i
//         for row c.
//   soft  online softmax in the exp2 domain on the unscaled scores (the
//         scale enters through the exponent's FMA): masked keys (after the
//         row's position; only the last tiles of a wave take the mask) get
//         weight 0; probabilities are rounded to the MFMA input type once,
//         and the running sum, P times a column of ones on the matrix cores,
//         adds exactly the rounded values.
//         With bf16 K/V the probability is split into a bf16 part and a bf16
//         remainder and PV runs on both: one bf16 rounding (2^-9 relative)
//         of a peaked softmax would otherwise move an output by up to
//         2^-9 x the spread of the V values it weights.
//   PV    A = P is the lane's own 8 probabilities (k-slot j = key 4q+j for
//         j < 4, 16+4q+j-4 otherwise); B = V read from its row-major LDS
//         copy with ds_read_tr16_b64 (two reads give a lane the 8 keys of one
//         head_dim column in that k-slot order); head_dim/16 MFMAs per row
//         block accumulate O[row][d] in fp32.
//
// With the write fused (16-bit KV), new tokens' K and V are read from the
// source rows, and the workgroup that owns a new token (its query rows)
// stores the token's K and V into its slot from the tile registers of its own
// main loop; no workgroup reads a slot another one writes.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;           // 4 waves
constexpr int kRB = 2;                  // 16-row MFMA blocks per wave
constexpr int kRows = 4 * 16 * kRB;     // (token, head) rows per workgroup
constexpr int kKeys = 32;               // keys per tile
constexpr int kMaxBt = 2048;            // block-table entries staged in LDS (longer tables are read in place)
constexpr float kSlack = 8.f;           // a row's weights stay below 2^8 between rescales

template <bool B>
struct MaskTag {   // selects the per-tile code with or without the causal mask
    static constexpr bool value = B;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max of x over lanes l, l ^ 16, l ^ 32 and l ^ 48, on the VALU: each
// v_permlane{16,32}_swap with both operands x leaves, in its two results,
// x of this lane and of lane l ^ 16 (l ^ 32), in some order
__device__ __forceinline__ float max_across_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
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
    static constexpr uint32_t kOne2 = 0x3C003C00u;   // two 1.0 values
    static __device__ __forceinline__ f32x4 run(Vec a, Vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t round(float x) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
    static __device__ __forceinline__ float widen(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
    // two values rounded (RNE) into one packed word, and back
    static __device__ __forceinline__ uint32_t round2(float x, float y) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
    }
    static __device__ __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
    static __device__ __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }
};

template <>
struct Mma<PA_BF16> {
    typedef bf16x8 Vec;
    static constexpr uint32_t kOne2 = 0x3F803F80u;
    static __device__ __forceinline__ f32x4 run(Vec a, Vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t round(float x) { return bf16_rne(x); }
    static __device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
    static __device__ __forceinline__ uint32_t round2(float x, float y) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
    }
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
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

template <int QT, int KVT, int D, int G, bool BT_LDS, bool WRITE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(PrefillArgs a) {
    using M = Mma<QT>;
    using Vec = typename M::Vec;
    constexpr int KB = KVT == PA_FP8_E4M3 ? 1 : 2;      // pool bytes per element
    constexpr int EPC = 16 / KB;                        // elements per 16-byte chunk
    constexpr int CPK = D / EPC;                        // chunks per key row
    constexpr int CHUNKS = kKeys * CPK;                 // chunks per K (or V) tile
    constexpr int U = (CHUNKS + kThreads - 1) / kThreads;
    constexpr int KS = D + 8;                           // LDS K row stride (elements)
    constexpr int VS = D + 16;                          // LDS V row stride: transposed reads of 4 rows x 16
                                                        // columns fall in distinct banks
    constexpr int KSTEPS = D / 32;
    constexpr int DT = D / 16;
    constexpr bool SPLIT = QT == PA_BF16 && KVT == PA_BF16;   // P = bf16 part + bf16 remainder
    static_assert(!WRITE || KVT != PA_FP8_E4M3, "the fused write moves 16-bit rows unchanged");

    __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kKeys * KS];
    __shared__ __attribute__((aligned(16))) uint16_t s_v[2][kKeys * VS];
    __shared__ int32_t s_bt[BT_LDS ? kMaxBt : 1];

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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15;
    const int q = lane >> 4;
    const int Hq = a.num_heads;
    const int row0 = tile * kRows + wave * 16 * kRB;     // this wave's first row

    // this lane's rows (B-operand column c of each 16-row block).  Scores
    // are kept unscaled and the (positive) scale enters in the exponent's
    // FMA; a negative scale is moved onto the queries as an exact sign flip.
    int pos[kRB];                                        // query positions
    Vec qop[kRB][KSTEPS];
    const uint32_t qsign = a.score_scale < 0.f ? 0x80008000u : 0u;
    // (a zero scale is raised to the least normal float, so that a masked
    // score, -inf, still scales to -inf and not to NaN)
    const float sscale = fmaxf(fabsf(a.score_scale), 1.17549435e-38f);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        const int r = min(row0 + 16 * rb + c, rows - 1);
        pos[rb] = L - n + r / G;
        const uint16_t* qp = static_cast<const uint16_t*>(a.query) +
                             ((int64_t)(first + r / G) * Hq + g * G + r % G) * D + 8 * q;
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k)
        {
            uint4 w = *reinterpret_cast<const uint4*>(qp + 32 * k);
            w.x ^= qsign;
            w.y ^= qsign;
            w.z ^= qsign;
            w.w ^= qsign;
            qop[rb][k] = __builtin_bit_cast(Vec, w);
        }
    }
    const int pos_first = L - n + row0 / G;              // the wave's earliest query
    const int last_row = min(tile * kRows + kRows, rows) - 1;
    const int p_max = L - n + last_row / G;              // the latest query of the workgroup
    const int n_tiles = p_max / kKeys + 1;

    // ---- the sequence's block table, staged in LDS when tables are short ----
    const int shift = a.block_shift;
    const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    if constexpr (BT_LDS) {
        const int nblk = (L + a.block_size - 1) >> shift;      // <= max_blocks_per_seq <= kMaxBt
        for (int i = tid; i < nblk; i += kThreads) s_bt[i] = bt_row[i];
        __syncthreads();
    }
    auto block_of = [&](int t) {
        int blk;
        if constexpr (BT_LDS) blk = s_bt[t >> shift];
        else blk = bt_row[t >> shift];
        return blk;
    };

    // ---- fused prompt-stage write ([CANN notes §4.2]: the prompt kernel
    // writes K and V as it goes).  This workgroup owns the new tokens its own
    // query rows belong to, i0 .. i1 - 1; the main loop loads every one of
    // them (they are its diagonal tiles), and the thread that holds a chunk
    // of an owned token's K and V stores it into the token's slot when it
    // moves the tile into LDS.  Every workgroup reads new tokens' K and V
    // from the source rows, so none waits for another's stores.
    const int i0 = tile * kRows / G;
    const int i1 = min(n, (tile + 1) * kRows / G);

    // ---- K/V tile loads ---------------------------------------------------------
    const int64_t row_bytes = (int64_t)Hkv * D * KB;
    const uint32_t half_bytes = (uint32_t)(row_bytes << shift);      // the K (or V) half of a block
    const uint32_t blk_bytes = 2u * half_bytes;
    const uint8_t* pool = static_cast<const uint8_t*>(a.kv_pool);

    // Each thread moves U chunks of K and of V per tile (chunk tid + 256u).
    // The loads are branch-free: where the tile has fewer chunks than
    // threads, the spare threads re-read chunk 0 and store nothing.
    static_assert(U <= 2, "at most two chunks per thread");
    struct Tile {
        uint4 k0, v0, k1, v1;
    };
    auto load_chunk = [&](int kt, int ci, uint4& kd, uint4& vd) {
        ci = ci < CHUNKS ? ci : 0;
        const int key = ci / CPK;
        const int ch = ci % CPK;
        const int t = min(kt * kKeys + key, L - 1);   // keys past the last position are masked
        if (WRITE && t >= L - n) {                    // a new token: its source row
            const int64_t src = ((int64_t)(first + t - (L - n)) * Hkv + g) * D + ch * EPC;
            kd = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.new_key) + src);
            vd = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.new_value) + src);
            return;
        }
        uint32_t blk = (uint32_t)block_of(t);
        blk = blk < (uint32_t)a.num_blocks ? blk : 0u;
        // a block is at most 4 GiB (checked on the host): 32-bit factors, one 64-bit product
        const uint32_t inner = (uint32_t)(t & (a.block_size - 1)) * (uint32_t)row_bytes + (uint32_t)((g * D + ch * EPC) * KB);
        const uint8_t* kp = pool + ((uint64_t)blk * blk_bytes + inner);
        kd = *reinterpret_cast<const uint4*>(kp);
        vd = *reinterpret_cast<const uint4*>(kp + half_bytes);
    };
    auto load_tile = [&](int kt) {
        Tile r;
        load_chunk(kt, tid, r.k0, r.v0);
        if constexpr (U > 1) load_chunk(kt, tid + kThreads, r.k1, r.v1);
        return r;
    };

    // K and V both row-major in LDS (fp8 widened to bf16 exactly)
    auto store_chunk = [&](int kt, int buf, int ci, uint4 kc, uint4 vc) {
        if (CHUNKS % kThreads != 0 && ci >= CHUNKS) return;
        const int key = ci / CPK;
        const int d0 = (ci % CPK) * EPC;
        if constexpr (WRITE) {
            const int t = kt * kKeys + key;              // not clamped: an owned token is < L
            const int i = t - (L - n);
            if (i >= i0 && i < i1) {
                const uint32_t blk = (uint32_t)block_of(t);
                if (blk < (uint32_t)a.num_blocks) {
                    const uint32_t inner = (uint32_t)(t & (a.block_size - 1)) * (uint32_t)row_bytes +
                                           (uint32_t)((g * D + d0) * KB);
                    uint8_t* kp = const_cast<uint8_t*>(pool) + ((uint64_t)blk * blk_bytes + inner);
                    *reinterpret_cast<uint4*>(kp) = kc;
                    *reinterpret_cast<uint4*>(kp + half_bytes) = vc;
                }
            }
        }
        if constexpr (KVT == PA_FP8_E4M3) {
            uint4 klo, khi, vlo, vhi;
            widen16_fp8(kc, klo, khi);
            widen16_fp8(vc, vlo, vhi);
            *reinterpret_cast<uint4*>(&s_k[buf][key * KS + d0]) = klo;
            *reinterpret_cast<uint4*>(&s_k[buf][key * KS + d0 + 8]) = khi;
            *reinterpret_cast<uint4*>(&s_v[buf][key * VS + d0]) = vlo;
            *reinterpret_cast<uint4*>(&s_v[buf][key * VS + d0 + 8]) = vhi;
        } else {
            *reinterpret_cast<uint4*>(&s_k[buf][key * KS + d0]) = kc;
            *reinterpret_cast<uint4*>(&s_v[buf][key * VS + d0]) = vc;
        }
    };
    auto store_tile = [&](int kt, int buf, const Tile& tl) {
        store_chunk(kt, buf, tid, tl.k0, tl.v0);
        if constexpr (U > 1) store_chunk(kt, buf, tid + kThreads, tl.k1, tl.v1);
    };

    // ---- per-tile math -------------------------------------------------------------
    // running max of row c (scaled, the same in the row's 4 lanes); the row
    // sums come from the matrix cores as P times a column of ones, in the C
    // layout of o (lane (c, q), register i: row 4q + i)
    float m_run[kRB];
    f32x4 oacc[kRB][DT], lacc[kRB];
    const Vec ones = __builtin_bit_cast(Vec, make_uint4(M::kOne2, M::kOne2, M::kOne2, M::kOne2));
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        m_run[rb] = -INFINITY;
        lacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[rb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    auto compute = [&](int kt, int buf, auto mask_tag) {
        constexpr bool kMasked = decltype(mask_tag)::value;
        const uint16_t* sk = s_k[buf];
        const uint16_t* sv = s_v[buf];
        // S^T = K Q^T for the tile's two 16-key halves; each K operand serves both row blocks
        // The matrix-core phases run at raised wave priority, so that a
        // wave in its softmax leaves the issue slots to the other wave of the
        // SIMD while that one has MFMAs to issue.
        f32x4 sacc[kRB][2];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) sacc[rb][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k) {
                const Vec kf = __builtin_bit_cast(Vec, *reinterpret_cast<const uint4*>(&sk[(16 * u + c) * KS + 32 * k + 8 * q]));
#pragma unroll
                for (int rb = 0; rb < kRB; ++rb) sacc[rb][u] = M::run(kf, qop[rb][k], sacc[rb][u]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // online softmax (lane: keys 4q+i and 16+4q+i of row c of each block).
        // Only tiles that reach past the wave's earliest query take the mask.
        Vec pop[kRB], pop_lo[kRB];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            float sc[8];
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = kt * kKeys + 16 * u + 4 * q + i;
                    float v = sacc[rb][u][i];
                    if constexpr (kMasked) v = key <= pos[rb] ? v : -INFINITY;
                    sc[4 * u + i] = v;
                    mx = fmaxf(mx, v);
                }
            }
            mx = max_across_rows(mx) * sscale;
            // The reference max moves only when a row's max grows by more
            // than kSlack (log2 units): the weights stay below 2^kSlack and
            // most tiles need no rescale of o at all.
            const bool grow = mx > m_run[rb] + kSlack;         // always on the first tile (m_run = -inf)
            const float m_new = grow ? mx : m_run[rb];         // finite: key 0 precedes every query
            const float alpha = grow ? fast_exp2(m_run[rb] - m_new) : 1.f;
            uint32_t pw[4], plw[4];     // packed probabilities (k-slot pairs)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = fast_exp2(fmaf(sc[2 * e], sscale, -m_new));     // masked: 2^-inf = 0
                const float p1 = fast_exp2(fmaf(sc[2 * e + 1], sscale, -m_new));
                pw[e] = M::round2(p0, p1);
                if constexpr (SPLIT) {
                    const float r0 = M::lo(pw[e]), r1 = M::hi(pw[e]);
                    plw[e] = M::round2(p0 - r0, p1 - r1);              // the differences are exact in fp32
                }
            }
            m_run[rb] = m_new;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                float ar[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) ar[i] = from_lane(alpha, 4 * q + i);
#pragma unroll
                for (int t = 0; t < DT; ++t) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) oacc[rb][t][i] *= ar[i];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) lacc[rb][i] *= ar[i];
            }
            pop[rb] = __builtin_bit_cast(Vec, make_uint4(pw[0], pw[1], pw[2], pw[3]));
            if constexpr (SPLIT) pop_lo[rb] = __builtin_bit_cast(Vec, make_uint4(plw[0], plw[1], plw[2], plw[3]));
        }
        // O += P V.  B operand: lane (n, q) needs V[key][16t + n] for its 8
        // k-slot keys 4q..4q+3 and 16+4q..16+4q+3.  ds_read_tr16_b64 gives
        // lane i of a 16-lane group element (i % 4) of the 8 bytes addressed
        // by lane 4j + (i % 16) / 4 as its element j, so lane 4j + m of the
        // group addresses V[4q + j][16t + 4m] (and the same 16 keys on).
        const int tr_key = 4 * q + (c >> 2);
        const int tr_col = 4 * (c & 3);
        if constexpr (!SPLIT) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(&sv[tr_key * VS + 16 * t + tr_col]));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(&sv[(16 + tr_key) * VS + 16 * t + tr_col]));
            const Vec vf = __builtin_bit_cast(Vec, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                oacc[rb][t] = M::run(pop[rb], vf, oacc[rb][t]);
                if constexpr (SPLIT) oacc[rb][t] = M::run(pop_lo[rb], vf, oacc[rb][t]);
            }
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            lacc[rb] = M::run(pop[rb], ones, lacc[rb]);
            if constexpr (SPLIT) lacc[rb] = M::run(pop_lo[rb], ones, lacc[rb]);
        }
        if constexpr (!SPLIT) __builtin_amdgcn_s_setprio(0);
    };

    // ---- main loop: two LDS buffers --------------------------------------------
    // Iteration kt computes tile kt from buffer kt & 1 while the loads of tile
    // kt + 1, issued one iteration earlier, are in flight; it then stores them
    // into the other buffer and issues the loads of tile kt + 2.  One barrier
    // per tile.
    Tile tl = load_tile(0);
    store_tile(0, 0, tl);
    if (n_tiles > 1) tl = load_tile(1);
    __syncthreads();
    // Tiles below the wave's earliest query need no mask: they run in a loop
    // of their own, the rest (at most kRows / kKeys + 1) in a second one.
    auto step = [&](int kt, auto mask_tag) {
        compute(kt, kt & 1, mask_tag);
        if (kt + 1 < n_tiles) {
            store_tile(kt + 1, (kt + 1) & 1, tl);
            if (kt + 2 < n_tiles) tl = load_tile(kt + 2);
        }
        __syncthreads();
    };
    const int n_plain = min((pos_first + 1) / kKeys, n_tiles);   // tiles with kt * kKeys + kKeys - 1 <= pos_first
    int kt = 0;
    for (; kt < n_plain; ++kt) step(kt, MaskTag<false>{});
    for (; kt < n_tiles; ++kt) step(kt, MaskTag<true>{});

    // ---- finish: row sums, normalise, store ----------------------------------
    uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int R = row0 + 16 * rb + 4 * q + i;
            if (R >= rows) continue;
            const float inv = a.v_scale / lacc[rb][i];
            uint16_t* dst = out + ((int64_t)(first + R / G) * Hq + g * G + R % G) * D + c;
#pragma unroll
            for (int t = 0; t < DT; ++t) dst[16 * t] = M::round(oacc[rb][t][i] * inv);
        }
    }
}

template <int QT, int KVT, int D, bool BT_LDS, bool WRITE>
int launch_g(const PrefillArgs& a, int group_size, int64_t grid, hipStream_t st) {
    const dim3 g3((unsigned)grid), block(kThreads);
    switch (group_size) {
        case 1: hipLaunchKernelGGL((prefill_kernel<QT, KVT, D, 1, BT_LDS, WRITE>), g3, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<QT, KVT, D, 2, BT_LDS, WRITE>), g3, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<QT, KVT, D, 4, BT_LDS, WRITE>), g3, block, 0, st, a); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<QT, KVT, D, 8, BT_LDS, WRITE>), g3, block, 0, st, a); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

template <int QT, int KVT, bool WRITE>
int launch_d(const PrefillArgs& a, int head_dim, int group_size, int64_t grid, hipStream_t st) {
    const bool bt_lds = a.max_blocks_per_seq <= kMaxBt;
    if (head_dim == 64)
        return bt_lds ? launch_g<QT, KVT, 64, true, WRITE>(a, group_size, grid, st)
                      : launch_g<QT, KVT, 64, false, WRITE>(a, group_size, grid, st);
    return bt_lds ? launch_g<QT, KVT, 128, true, WRITE>(a, group_size, grid, st)
                  : launch_g<QT, KVT, 128, false, WRITE>(a, group_size, grid, st);
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
    const bool w = a.new_key != nullptr;                 // fused write: 16-bit KV only
    if (kv_dtype == PA_F16)
        return w ? launch_d<PA_F16, PA_F16, true>(a, head_dim, group_size, grid, st)
                 : launch_d<PA_F16, PA_F16, false>(a, head_dim, group_size, grid, st);
    if (kv_dtype == PA_BF16)
        return w ? launch_d<PA_BF16, PA_BF16, true>(a, head_dim, group_size, grid, st)
                 : launch_d<PA_BF16, PA_BF16, false>(a, head_dim, group_size, grid, st);
    if (w) return (int)hipErrorInvalidValue;
    return launch_d<PA_BF16, PA_FP8_E4M3, false>(a, head_dim, group_size, grid, st);
}

}  // namespace pa
