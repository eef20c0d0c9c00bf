// pa_decode for grouped-query attention over a 16-bit (fp16 or bf16) KV
// cache on the matrix cores ([nano-vllm blog §2.3] decode attention).  With
// G = 2, 4 or 8 query heads per KV head, QK and PV are small dense products
// per 16-token step: the 2G multiply-adds per KV element that would bind the
// vector ALUs (the vector kernel reads bf16 GQA-8 at about 2.5 TB/s) run on
// the matrix cores, and the kernel stays bound by HBM.
//
// Work decomposition (as the fp8 GQA kernel): workgroup = (sequence, group of
// 4 KV heads, partition); wave w owns KV head 4*group + w for the whole
// partition, so the waves never exchange softmax state.  A wave walks its
// partition in 16-token steps (a step never crosses a block for block size 16
// or 32), keeping two steps of K/V loads in flight.
//
// Per step, per wave (lane l: n = l % 16, q = l / 16):
//   load  each load instruction reads 4 whole 256-byte head rows (16 lanes x
//         16 bytes per token); the rows are staged in this wave's LDS.
//   QK    v_mfma_f32_16x16x32_{f16,bf16}: A = K rows (lane: token n, head_dim
//         32c + 8q .. + 7 of k-step c), B = queries (lane: head n, the same
//         head_dim positions; zero for n >= G).  4 MFMAs give S[token][head],
//         lane (q, n) holding tokens 4q .. 4q + 3 of head n.
//   soft  running max over the step (in-lane, then across the 4 lane rows by
//         permlane swaps), exp2-domain probabilities rounded to the MFMA type
//         (bf16: plus a rounded remainder, see PV); the reference max moves
//         only when a head's max grows by more than 2^8.
//   PV    v_mfma_f32_16x16x16_{f16,bf16}: A = P, exactly the lane's own 4
//         probabilities (k-slot 4q + j is token 4q + j); B = V read from its
//         row-major LDS copy with ds_read_b64_tr_b16 -- within a 16-lane group
//         lane i's element j is element i % 4 of the 8 bytes addressed by lane
//         4j + i / 4, so lane 4j + m addresses V[4q + j][16t + 4m] and lane i
//         receives column 16t + i of tokens 4q .. 4q + 3.  8 MFMAs (16
//         head_dim columns each) accumulate O[head][d] in fp32, and one more,
//         P times a column of ones, the running sums.  With bf16 KV the
//         probabilities are split into a bf16 part and a bf16 remainder and
//         both go through PV and the sums: one bf16 rounding (2^-9 relative)
//         would move an output of a peaked softmax by up to 2^-9 times the
//         spread of the V rows it weights, while the pair carries about 16
//         significant bits.  fp16 (2^-11) keeps a single rounding.
//
// Output, partials and the merge are shared with the other decode kernels.
// With WRITE (pa_decode_write) the 16 lanes whose loads will cover a
// sequence's newest token store its K/V row first, each lane the 16 bytes it
// later reads itself.  With RUN (pa_decode_shared, one query head per KV
// head) the query rows are head g of a shared run's sequences and the
// workgroup covers a partition the run shares: each K/V row is read once for
// the whole run.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "decode_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;                  // head_dim
constexpr int kStep = 16;                // tokens per step
constexpr int kKS = kD + 8;              // LDS K row stride (elements)
constexpr int kVS = kD + 16;             // LDS V row stride (elements): the transposed reads of 4 rows
                                         // x 16 columns fall in distinct banks
constexpr int kStages = 2;               // steps of K/V loads each wave keeps in flight
constexpr float kSlack = 8.f;            // a head's weights stay below 2^8 between rescales

template <int KVT>
struct Mma16;

template <>
struct Mma16<PA_F16> {
    typedef f16x8 V8;
    static __device__ __forceinline__ f32x4 qk(V8 a, V8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 pv(uint2 a, uint2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b),
                                                    c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t round2(float x, float y) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
    }
    static __device__ __forceinline__ uint16_t round(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
    static constexpr uint32_t kOne2 = 0x3C003C00u;      // two 1.0 values
    static constexpr bool kSplit = false;               // P rounded once (2^-11 relative)
};

template <>
struct Mma16<PA_BF16> {
    typedef bf16x8 V8;
    static __device__ __forceinline__ f32x4 qk(V8 a, V8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 pv(uint2 a, uint2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                        c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t round2(float x, float y) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
    }
    static __device__ __forceinline__ uint16_t round(float x) {
        const uint32_t b = __float_as_uint(x);
        if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);   // NaN
        return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
    }
    static constexpr uint32_t kOne2 = 0x3F803F80u;
    static constexpr bool kSplit = true;                // P = bf16 part + bf16 remainder
    // the two values of a packed pair, widened exactly
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4 stream_load(const uint8_t* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ uint4 cached_load(const uint8_t* p) {
    return __builtin_bit_cast(uint4, *reinterpret_cast<const u32x4*>(p));
}

// max of x over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the 4 rows holding one
// head), on the VALU: each v_permlane{16,32}_swap with both operands x
// leaves, in its two results, x of this lane and of lane l ^ 16 (l ^ 32)
__device__ __forceinline__ float max_across_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float from_lane(float x, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

// RUN: the shared-run form (one query head per KV head): query row n of KV
// head g is head g of sequence s + n, for the G sequences of run s / G, over a
// partition the run shares (read once, streamed).
template <int KVT, int G, bool WRITE, bool RUN = false>
__global__ __launch_bounds__(kDecodeThreads) void decode_gqa16_mfma_kernel(DecodeArgs a) {
    static_assert(G == 2 || G == 4 || G == 8, "query heads per KV head");
    static_assert(!(RUN && WRITE), "a shared partition never holds a newest token");
    using M = Mma16<KVT>;
    using V8 = typename M::V8;
    constexpr int NW = kDecodeWaves;
    __shared__ __attribute__((aligned(16))) uint16_t s_k[NW][kStep * kKS];
    __shared__ __attribute__((aligned(16))) uint16_t s_v[NW][kStep * kVS];

    // ---- which (sequence, KV-head group, partition) -------------------------
    WorkItem w;
    if (!(RUN ? find_run_work(a, blockIdx.x, w) : begin_work(a, blockIdx.x, w))) return;
    const int group = w.group;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = group * NW + wave;                 // this wave's KV head
    if (g >= a.num_kv_heads) return;                 // no barriers below: idle waves may leave
    const int Hq = a.num_heads;
    uint16_t* out = static_cast<uint16_t*>(a.out);

    // one segment (tokens [t0, t1) of one sequence) per pass
    do {
    if (!RUN) publish_segments(a, w);                // (thread 0: wave 0 always holds a KV head)
    const int lane = opaque(threadIdx.x) & 63;       // (derived in every pass, see decode.hip)
    const int n = lane & 15;
    const int q = lane >> 4;
    const int s = w.s, L = w.L;
    const int64_t seg_slot = w.seg_slot;
    const bool whole = RUN ? w.n_part == 1 : whole_sequence(w);

    if (!RUN && L <= 0) {
        uint16_t* dst = out + ((int64_t)s * Hq + g * G) * kD;
        const uint32_t z = opaque(0);
        for (int i = lane * 8; i < G * kD; i += 64 * 8) *reinterpret_cast<uint4*>(dst + i) = make_uint4(z, z, z, z);
        continue;
    }

    // ---- query operand: head n of this KV head's group, head_dim 32c + 8q ----
    // Scores stay unscaled out of the MFMA and the positive scale enters in
    // the exponent's FMA; a negative scale is moved onto the queries as an
    // exact sign flip, and a zero scale is raised to the least normal float
    // (so a masked -inf score still scales to -inf).
    const uint32_t qsign = a.score_scale < 0.f ? 0x80008000u : 0u;
    const float sscale = fmaxf(fabsf(a.score_scale), 1.17549435e-38f);
    V8 qop[4];
    {
        const int nq = n < G ? n : 0;
        const uint16_t* qp = static_cast<const uint16_t*>(a.query) +
                             (RUN ? (int64_t)(s + nq) * Hq + g : (int64_t)s * Hq + g * G + nq) * kD + 8 * q;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint4 v = n < G ? *reinterpret_cast<const uint4*>(qp + 32 * c) : make_uint4(0, 0, 0, 0);
            v.x ^= qsign;
            v.y ^= qsign;
            v.z ^= qsign;
            v.w ^= qsign;
            qop[c] = __builtin_bit_cast(V8, v);
        }
    }

    const int t_begin = w.t0;
    const int t_end = w.t1;
    const int shift = a.block_shift;
    const uint32_t row_bytes = (uint32_t)(a.num_kv_heads * kD * 2);          // one token row, all heads
    const uint32_t half_bytes = row_bytes << shift;                           // K half -> V half
    const uint32_t lane_col = (uint32_t)(g * kD * 2 + 16 * n);                // this lane's 16 bytes of the row
    const uint8_t* pool = static_cast<const uint8_t*>(a.kv_pool);
    const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    // the fused write applies to lengths the table holds (as pa_cache_write)
    const bool write_len = WRITE && w.L_raw == L;

    uint16_t* sk = s_k[wave];
    uint16_t* sv = s_v[wave];
    // transposed-read address of this lane: V[4q + n / 4][16t + 4 (n % 4)]
    const uint32_t tr_off = (uint32_t)((4 * q + (n >> 2)) * kVS + 4 * (n & 3));

    float m_run = -INFINITY;       // running max of head n (identical in all 4 lane rows)
    // O and the running sums in the MFMA C layout: register i is head 4q + i
    f32x4 oacc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
    const uint2 ones = make_uint2(M::kOne2, M::kOne2);

    const int lb_first = t_begin >> shift;
    const int lb_last = (t_end - 1) >> shift;
    for (int seg0 = lb_first; seg0 <= lb_last; seg0 += 64) {
        const int seg_blocks = min(64, lb_last - seg0 + 1);
        const bool in_seg = lane < seg_blocks;
        const int my_blk = in_seg ? bt_row[seg0 + lane] : 0;
        // blocks a neighbouring sequence maps at the same logical index (a
        // shared prefix) go through the caches; the rest are streamed
        const int prev_blk = in_seg && s > 0 ? bt_row[seg0 + lane - a.max_blocks_per_seq] : -1;
        const int next_blk = in_seg && s + 1 < a.num_seqs ? bt_row[seg0 + lane + a.max_blocks_per_seq] : -1;
        // (the run form reads each block once: streamed)
        const uint64_t shared = RUN ? 0ull : __builtin_amdgcn_ballot_w64(in_seg && (my_blk == prev_blk || my_blk == next_blk));
        const int seg_t0 = max(t_begin, seg0 << shift);
        const int seg_t1 = min(t_end, (seg0 + seg_blocks) << shift);
        const int n_steps = (seg_t1 - seg_t0 + kStep - 1) / kStep;

        // Fused cache write ([CANN notes §4.3]: write the new token, then read
        // every block).  Before this segment's first load, the 16 lanes whose
        // loads will cover the newest token store its row, each lane the 16
        // bytes it later reads itself: one lane's global accesses to one
        // address take effect in program order, so the loads see the new
        // bytes with no wait on the stores.
        if (write_len && L - 1 >= seg_t0 && L - 1 < seg_t1) {
            const int t_new = L - 1;
            const int blk = __builtin_amdgcn_readlane(my_blk, (t_new >> shift) - seg0);
            if (blk >= 0 && blk < a.num_blocks && q == (t_new & 3)) {
                const int64_t row = ((int64_t)blk * 2 << shift) + (t_new & (a.block_size - 1));
                uint8_t* kp = const_cast<uint8_t*>(pool) + row * row_bytes + lane_col;
                const int64_t src = ((int64_t)s * a.num_kv_heads + g) * kD + 8 * n;
                *reinterpret_cast<uint4*>(kp) = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.new_key) + src);
                *reinterpret_cast<uint4*>(kp + half_bytes) =
                    *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.new_value) + src);
            }
        }
        // Issue the K and V loads of step k: load u reads tokens 4u .. 4u + 3
        // of the step (lane: token 4u + q, 16 bytes n).  Tokens past the end
        // are redirected to the step's first token, which is always valid, and
        // masked out of the softmax.  `load` is the segment's policy: cached
        // when a neighbouring sequence maps one of its blocks, else streamed.
        auto issue = [&](int k, uint4 (&kr)[4], uint4 (&vr)[4], auto load) {
            const int kk = min(k, n_steps - 1);
            const int th = seg_t0 + kk * kStep;
            const int blk = __builtin_amdgcn_readlane(my_blk, (th >> shift) - seg0);
            const bool ok = blk >= 0 && blk < a.num_blocks;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = th + 4 * u + q;
                const int tok = t < seg_t1 ? t : th;
                const int64_t row = ((int64_t)(ok ? blk : 0) * 2 << shift) + (tok & (a.block_size - 1));
                const uint8_t* kp = pool + row * row_bytes + lane_col;
                kr[u] = load(kp);
                vr[u] = load(kp + half_bytes);
            }
        };

        auto compute = [&](int k, const uint4 (&kr)[4], const uint4 (&vr)[4]) {
            if (k >= n_steps) return;
            const int th = seg_t0 + k * kStep;
            const int blk = __builtin_amdgcn_readlane(my_blk, (th >> shift) - seg0);
            const bool step_ok = blk >= 0 && blk < a.num_blocks;     // a block id outside the pool drops the step
            const bool full = step_ok && th + kStep <= seg_t1;          // uniform
            // stage the step's K and V rows (row 4u + q, 16 bytes n).  V rows
            // past the end (or of a dropped step) are staged as zeros: their
            // weight is 0, and 0 times whatever a redirected load returned
            // (the slot being written, a NaN) must not reach O.  (K rows need
            // no care: their scores are masked.)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                *reinterpret_cast<uint4*>(sk + (4 * u + q) * kKS + 8 * n) = kr[u];
                *reinterpret_cast<uint4*>(sv + (4 * u + q) * kVS + 8 * n) = vr[u];
            }
            if (!full) {      // the masked rows' V, overwritten (one wave's LDS stores land in order)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (!(step_ok && th + 4 * u + q < seg_t1))
                        *reinterpret_cast<uint4*>(sv + (4 * u + q) * kVS + 8 * n) = make_uint4(0, 0, 0, 0);
            }
            // QK: S[token][head]; A operand of lane (token n, k-group q)
            f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const V8 kf = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(sk + n * kKS + 32 * c + 8 * q));
                sacc = M::qk(kf, qop[c], sacc);
            }
            __builtin_amdgcn_s_setprio(0);
            // online softmax over the step's 16 tokens (lane: tokens 4q + i, head n).
            // Only a step that reaches past the segment, or a dropped step,
            // takes the mask (a uniform branch).
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = sacc[i];
            if (!full) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!(step_ok && th + 4 * q + i < seg_t1)) sc[i] = -INFINITY;
            }
            float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            mx = max_across_rows(mx) * sscale;
            const bool grow = mx > m_run + kSlack;
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
            const float m_sub = m_new == -INFINITY ? 0.f : m_new;   // no finite score yet: every weight is 0
            m_run = m_new;
            // rescale O rows (head 4q + i in register i) when some real head's max moved
            if (__builtin_amdgcn_ballot_w64(n < G && grow)) {
                float ar[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) ar[i] = from_lane(alpha, 4 * q + i);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) oacc[t][i] *= ar[i];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) lacc[i] *= ar[i];
            }
            // probabilities rounded (RNE, in pairs): the same values feed the
            // PV product and the running sum.  bf16: the remainder p - hi is
            // exact in fp32 and rounded once more.
            float pf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pf[i] = fast_exp2(fmaf(sc[i], sscale, -m_sub));
            const uint2 pop = make_uint2(M::round2(pf[0], pf[1]), M::round2(pf[2], pf[3]));
            uint2 pop_lo = make_uint2(0u, 0u);
            if constexpr (M::kSplit)
                pop_lo = make_uint2(M::round2(pf[0] - M::lo(pop.x), pf[1] - M::hi(pop.x)),
                                    M::round2(pf[2] - M::lo(pop.y), pf[3] - M::hi(pop.y)));
            // PV, and the row sums (split: the 8 remainder products after the
            // 8 leading ones, so no MFMA waits on the one before it)
            __builtin_amdgcn_s_setprio(1);
            uint2 vop[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                vop[t] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(sv + tr_off + 16 * t)));
                oacc[t] = M::pv(pop, vop[t], oacc[t]);
            }
            lacc = M::pv(pop, ones, lacc);
            if constexpr (M::kSplit) {
#pragma unroll
                for (int t = 0; t < 8; ++t) oacc[t] = M::pv(pop_lo, vop[t], oacc[t]);
                lacc = M::pv(pop_lo, ones, lacc);
            }
            __builtin_amdgcn_s_setprio(0);
        };

        // the step loop, instantiated once per load policy (a per-step choice
        // between two load forms writing the same registers makes the
        // compiler wait for every outstanding load in between)
        auto run_steps = [&](auto load) {
            constexpr int NS = kStages;
            uint4 kr[NS][4], vr[NS][4];
#pragma unroll
            for (int st = 0; st < NS - 1; ++st) issue(st, kr[st], vr[st], load);
            for (int k = 0; k < n_steps; k += NS) {
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    const int nxt = (st + NS - 1) % NS;
                    issue(k + st + NS - 1, kr[nxt], vr[nxt], load);
                    compute(k + st, kr[st], vr[st]);
                }
            }
        };
        if (shared) run_steps(cached_load);
        else run_steps(stream_load);
    }

    // ---- finish: the output or a split-K partial ---------------------------
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float mr = from_lane(m_run, 4 * q + i);
        const int hl = 4 * q + i;                     // head within the group (RUN: sequence within the run)
        if (hl >= G) continue;
        const int h = RUN ? g : g * G + hl;
        const int so = RUN ? s + hl : s;              // the output's sequence
        if (whole) {
            const float inv = a.v_scale / lacc[i];
            uint16_t* dst = out + ((int64_t)so * Hq + h) * kD + n;
#pragma unroll
            for (int t = 0; t < 8; ++t) dst[16 * t] = M::round(oacc[t][i] * inv);
        } else {
            // (a run member's partial: its own sequence's slot of the partition)
            const int64_t slot = (RUN ? seg_slot + (int64_t)hl * a.max_partitions : seg_slot) * Hq + h;
            float* po = a.part_o + slot * kD + n;
#pragma unroll
            for (int t = 0; t < 8; ++t) po[16 * t] = oacc[t][i];
            if (n == 0) {
                a.part_ml[slot * 2] = mr;
                a.part_ml[slot * 2 + 1] = lacc[i];
            }
        }
    }
    } while (!RUN && next_segment(a, w));
}

}  // namespace

bool gqa16_mfma_supported(pa_dtype q_dtype, pa_dtype kv_dtype, int head_dim, int group_size) {
    return (kv_dtype == PA_F16 || kv_dtype == PA_BF16) && q_dtype == kv_dtype && head_dim == kD &&
           (group_size == 2 || group_size == 4 || group_size == 8);
}

int launch_decode_gqa16_mfma(const DecodeArgs& args, const DecodePlan& plan, pa_dtype kv_dtype, int group_size,
                             void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    void (*kernel)(DecodeArgs);
    const bool w = args.new_key != nullptr;
    const bool f16 = kv_dtype == PA_F16;
    switch (group_size) {
        case 2:
            kernel = f16 ? (w ? decode_gqa16_mfma_kernel<PA_F16, 2, true> : decode_gqa16_mfma_kernel<PA_F16, 2, false>)
                         : (w ? decode_gqa16_mfma_kernel<PA_BF16, 2, true> : decode_gqa16_mfma_kernel<PA_BF16, 2, false>);
            break;
        case 4:
            kernel = f16 ? (w ? decode_gqa16_mfma_kernel<PA_F16, 4, true> : decode_gqa16_mfma_kernel<PA_F16, 4, false>)
                         : (w ? decode_gqa16_mfma_kernel<PA_BF16, 4, true> : decode_gqa16_mfma_kernel<PA_BF16, 4, false>);
            break;
        case 8:
            kernel = f16 ? (w ? decode_gqa16_mfma_kernel<PA_F16, 8, true> : decode_gqa16_mfma_kernel<PA_F16, 8, false>)
                         : (w ? decode_gqa16_mfma_kernel<PA_BF16, 8, true> : decode_gqa16_mfma_kernel<PA_BF16, 8, false>);
            break;
        default:
            return (int)hipErrorInvalidValue;
    }
    DecodeArgs a = args;
    const int64_t grid = decode_grid(&a, plan, reinterpret_cast<const void*>(kernel), 0);
    if (grid <= 0 || grid > INT32_MAX) return grid == 0 ? 0 : (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kDecodeThreads), 0, st, a);
    return (int)hipGetLastError();
}

int launch_run_gqa16_mfma(const DecodeArgs& a, pa_dtype kv_dtype, void* stream) {
    const int64_t grid = (int64_t)(a.num_seqs / a.share_run) * a.groups * a.max_partitions;
    if (grid == 0) return 0;
    if (grid > INT32_MAX) return (int)hipErrorInvalidValue;
    const bool f16 = kv_dtype == PA_F16;
    void (*kernel)(DecodeArgs);
    switch (a.share_run) {
        case 2: kernel = f16 ? decode_gqa16_mfma_kernel<PA_F16, 2, false, true> : decode_gqa16_mfma_kernel<PA_BF16, 2, false, true>; break;
        case 4: kernel = f16 ? decode_gqa16_mfma_kernel<PA_F16, 4, false, true> : decode_gqa16_mfma_kernel<PA_BF16, 4, false, true>; break;
        case 8: kernel = f16 ? decode_gqa16_mfma_kernel<PA_F16, 8, false, true> : decode_gqa16_mfma_kernel<PA_BF16, 8, false, true>; break;
        default: return (int)hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kDecodeThreads), 0, static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

}  // namespace pa
