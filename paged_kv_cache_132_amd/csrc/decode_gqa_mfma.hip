// pa_decode for grouped-query attention over an fp8 (OCP e4m3) KV cache on
// the matrix cores ([nano-vllm blog §2.3] decode attention; fp8 KV of
// [nano-vllm blog §1.1, §6.3]).  Several query heads (G = 2, 4 or 8) read one
// KV head, so QK and PV become small dense products per 32-token step; the
// 4-to-8 multiply-adds per KV byte that would saturate the vector ALUs run on
// v_mfma_f32_16x16x32_bf16 instead, and the kernel stays bound by HBM.
//
// Work decomposition
//   Workgroup = (sequence, group of 4 KV heads, partition); wave w owns KV
//   head 4*group + w for the whole partition, so the waves never exchange
//   softmax state.  A wave walks its partition in steps of 32 tokens (two
//   16-token halves; a half never crosses a block boundary for block size 16
//   or 32), keeping kGqaStages steps of K/V loads in flight (at two waves
//   per SIMD the in-flight bytes, not the ALUs, set the rate).
//
// Per step, per wave (lane l: n = l % 16, q = l / 16):
//   load each load instruction reads 8 whole 128-byte head rows (8 lanes x
//        16 bytes per token); the rows are staged in this wave's LDS and read
//        back in operand layout.  (Operand-layout loads -- 16 tokens x 64
//        bytes per instruction -- reached only ~3.9 TB/s even with no
//        arithmetic at all; whole-row loads ~5.4 TB/s.)
//   QK   A = K rows: lane (token n of the half, head_dim 16q..16q+15 and
//        64+16q..64+16q+15), widened fp8 -> bf16 (exact); B = query: lane
//        (head n, the same 32 head_dim positions), zero for n >= G.  4 MFMAs
//        per half give S[token][head] with lane (q, n) holding tokens
//        4q..4q+3 of head n.
//   soft running max over the 32 tokens (in-lane, then across the 4 rows),
//        exp2-domain probabilities; masked tokens get weight 0.
//   PV   A = P: exactly the lane's own 8 probabilities (k-slot 8q+j is token
//        4q+j of half 0 for j < 4, token 4q+j-4 of half 1 for j >= 4), bf16.
//        B = V: the 32 V rows are staged in LDS and read back transposed with
//        ds_read_tr8_b64 -- within each 16-lane group, lane i receives byte
//        (i & 7) of the 8 rows addressed by lanes 2j + (i >> 3) -- so each lane
//        gets the 8 k-slot tokens of one head_dim column, widened to bf16.
//        8 MFMAs (16 head_dim columns each) accumulate O[head][d] in fp32.
//
// Output, partials and the merge are shared with the vector kernel.  With
// WRITE (pa_decode_write) the 8 lanes whose loads will cover a sequence's
// newest token store its encoded K/V row first, in the segment that holds it.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "decode_common.h"
#include "kv_encode.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;                  // head_dim
constexpr int kRowStride = 144;          // LDS bytes per staged V row (128 + 16 against bank conflicts)
constexpr int kStepTokens = 32;
constexpr int kGqaStages = 2;            // 32-token steps of K/V loads each wave keeps in flight
constexpr float kSlack = 8.f;            // a head's weights stay below 2^8 between rescales

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4 stream_load(const uint8_t* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ uint4 cached_load(const uint8_t* p) {
    return __builtin_bit_cast(uint4, *reinterpret_cast<const u32x4*>(p));
}

// 8 fp8 codes (two dwords) -> 8 bf16, exactly.
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    const uint32_t b = __float_as_uint(x);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
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

template <int G, bool WRITE>
__global__ __launch_bounds__(kDecodeThreads) void decode_gqa_fp8_mfma_kernel(DecodeArgs a) {
    static_assert(G == 2 || G == 4 || G == 8, "query heads per KV head");
    constexpr int NW = kDecodeWaves;
    __shared__ __attribute__((aligned(16))) uint8_t s_kv[NW][2][kStepTokens * kRowStride];

    // ---- which (sequence, KV-head group, partition) -------------------------
    WorkItem w;
    if (!begin_work(a, blockIdx.x, w)) return;
    const int group = w.group;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = group * NW + wave;                 // this wave's KV head
    if (g >= a.num_kv_heads) return;                 // no barriers below: idle waves may leave
    const int Hq = a.num_heads;
    uint16_t* out = static_cast<uint16_t*>(a.out);

    // one segment (tokens [t0, t1) of one sequence) per pass
    do {
    publish_segments(a, w);                          // (thread 0: wave 0 always holds a KV head)
    const int lane = opaque(threadIdx.x) & 63;       // (derived in every pass, see decode.hip)
    const int n = lane & 15;
    const int q = lane >> 4;
    const int s = w.s, L = w.L;
    const int64_t seg_slot = w.seg_slot;
    const bool whole = whole_sequence(w);

    if (L <= 0) {
        uint16_t* dst = out + ((int64_t)s * Hq + g * G) * kD;
        const uint32_t z = opaque(0);
        for (int i = lane * 8; i < G * kD; i += 64 * 8) *reinterpret_cast<uint4*>(dst + i) = make_uint4(z, z, z, z);
        continue;
    }

    // ---- query operand: head n of this KV head's group, head_dim 32q.. ----
    // Scores stay unscaled out of the MFMA and the positive scale enters in
    // the exponent's FMA; a negative scale is moved onto the queries as an
    // exact sign flip, and a zero scale is raised to the least normal float
    // (so a masked -inf score still scales to -inf).
    const uint32_t qsign = a.score_scale < 0.f ? 0x80008000u : 0u;
    const float sscale = fmaxf(fabsf(a.score_scale), 1.17549435e-38f);
    bf16x8 qop[4];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.query) + ((int64_t)s * Hq + g * G + (n < G ? n : 0)) * kD + 16 * q;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int d0 = (c >> 1) * 64 + (c & 1) * 8;
            uint4 v = n < G ? *reinterpret_cast<const uint4*>(qp + d0) : make_uint4(0, 0, 0, 0);
            v.x ^= qsign;
            v.y ^= qsign;
            v.z ^= qsign;
            v.w ^= qsign;
            qop[c] = __builtin_bit_cast(bf16x8, v);
        }
    }

    const int t_begin = w.t0;
    const int t_end = w.t1;
    const int shift = a.block_shift;
    const uint32_t row_bytes = (uint32_t)(a.num_kv_heads * kD);               // fp8: 1 byte per element
    const uint32_t half_bytes = row_bytes << shift;                           // K half -> V half
    const uint32_t lane_col = (uint32_t)(g * kD + 16 * (lane & 7));           // 16-byte chunk of the head's row
    const uint8_t* pool = static_cast<const uint8_t*>(a.kv_pool);
    const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    // the fused write applies to lengths the table holds (as pa_cache_write)
    const bool write_len = WRITE && w.L_raw == L;

    // LDS: this wave's K and V staging rows; transposed-read base address of this lane
    uint8_t* sk = s_kv[wave][0];
    uint8_t* sv = s_kv[wave][1];
    const int jj = n >> 1;
    const uint32_t tr_off = (uint32_t)((16 * (jj >> 2) + 4 * q + (jj & 3)) * kRowStride + 8 * (lane & 1));

    float m_run = -INFINITY;       // running max of head n (identical in all 4 rows)
    // running sums as P times a column of ones on the matrix cores, in the C
    // layout of O (register i: head 4q + i)
    f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
    f32x4 oacc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

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
        const uint64_t shared = __builtin_amdgcn_ballot_w64(in_seg && (my_blk == prev_blk || my_blk == next_blk));
        const int seg_t0 = max(t_begin, seg0 << shift);
        const int seg_t1 = min(t_end, (seg0 + seg_blocks) << shift);
        const int n_steps = (seg_t1 - seg_t0 + kStepTokens - 1) / kStepTokens;

        // Fused cache write ([CANN notes §4.3]: write the new token, then read
        // every block).  Before this segment's first load, the 8 lanes whose
        // loads will cover the newest token store its encoded row, each lane
        // the 16 bytes it later reads itself: one lane's global accesses to
        // one address take effect in program order, so the loads see the new
        // bytes with no wait on the stores.
        if (write_len && L - 1 >= seg_t0 && L - 1 < seg_t1) {
            const int t_new = L - 1;
            const int blk = __builtin_amdgcn_readlane(my_blk, (t_new >> shift) - seg0);
            if (blk >= 0 && blk < a.num_blocks && (lane >> 3) == (t_new & 7)) {
                const int64_t row = ((int64_t)blk * 2 << shift) + (t_new & (a.block_size - 1));
                uint8_t* kp = const_cast<uint8_t*>(pool) + row * row_bytes + lane_col;
                const int64_t src = ((int64_t)s * a.num_kv_heads + g) * kD + 16 * (lane & 7);
                *reinterpret_cast<uint4*>(kp) = encode_chunk16<PA_BF16, PA_FP8_E4M3>(
                    static_cast<const uint16_t*>(a.new_key) + src, a.write_k_scale);
                *reinterpret_cast<uint4*>(kp + half_bytes) = encode_chunk16<PA_BF16, PA_FP8_E4M3>(
                    static_cast<const uint16_t*>(a.new_value) + src, a.write_v_scale);
            }
        }
        // Issue the K and V loads of step k.  Each load instruction reads 8
        // whole 128-byte head rows (8 lanes x 16 bytes per token): long runs
        // keep the request count per byte low.  Rows past the end are
        // redirected to the first row of their half, which is always valid,
        // and are masked out of the softmax.
        auto issue = [&](int k, uint4 (&kr)[4], uint4 (&vr)[4]) {
            const int kk = min(k, n_steps - 1);
            const int t0 = seg_t0 + kk * kStepTokens;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int th = min(t0 + 16 * u, seg_t1 - 1) & ~15;       // half start (clamped into range)
                const int blk = __builtin_amdgcn_readlane(my_blk, (th >> shift) - seg0);
                const bool ok = blk >= 0 && blk < a.num_blocks;
                auto load_half = [&](auto load) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int t = th + 8 * j + (lane >> 3);
                        const int tok = t < seg_t1 ? t : th;
                        const int64_t row = ((int64_t)(ok ? blk : 0) * 2 << shift) + (tok & (a.block_size - 1));
                        const uint8_t* kp = pool + row * row_bytes + lane_col;
                        kr[2 * u + j] = load(kp);
                        vr[2 * u + j] = load(kp + half_bytes);
                    }
                };
                if ((shared >> ((th >> shift) - seg0)) & 1) load_half(cached_load);
                else load_half(stream_load);

            }
        };

        auto compute = [&](int k, const uint4 (&kr)[4], const uint4 (&vr)[4]) {
            if (k >= n_steps) return;
            const int t0 = seg_t0 + k * kStepTokens;
            // block ids outside the pool drop the whole half
            bool half_ok[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int th = t0 + 16 * u;
                const int blk = th < seg_t1 ? __builtin_amdgcn_readlane(my_blk, (th >> shift) - seg0) : -1;
                half_ok[u] = th < seg_t1 && blk >= 0 && blk < a.num_blocks;
            }
            // stage the step's K and V rows (row 16u + 8j + lane/8, chunk
            // lane%8).  V rows past the end (or of a dropped half) are staged
            // as zeros: their weight is 0, and 0 times whatever a redirected
            // load returned (the slot the fused write is storing, a NaN) must
            // not reach O.  (K rows need no care: their scores are masked.)
            const bool full = half_ok[0] && half_ok[1] && t0 + kStepTokens <= seg_t1;   // uniform
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint32_t off = (uint32_t)((16 * u + 8 * j + (lane >> 3)) * kRowStride + 16 * (lane & 7));
                    *reinterpret_cast<uint4*>(sk + off) = kr[2 * u + j];
                    *reinterpret_cast<uint4*>(sv + off) = vr[2 * u + j];
                }
            }
            if (!full) {      // the masked rows' V, overwritten (one wave's LDS stores land in order)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const uint32_t off = (uint32_t)((16 * u + 8 * j + (lane >> 3)) * kRowStride + 16 * (lane & 7));
                        if (!(half_ok[u] && t0 + 16 * u + 8 * j + (lane >> 3) < seg_t1))
                            *reinterpret_cast<uint4*>(sv + off) = make_uint4(0, 0, 0, 0);
                    }
                }
            }
            // QK: S[token][head] for both halves; A operand of lane (token n,
            // k-group q) = head_dim 16q..16q+15 and 64+16q..64+16q+15
            f32x4 sacc[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint8_t* rowp = sk + (16 * u + n) * kRowStride + 16 * q;
                const uint4 lo = *reinterpret_cast<const uint4*>(rowp);
                const uint4 hi = *reinterpret_cast<const uint4*>(rowp + 64);
                const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(w[2 * c], w[2 * c + 1]), qop[c], acc, 0, 0, 0);
                sacc[u] = acc;
            }
            // online softmax over the step's 32 tokens (lane: tokens 4q+i of each half, head n)
            // Only a step that reaches past the segment, or holds a dropped
            // half, takes the mask (a uniform branch).
            float sc[8];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[4 * u + i] = sacc[u][i];
            }
            if (!full) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tt = t0 + 16 * u + 4 * q + i;
                        if (!(half_ok[u] && tt < seg_t1)) sc[4 * u + i] = -INFINITY;
                    }
                }
            }
            float mx = sc[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
            mx = max_across_rows(mx) * sscale;
            // The reference max moves only when a head's max grows by more
            // than kSlack (log2 units): weights stay below 2^kSlack and most
            // steps skip the rescale of O (an AGPR round trip).  A step whose
            // halves are all dropped leaves mx, and maybe m_run, at -inf.
            const bool grow = mx > m_run + kSlack;
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
            const float m_sub = m_new == -INFINITY ? 0.f : m_new;   // no finite score yet: every weight is 0
            // probabilities rounded to bf16 once (RNE, in pairs): the same
            // values feed the PV product and the running sum, so the weights
            // normalise exactly
            uint32_t pw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = fast_exp2(fmaf(sc[2 * e], sscale, -m_sub));      // masked: 2^-inf = 0
                const float p1 = fast_exp2(fmaf(sc[2 * e + 1], sscale, -m_sub));
                pw[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
            }
            m_run = m_new;
            // rescale O rows (head 4q+i in register i) when some real head's max moved
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
            // PV, and the row sums
            const bf16x8 pop = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
            lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pop, ones, lacc, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const i32x2 v8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) i32x2*)(sv + tr_off + 16 * t));
                oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pop, widen8((uint32_t)v8[0], (uint32_t)v8[1]),
                                                                oacc[t], 0, 0, 0);
            }
        };

        constexpr int NS = kGqaStages;
        uint4 kr[NS][4], vr[NS][4];
#pragma unroll
        for (int st = 0; st < NS - 1; ++st) issue(st, kr[st], vr[st]);
        for (int k = 0; k < n_steps; k += NS) {
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const int nxt = (st + NS - 1) % NS;
                issue(k + st + NS - 1, kr[nxt], vr[nxt]);
                compute(k + st, kr[st], vr[st]);
            }
        }
    }

    // ---- finish: per-head sums, then the output or a split-K partial -------
    float lr[4], mr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lr[i] = lacc[i];
        mr[i] = from_lane(m_run, 4 * q + i);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hl = 4 * q + i;                     // head within the group
        if (hl >= G) continue;
        const int h = g * G + hl;
        if (whole) {
            const float inv = a.v_scale / lr[i];
            uint16_t* dst = out + ((int64_t)s * Hq + h) * kD + n;
#pragma unroll
            for (int t = 0; t < 8; ++t) dst[16 * t] = bf16_bits(oacc[t][i] * inv);
        } else {
            const int64_t slot = seg_slot * Hq + h;
            float* po = a.part_o + slot * kD + n;
#pragma unroll
            for (int t = 0; t < 8; ++t) po[16 * t] = oacc[t][i];
            if (n == 0) {
                a.part_ml[slot * 2] = mr[i];
                a.part_ml[slot * 2 + 1] = lr[i];
            }
        }
    }
    } while (next_segment(a, w));
}

}  // namespace

bool gqa_mfma_supported(pa_dtype q_dtype, pa_dtype kv_dtype, int head_dim, int group_size) {
    return q_dtype == PA_BF16 && kv_dtype == PA_FP8_E4M3 && head_dim == kD &&
           (group_size == 2 || group_size == 4 || group_size == 8);
}

int launch_decode_gqa_mfma(const DecodeArgs& args, const DecodePlan& plan, int group_size, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    void (*kernel)(DecodeArgs);
    const bool w = args.new_key != nullptr;
    switch (group_size) {
        case 2: kernel = w ? decode_gqa_fp8_mfma_kernel<2, true> : decode_gqa_fp8_mfma_kernel<2, false>; break;
        case 4: kernel = w ? decode_gqa_fp8_mfma_kernel<4, true> : decode_gqa_fp8_mfma_kernel<4, false>; break;
        case 8: kernel = w ? decode_gqa_fp8_mfma_kernel<8, true> : decode_gqa_fp8_mfma_kernel<8, false>; break;
        default: return (int)hipErrorInvalidValue;
    }
    // Two waves per SIMD: built with VGPR accumulators the kernel needs about
    // 156 VGPRs, which would admit three, and three measured slower (the
    // in-flight loads of two waves already cover the latency, a third adds
    // contention).  Unused dynamic LDS caps a CU at two workgroups.
    constexpr size_t kStaticLds = (size_t)kDecodeWaves * 2 * kStepTokens * kRowStride;
    constexpr size_t kCapLds = 18432;
    static_assert(3 * (kStaticLds + kCapLds) > 160 * 1024 && 2 * (kStaticLds + kCapLds) <= 160 * 1024,
                  "two workgroups of LDS per CU, not three");
    DecodeArgs a = args;
    const int64_t grid = decode_grid(&a, plan, reinterpret_cast<const void*>(kernel), kCapLds);
    if (grid <= 0 || grid > INT32_MAX) return grid == 0 ? 0 : (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kDecodeThreads), kCapLds, st, a);
    return (int)hipGetLastError();
}

}  // namespace pa
