// pa_decode kernels: paged decode attention with split-K over token
// partitions and a second merge pass ([nano-vllm blog §2.3], [CANN notes §4.3
// step 4]; the FlashAttention-style tiling of the computation inside a paged
// layout that [nano-vllm blog §2.3] says composes with paging).
//
// Work decomposition
//   A workgroup (4 waves) owns one (sequence, group of KV heads, partition of
//   `partition` consecutive tokens).  One wave-wide 16-byte-per-lane load
//   covers `rows` consecutive KV heads of ONE token: lane = (row r, slice j),
//   `row_lanes` lanes per head row (head_dim 128 fp16: 16 lanes x 8 halves,
//   4 heads = 1 KiB contiguous per token).  Each 16-lane/8-lane row therefore
//   owns one KV head and keeps that head's online-softmax state on its own,
//   with no cross-row traffic.
//   The 4 waves take interleaved chunks of 4 tokens (chunk c -> wave c % 4),
//   so the four waves of a workgroup stream neighbouring token rows of the
//   same physical block together.  Each wave keeps two chunks in flight:
//   16 x 16-byte loads per lane before it first waits.
//
// Per chunk (4 tokens), per lane:
//   QK:   packed dot products (v_dot2_f32_f16 / v_dot2_f32_bf16) over the
//         lane's 8 or 16 elements, then a 2-4 step DPP reduction inside the
//         row; every lane of the row ends with the full score.
//   mask: tokens at or beyond the end of the partition get weight 0 and are
//         never loaded from their own slot (their load is redirected to the
//         first token of the chunk, which is always valid), so poisoned or
//         stale slots never reach the arithmetic.
//   softmax: running max m and sum l in the exp2 domain (scores are
//         pre-scaled by scale * log2 e), rescaling o when m grows.
//   PV:   o[e] += p * v[e] in float32 for the lane's slice of head_dim.
//
// End of the workgroup: the 4 waves' states are merged through LDS.  A
// sequence with a single partition writes its output directly; otherwise the
// workgroup stores its partial (max, sum, unnormalised o) in the workspace
// and the merge kernel, launched next on the same stream, combines them
//     M = max_p m_p,  out = sum_p 2^(m_p-M) o_p / sum_p 2^(m_p-M) l_p.
// Two launches instead of a last-arriving-workgroup merge: publishing
// partials between workgroups inside one kernel needs device-scope fences,
// and on this part each one writes back and invalidates the XCD's L2.
//
// With WRITE (pa_decode_write) the wave that will load a sequence's newest
// token first stores that token's encoded K/V rows, each lane the bytes it
// later reads back itself (see the block before the main loop).
//
// With RUN (pa_decode_shared, one query head per KV head) the same kernel is
// the run kernel of shared runs where the matrix-core form does not apply
// (fp8 KV, head_dim 64, block 8): its G "query heads" are head g of the run's
// G sequences, over a partition the run shares, each K/V row read once.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "decode_common.h"
#include "kv_encode.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTokensPerChunk = 4;   // tokens one wave takes per step
constexpr int kStages = 2;           // chunks of loads each wave keeps in flight

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N = 4, 8, 16); every lane of the group
// receives the same total.  quad_perm [1,0,3,2] and [2,3,0,1], then
// row_half_mirror (8-lane halves) and row_mirror (16-lane rows).
template <int N>
__device__ __forceinline__ float row_sum(float x) {
    static_assert(N == 4 || N == 8 || N == 16, "row width");
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    if constexpr (N >= 8) x += dpp<0x141>(x);
    if constexpr (N >= 16) x += dpp<0x140>(x);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// K/V rows are read exactly once per call: load them with the nontemporal
// hint so the stream does not displace other lines in L2 and the MALL.
__device__ __forceinline__ uint4 stream_load(const uint8_t* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ uint4 cached_load(const uint8_t* p) {
    return __builtin_bit_cast(uint4, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int QT>
__device__ __forceinline__ uint16_t to_out_bits(float x) {
    if constexpr (QT == PA_F16) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    } else {
        const uint32_t b = __float_as_uint(x);
        if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);   // NaN
        return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
    }
}

// Dot product of a lane's K slice with a packed 16-bit query slice.
//   16-bit KV: 4 dwords = 8 elements, q as 4 packed pairs.
//   fp8 KV:    4 dwords = 16 codes, q as 8 packed bf16 pairs.
template <int KVT>
__device__ __forceinline__ float dot_slice(const uint4& k, const uint32_t* q) {
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
    float acc = 0.f;
    if constexpr (KVT == PA_F16) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, q[w]),
                                         __builtin_bit_cast(f16x2, kw[w]), acc, false);
    } else if constexpr (KVT == PA_BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[w]),
                                                  __builtin_bit_cast(bf16x2, kw[w]), acc, false);
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[w], 1.0f, false);
            const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[w], 1.0f, true);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[2 * w]), lo, acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[2 * w + 1]), hi, acc, false);
        }
    }
    return acc;
}

// o[e] += p * v[e] over a lane's V slice (8 or 16 elements).
template <int KVT, int EPL>
__device__ __forceinline__ void accumulate_v(float (&o)[EPL], float p, const uint4& v) {
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
    if constexpr (KVT == PA_F16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const f16x2 h = __builtin_bit_cast(f16x2, vw[w]);
            o[2 * w] = fmaf(p, (float)h.x, o[2 * w]);
            o[2 * w + 1] = fmaf(p, (float)h.y, o[2 * w + 1]);
        }
    } else if constexpr (KVT == PA_BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            o[2 * w] = fmaf(p, bf16_lo(vw[w]), o[2 * w]);
            o[2 * w + 1] = fmaf(p, bf16_hi(vw[w]), o[2 * w + 1]);
        }
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(vw[w], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(vw[w], true);
            o[4 * w + 0] = fmaf(p, lo[0], o[4 * w + 0]);
            o[4 * w + 1] = fmaf(p, lo[1], o[4 * w + 1]);
            o[4 * w + 2] = fmaf(p, hi[0], o[4 * w + 2]);
            o[4 * w + 3] = fmaf(p, hi[1], o[4 * w + 3]);
        }
    }
}


// RUN: the run kernel.  G is then the run length: "query head" gi of KV
// head g is head g of sequence s + gi (num_heads == num_kv_heads), and the
// workgroup's partition is one its run shares, read once for all of them.
template <int QT, int KVT, int D, int G, bool WRITE, bool RUN = false>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeArgs a) {
    static_assert(!(RUN && WRITE), "a shared partition never holds a newest token");
    constexpr int KVB = KVT == PA_FP8_E4M3 ? 1 : 2;
    constexpr int ROWL = D * KVB / 16;      // lanes per KV-head row
    constexpr int ROWS = 64 / ROWL;         // KV heads per workgroup
    constexpr int EPL = 16 / KVB;           // KV elements per lane per token
    constexpr int QDW = EPL / 2;            // packed 16-bit query pairs per lane
    constexpr int NW = kDecodeWaves;
    constexpr int TPC = kTokensPerChunk;
    constexpr int NS = kStages;
    constexpr int OPT = EPL / NW;           // output elements per thread in the merge

    __shared__ float s_m[NW][ROWS];
    __shared__ float s_l[NW][ROWS];
    __shared__ float s_o[NW][64 * EPL];

    // ---- which KV-head group, and which sequences' tokens -------------------
    WorkItem w;
    if (!(RUN ? find_run_work(a, blockIdx.x, w) : begin_work(a, blockIdx.x, w))) return;
    const int group = w.group;

    const int Hq = a.num_heads;
    uint16_t* out = static_cast<uint16_t*>(a.out);

    // one segment (tokens [t0, t1) of one sequence) per pass; every wave of
    // the workgroup walks the same segments
    do {
    // The lane's indices are derived afresh in every pass (from a value the
    // compiler cannot see through): computed once before the loop they would
    // stay live through the main loop and cost a wave per SIMD.
    const int tid = opaque(threadIdx.x);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane / ROWL;
    const int j = lane % ROWL;
    const int g_row = group * ROWS + r;
    const bool row_ok = g_row < a.num_kv_heads;
    const int g = row_ok ? g_row : a.num_kv_heads - 1;   // rows past the last head idle on a valid one
    const int s = w.s, L = w.L;
    const int64_t seg_slot = w.seg_slot;
    // the output is written here, with no merge: the segment is its sequence's whole range
    const bool whole = RUN ? w.n_part == 1 : whole_sequence(w);
    if (!RUN) publish_segments(a, w);
    if (!RUN && L <= 0) {                                  // empty sequence: zero output
        if (wave == 0 && row_ok) {
            const uint32_t z = opaque(0);                  // (a zero made here, not held through the loop)
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                uint16_t* dst = out + ((int64_t)s * Hq + g * G + gi) * D + j * EPL;
#pragma unroll
                for (int e = 0; e < EPL; e += 8) *reinterpret_cast<uint4*>(dst + e) = make_uint4(z, z, z, z);
            }
        }
        continue;
    }

    // ---- query slices of the G query heads that read KV head g ------------
    // (RUN: head g of the run's G sequences)
    uint32_t q[G][QDW];
    {
        const uint16_t* qb = static_cast<const uint16_t*>(a.query) + ((int64_t)s * Hq + g * (RUN ? 1 : G)) * D + j * EPL;
        const int64_t qstride = RUN ? (int64_t)Hq * D : D;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
#pragma unroll
            for (int w = 0; w < QDW; w += 4) {
                const uint4 v = *reinterpret_cast<const uint4*>(qb + gi * qstride + 2 * w);
                q[gi][w] = v.x; q[gi][w + 1] = v.y; q[gi][w + 2] = v.z; q[gi][w + 3] = v.w;
            }
        }
    }

    // ---- the partition's token range and this lane's K/V addressing -------
    const int t_begin = w.t0;
    const int t_end = w.t1;
    const int shift = a.block_shift;
    const uint32_t row_bytes = (uint32_t)(a.num_kv_heads * D * KVB);        // one token row, all heads
    const uint32_t half_bytes = row_bytes << shift;                       // K half -> V half
    const uint32_t lane_off = (uint32_t)((g * D + j * EPL) * KVB);         // this lane's 16 bytes
    const uint8_t* pool = static_cast<const uint8_t*>(a.kv_pool);
    const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    // the fused write applies to lengths the table holds (as pa_cache_write)
    const bool write_len = WRITE && w.L_raw == L;

    float m[G], l[G], o[G][EPL];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        m[gi] = -INFINITY;
        l[gi] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[gi][e] = 0.f;
    }

    auto compute_chunk = [&](int nvalid, const uint4 (&kr)[TPC], const uint4 (&vr)[TPC]) {
        if (nvalid <= 0) return;
        float sc[TPC][G];
#pragma unroll
        for (int i = 0; i < TPC; ++i) {
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
                sc[i][gi] = row_sum<ROWL>(dot_slice<KVT>(kr[i], q[gi])) * a.score_scale;
        }
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            float mx = sc[0][gi];
#pragma unroll
            for (int i = 1; i < TPC; ++i) mx = i < nvalid ? fmaxf(mx, sc[i][gi]) : mx;
            const float m_new = fmaxf(m[gi], mx);
            const float alpha = fast_exp2(m[gi] - m_new);   // m_new is finite: token 0 is valid
            float pr[TPC];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < TPC; ++i) {
                pr[i] = i < nvalid ? fast_exp2(sc[i][gi] - m_new) : 0.f;
                psum += pr[i];
            }
            l[gi] = l[gi] * alpha + psum;
            m[gi] = m_new;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[gi][e] *= alpha;
#pragma unroll
            for (int i = 0; i < TPC; ++i) accumulate_v<KVT, EPL>(o[gi], pr[i], vr[i]);
        }
    };

    // ---- main loop --------------------------------------------------------
    // The partition is walked in segments of up to 64 logical blocks.  Each
    // wave holds the segment's physical block ids in one VGPR (lane k = entry
    // k) and picks them out with readlane, so no memory access sits between
    // one chunk's loads and the next.  Chunks of TPC tokens go round-robin to
    // the 4 waves; every wave keeps NS chunks of loads in flight, issuing
    // chunk c + (NS-1)*4 right before it consumes chunk c.  Loads past the
    // wave's last chunk re-read a valid chunk and are masked out (nvalid 0).
    //
    // Blocks that a neighbouring sequence (s - 1 or s + 1) maps at the same
    // logical index -- a shared prefix -- will be read again by that
    // sequence's workgroups at about the same time: they are loaded through
    // the caches.  Every other block is streamed with nontemporal loads.
    const int lb_first = t_begin >> shift;
    const int lb_last = (t_end - 1) >> shift;

    // Fused cache write ([CANN notes §4.3]: write the new token, then read
    // every block).  The newest token sits in the last partition, in the
    // segment and chunk found below.  The wave that will load that chunk
    // stores the token's encoded rows before it issues any load, each lane
    // the 16 bytes it later reads itself: one lane's global accesses to one
    // address take effect in program order, so the loads see the new bytes
    // with no wait on the stores.
    if (WRITE && write_len && t_end == L) {
        const int t_new = L - 1;
        const int sg = lb_first + (((t_new >> shift) - lb_first) & ~63);
        const int cn = (t_new - max(t_begin, sg << shift)) / TPC;
        const int blk = bt_row[t_new >> shift];
        if (cn % NW == wave && row_ok && blk >= 0 && blk < a.num_blocks) {
            const int64_t src = ((int64_t)s * a.num_kv_heads + g) * D + j * EPL;
            const int64_t row = ((int64_t)blk * 2 << shift) + (t_new & (a.block_size - 1));
            uint8_t* kdst = const_cast<uint8_t*>(pool) + row * row_bytes + lane_off;
            *reinterpret_cast<uint4*>(kdst) =
                encode_chunk16<QT, KVT>(static_cast<const uint16_t*>(a.new_key) + src, a.write_k_scale);
            *reinterpret_cast<uint4*>(kdst + half_bytes) =
                encode_chunk16<QT, KVT>(static_cast<const uint16_t*>(a.new_value) + src, a.write_v_scale);
        }
    }
    for (int seg0 = lb_first; seg0 <= lb_last; seg0 += 64) {
        const int seg_blocks = min(64, lb_last - seg0 + 1);
        const bool in_seg = lane < seg_blocks;
        const int my_blk = in_seg ? bt_row[seg0 + lane] : 0;
        const int prev_blk = in_seg && s > 0 ? bt_row[seg0 + lane - a.max_blocks_per_seq] : -1;
        const int next_blk = in_seg && s + 1 < a.num_seqs ? bt_row[seg0 + lane + a.max_blocks_per_seq] : -1;
        // (the run kernel reads each block once: streamed)
        const uint64_t shared = RUN ? 0ull : __builtin_amdgcn_ballot_w64(in_seg && (my_blk == prev_blk || my_blk == next_blk));
        const int seg_t0 = max(t_begin, seg0 << shift);
        const int seg_t1 = min(t_end, (seg0 + seg_blocks) << shift);
        const int n_chunks = (seg_t1 - seg_t0 + TPC - 1) / TPC;
        if (wave >= n_chunks) continue;
        const int n_mine = (n_chunks - wave + NW - 1) / NW;

        auto issue = [&](int c, uint4 (&kr)[TPC], uint4 (&vr)[TPC]) -> int {
            const int cc = min(c, n_chunks - 1);
            const int tc = seg_t0 + cc * TPC;
            const int blk = __builtin_amdgcn_readlane(my_blk, (tc >> shift) - seg0);
            const bool blk_ok = blk >= 0 && blk < a.num_blocks;
            const int nvalid = (c < n_chunks && blk_ok) ? min(TPC, seg_t1 - tc) : 0;
            const int64_t row0 = ((int64_t)(blk_ok ? blk : 0) * 2 << shift) + (tc & (a.block_size - 1));
            const uint8_t* kbase = pool + row0 * row_bytes;
            auto load_chunk = [&](auto load) {
#pragma unroll
                for (int i = 0; i < TPC; ++i) {
                    const uint32_t ti = (uint32_t)(i < nvalid ? i : 0) * row_bytes;
                    kr[i] = load(kbase + ti + lane_off);
                }
#pragma unroll
                for (int i = 0; i < TPC; ++i) {
                    const uint32_t ti = (uint32_t)(i < nvalid ? i : 0) * row_bytes;
                    vr[i] = load(kbase + half_bytes + ti + lane_off);
                }
            };
            if ((shared >> ((tc >> shift) - seg0)) & 1) load_chunk(cached_load);
            else load_chunk(stream_load);
            return nvalid;
        };

        uint4 kr[NS][TPC], vr[NS][TPC];
        int nv[NS];
#pragma unroll
        for (int st = 0; st < NS - 1; ++st) nv[st] = issue(wave + st * NW, kr[st], vr[st]);
        int c = wave;
        for (int it = 0; it < n_mine; it += NS) {
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const int nxt = (st + NS - 1) % NS;
                nv[nxt] = issue(c + (NS - 1) * NW, kr[nxt], vr[nxt]);
                compute_chunk(nv[st], kr[st], vr[st]);
                c += NW;
            }
        }
    }

    // ---- merge the 4 waves, then finish or publish a partial ---------------
    const int ln = tid & 63;          // lane slot this thread merges
    const int part = tid >> 6;        // which quarter of that slot's elements
    const int mr = ln / ROWL;
    const int mj = ln % ROWL;
    const int mg_row = group * ROWS + mr;
    const bool m_ok = mg_row < a.num_kv_heads;

#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        if (j == 0) {
            s_m[wave][r] = m[gi];
            s_l[wave][r] = l[gi];
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_o[wave][lane * EPL + e] = o[gi][e];
        __syncthreads();

        float M = s_m[0][mr];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][mr]);
        float fw[NW];
        float Lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            fw[w] = fast_exp2(s_m[w][mr] - M);            // idle waves: 2^-inf = 0
            Lsum += fw[w] * s_l[w][mr];
        }
        float acc[OPT];
#pragma unroll
        for (int e = 0; e < OPT; ++e) {
            float x = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) x = fmaf(fw[w], s_o[w][ln * EPL + part * OPT + e], x);
            acc[e] = x;
        }
        const int h = RUN ? mg_row : mg_row * G + gi;
        const int so = RUN ? s + gi : s;                  // the output's sequence
        const int d0 = mj * EPL + part * OPT;
        if (m_ok) {
            if (whole) {
                const float inv = a.v_scale / Lsum;
                uint16_t* dst = out + ((int64_t)so * Hq + h) * D + d0;
#pragma unroll
                for (int e = 0; e < OPT; ++e) dst[e] = to_out_bits<QT>(acc[e] * inv);
            } else {
                // (a run member's partial: its own sequence's slot of the partition)
                const int64_t slot = (RUN ? seg_slot + (int64_t)gi * a.max_partitions : seg_slot) * Hq + h;
                float* po = a.part_o + slot * D + d0;
#pragma unroll
                for (int e = 0; e < OPT; ++e) po[e] = acc[e];
                if (mj == 0 && part == 0) {
                    a.part_ml[slot * 2] = M;
                    a.part_ml[slot * 2 + 1] = Lsum;
                }
            }
        }
        __syncthreads();
    }
    } while (!RUN && next_segment(a, w));
}

// Split-K merge of one sequence's partitions for NE consecutive output
// elements [d0, d0 + NE) of query head h:
//     M = max_p m_p,  out = v_scale * sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p
template <int QT, int D, int NE>
__device__ __forceinline__ void merge_partials(const DecodeArgs& a, int s, int h, int d0, const MergeList& list) {
    // A running maximum over batches of 8 partials: each batch's loads are
    // all issued before the first is used, so most sequences take one round
    // trip to memory.
    constexpr int kBatch = 8;
    float M = -INFINITY;
    float den = 0.f;
    float num[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) num[e] = 0.f;
    for (int i0 = 0; i0 < list.n; i0 += kBatch) {
        float mp[kBatch], lp[kBatch], op[kBatch][NE];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int64_t slot = list.slot(min(i0 + k, list.n - 1)) * a.num_heads + h;
            mp[k] = a.part_ml[slot * 2];
            lp[k] = a.part_ml[slot * 2 + 1];
            const float* po = a.part_o + slot * D + d0;
            if constexpr (NE == 4) {
                const float4 v = *reinterpret_cast<const float4*>(po);
                op[k][0] = v.x; op[k][1] = v.y; op[k][2] = v.z; op[k][3] = v.w;
            } else {
#pragma unroll
                for (int e = 0; e < NE; ++e) op[k][e] = po[e];
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (i0 + k < list.n) {                      // uniform: one sequence per workgroup
                const float m_new = fmaxf(M, mp[k]);
                const float alpha = fast_exp2(M - m_new);   // 0 on the first partial
                const float f = fast_exp2(mp[k] - m_new);
                den = fmaf(den, alpha, f * lp[k]);
#pragma unroll
                for (int e = 0; e < NE; ++e) num[e] = fmaf(num[e], alpha, f * op[k][e]);
                M = m_new;
            }
        }
    }
    const float inv = a.v_scale / den;
    uint16_t* dst = static_cast<uint16_t*>(a.out) + ((int64_t)s * a.num_heads + h) * D + d0;
#pragma unroll
    for (int e = 0; e < NE; ++e) dst[e] = to_out_bits<QT>(num[e] * inv);
}

// Second pass of split-K: one thread per output element of every sequence
// whose range was split between workgroups.
// A workgroup takes kMergeHeads query heads of one sequence, a thread NE
// consecutive output elements of one head (16-byte loads of the partial o at
// head_dim 128): few workgroups, most of which leave after one load when
// their sequence was not split.
constexpr int kMergeHeads = 8;

template <int QT, int D>
__global__ __launch_bounds__(kDecodeThreads) void merge_kernel(DecodeArgs a) {
    constexpr int NE = kMergeHeads * D / kDecodeThreads;   // output elements per thread
    constexpr int TPH = D / NE;                            // threads per head
    const int chunks = (a.num_heads + kMergeHeads - 1) / kMergeHeads;
    const int s = blockIdx.x / chunks;
    const int h = (blockIdx.x % chunks) * kMergeHeads + threadIdx.x / TPH;
    const int d0 = (threadIdx.x % TPH) * NE;
    const MergeList list = merge_list(a, s);
    if (list.n <= 1 || h >= a.num_heads) return;
    merge_partials<QT, D, NE>(a, s, h, d0, list);
}

template <int QT, int KVT, int D>
int launch_d(const DecodeArgs& args, const DecodePlan& plan, int group_size, hipStream_t st) {
    void (*kernel)(DecodeArgs);
    const bool w = args.new_key != nullptr;
    switch (group_size) {
        case 1: kernel = w ? decode_kernel<QT, KVT, D, 1, true> : decode_kernel<QT, KVT, D, 1, false>; break;
        case 2: kernel = w ? decode_kernel<QT, KVT, D, 2, true> : decode_kernel<QT, KVT, D, 2, false>; break;
        case 4: kernel = w ? decode_kernel<QT, KVT, D, 4, true> : decode_kernel<QT, KVT, D, 4, false>; break;
        case 8: kernel = w ? decode_kernel<QT, KVT, D, 8, true> : decode_kernel<QT, KVT, D, 8, false>; break;
        default: return (int)hipErrorInvalidValue;
    }
    DecodeArgs a = args;
    const int64_t grid = decode_grid(&a, plan, reinterpret_cast<const void*>(kernel), 0);
    if (grid <= 0 || grid > INT32_MAX) return grid == 0 ? 0 : (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kDecodeThreads), 0, st, a);
    return (int)hipGetLastError();
}

// the run kernel: one workgroup per (run, KV-head group, partition); those
// whose partition the run does not share leave at once
template <int QT, int KVT, int D>
int launch_run(const DecodeArgs& a, hipStream_t st) {
    const int64_t grid = (int64_t)(a.num_seqs / a.share_run) * a.groups * a.max_partitions;
    if (grid == 0) return 0;
    if (grid > INT32_MAX) return (int)hipErrorInvalidValue;
    void (*kernel)(DecodeArgs);
    switch (a.share_run) {
        case 2: kernel = decode_kernel<QT, KVT, D, 2, false, true>; break;
        case 4: kernel = decode_kernel<QT, KVT, D, 4, false, true>; break;
        case 8: kernel = decode_kernel<QT, KVT, D, 8, false, true>; break;
        default: return (int)hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kDecodeThreads), 0, st, a);
    return (int)hipGetLastError();
}

template <int QT, int KVT>
int launch_run_t(const DecodeArgs& a, int head_dim, hipStream_t st) {
    if (head_dim == 64) return launch_run<QT, KVT, 64>(a, st);
    return launch_run<QT, KVT, 128>(a, st);
}

template <int QT, int D>
int launch_merge(const DecodeArgs& a, hipStream_t st) {
    const int chunks = (a.num_heads + kMergeHeads - 1) / kMergeHeads;
    hipLaunchKernelGGL((merge_kernel<QT, D>), dim3((unsigned)(a.num_seqs * chunks)), dim3(kDecodeThreads), 0, st, a);
    return (int)hipGetLastError();
}

template <int QT, int KVT>
int launch_t(const DecodeArgs& a, const DecodePlan& plan, int head_dim, int group_size, hipStream_t st) {
    if (head_dim == 64) return launch_d<QT, KVT, 64>(a, plan, group_size, st);
    return launch_d<QT, KVT, 128>(a, plan, group_size, st);
}

}  // namespace

int launch_decode(const DecodeArgs& a, const DecodePlan& plan, pa_dtype q_dtype, pa_dtype kv_dtype,
                  int head_dim, int group_size, int phases, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (plan.grid == 0) return 0;
    int err = 0;
    if (phases & kPhasePartials) {
        if (a.share_run > 1) {             // the runs' shared partitions first (one query head per KV head)
            if (gqa16_mfma_supported(kv_dtype, kv_dtype, head_dim, a.share_run) && a.block_size >= 16)
                err = launch_run_gqa16_mfma(a, kv_dtype, stream);
            else if (kv_dtype == PA_F16) err = launch_run_t<PA_F16, PA_F16>(a, head_dim, st);
            else if (kv_dtype == PA_BF16) err = launch_run_t<PA_BF16, PA_BF16>(a, head_dim, st);
            else err = launch_run_t<PA_BF16, PA_FP8_E4M3>(a, head_dim, st);
            if (err != 0) return err;
        }
        if (plan.geo.mfma)
            err = kv_dtype == PA_FP8_E4M3 ? launch_decode_gqa_mfma(a, plan, group_size, stream)
                                          : launch_decode_gqa16_mfma(a, plan, kv_dtype, group_size, stream);
        else if (kv_dtype == PA_F16) err = launch_t<PA_F16, PA_F16>(a, plan, head_dim, group_size, st);
        else if (kv_dtype == PA_BF16) err = launch_t<PA_BF16, PA_BF16>(a, plan, head_dim, group_size, st);
        else err = launch_t<PA_BF16, PA_FP8_E4M3>(a, plan, head_dim, group_size, st);
    }
    // no merge when no sequence can be split: one fixed partition holds every
    // table, and (partition 0) a single chunk the whole batch
    const bool can_split = plan.max_partitions > 1 || (a.partition == 0 && plan.max_chunks > 1);
    if (err != 0 || !(phases & kPhaseMerge) || !can_split) return err;
    const bool f16 = q_dtype == PA_F16;
    if (head_dim == 64) return f16 ? launch_merge<PA_F16, 64>(a, st) : launch_merge<PA_BF16, 64>(a, st);
    return f16 ? launch_merge<PA_F16, 128>(a, st) : launch_merge<PA_BF16, 128>(a, st);
}

}  // namespace pa
