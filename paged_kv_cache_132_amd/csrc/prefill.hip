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
//   32w .. 32w+31 of the tile as one 32-row block of 32x32x16 MFMAs.  Tiles
//   are dispatched last tile first: the latest queries see the most keys.
//   The sequence's block table is staged in LDS once (tables of up to 2048
//   blocks).
//
// Per 32-key tile (lane l: n = l % 32, h = l / 32):
//   load  the 256 threads read the tile's K and V rows through the block
//         table (16 bytes each) and store them row-major into LDS (fp8
//         widened to bf16 exactly): two K buffers and three V buffers.
//   S^T = K Q^T on v_mfma_f32_32x32x16_{f16,bf16}: A = K rows (lane: key n,
//         head_dim 8h..8h+7 of each 16-wide step), B = the queries (lane:
//         row n, the same head_dim positions, held in registers).  Lane
//         (n, h) gets the scores of row n for keys 8(r/4) + 4h + r%4,
//         r = 0..15.
//   soft  online softmax in the exp2 domain on the unscaled scores (the
//         scale enters through the exponent's FMA): masked keys (after the
//         row's position; only the last tiles of a wave take the mask) get
//         weight 0; probabilities are rounded to the MFMA input type once,
//         and the running sum adds exactly those rounded values (dot2 with
//         ones; lanes n and n + 32 each sum half of the row's keys).
//         With bf16 K/V the probability is split into a bf16 part and a bf16
//         remainder and PV runs on both: one bf16 rounding (2^-9 relative)
//         of a peaked softmax would otherwise move an output by up to
//         2^-9 x the spread of the V values it weights.
//   PV    A = P, the lane's own probabilities (registers 8k..8k+7 for key
//         step k); B = V read from its row-major LDS copy with
//         ds_read_tr16_b64 (two reads give a lane the 8 keys of one head_dim
//         column in that k-slot order); head_dim/32 MFMAs per key step
//         accumulate O[row][d] in fp32.
//   The steps are software-pipelined: iteration kt issues the QK MFMAs of
//   tile kt + 1 next to the softmax of tile kt, then the PV of tile kt, then
//   stores tile kt + 2 into LDS and issues the loads of tile kt + 3; one
//   barrier per tile.
//
// With the write fused (16-bit KV), new tokens' K and V are read from the
// source rows, and the workgroup that owns a new token (its query rows)
// stores the token's K and V into its slot from the tile registers of its own
// main loop; no workgroup reads a slot another one writes.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;           // 4 waves
constexpr int kRows = 4 * 32;           // (token, head) rows per workgroup: 32 per wave
constexpr int kKeys = 32;               // keys per tile
constexpr int kKBufs = 2;               // K tiles in LDS
constexpr int kVBufs = 3;               // V tiles in LDS: V of tile kt is read one iteration after K
constexpr int kMaxBt = 2048;            // block-table entries staged in LDS (longer tables are read in place)
constexpr float kSlack = 8.f;           // a row's weights stay below 2^8 between rescales

template <bool B>
struct MaskTag {   // selects the per-tile code with or without the causal mask
    static constexpr bool value = B;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// the values of x in this lane and in lane l ^ 32, in some order
__device__ __forceinline__ f32x2 with_other_half(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return f32x2{__uint_as_float(a[0]), __uint_as_float(a[1])};
}

__device__ __forceinline__ float from_lane(float x, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

// wave-wide sum and max of an int, returned as a uniform value (DPP within
// rows of 16 lanes, then lane swaps across rows and halves)
template <typename Op>
__device__ __forceinline__ int wave_reduce(int x, Op op) {
    x = op(x, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
    x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
    x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false));   // row_ror:4
    x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));   // row_ror:8
    const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = op((int)a[0], (int)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return __builtin_amdgcn_readfirstlane(op((int)b[0], (int)b[1]));
}
__device__ __forceinline__ int wave_sum(int x) {
    return wave_reduce(x, [](int u, int v) { return u + v; });
}
__device__ __forceinline__ int wave_max(int x) {
    return wave_reduce(x, [](int u, int v) { return max(u, v); });
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
    static __device__ __forceinline__ f32x16 run(Vec a, Vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t round(float x) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
    // two values rounded (RNE) into one packed word, and back
    static __device__ __forceinline__ uint32_t round2(float x, float y) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
    }
    static __device__ __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
    static __device__ __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }
    // acc + both values of a packed word, in fp32
    static __device__ __forceinline__ float add2(uint32_t w, float acc) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), f16x2{(_Float16)1.f, (_Float16)1.f}, acc, false);
    }
};

template <>
struct Mma<PA_BF16> {
    typedef bf16x8 Vec;
    static __device__ __forceinline__ f32x16 run(Vec a, Vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t round(float x) { return bf16_rne(x); }
    static __device__ __forceinline__ uint32_t round2(float x, float y) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
    }
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
    static __device__ __forceinline__ float add2(uint32_t w, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                               acc, false);
    }
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

// ---- the order of the work -----------------------------------------------------
// A job is (sequence, tile of kRows query rows); its work is the number of
// 32-key tiles its latest query reads.  Workgroups take the jobs in
// decreasing order of work (longest first), so that the longest ones start
// at once and the short ones fill the end of the launch: workgroup b runs job
// b / Hkv for KV head b % Hkv.  Jobs of equal work go by sequence, then
// latest tile first.
struct SeqShape {
    int first, n, off, T;   // first packed row, new tokens, cached prefix L - n, row tiles (0: no work)
};

template <int G>
__device__ __forceinline__ SeqShape seq_shape(const PrefillArgs& a, int s) {
    if (s >= a.num_seqs) return {0, 0, 0, 0};
    const int first = a.cu_seqlens[s];
    const int n = a.cu_seqlens[s + 1] - first;
    const int L = min(a.context_lens[s], a.max_blocks_per_seq << a.block_shift);
    // nothing new, an impossible run, or more new tokens than the launch was sized for
    if (n <= 0 || n > L || n > a.max_new_tokens || first < 0 || first + n > a.num_tokens) return {0, 0, 0, 0};
    return {first, n, L - n, (n * G + kRows - 1) / kRows};
}

// Tiles of a sequence whose work is at least w.  Tile t's latest query is
// token min(kRows (t + 1), n G) / G - 1 (rows are token-major), at position
// off + that token, and its work is position / kKeys + 1; the work grows
// with t, so the tiles that reach w are the last ones, from
// t = floor(A G / kRows) on, where A = kKeys (w - 1) - off is the token the
// latest query must reach.
template <int G>
__device__ __forceinline__ int tiles_with_work(const SeqShape& q, int w) {
    const int A = kKeys * (w - 1) - q.off;
    if (A <= 0) return q.T;
    if (A >= q.n) return 0;
    return q.T - (A * G) / kRows;
}

// Inclusive prefix sum over the lanes of the wave (DPP shifts within rows
// of 16, then row broadcasts).
__device__ __forceinline__ int wave_prefix_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);    // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);    // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);    // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);    // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2 and 3
    return x;
}

// Job j in that order, as (sequence, its shape, tile); false past the last
// job.  Every lane of the wave takes part; the results are uniform.  The
// lanes search in parallel: each counts the jobs of work >= its own
// candidate w (up to 64 candidates per pass, narrowing the range 64-fold),
// then the rank among equal work comes from a prefix sum over sequences.
template <int G>
__device__ bool find_job(const PrefillArgs& a, int j, int& seq, SeqShape& job, int& tile) {
    const int lane = threadIdx.x & 63;
    const int S = a.num_seqs;
    const SeqShape q0 = seq_shape<G>(a, lane);           // lane l: sequence l (the rest are read when needed)
    int w_top = q0.T ? (q0.off + q0.n - 1) / kKeys + 1 : 0;   // the work of a sequence's last tile
    for (int s = lane + 64; s < S; s += 64) {
        const SeqShape q = seq_shape<G>(a, s);
        w_top = max(w_top, q.T ? (q.off + q.n - 1) / kKeys + 1 : 0);
    }
    // jobs of work >= w, for this lane's w, over all sequences
    auto count = [&](int w) {
        int c = 0;
        for (int s = 0; s < min(S, 64); ++s) {
            const SeqShape q = {0, __builtin_amdgcn_readlane(q0.n, s), __builtin_amdgcn_readlane(q0.off, s),
                                __builtin_amdgcn_readlane(q0.T, s)};
            c += tiles_with_work<G>(q, w);
        }
        for (int s = 64; s < S; ++s) c += tiles_with_work<G>(seq_shape<G>(a, s), w);
        return c;
    };
    // the job's work: the largest w with count(w) > j; count(lo) > j >= count(hi) = c_hi
    int lo = 1, hi = wave_max(w_top) + 1, c_hi = 0;
    for (bool first = true; first || hi - lo > 1; first = false) {
        const int step = (hi - lo + 63) / 64;
        const int w = lo + lane * step;
        const int c = count(w);
        if (first && j >= __builtin_amdgcn_readlane(c, 0)) return false;   // count(1): all the jobs
        const uint64_t above = __builtin_amdgcn_ballot_w64(w < hi && c > j);   // lane 0 at least
        const int k = 63 - __builtin_clzll(above);
        if (k < 63 && lo + (k + 1) * step < hi) c_hi = __builtin_amdgcn_readlane(c, k + 1);
        hi = min(lo + (k + 1) * step, hi);
        lo += k * step;
    }
    // rank r among the jobs of work exactly lo, which go by sequence, then
    // latest tile first: sequence s has tiles T - ge .. T - gt - 1 of it
    int r = j - c_hi;
    for (int base = 0; base < S; base += 64) {
        const SeqShape q = base == 0 ? q0 : seq_shape<G>(a, base + lane);
        const int ge = tiles_with_work<G>(q, lo), gt = tiles_with_work<G>(q, lo + 1);
        const int upto = wave_prefix_sum(ge - gt);       // jobs of work lo in sequences base .. base + lane
        const uint64_t past = __builtin_amdgcn_ballot_w64(upto > r && base + lane < S);
        if (past) {
            const int l = __builtin_ctzll(past);
            seq = base + l;
            job = {__builtin_amdgcn_readlane(q.first, l), __builtin_amdgcn_readlane(q.n, l),
                   __builtin_amdgcn_readlane(q.off, l), __builtin_amdgcn_readlane(q.T, l)};
            const int before = __builtin_amdgcn_readlane(upto - (ge - gt), l);
            tile = __builtin_amdgcn_readlane(q.T - gt, l) - 1 - (r - before);
            return tile >= 0 && tile < job.T;            // (always, when the search is right)
        }
        r -= __builtin_amdgcn_readlane(upto, 63);
    }
    return false;   // not reached: r < the number of jobs of work lo
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
    constexpr int KSTEPS = D / 16;                      // QK: 16 of head_dim per MFMA
    constexpr int DB = D / 32;                          // PV: 32-column blocks of O
    constexpr bool SPLIT = QT == PA_BF16 && KVT == PA_BF16;   // P = bf16 part + bf16 remainder
    static_assert(!WRITE || KVT != PA_FP8_E4M3, "the fused write moves 16-bit rows unchanged");

    // K buffers, then V buffers, in one region: the epilogue stages the
    // output rows there
    constexpr int kKvElems = kKBufs * kKeys * KS + kVBufs * kKeys * VS;
    constexpr int OS = D + 8;                           // epilogue row stride (elements)
    static_assert(4 * 32 * OS <= kKvElems, "the output tile fits in the K/V buffers");
    __shared__ __attribute__((aligned(16))) uint16_t s_kv[kKvElems];
    uint16_t (*s_k)[kKeys * KS] = reinterpret_cast<uint16_t (*)[kKeys * KS]>(s_kv);
    uint16_t (*s_v)[kKeys * VS] = reinterpret_cast<uint16_t (*)[kKeys * VS]>(s_kv + kKBufs * kKeys * KS);
    __shared__ int32_t s_bt[BT_LDS ? kMaxBt : 1];

    // ---- work item: job blockIdx / Hkv in decreasing order of work ---------
    const int Hkv = a.num_kv_heads;
    const int g = blockIdx.x % Hkv;
    SeqShape job;
    int s, tile;
    if (!find_job<G>(a, blockIdx.x / Hkv, s, job, tile)) return;
    const int first = job.first;
    const int n = job.n;
    const int L = job.off + n;
    const int rows = n * G;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 31;                           // row (S, P), key (K operand) or column (V, O)
    const int h = lane >> 5;
    const int Hq = a.num_heads;
    const int row0 = tile * kRows + wave * 32;          // this wave's first row

    // this lane's row (B-operand column ln of S^T).  Scores are kept
    // unscaled and the (positive) scale enters in the exponent's FMA; a
    // negative scale is moved onto the queries as an exact sign flip.
    Vec qop[KSTEPS];
    const uint32_t qsign = a.score_scale < 0.f ? 0x80008000u : 0u;
    // (a zero scale is raised to the least normal float, so that a masked
    // score, -inf, still scales to -inf and not to NaN)
    const float sscale = fmaxf(fabsf(a.score_scale), 1.17549435e-38f);
    const int r_own = min(row0 + ln, rows - 1);
    const int pos = L - n + r_own / G;                  // the row's query position
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.query) +
                             ((int64_t)(first + r_own / G) * Hq + g * G + r_own % G) * D + 8 * h;
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k) {
            uint4 w = *reinterpret_cast<const uint4*>(qp + 16 * k);
            w.x ^= qsign;
            w.y ^= qsign;
            w.z ^= qsign;
            w.w ^= qsign;
            qop[k] = __builtin_bit_cast(Vec, w);
        }
    }
    const int pos_first = L - n + row0 / G;              // the wave's earliest query
    // the wave's last tile with a key its latest query sees (the workgroup's
    // later waves may need up to kRows / kKeys - 1 tiles more)
    const int kt_last = __builtin_amdgcn_readfirstlane((L - n + min(row0 + 31, rows - 1) / G) / kKeys);
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
    // The loads are branch-free and clamped to the sequence: where the tile
    // has fewer chunks than threads, the spare threads re-read chunk 0 and
    // store nothing; tiles past the last one (the pipeline runs up to three
    // tiles ahead) re-read the last key and their LDS copies are never used.
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
    auto store_chunk = [&](int kt, int kbuf, int vbuf, int ci, uint4 kc, uint4 vc) {
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
            *reinterpret_cast<uint4*>(&s_k[kbuf][key * KS + d0]) = klo;
            *reinterpret_cast<uint4*>(&s_k[kbuf][key * KS + d0 + 8]) = khi;
            *reinterpret_cast<uint4*>(&s_v[vbuf][key * VS + d0]) = vlo;
            *reinterpret_cast<uint4*>(&s_v[vbuf][key * VS + d0 + 8]) = vhi;
        } else {
            *reinterpret_cast<uint4*>(&s_k[kbuf][key * KS + d0]) = kc;
            *reinterpret_cast<uint4*>(&s_v[vbuf][key * VS + d0]) = vc;
        }
    };
    auto store_tile = [&](int kt, int kbuf, int vbuf, const Tile& tl) {
        store_chunk(kt, kbuf, vbuf, tid, tl.k0, tl.v0);
        if constexpr (U > 1) store_chunk(kt, kbuf, vbuf, tid + kThreads, tl.k1, tl.v1);
    };

    // ---- per-tile math -------------------------------------------------------------
    // m_run: running reference max of row ln (scaled; the same in lanes ln
    // and ln + 32); l_part: this lane's half of the row's weight sum; o: the
    // C layout of O (lane (column ln, h), register r: row 8(r/4) + 4h + r%4)
    float m_run = -INFINITY, l_part = 0.f;
    f32x16 oacc[DB];
#pragma unroll
    for (int t = 0; t < DB; ++t) oacc[t] = f32x16{};

    // this lane's element of a V buffer for the transposed reads (see below)
    const int v_lane = (4 * h + ((lane & 15) >> 2)) * VS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // S^T = K Q^T of the tile in K buffer kbuf
    auto qk = [&](int kbuf) {
        const uint16_t* sk = &s_k[kbuf][ln * KS + 8 * h];
        f32x16 acc = {};
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k)
            acc = M::run(__builtin_bit_cast(Vec, *reinterpret_cast<const uint4*>(sk + 16 * k)), qop[k], acc);
        return acc;
    };

    // online softmax of tile kt's scores (lane: keys 8(r/4) + 4h + r%4 of
    // row ln), the rescale of o, then O += P V from V buffer vbuf.  Only
    // tiles that reach past the wave's earliest query take the mask.
    auto softmax_pv = [&](int kt, int vbuf, f32x16 sc, auto mask_tag) {
        constexpr bool kMasked = decltype(mask_tag)::value;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (kMasked) {
                const int key = kt * kKeys + 8 * (r >> 2) + 4 * h + (r & 3);
                sc[r] = key <= pos ? sc[r] : -INFINITY;
            }
            mx = fmaxf(mx, sc[r]);
        }
        const f32x2 mm = with_other_half(mx);
        mx = fmaxf(mm[0], mm[1]) * sscale;
        // The reference max moves only when a row's max grows by more than
        // kSlack (log2 units): the weights stay below 2^kSlack and most
        // tiles need no rescale of o at all.
        const bool grow = mx > m_run + kSlack;          // always on the first tile (m_run = -inf)
        const float m_new = grow ? mx : m_run;          // finite: key 0 precedes every query
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
        uint32_t pw[8], plw[8];                         // packed probabilities (register pairs)
        float lsum = l_part * alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p0 = fast_exp2(fmaf(sc[2 * e], sscale, -m_new));       // masked: 2^-inf = 0
            const float p1 = fast_exp2(fmaf(sc[2 * e + 1], sscale, -m_new));
            pw[e] = M::round2(p0, p1);
            lsum = M::add2(pw[e], lsum);
            if constexpr (SPLIT) {
                plw[e] = M::round2(p0 - M::lo(pw[e]), p1 - M::hi(pw[e]));    // the differences are exact in fp32
                lsum = M::add2(plw[e], lsum);
            }
        }
        l_part = lsum;
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float ar = from_lane(alpha, 8 * (r >> 2) + 4 * h + (r & 3));
#pragma unroll
                for (int t = 0; t < DB; ++t) oacc[t][r] *= ar;
            }
        }
        // B operand: lane (column ln, h) needs V[key][32t + ln] for the keys
        // of its k-slots, 16k + 4h + j and 16k + 8 + 4h + j (j < 4).
        // ds_read_tr16_b64 gives lane i of a 16-lane group element (i % 4)
        // of the 8 bytes addressed by lane 4j + (i % 16) / 4 as its element
        // j, so lane 4j + m of the group addresses V[k0 + j][c0 + 4m].
        const uint16_t* sv = &s_v[0][0] + __builtin_amdgcn_readfirstlane(vbuf * (kKeys * VS)) + v_lane;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const Vec pop = __builtin_bit_cast(Vec, make_uint4(pw[4 * k], pw[4 * k + 1], pw[4 * k + 2], pw[4 * k + 3]));
            Vec pop_lo;
            if constexpr (SPLIT)
                pop_lo = __builtin_bit_cast(Vec, make_uint4(plw[4 * k], plw[4 * k + 1], plw[4 * k + 2], plw[4 * k + 3]));
#pragma unroll
            for (int t = 0; t < DB; ++t) {
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16*)(sv + (16 * k) * VS + 32 * t));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16*)(sv + (16 * k + 8) * VS + 32 * t));
                const Vec vf = __builtin_bit_cast(Vec, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
                oacc[t] = M::run(pop, vf, oacc[t]);
                if constexpr (SPLIT) oacc[t] = M::run(pop_lo, vf, oacc[t]);
            }
        }
    };

    // ---- main loop ------------------------------------------------------------------
    // Before iteration kt: the scores of tile kt are in registers, K of tile
    // kt + 1 and V of tiles kt and kt + 1 are in LDS, the loads of tile kt + 2
    // are in flight.  Iteration kt stores tile kt + 2 (K into the buffer K of
    // tile kt left, V into the one V of tile kt - 1 left), issues the loads of
    // tile kt + 3, computes the scores of tile kt + 1 beside the softmax of
    // tile kt, then the PV of tile kt; the barrier at its end makes tile
    // kt + 2 visible and frees the buffers of tile kt.  (The second barrier
    // of the prologue keeps the store of tile 2 in iteration 0 after every
    // wave's reads of K of tile 0.)
    Tile tl = load_tile(0);
    {
        const Tile t1 = load_tile(1);
        store_tile(0, 0, 0, tl);
        store_tile(1, 1, 1, t1);
    }
    tl = load_tile(2);
    __syncthreads();
    f32x16 s0 = qk(0), s1;
    __syncthreads();
    auto step = [&](int kt, const f32x16& cur, f32x16& next, auto mask_tag) {
        store_tile(kt + 2, kt & 1, (kt + 2) % kVBufs, tl);
        tl = load_tile(kt + 3);
        // (tiles past the wave's last visible key only move data for the
        // other waves; the scores of the tile after the wave's last one, or
        // after the workgroup's last one, are computed and not used)
        if (!decltype(mask_tag)::value || kt <= kt_last) {
            next = qk((kt + 1) & 1);
            softmax_pv(kt, kt % kVBufs, cur, mask_tag);
        }
        __syncthreads();
    };
    // Tiles below the wave's earliest query need no mask: they run in a loop
    // of their own, the rest (at most kRows / kKeys + 1) in a second one.
    // Both are unrolled by two, so that the score registers of even and odd
    // tiles keep their roles without copies.
    const int n_plain = min((pos_first + 1) / kKeys, n_tiles);   // tiles with kt * kKeys + kKeys - 1 <= pos_first
    int kt = 0;
    for (; kt + 1 < n_plain; kt += 2) {
        step(kt, s0, s1, MaskTag<false>{});
        step(kt + 1, s1, s0, MaskTag<false>{});
    }
    if (kt < n_plain) step(kt++, s0, s1, MaskTag<false>{});
    if ((kt & 1) && kt < n_tiles) step(kt++, s1, s0, MaskTag<true>{});
    for (; kt + 1 < n_tiles; kt += 2) {
        step(kt, s0, s1, MaskTag<true>{});
        step(kt + 1, s1, s0, MaskTag<true>{});
    }
    if (kt < n_tiles) step(kt, s0, s1, MaskTag<true>{});

    // ---- finish: row sums, normalise, store ----------------------------------
    // Each wave puts its 32 normalised rows into the (now free) K/V region,
    // row-major, then stores them as 16-byte pieces of whole rows.
    const f32x2 ls = with_other_half(l_part);
    const float l_row = ls[0] + ls[1];                   // the whole row's sum, in lanes ln and ln + 32
    uint16_t* o_lds = s_kv + wave * (32 * OS);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int rr = 8 * (r >> 2) + 4 * h + (r & 3);
        const float inv = a.v_scale / from_lane(l_row, rr);
#pragma unroll
        for (int t = 0; t < DB; ++t) o_lds[rr * OS + 32 * t + ln] = M::round(oacc[t][r] * inv);
    }
    __syncthreads();
    uint16_t* out = static_cast<uint16_t*>(a.out);
    constexpr int PIECES = 32 * D / 8;                   // 16-byte pieces of the wave's rows
#pragma unroll
    for (int i = 0; i < PIECES / 64; ++i) {
        const int c = lane + 64 * i;
        const int rr = c / (D / 8), col = 8 * (c % (D / 8));
        const int R = row0 + rr;
        if (R < rows)
            *reinterpret_cast<uint4*>(out + ((int64_t)(first + R / G) * Hq + g * G + R % G) * D + col) =
                *reinterpret_cast<const uint4*>(o_lds + rr * OS + col);
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

// One workgroup per (job, KV head).  A sequence has at most
// ceil(max_new_tokens G / kRows) jobs, and since the runs are disjoint rows of
// the num_tokens packed ones, all sequences together at most
// (num_tokens G + (kRows - 1) num_seqs) / kRows.
int64_t prefill_grid(int num_seqs, int num_kv_heads, int group_size, int max_new_tokens, int num_tokens) {
    const int64_t per_seq = ((int64_t)max_new_tokens * group_size + kRows - 1) / kRows;
    const int64_t all = ((int64_t)num_tokens * group_size + (int64_t)(kRows - 1) * num_seqs) / kRows;
    return std::min(per_seq * num_seqs, all) * num_kv_heads;
}

int launch_prefill(const PrefillArgs& a, pa_dtype kv_dtype, int head_dim, int group_size, int max_new_tokens,
                   void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t grid = prefill_grid(a.num_seqs, a.num_kv_heads, group_size, max_new_tokens, a.num_tokens);
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
