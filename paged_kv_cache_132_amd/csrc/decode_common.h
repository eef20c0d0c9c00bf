// Device helpers shared by the decode kernels: which tokens of which
// sequences a workgroup attends over, where its partial results go, and how
// the merge finds them again.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pa_internal.h"

namespace pa {

constexpr int kXcds = 8;                          // accelerator complex dies of the chip

// Where the chunks lie: chunk c starts at block floor(c * units / n) of the
// padded batch, so chunks differ in length by at most one block.  (Odd XCDs
// of this part stream about 8 % slower than even ones whichever chunks they
// get, but chunks weighted by XCD did not shorten the kernel.)
struct ChunkLayout {
    int n, units, block_size;
    // first padded token of chunk c (c = 0 .. n)
    __device__ __forceinline__ int start(int c) const {
        return (int)((int64_t)c * units / n) * block_size;
    }
};

// One segment of a workgroup's work: tokens [t0, t1) of sequence s, for the
// KV heads of group `group`.
//
// Fixed partitions (a.partition > 0): a workgroup owns partition p of one
// sequence (one segment).  Token chunks (a.partition == 0): a workgroup owns
// chunk c of the batch's tokens laid end to end, and walks the one or more
// sequences the chunk covers, one segment each.
struct WorkItem {
    int s, p, group;
    int L;          // context length, cut to the table's capacity
    int L_raw;      // context_lens[s] as given
    int n_part;     // fixed partitions: partitions of sequence s (0 for an empty sequence)
    int t0, t1;     // the segment's tokens [t0, t1)
    // token chunks: the chunk, the chunk's padded token range [pos, end),
    // and sequence s's padded offset
    int chunk, pos, end, off;
    int64_t seg_slot;   // partial-result slot of this segment (times num_heads, plus the head)
};

constexpr int kCachedChunks = 8;                  // sequences 0..511 keep their length in registers

// Items a sequence of length L is cut into with item length T; an empty
// sequence still has one item, which writes its zero output.
__device__ __forceinline__ int items_for(int L, int T) { return L > 0 ? (L + T - 1) / T : 1; }

// Tokens a sequence occupies in the chunk layout: its length rounded up to
// whole blocks, so every chunk boundary falls on a block boundary of the
// sequence it cuts; an empty sequence takes one block (its zero output).
__device__ __forceinline__ int padded_len(int L, int block_size) {
    return L > 0 ? (L + block_size - 1) & ~(block_size - 1) : block_size;
}

// x, through an empty asm statement: values computed from the result are
// computed where they are used, not hoisted out of a loop around them.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

// Sum of v over the 64 lanes of the wave, returned in every lane.
__device__ __forceinline__ int wave_total(int v) {
    v += dpp_i<0xB1>(v);      // quad_perm [1,0,3,2]
    v += dpp_i<0x4E>(v);      // quad_perm [2,3,0,1]
    v += dpp_i<0x141>(v);     // row_half_mirror
    v += dpp_i<0x140>(v);     // row_mirror: every lane holds its 16-lane row's sum
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Whether the batch shares prefix blocks between neighbouring sequences, as
// prefix caching and parallel sampling produce: some probe pair of
// neighbours (four pairs spread over the batch) maps its first logical block
// to the same physical block.  Lanes 0..3 load one pair each, all at once;
// every wave gets the same answer.
__device__ inline bool batch_shares_prefix(const DecodeArgs& a) {
    const int B = a.num_seqs;
    if (B < 2) return false;
    const int lane = threadIdx.x & 63;
    bool pair = false;
    if (lane < 4) {
        const int s = lane * (B - 2) / 3;                  // 0 .. B - 2
        const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
        const int l0 = a.context_lens[s], l1 = a.context_lens[s + 1];
        const int b0 = bt[0], b1 = bt[a.max_blocks_per_seq];
        pair = l0 > 0 && l1 > 0 && b0 == b1;
    }
    return __builtin_amdgcn_ballot_w64(pair) != 0;
}

// Whether run k (sequences R*k .. R*k + R - 1, R = a.share_run) shares
// partition p: every sequence of the run holds the partition whole with at
// least one token after it (so neither the newest token nor a ragged tail
// falls into it) and maps each of its blocks to the run leader's physical
// block.  Each wave computes it on its own from the tables; all waves agree.
__device__ inline bool run_shares_partition(const DecodeArgs& a, int k, int p) {
    const int R = a.share_run;
    const int s0 = k * R;
    if (R < 2 || s0 + R > a.num_seqs) return false;
    const int shift = a.block_shift;
    const int max_tokens = a.max_blocks_per_seq << shift;
    const int t1 = (p + 1) * a.partition;          // end of partition p
    if (t1 >= max_tokens) return false;            // no token can follow it in any table
    const int lane = threadIdx.x & 63;
    bool ok = true;
    if (lane < R) ok = a.context_lens[s0 + lane] > t1;
    const int b0 = (p * a.partition) >> shift;
    const int nb = a.partition >> shift;
    const int MB = a.max_blocks_per_seq;
    const int32_t* lead = a.block_tables + (int64_t)s0 * MB;
    for (int x = lane; x < (R - 1) * nb; x += 64) {
        const int i = 1 + x / nb, jb = b0 + x % nb;
        ok = ok && lead[(int64_t)i * MB + jb] == lead[jb];
    }
    return __builtin_amdgcn_ballot_w64(!ok) == 0;
}

// Lengths of sequences lane + 64 i, i < kCachedChunks (0 past the batch):
// one load per lane and chunk of 64, all issued together.
__device__ __forceinline__ void load_lengths(const DecodeArgs& a, int (&len_raw)[kCachedChunks]) {
    const int lane = threadIdx.x & 63;
    const int chunks = (a.num_seqs + 63) >> 6;                 // uniform
#pragma unroll
    for (int i = 0; i < kCachedChunks; ++i) {
        const int s = lane + 64 * i;
        len_raw[i] = (i < chunks && s < a.num_seqs) ? a.context_lens[s] : 0;
    }
}

// Value of v held by lane (s & 63) of register (s >> 6), s < 512 and uniform.
// (Each register is read out on its own and the results selected, so that
// the array is never indexed by a variable and stays in registers.)
__device__ __forceinline__ int cached_at(const int (&v)[kCachedChunks], int s) {
    int x = 0;
#pragma unroll
    for (int i = 0; i < kCachedChunks; ++i) {
        const int vi = __builtin_amdgcn_readlane(v[i], s & 63);
        x = (s >> 6) == i ? vi : x;
    }
    return x;
}

// ---------------------------------------------------------------------------
// Token chunks (partition 0, the library's choice).
//
// The sequences' tokens are laid end to end, each sequence padded to whole
// blocks and preceded by a head of seg_head tokens that holds no work
// (`units` blocks in all), and cut at block boundaries into N chunks of
// near-equal length: chunk c holds blocks [c*units/N, (c+1)*units/N).  N is
// the number of workgroup slots the GPU holds at once divided among the
// KV-head groups, so that every workgroup starts in the first dispatch round
// and every compute unit is dealt about the same work -- a compute unit
// streams at about a fixed rate, so it is the work per unit, not per
// workgroup, that decides when the last one finishes.  The heads make that
// work more than tokens: each sequence a workgroup starts costs it the round
// trips of a fresh start (length, query, table, first K/V), so a chunk with
// many short sequences takes fewer tokens.  Chunks are not shorter than
// part_min tokens, so small batches take fewer of them.  A chunk covers the
// end of one sequence, whole sequences, and the start of another, each a
// segment; a segment that is not its sequence's whole range leaves a partial
// result for the merge, in slot 2c (the chunk's first segment) or 2c + 1
// (its last), which no other segment of the chunk can need.

// Segment of sequence w.s (layout offset w.off, its tokens from seg_head on)
// that chunk [pos, end) holds: tokens [t0, t1); false when it holds none.
// An empty sequence counts its one padded block.
__device__ __forceinline__ bool chunk_segment(const DecodeArgs& a, WorkItem& w) {
    const int r0 = w.off + a.seg_head;
    w.t0 = max(w.pos - r0, 0);
    w.t1 = min(w.L, w.end - r0);
    return r0 < w.end && r0 + max(w.L, 1) > w.pos;
}

// On to the sequence after w.s, if its layout starts inside the chunk.
__device__ __forceinline__ bool next_chunk_sequence(const DecodeArgs& a, WorkItem& w) {
    w.off += a.seg_head + padded_len(w.L, a.block_size);
    ++w.s;
    if (w.off >= w.end || w.s >= a.num_seqs) return false;
    w.L_raw = a.context_lens[w.s];
    w.L = min(w.L_raw, a.max_blocks_per_seq << a.block_shift);
    return true;
}

__device__ inline bool begin_chunk_work(const DecodeArgs& a, int wg, WorkItem& w) {
    const int lane = threadIdx.x & 63;
    const int B = a.num_seqs;
    const int U = a.block_size;
    const int E = a.seg_head;
    const int max_tokens = a.max_blocks_per_seq << a.block_shift;
    int len_raw[kCachedChunks], padded[kCachedChunks];
    load_lengths(a, len_raw);
#pragma unroll
    for (int i = 0; i < kCachedChunks; ++i)
        padded[i] = lane + 64 * i < B ? E + padded_len(min(len_raw[i], max_tokens), U) : 0;
    // layout tokens of sequences [0, s): every wave computes the same sums
    auto offset_of = [&](int s) {
        int acc = 0;
#pragma unroll
        for (int i = 0; i < kCachedChunks; ++i) acc += lane + 64 * i < s ? padded[i] : 0;
        for (int x = lane + 64 * kCachedChunks; x < s; x += 64)
            acc += E + padded_len(min(a.context_lens[x], max_tokens), U);
        return wave_total(acc);
    };
    const int total = offset_of(B);
    const int units = total / U;
    const int slots = max(a.target_items / a.groups, 1);
    const int n = max(1, min(min(min(slots, (total + a.part_min - 1) / a.part_min), units), a.max_chunks));
    const int items = n * a.groups;
    if (wg >= items) return false;
    // The hardware deals workgroup ids round-robin to the XCDs (id % kXcds);
    // renumber so that each XCD takes a contiguous run of chunks: the
    // KV-head groups of one chunk, and neighbouring sequences (which may
    // share prefix blocks), then share that XCD's L2.
    const int x = wg % kXcds, j = wg / kXcds;
    const int per = items / kXcds, rem = items % kXcds;
    const int item = x * per + min(x, rem) + j;
    w.chunk = item / a.groups;
    w.group = item % a.groups;
    const ChunkLayout layout{n, units, U};
    w.pos = layout.start(w.chunk);
    w.end = layout.start(w.chunk + 1);
    // the sequence holding the chunk's first token: the last s with
    // offset(s) <= pos (offsets grow strictly: every sequence takes a block)
    int lo = 0, hi = B;                                           // offset(lo) <= pos < offset(hi)
    int off_lo = 0;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        const int off_mid = offset_of(mid);
        if (off_mid <= w.pos) { lo = mid; off_lo = off_mid; }
        else hi = mid;
    }
    w.s = lo;
    w.off = off_lo;
    w.L_raw = lo < 64 * kCachedChunks ? cached_at(len_raw, lo) : a.context_lens[lo];
    w.L = min(w.L_raw, max_tokens);
    w.p = 0;
    w.n_part = 0;
    w.seg_slot = 2 * (int64_t)w.chunk;
    // the chunk's first segment: that sequence's, unless the chunk starts
    // past its tokens (in its last block's padding) or in the head of the next
    while (!chunk_segment(a, w))
        if (!next_chunk_sequence(a, w)) return false;
    return true;
}

// The next sequence of the chunk, if the chunk holds some of its tokens.
// Its length is loaded here, together with whatever the segment loads next.
__device__ inline bool next_chunk_segment(const DecodeArgs& a, WorkItem& w) {
    if (!next_chunk_sequence(a, w)) return false;
    w.seg_slot = 2 * (int64_t)w.chunk + 1;
    return chunk_segment(a, w);
}

// ---------------------------------------------------------------------------
// Fixed partitions.
//
// Items are (sequence s, partition p < items(s), KV-head group) with
// items(s) = max(n_part(s), 1) (an empty sequence has one item, which writes
// its zero output).  They are ordered by partition first: every sequence's
// partition p runs at about the same time as the others', and no workgroup
// slot is spent on a partition past a sequence's end.  Within partition p:
//   - no shared prefixes: group fastest, then sequence, so one sequence's
//     KV-head groups (whole token rows) are read together;
//   - shared prefixes: sequence fastest, then group, so the workgroups of
//     the sequences that share a block start together and read it once into
//     L2 (13B shared-prefix batch: 549 -> 470 us; the order costs the
//     unshared 7B batch 1.5 %, hence the probe).
// The grid is sized for every sequence at full table length; its surplus is
// a run of workgroups at the end that leave at once.
//
// Items before partition p:  C(p) * groups, C(p) = sum_s min(items(s), p)
// (monotone in p).  The item's partition is the largest p with
// C(p) <= item / groups (binary search); n_p = C(p + 1) - C(p) sequences have
// a partition p, and the item's sequence is one of them, in order.
// Each wave computes this on its own -- no LDS, no barriers -- so waves of a
// workgroup may call it independently; they all reach the same answer.
//
// With partition 0 this is the layout of batches that share prefix blocks:
// there the sharers of a block must read it at about the same time, and
// fixed partitions restart them together at every partition.
__device__ __forceinline__ int fixed_partition(const DecodeArgs& a) {
    return a.partition > 0 ? a.partition : a.fallback_partition;
}

__device__ inline bool begin_partition_work(const DecodeArgs& a, int wg, WorkItem& w, bool shares) {
    constexpr int kCached = kCachedChunks;
    const int lane = threadIdx.x & 63;
    const int B = a.num_seqs;
    const int P = a.max_partitions;
    const int T = fixed_partition(a);
    const int max_tokens = a.max_blocks_per_seq << a.block_shift;
    int len_raw[kCached];
    load_lengths(a, len_raw);
    int cached[kCached];
#pragma unroll
    for (int i = 0; i < kCached; ++i) cached[i] = lane + 64 * i < B ? items_for(min(len_raw[i], max_tokens), T) : 0;
    auto items_of = [&](int s) { return items_for(min(a.context_lens[s], max_tokens), T); };
    auto C = [&](int p) {
        int acc = 0;
#pragma unroll
        for (int i = 0; i < kCached; ++i) acc += min(cached[i], p);
        for (int s = lane + 64 * kCached; s < B; s += 64) acc += min(items_of(s), p);
        return wave_total(acc);
    };
    // Live items are workgroups 0 .. total-1, renumbered per XCD as in the
    // chunk layout
    const int total = C(P) * a.groups;
    if (wg >= total) return false;                // past the last item
    const int x = wg % kXcds, j = wg / kXcds;
    const int per = total / kXcds, rem = total % kXcds;
    // (with shared runs the per-sequence kernel skips the runs' shared
    // partitions, a contiguous range of items: dealt round-robin, the live
    // items still reach every XCD)
    const int item = a.share_run > 1 ? wg : x * per + min(x, rem) + j;
    const int k = item / a.groups;                // item index ignoring the group
    int lo = 0, hi = P;                           // C(lo) <= k < C(hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (C(mid) <= k) lo = mid;
        else hi = mid;
    }
    const int p = lo;
    const int c_p = C(p);
    int rank, group;                              // rank: among sequences with items(s) > p, ascending s
    if (shares) {
        const int n_p = C(p + 1) - c_p;           // >= 1: the item lies in partition p
        const int local = item - c_p * a.groups;
        group = local / n_p;
        rank = local - group * n_p;
    } else {
        group = item % a.groups;
        rank = k - c_p;
    }
    // the rank-th sequence (ascending) with more than p items: count them 64
    // at a time (registers first, then loads past 512)
    int s_found = -1;
    auto pick = [&](int c0, bool has_item) {
        const uint64_t bits = __builtin_amdgcn_ballot_w64(has_item);
        const int cnt = __builtin_popcountll(bits);
        if (s_found < 0 && rank < cnt) {
            // lane whose bit is set with exactly `rank` set bits below it
            const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
            const uint64_t hit = __builtin_amdgcn_ballot_w64(((bits >> lane) & 1ull) && (int)below == rank);
            s_found = c0 + (int)__builtin_ctzll(hit);
        }
        rank -= cnt;
    };
#pragma unroll
    for (int i = 0; i < kCached; ++i)
        if (s_found < 0 && 64 * i < B) pick(64 * i, cached[i] > p);
    for (int c0 = 64 * kCached; s_found < 0 && c0 < B; c0 += 64) pick(c0, c0 + lane < B && items_of(c0 + lane) > p);
    if (s_found < 0) return false;
    w.s = s_found;
    w.p = p;
    w.group = group;
    w.L_raw = s_found < 64 * kCached ? cached_at(len_raw, s_found) : a.context_lens[s_found];
    w.L = min(w.L_raw, max_tokens);
    w.n_part = w.L > 0 ? (w.L + T - 1) / T : 0;
    w.t0 = p * T;
    w.t1 = min(w.L, w.t0 + T);
    w.chunk = -1;
    w.seg_slot = (int64_t)s_found * P + p;
    // a partition a shared run holds is the run kernel's
    if (a.share_run > 1 && run_shares_partition(a, s_found / a.share_run, p)) return false;
    return true;
}

// Whether a launch with partition 0 lays out token chunks: unless the batch
// shares prefix blocks (then fixed partitions of fallback_partition tokens).
__device__ __forceinline__ bool uses_chunks(const DecodeArgs& a, bool shares) {
    return a.partition == 0 && !shares;
}

// The first segment of workgroup `wg` of a per-sequence decode kernel.  (The
// grid covers both layouts; workgroups past the chosen one's items leave.)
__device__ __forceinline__ bool begin_work(const DecodeArgs& a, int wg, WorkItem& w) {
    const bool shares = batch_shares_prefix(a);                   // its loads go out with the lengths'
    return uses_chunks(a, shares) ? begin_chunk_work(a, wg, w) : begin_partition_work(a, wg, w, shares);
}

// Advance to the workgroup's next segment; false when it has none.
__device__ __forceinline__ bool next_segment(const DecodeArgs& a, WorkItem& w) {
    return w.chunk >= 0 ? next_chunk_segment(a, w) : false;
}

// Whether the segment is its sequence's whole range (the output is written
// directly, no partial).
__device__ __forceinline__ bool whole_sequence(const WorkItem& w) { return w.t0 == 0 && w.t1 >= w.L; }

// Token chunks: where each sequence's partials lie, for the merge.  The
// workgroup of group 0 that holds a sequence's first token records that
// chunk and the slot its segment took there (0: it starts the chunk); the
// one that holds its last token records that chunk.  Thread 0, once per
// sequence and call.
__device__ __forceinline__ void publish_segments(const DecodeArgs& a, const WorkItem& w) {
    if (w.chunk < 0 || w.group != 0 || threadIdx.x != 0) return;
    int32_t* h = a.part_n + 4 * (int64_t)w.s;
    if (w.t0 == 0) {
        h[1] = w.chunk;
        h[2] = (int)(w.seg_slot - 2 * (int64_t)w.chunk);
    }
    if (w.t1 >= w.L) h[0] = w.chunk;
}

// Partials of sequence s for the merge: their count (0 or 1: no merge), and
// slot(i) of the i-th, in token order.
struct MergeList {
    int n;
    int64_t base;       // fixed partitions: s * P; token chunks: 2 * first chunk + its slot
    bool chunked;
    __device__ __forceinline__ int64_t slot(int i) const {
        return chunked ? (i == 0 ? base : (base & ~1ll) + 2 * (int64_t)i) : base + i;
    }
};

__device__ __forceinline__ MergeList merge_list(const DecodeArgs& a, int s) {
    MergeList m;
    m.chunked = uses_chunks(a, batch_shares_prefix(a));
    // the length and (token chunks) the record of the attention pass, loaded together
    const int L = min(a.context_lens[s], a.max_blocks_per_seq << a.block_shift);
    int4 rec = make_int4(0, 0, 0, 0);
    if (m.chunked) rec = *reinterpret_cast<const int4*>(a.part_n + 4 * (int64_t)s);
    if (L <= 0) {
        m.n = 0;
        m.base = 0;
    } else if (!m.chunked) {
        const int T = fixed_partition(a);
        m.n = (L + T - 1) / T;
        m.base = (int64_t)s * a.max_partitions;
    } else {
        // as the attention pass recorded it (first chunk, slot there, last
        // chunk), kept within the workspace
        const int first = min(max(rec.y, 0), a.max_chunks - 1);
        const int last = min(max(rec.x, first), a.max_chunks - 1);
        m.n = last - first + 1;
        m.base = 2 * (int64_t)first + (rec.z & 1);
    }
    return m;
}

// Map workgroup `wg` of the run kernel to (run k, KV-head group, partition p):
// group fastest, then run, then partition.  False when that partition is not
// shared by the run (the per-sequence kernel computes it) or past the grid.
__device__ inline bool find_run_work(const DecodeArgs& a, int wg, WorkItem& w) {
    const int runs = a.num_seqs / a.share_run;
    const int group = wg % a.groups;
    const int k = (wg / a.groups) % runs;
    const int p = wg / (a.groups * runs);
    if (p >= a.max_partitions || !run_shares_partition(a, k, p)) return false;
    w.s = k * a.share_run;
    w.p = p;
    w.group = group;
    w.L_raw = a.context_lens[w.s];
    w.L = min(w.L_raw, a.max_blocks_per_seq << a.block_shift);
    w.n_part = (w.L + a.partition - 1) / a.partition;
    w.t0 = p * a.partition;
    w.t1 = min(w.L, w.t0 + a.partition);
    w.chunk = -1;
    w.seg_slot = (int64_t)w.s * a.max_partitions + p;    // run member i: (s + i) * max_partitions + p
    return true;
}

}  // namespace pa
