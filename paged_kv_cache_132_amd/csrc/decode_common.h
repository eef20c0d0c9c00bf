// Device helpers shared by the two decode kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pa_internal.h"

namespace pa {

// One decode work item: partition p of sequence s for KV-head group `group`.
struct WorkItem {
    int s, p, group;
    int L;        // context length, cut to the table's capacity
    int n_part;   // partitions of sequence s (0 for an empty sequence)
};

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
// to the same physical block.  A handful of scalar loads; every wave gets
// the same answer.
__device__ inline bool batch_shares_prefix(const DecodeArgs& a) {
    const int B = a.num_seqs;
    if (B < 2) return false;
    bool shared = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int s = k * (B - 2) / 3;                     // 0 .. B - 2
        if (a.context_lens[s] > 0 && a.context_lens[s + 1] > 0) {
            const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
            shared |= bt[0] == bt[a.max_blocks_per_seq];
        }
    }
    return shared;
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

// Map workgroup `wg` to the wg-th live work item.
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
constexpr int kXcds = 8;                          // accelerator complex dies of the chip

__device__ inline bool find_work(const DecodeArgs& a, int wg, WorkItem& w) {
    constexpr int kCached = 8;                    // sequences 0..511 keep their count in registers
    const int lane = threadIdx.x & 63;
    const int B = a.num_seqs;
    const int P = a.max_partitions;
    const int max_tokens = a.max_blocks_per_seq << a.block_shift;
    auto items_of = [&](int s) {
        const int L = min(a.context_lens[s], max_tokens);
        return L > 0 ? (L + a.partition - 1) / a.partition : 1;
    };
    int cached[kCached];
#pragma unroll
    for (int i = 0; i < kCached; ++i) {
        const int s = lane + 64 * i;
        cached[i] = s < B ? items_of(s) : 0;
    }
    auto items_at = [&](int i, int s) { return i < kCached ? cached[i] : (s < B ? items_of(s) : 0); };
    auto C = [&](int p) {
        int acc = 0;
#pragma unroll
        for (int i = 0; i < kCached; ++i) acc += min(cached[i], p);
        for (int s = lane + 64 * kCached; s < B; s += 64) acc += min(items_of(s), p);
        return wave_total(acc);
    };
    // Live items are workgroups 0 .. total-1.  The hardware deals workgroup
    // ids round-robin to the XCDs (id % kXcds); renumber so that each XCD
    // takes a contiguous run of items: the KV-head groups of one (sequence,
    // partition) and neighbouring sequences then share that XCD's L2.
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
    if (batch_shares_prefix(a)) {
        const int n_p = C(p + 1) - c_p;           // >= 1: the item lies in partition p
        const int local = item - c_p * a.groups;
        group = local / n_p;
        rank = local - group * n_p;
    } else {
        group = item % a.groups;
        rank = k - c_p;
    }
    int s_found = -1;
    for (int c0 = 0, i = 0; c0 < B; c0 += 64, ++i) {
        const int s = c0 + lane;
        const uint64_t bits = __builtin_amdgcn_ballot_w64(s < B && items_at(i, s) > p);
        const int cnt = __builtin_popcountll(bits);
        if (rank < cnt) {
            // lane whose bit is set with exactly `rank` set bits below it
            const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
            const uint64_t hit = __builtin_amdgcn_ballot_w64(((bits >> lane) & 1ull) && (int)below == rank);
            s_found = c0 + (int)__builtin_ctzll(hit);
            break;
        }
        rank -= cnt;
    }
    if (s_found < 0) return false;
    w.s = s_found;
    w.p = p;
    w.group = group;
    w.L = min(a.context_lens[s_found], max_tokens);
    w.n_part = w.L > 0 ? (w.L + a.partition - 1) / a.partition : 0;
    // a partition a shared run holds is the run kernel's
    if (a.share_run > 1 && run_shares_partition(a, s_found / a.share_run, p)) return false;
    return true;
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
    w.L = min(a.context_lens[w.s], a.max_blocks_per_seq << a.block_shift);
    w.n_part = (w.L + a.partition - 1) / a.partition;
    return true;
}

}  // namespace pa
