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

// Block-wide inclusive prefix sum of one int per thread; `total` receives
// the sum over the whole block.  All threads must call it.
__device__ inline int block_scan(int v, int* s_tmp, int& total) {
    const int tid = threadIdx.x;
    s_tmp[tid] = v;
    __syncthreads();
#pragma unroll
    for (int off = 1; off < kDecodeThreads; off <<= 1) {
        const int x = tid >= off ? s_tmp[tid - off] : 0;
        __syncthreads();
        s_tmp[tid] += x;
        __syncthreads();
    }
    const int r = s_tmp[tid];
    total = s_tmp[kDecodeThreads - 1];
    __syncthreads();
    return r;
}

// Partition-major ordering is used while the partition count fits this many
// histogram bins in LDS; beyond it the items are taken sequence by sequence.
constexpr int kMaxPartitionBins = 1024;

// Map workgroup `wg` to the wg-th live work item.
//
// Items are (sequence s, partition p < max(n_part(s), 1), KV-head group); an
// empty sequence has one item, which writes its zero output.  They are
// ordered group fastest, then sequence, then partition: the order of a dense
// (partition, sequence, group) grid with its idle entries squeezed out, so
// every sequence's partition p runs at about the same time as the others'
// (sequences that share prefix blocks read them together) and no workgroup
// slot is spent on a partition past a sequence's end.  The grid is sized for
// every sequence at full table length; its surplus is a run of workgroups at
// the end that leave at once.  Every thread of the workgroup must call this
// (it uses LDS and barriers).  Returns false for a surplus workgroup.
__device__ inline bool find_work(const DecodeArgs& a, int wg, WorkItem& w) {
    constexpr int NT = kDecodeThreads;
    __shared__ int s_tmp[NT];
    __shared__ int s_hist[kMaxPartitionBins + 1];
    __shared__ int s_sel[3];       // partition found, rank within it, sequence found
    const int tid = threadIdx.x;
    const int B = a.num_seqs;
    const int P = a.max_partitions;
    const int max_tokens = a.max_blocks_per_seq << a.block_shift;
    const int k = wg / a.groups;   // item index ignoring the group
    auto items_of = [&](int s) {
        const int L = min(a.context_lens[s], max_tokens);
        return L > 0 ? (L + a.partition - 1) / a.partition : 1;
    };

    if (tid == 0) {
        s_sel[0] = -1;
        s_sel[1] = 0;
        s_sel[2] = -1;
    }
    int pp = -1, rank = 0;
    if (P <= kMaxPartitionBins) {
        // hist[v] = sequences with exactly v items (v = 1 .. P)
        for (int i = tid; i <= P; i += NT) s_hist[i] = 0;
        __syncthreads();
        for (int s = tid; s < B; s += NT) atomicAdd(&s_hist[items_of(s)], 1);
        __syncthreads();
        // cnt(p) = sequences with more than p items = B - sum_{v <= p} hist[v];
        // partition p holds items [C(p), C(p) + cnt(p)), C = running sum of cnt
        int le_base = 0, c_base = 0;
        for (int p0 = 0; p0 < P; p0 += NT) {
            const int p = p0 + tid;
            int tot_h, tot_c;
            const int le = le_base + block_scan((p >= 1 && p <= P) ? s_hist[p] : 0, s_tmp, tot_h);
            const int cnt = p < P ? B - le : 0;
            const int incl = c_base + block_scan(cnt, s_tmp, tot_c);
            if (p < P && k >= incl - cnt && k < incl) {
                s_sel[0] = p;
                s_sel[1] = k - (incl - cnt);
            }
            __syncthreads();
            pp = s_sel[0];
            rank = s_sel[1];
            if (pp >= 0) break;
            le_base += tot_h;
            c_base += tot_c;
        }
        if (pp < 0) return false;
        // the rank-th sequence (ascending) with more than pp items
        int r_base = 0;
        for (int c0 = 0; c0 < B; c0 += NT) {
            const int s = c0 + tid;
            const int ind = (s < B && items_of(s) > pp) ? 1 : 0;
            int tot;
            const int incl = r_base + block_scan(ind, s_tmp, tot);
            if (ind && incl == rank + 1) s_sel[2] = s;
            __syncthreads();
            if (s_sel[2] >= 0) break;
            r_base += tot;
        }
    } else {
        // sequence-major: item k is partition k - C(s) of the sequence s with
        // C(s) <= k < C(s) + items(s)
        int base = 0;
        for (int c0 = 0; c0 < B; c0 += NT) {
            const int s = c0 + tid;
            const int items = s < B ? items_of(s) : 0;
            int tot;
            const int incl = base + block_scan(items, s_tmp, tot);
            if (s < B && k >= incl - items && k < incl) {
                s_sel[2] = s;
                s_sel[1] = k - (incl - items);
            }
            __syncthreads();
            if (s_sel[2] >= 0) break;
            base += tot;
        }
        pp = s_sel[1];
    }
    const int s = s_sel[2];
    if (s < 0) return false;
    w.s = s;
    w.p = pp;
    w.group = wg % a.groups;
    w.L = min(a.context_lens[s], max_tokens);
    w.n_part = w.L > 0 ? (w.L + a.partition - 1) / a.partition : 0;
    return true;
}

}  // namespace pa
