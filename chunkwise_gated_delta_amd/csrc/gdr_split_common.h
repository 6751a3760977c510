// Sequence planning shared by the two-kernel (prep / state) paths (internal header).
//
// Both paths cut every sequence into chunks of C tokens; packed sequences
// (cu_seqlens) restart the chunking at each sequence start.  The prep kernels
// walk the chunks of all sequences as one flat list, the state kernels walk the
// chunks of one sequence; the plan below gives both the same numbering.
#pragma once

#include "gdr_common.h"

namespace gdr {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanBins = 4096;

// Bin of a sequence's chunk count for the longest-first order: the count itself below
// 2048; from 2048 on, its power of two and the six bits below the leading one (so the
// bins are monotone in the count, and counts in one bin differ by less than 1/64).
__device__ __forceinline__ int plan_bin(int c) {
    if (c < 2048) return c;
    const int e = 31 - __builtin_clz((unsigned)c);  // 11 .. 30
    return 2048 + ((e - 11) << 6) + ((c >> (e - 6)) & 63);
}

// Exclusive prefix sum of x over the workgroup's kPlanThreads threads: a scan inside
// each wave, then the wave totals through LDS (buf: one int per wave); *total receives
// the sum of all of them.
__device__ __forceinline__ int plan_scan(int x, int *buf, int *total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    if (lane == 63) buf[w] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kPlanThreads / 64; ++i) {
        const int t = buf[i];
        before += i < w ? t : 0;
        all += t;
    }
    *total = all;
    __syncthreads();  // buf may be reused
    return before + incl - x;
}

// Chunk offsets of packed sequences: coff[n] = sum over m < n of ceil(len_m / C);
// and the sequences ordered longest first (ties by index), so that a state kernel,
// whose work per sequence is serial, starts the longest ones first when there are
// more workgroups than slots.  The order is a stable counting sort over plan_bin of
// the chunk counts (exact below 2048 chunks): O(n_seq) work, one workgroup.  Malformed
// offsets are clamped here (and flagged) exactly as the other kernels clamp them, so
// all of them agree on every sequence's bounds.  P provides cu, T, total, err, coff,
// order, n_seq and C.
template <class P>
__global__ __launch_bounds__(kPlanThreads) void chunk_plan_kernel(P p) {
    __shared__ int buf[kPlanThreads / 64];
    __shared__ int bins[kPlanBins];  // per bin: its count, then its next free rank
    __shared__ int tkey[kPlanThreads];
    const int tid = threadIdx.x, N = p.n_seq, C = p.C;
    // (1) chunk offsets: each thread sums a contiguous range of sequences
    const int per = (N + kPlanThreads - 1) / kPlanThreads;
    const int a = min(N, tid * per), b = min(N, a + per);
    int s = 0;
    for (int n = a; n < b; ++n) {
        long t0, t1;
        seq_bounds(p.cu, n, p.T, p.total, t0, t1, p.err);
        s += (int)((t1 - t0 + C - 1) / C);
    }
    int all = 0;
    s = plan_scan(s, buf, &all);
    if (tid == 0) p.coff[N] = all;
    for (int n = a; n < b; ++n) {
        p.coff[n] = s;
        long t0, t1;
        seq_bounds(p.cu, n, p.T, p.total, t0, t1, nullptr);
        s += (int)((t1 - t0 + C - 1) / C);
    }
    // (2) histogram of the bins
    for (int i = tid; i < kPlanBins; i += kPlanThreads) bins[i] = 0;
    __syncthreads();  // also orders the coff writes above before the reads below
    for (int n = tid; n < N; n += kPlanThreads) atomicAdd(&bins[plan_bin(p.coff[n + 1] - p.coff[n])], 1);
    __syncthreads();
    // (3) first rank of each bin = the number of sequences in higher bins: thread t owns
    // bins [BPT t, BPT t + BPT), sums them from the top, and adds the totals of the
    // threads above it
    constexpr int BPT = kPlanBins / kPlanThreads;
    int loc[BPT];
    s = 0;
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {
        loc[i] = s;
        s += bins[BPT * tid + i];
    }
    const int below = plan_scan(s, buf, &all);  // sequences in the bins below this thread's
    const int above = all - below - s;
#pragma unroll
    for (int i = 0; i < BPT; ++i) bins[BPT * tid + i] = above + loc[i];
    __syncthreads();
    // (4) ranks, kPlanThreads sequences at a time in index order: a sequence goes after
    // those of its bin in earlier tiles and in this tile before it
    for (int base = 0; base < N; base += kPlanThreads) {
        const int n = base + tid;
        const int key = n < N ? plan_bin(p.coff[n + 1] - p.coff[n]) : -1;
        tkey[tid] = key;
        __syncthreads();
        if (n < N) {
            int same = 0;
            for (int j = 0; j < tid; ++j) same += tkey[j] == key;
            const int r = bins[key] + same;
            if (r < N) p.order[r] = n;
        }
        __syncthreads();
        if (n < N) atomicAdd(&bins[key], 1);
        __syncthreads();
    }
}

// Sequence n and chunk c of global chunk j; false when j is past the last chunk.
// P provides coff (NULL for a fixed-length batch), nc, n_seq and max_chunks.
template <class P>
__device__ __forceinline__ bool chunk_of(const P &p, int j, int &n, int &c) {
    if (p.coff == nullptr) {
        n = j / p.nc;
        c = j - n * p.nc;
        return true;
    }
    const int last = min(p.coff[p.n_seq], p.max_chunks);
    if (j >= last) return false;
    int lo = 0, hi = p.n_seq - 1;  // last n with coff[n] <= j
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.coff[mid] <= j) lo = mid;
        else hi = mid - 1;
    }
    n = lo;
    c = j - p.coff[lo];
    return true;
}

// Workspace of a two-kernel path: [error flag header][chunk offsets and order of
// packed sequences][one block of blk_bytes per (chunk, head)].
struct SplitLayout {
    size_t coff_off, blk_off, total;
    int nc;          // chunks per sequence (fixed-length batch), 0 for packed sequences
    int max_chunks;  // blocks per head
};

inline SplitLayout split_layout(const FwdArgs &a, int N, size_t blk_bytes) {
    SplitLayout L;
    const int ncT = (a.T + a.C - 1) / a.C;
    L.coff_off = kWorkspaceHeader;
    if (a.cu_seqlens != nullptr) {
        // every sequence may end in a partial chunk: at most ceil(T / C) + N chunks
        L.nc = 0;
        L.max_chunks = ncT + N;
        L.blk_off = L.coff_off + (((size_t)(2 * N + 1) * 4 + 255) / 256) * 256;  // coff, order
    } else {
        L.nc = ncT;
        L.max_chunks = N * ncT;
        L.blk_off = L.coff_off;
    }
    L.total = L.blk_off + (size_t)a.H * L.max_chunks * blk_bytes;
    return L;
}

}  // namespace
}  // namespace gdr
