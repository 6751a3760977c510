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

// Chunk offsets of packed sequences: coff[n] = sum over m < n of ceil(len_m / C);
// and the sequences ordered longest first (ties by index), so that a state kernel,
// whose work per sequence is serial, starts the longest ones first when there are
// more workgroups than slots.  Malformed offsets are clamped here (and flagged)
// exactly as the other kernels clamp them, so all of them agree on every
// sequence's bounds.  P provides cu, T, total, err, coff, order, n_seq and C.
template <class P>
__global__ __launch_bounds__(kPlanThreads) void chunk_plan_kernel(P p) {
    __shared__ int part[kPlanThreads];
    const int tid = threadIdx.x, N = p.n_seq, C = p.C;
    const int per = (N + kPlanThreads - 1) / kPlanThreads;
    const int a = min(N, tid * per), b = min(N, a + per);
    int s = 0;
    for (int n = a; n < b; ++n) {
        long t0, t1;
        seq_bounds(p.cu, n, p.T, p.total, t0, t1, p.err);
        s += (int)((t1 - t0 + C - 1) / C);
    }
    part[tid] = s;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int i = 0; i < kPlanThreads; ++i) {
            const int x = part[i];
            part[i] = acc;
            acc += x;
        }
        p.coff[N] = acc;
    }
    __syncthreads();
    s = part[tid];
    for (int n = a; n < b; ++n) {
        p.coff[n] = s;
        long t0, t1;
        seq_bounds(p.cu, n, p.T, p.total, t0, t1, nullptr);
        s += (int)((t1 - t0 + C - 1) / C);
    }
    __syncthreads();
    // rank of sequence n: how many sequences are longer, or as long with a lower index
    for (int n = tid; n < N; n += kPlanThreads) {
        const int cn = p.coff[n + 1] - p.coff[n];
        int rank = 0;
        for (int m2 = 0; m2 < N; ++m2) {
            const int cm = p.coff[m2 + 1] - p.coff[m2];
            rank += (cm > cn) || (cm == cn && m2 < n);
        }
        p.order[rank] = n;
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
