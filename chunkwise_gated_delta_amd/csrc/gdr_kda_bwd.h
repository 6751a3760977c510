// Backward pass of the chunkwise KDA form (internal header, included by
// gdr_kda_split.hip after the forward kernels).
//
// Gradients of L = <dO, O> + <dS_final, S_final> ("Kimi Delta Attention backward"
// notes), per chunk of C = 64 tokens with the notation of the forward kernels:
//   g = in-chunk prefix sum of log alpha, Gamma = e^g, gamma_C = Gamma[last row]
//   Q<- = Q Gamma, K<- = K Gamma, K-> = K / Gamma
//   KK = K<- K->^T strictly lower, At = (I + Diag(beta) KK)^-1, Ab = At Diag(beta)
//   A_qk = Q<- K->^T on and below the diagonal, W = Ab K<-, U = Ab V
//   V_new = U - W S_p^T,  O = Q<- S_p^T + A_qk V_new,  S_n = (S_p + V_new^T K->) Diag(gamma_C)
// Three passes produce the states the per-chunk gradients need:
//   forward   the forward state kernel, saving S_p (the state entering each chunk)
//   reverse   dS_p = dS_n Diag(gamma_C) + (K^ dS_n^T)^T W' + dO^T Q~ over the chunks in
//             reverse order (the forward state kernel on the forward blocks, with K^,
//             W' and Q~ transposed in LDS as it reads them), saving
//             dS_n (the gradient of the state leaving each chunk); K^ = K-> gamma_C,
//             W' = -W and Q~ = Q<- - A_qk W come from the forward prep blocks
//   post      one workgroup per (chunk, head), with dSg = dS_n Diag(gamma_C):
//     dV_new = K-> dSg^T + A_qk^T dO                  dV = Diag(beta) At^T dV_new
//     dW = -dV_new S_p,   dA = dO V_new^T (lower),    dKg = V_new dSg
//     Y = dW K<-^T + dV_new V^T,  Z = At^T Y,  dXt = -Z Ab^T
//     dbeta = diag(Z) + rowsum(dXt * KK),             dXm = Diag(beta) dXt (strictly lower)
//     dK<- = Diag(beta) At^T dW + dXm K->
//     dK-> = dKg + dA^T Q<- + dXm^T K<-
//     dQ<- = dO S_p + dA K->
//     dQ = dQ<- Gamma,  dK = dK<- Gamma + dK-> / Gamma
//     dg = dQ<- Q<- + dK<- K<- - dK-> K->, plus sum_i S_n[i][j] dS_n[i][j] on the last row,
//          which is sum_i S_p dSg + sum_r K-> dKg by the state update
//     dlog alpha = suffix sum of dg over the chunk's rows (summed over channels for a
//     head gate)
// The notes' dbeta divides diag(At^T dAt) by beta; diag(Z) is the same number written
// without the division (it is the diagonal of the first line of their derivation).
#pragma once

namespace gdr {
namespace {

// ---------------------------------------------------------------------------------
// Per-chunk gradients.
// ---------------------------------------------------------------------------------
struct BwdParams {
    const bf16 *q, *k, *v, *dO;
    const bf16 *a, *b;  // DPLR only
    const float *la, *beta;
    const uint16_t *S, *dS;  // bf16 [chunk][head][dv][dk]: S_p, dS_n
    bf16 *dq, *dk, *dv;
    bf16 *da, *db;      // DPLR only
    float *dla, *dbeta;
    const int32_t *cu;
    const int32_t *coff;
    int *err;  // workspace error word: bit 2 when a chunk's gate falls beyond kBwdGateRange
    long total;
    int H, T, dv_, n_seq, nc, max_chunks, C;
};

// The gate inside a chunk, referred to the middle of its range: g' = g - r with
// r = n ln 2, n the integer nearest g_C / (2 ln 2).  Every factor these kernels form from
// it (Q<-, K<-, K->, Gamma) is e^g' or its inverse, which stays within about e^(|g_C|/2)
// both ways; the products they enter (K<- K->^T, Q<- K->^T, ...) are unchanged by the
// shift, and the terms with the states take S_p 2^n and dS_n e^(g_C - r) per column:
// (S_p 2^n)(W' 2^-n)^T = S_p W^T, and dS_n Diag(gamma_C) 2^-n pairs with K-> 2^n.  The
// gradients of the shifted operands map back through the shifted Gamma in the same way,
// and the gate gradient (elementwise products of an operand and its gradient) is
// unchanged.  A power of two keeps the bf16 S_p exact when scaled.
//
// g[i][e] holds the prefix of the thread's row-group (rows 8 rg + i); part[r2 * DK + e]
// (r2 < 8) holds each row-group's total for the same channel; row-group 0 writes 2^n to
// spf[e].  part and spf point at the thread's first channel (one vector read per
// row-group; the sums run in row-group order).
template <int CPT>
__device__ __forceinline__ void g_shift_all(float (&g)[8][CPT], const float *part, int rg, float *spf) {
    constexpr int DKP = CPT * 32;
    float acc[CPT], carry[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) acc[e] = carry[e] = 0.f;
#pragma unroll
    for (int r2 = 0; r2 < 8; ++r2) {
        float v[CPT];
        if constexpr (CPT == 4) {
            const float4 x = *(const float4 *)(part + r2 * DKP);
            v[0] = x.x; v[CPT > 1 ? 1 : 0] = x.y; v[CPT > 2 ? 2 : 0] = x.z; v[CPT > 3 ? 3 : 0] = x.w;
        } else {
#pragma unroll
            for (int e = 0; e < CPT; ++e) v[e] = part[r2 * DKP + e];
        }
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            if (r2 == rg) carry[e] = acc[e];  // the sum of the row-groups before this one
            acc[e] += v[e];
        }
    }
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
        const float n = rintf(0.5f * acc[e] * kLog2e);
        const float shift = carry[e] - n * kLn2;
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i][e] += shift;
        if (rg == 0) spf[e] = exp2f(n);
    }
}

// With the shift above, a chunk whose gate falls by more than twice this in some channel
// (natural log; e^66.54 = 2^96) is beyond the kernels' float range, which the error word
// reports.
constexpr float kBwdGateRange = 66.54f;

// Wave 3's lanes 32-63 hold the chunk's last row (rows 8 rg + i, rg = 7) of the shifted
// gate, g_C/2; flag the call when any channel falls beyond 2 kBwdGateRange.
template <int CPT>
__device__ __forceinline__ void flag_wide_gate(const float (&g)[8][CPT], int wave, int lane, int *err) {
    if (wave != 3) return;
    bool wide = false;
#pragma unroll
    for (int e = 0; e < CPT; ++e) wide = wide || !(g[7][e] >= -kBwdGateRange);
    if (__builtin_amdgcn_ballot_w64(wide && lane >= 32) != 0 && lane == 0) atomicOr(err, 2);
}

// One 16x16 output tile of A B on the 16x16x32 MFMA: lane l ends with
// D[m0 + l%16][n0 + 4(l/16) + e] in register e.  A is read from a row-major [m][k]
// array (AT = false) or from one stored [k][m] (AT = true); B from [k][n] (BT =
// false) or [n][k] (BT = true).  The contraction runs over [k0, k1) (at most KMAX
// long) in steps of 32; every step's operands are read before the first product so
// that the LDS latency is paid once per tile.
template <bool AT, bool BT, int KMAX>
__device__ __forceinline__ f32x4 mma_tile(const uint16_t *A, int lda, const uint16_t *B, int ldb,
                                          int m0, int n0, int k0, int k1, f32x4 acc, int lane) {
    constexpr int NS = KMAX / 32;
    const int r = lane & 15, g = lane >> 4;
    bf16x8 fa[NS], fb[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const int k = k0 + 32 * st;
        if (k < k1) {
            fa[st] = AT ? frag_tr(A, k, lda, m0, lane) : frag(A, m0 + r, lda, k + 8 * g);
            fb[st] = BT ? frag(B, n0 + r, ldb, k + 8 * g) : frag_tr(B, k, ldb, n0, lane);
        }
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
        if (k0 + 32 * st < k1) acc = mfma(fb[st], fa[st], acc);
    return acc;
}

// The same product split in two, for a row block whose A fragments serve several output
// tiles: load_a reads them once, mma_b multiplies them by one B tile (same steps, same
// order, same result as mma_tile).
template <bool AT, int KMAX>
__device__ __forceinline__ void load_a(bf16x8 (&fa)[KMAX / 32], const uint16_t *A, int lda, int m0,
                                       int k0, int k1, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int st = 0; st < KMAX / 32; ++st) {
        const int k = k0 + 32 * st;
        if (k < k1) fa[st] = AT ? frag_tr(A, k, lda, m0, lane) : frag(A, m0 + r, lda, k + 8 * g);
    }
}
template <bool BT, int KMAX>
__device__ __forceinline__ f32x4 mma_b(const bf16x8 (&fa)[KMAX / 32], const uint16_t *B, int ldb, int n0,
                                       int k0, int k1, f32x4 acc, int lane) {
    constexpr int NS = KMAX / 32;
    const int r = lane & 15, g = lane >> 4;
    bf16x8 fb[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const int k = k0 + 32 * st;
        if (k < k1) fb[st] = BT ? frag(B, n0 + r, ldb, k + 8 * g) : frag_tr(B, k, ldb, n0, lane);
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
        if (k0 + 32 * st < k1) acc = mfma(fb[st], fa[st], acc);
    return acc;
}

// Two row blocks against one B tile over the same range: the B fragments read once.
template <bool BT, int KMAX>
__device__ __forceinline__ void mma_b2(const bf16x8 (&fa)[KMAX / 32], const bf16x8 (&fa2)[KMAX / 32],
                                       const uint16_t *B, int ldb, int n0, int k0, int k1, f32x4 &acc,
                                       f32x4 &acc2, int lane) {
    constexpr int NS = KMAX / 32;
    const int r = lane & 15, g = lane >> 4;
    bf16x8 fb[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const int k = k0 + 32 * st;
        if (k < k1) fb[st] = BT ? frag(B, n0 + r, ldb, k + 8 * g) : frag_tr(B, k, ldb, n0, lane);
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
        if (k0 + 32 * st < k1) {
            acc = mfma(fb[st], fa[st], acc);
            acc2 = mfma(fb[st], fa2[st], acc2);
        }
}

// Operand fragments of v_mfma_f32_16x16x16_bf16 (lane l: index l%16, contraction
// 4(l/16)+0..3): from a row-major [m][k] array (8-byte read) or, gathered with one
// LDS transpose read, from an array whose rows run along the contraction.
__device__ __forceinline__ bf16x4 frag4(const uint16_t *base, int row, int stride, int col) {
    return *(const bf16x4 *)(base + row * stride + col);
}
__device__ __forceinline__ bf16x4 frag4_tr(const uint16_t *base, int k0, int stride, int col0, int lane) {
    const int G = lane >> 4, q = lane & 15;
    const uint16_t *ptr = base + (k0 + 4 * G + (q >> 2)) * stride + col0 + 4 * (q & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)ptr);
}

template <int DK>
struct BwdSmem {
    static constexpr int KS = DK + 8;           // bf16 stride of [64][DK] arrays
    static constexpr int CS = kC + 8;           // bf16 stride of [64][64] arrays
    static constexpr int VS = 32 + 8;           // bf16 stride of [64][32] value tiles
    static constexpr int QK = kC * KS * 2;      // bytes of one [64][KS] array
    static constexpr int CC = kC * CS * 2;      // bytes of one [64][CS] array
    static constexpr int oQl = 0;               // Q<-
    static constexpr int oKl = oQl + QK;        // K<-
    static constexpr int oKr = oKl + QK;        // K->
    static constexpr int oA = oKr + QK;         // At
    static constexpr int oAb = oA + CC;         // Ab
    static constexpr int oAqk = oAb + CC;       // A_qk
    static constexpr int oW = oAqk + CC;        // W, then dW
    static constexpr int oT = oW + QK;          // per-dv-tile region, reused below
    //   dv tile: S_p [32][KS], dSg [32][KS], V, dO, V_new, dV_new [64][VS]
    static constexpr int tSp = 0, tdS = tSp + 32 * KS * 2, tV = tdS + 32 * KS * 2;
    static constexpr int tdO = tV + kC * VS * 2, tVn = tdO + kC * VS * 2, tdVn = tVn + kC * VS * 2;
    static constexpr int tEnd = tdVn + kC * VS * 2;
    //   after the dv loop: dA, dXm (Y first), Z at tSp..; the inverse's KK fp32 [64][68] at 0
    static constexpr int tdA = 0, tY = CC, tZ = 2 * CC;
    //   the inverse: KK fp32 [64][68], then L and the middle factor bf16 [64][CS] each
    static constexpr int tInv = kC * 68 * 4 + 2 * CC;
    static constexpr int Tbytes = tEnd > 3 * CC ? (tEnd > tInv ? tEnd : tInv) : (3 * CC > tInv ? 3 * CC : tInv);
    static constexpr int oBeta = oT + Tbytes;   // fp32 [64]
    static constexpr int oGam = oBeta + kC * 4; // fp32 [DK] gamma_C
    static constexpr int oGp = oGam + DK * 4;   // fp32 [8][DK] gate partial sums
    static constexpr int oDb = oGp + 8 * DK * 4;  // fp32 [64] dbeta
    // fp32 [8][DK] last-row term of dg: slot w the S_p dSg part of wave w, slot 4 + w its
    // K-> dKg part (each written once per job: no clearing, no read-modify-write)
    static constexpr int oDg = oDb + kC * 4;
    static constexpr int oSpf = oDg + 8 * DK * 4;  // fp32 [DK] 2^n, the state's scale
    static constexpr int bytes = oSpf + DK * 4;
    // final stage: Gamma fp32 [64][DK] over Q<-..K-> (free by then), dg fp32 [64][DK] over T
    static_assert(kC * DK * 4 <= 3 * QK, "Gamma fits over the operand arrays");
    static_assert(kC * DK * 4 <= Tbytes, "dg fits over the tile region");
    static_assert(bytes <= 160 * 1024, "LDS");
};

template <int DK, int GATE>
__global__ __launch_bounds__(kThreads, 1) void kda_bwd_post_kernel(BwdParams p) {
    using L = BwdSmem<DK>;
    constexpr int KS = L::KS, CS = L::CS, VS = L::VS;
    constexpr int NT = DK / 16;   // 16-column tiles of dk
    constexpr int CPT = DK / 32;  // gate stage: channels per thread
    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    uint16_t *sQl = (uint16_t *)(smem + L::oQl), *sKl = (uint16_t *)(smem + L::oKl);
    uint16_t *sKr = (uint16_t *)(smem + L::oKr), *sA = (uint16_t *)(smem + L::oA);
    uint16_t *sAb = (uint16_t *)(smem + L::oAb), *sAqk = (uint16_t *)(smem + L::oAqk);
    uint16_t *sW = (uint16_t *)(smem + L::oW);
    char *sT = smem + L::oT;
    uint16_t *sSp = (uint16_t *)(sT + L::tSp), *sdS = (uint16_t *)(sT + L::tdS);
    uint16_t *sV = (uint16_t *)(sT + L::tV), *sdO = (uint16_t *)(sT + L::tdO);
    uint16_t *sVn = (uint16_t *)(sT + L::tVn), *sdVn = (uint16_t *)(sT + L::tdVn);
    float *sBeta = (float *)(smem + L::oBeta), *sGam = (float *)(smem + L::oGam);
    float *sGp = (float *)(smem + L::oGp), *sDb = (float *)(smem + L::oDb);
    float *sDg = (float *)(smem + L::oDg);
    float *sSpf = (float *)(smem + L::oSpf);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, DV = p.dv_;
    const int R0 = 16 * wave;  // this wave's 16 rows of every row-block output
    const int rg = tid >> 5, c0 = CPT * (tid & 31);
    constexpr int WPR = CPT / 2;  // bf16 words per row and thread in the gate layout

    // The grid is persistent: workgroup w takes jobs (chunk, head) w, w + gridDim.x, ...
    // While one job finishes, the next job's inputs are already being loaded.
    struct Job {
        int job, h, m;
        long tok0;
        size_t sbase;  // (chunk, head) index of the state buffers
        bool ok;
    };
    auto decode = [&](int job) {
        Job J;
        J.job = job;
        J.h = job % H;
        J.m = 1;
        J.tok0 = 0;
        J.sbase = (size_t)job;
        int n = 0, c = 0;
        J.ok = job < p.H * p.max_chunks && chunk_of(p, job / H, n, c);
        if (J.ok) {
            long t0, t1;
            seq_bounds(p.cu, n, p.T, p.total, t0, t1, nullptr);
            J.tok0 = t0 + (long)c * kC;
            J.m = (int)((t1 - J.tok0) < kC ? (t1 - J.tok0) : kC);
        }
        return J;
    };
    // One dv tile's S_p and dS_n rows j0..j0+31, value and dO tiles, loaded a tile ahead.
    constexpr int kSPT = 32 * DK / 8 / kThreads;  // 16-byte pieces of a state tile per thread
    struct Tile {
        uint4 s[kSPT], d[kSPT], v, o;
    } pf;
    auto issue = [&](const Job &J, int j0) {
        const uint16_t *ps = p.S + (J.sbase * DV + j0) * DK;
        const uint16_t *pd = p.dS + (J.sbase * DV + j0) * DK;
#pragma unroll
        for (int i = 0; i < kSPT; ++i) {
            const int idx = tid + kThreads * i, r = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
            pf.s[i] = *(const uint4 *)(ps + (size_t)r * DK + c8);
            pf.d[i] = *(const uint4 *)(pd + (size_t)r * DK + c8);
        }
        const int r = tid >> 2, c8 = 8 * (tid & 3);
        const size_t off = ((size_t)(J.tok0 + (r < J.m ? r : 0)) * H + J.h) * DV + j0 + c8;
        pf.v = *(const uint4 *)(p.v + off);  // rows past the end are zeroed when stored
        pf.o = *(const uint4 *)(p.dO + off);
    };
    // A job's q, k and log alpha in the gate layout (rows 8rg + i, channels c0 + e) and
    // beta of row tid; rows past the end are zeroed where they are used.
    struct In {
        uint32_t qw[8][WPR], kw[8][WPR];
        float la[8][CPT];
        float beta;
    } in;
    auto load_in = [&](const Job &J) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * rg + i;
            const size_t th = (size_t)(J.tok0 + (r < J.m ? r : 0)) * H + J.h;
            if constexpr (WPR == 2) {
                const uint2 qa = *(const uint2 *)(p.q + th * DK + c0), ka = *(const uint2 *)(p.k + th * DK + c0);
                in.qw[i][0] = qa.x; in.qw[i][WPR - 1] = qa.y; in.kw[i][0] = ka.x; in.kw[i][WPR - 1] = ka.y;
            } else {
                in.qw[i][0] = *(const uint32_t *)(p.q + th * DK + c0);
                in.kw[i][0] = *(const uint32_t *)(p.k + th * DK + c0);
            }
            if (GATE == kGateChannel) {
                if constexpr (CPT == 4) {
                    const float4 x = *(const float4 *)(p.la + th * DK + c0);
                    in.la[i][0] = x.x; in.la[i][CPT > 1 ? 1 : 0] = x.y;
                    in.la[i][CPT > 2 ? 2 : 0] = x.z; in.la[i][CPT > 3 ? 3 : 0] = x.w;
                } else {
                    const float2 x = *(const float2 *)(p.la + th * DK + c0);
                    in.la[i][0] = x.x; in.la[i][CPT > 1 ? 1 : 0] = x.y;
                }
            } else if (GATE == kGateHead) {
                const float x = p.la[th];
#pragma unroll
                for (int e = 0; e < CPT; ++e) in.la[i][e] = x;
            } else {
#pragma unroll
                for (int e = 0; e < CPT; ++e) in.la[i][e] = 0.f;
            }
        }
        in.beta = p.beta[(size_t)(J.tok0 + (tid < J.m ? tid : 0)) * H + J.h];
    };

    Job J = decode(blockIdx.x);
    if (J.ok) {
        load_in(J);
        issue(J, 0);
    }
    while (J.ok) {  // workgroup-uniform
    const Job Nx = decode(J.job + gridDim.x);  // the next job
    // lane indices are re-derived each job so that the compiler keeps no per-lane
    // addresses alive across jobs
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
    const int rg = tid >> 5, c0 = CPT * (tid & 31);  // the gate layout, as in load_in
    const int h = J.h, m = J.m;
    const long tok0 = J.tok0;

    // ---- gate: g for rows 8rg + i, channels c0 + e (natural log, inclusive prefix) ----
    auto gate = [&](float (&g)[8][CPT]) {
        float run[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) run[e] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                run[e] += 8 * rg + i < m ? in.la[i][e] : 0.f;
                g[i][e] = run[e];
            }
#pragma unroll
        for (int e = 0; e < CPT; ++e) sGp[rg * DK + c0 + e] = run[e];
        lds_barrier();
        g_shift_all(g, sGp + c0, rg, sSpf + c0);
        lds_barrier();  // sGp may be reused
    };

    // ---- stage 0: scaled operands ---------------------------------------------------
    float g[8][CPT];  // kept for the chain rule at the end
    {
        gate(g);
        flag_wide_gate(g, wave, lane, p.err);
        if (tid < kC) sBeta[tid] = tid < m ? in.beta : 0.f;
        uint32_t qw[8][WPR], kw[8][WPR];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int w = 0; w < WPR; ++w) {
                const bool ok = 8 * rg + i < m;
                qw[i][w] = ok ? in.qw[i][w] : 0u;
                kw[i][w] = ok ? in.kw[i][w] : 0u;
            }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * rg + i;
            uint32_t oq[WPR], ol[WPR], orr[WPR];
#pragma unroll
            for (int w = 0; w < WPR; ++w) {
                const float G0 = exp2_fast(g[i][2 * w] * kLog2e), G1 = exp2_fast(g[i][2 * w + 1] * kLog2e);
                const float q0 = bf16_lo(qw[i][w]), q1 = bf16_hi(qw[i][w]);
                const float k0 = bf16_lo(kw[i][w]), k1 = bf16_hi(kw[i][w]);
                oq[w] = pack_bf16x2(q0 * G0, q1 * G1);
                ol[w] = pack_bf16x2(k0 * G0, k1 * G1);
                orr[w] = pack_bf16x2(k0 * exp2_fast(-g[i][2 * w] * kLog2e), k1 * exp2_fast(-g[i][2 * w + 1] * kLog2e));
                if (r == kC - 1) {
                    sGam[c0 + 2 * w] = G0;
                    sGam[c0 + 2 * w + 1] = G1;
                }
            }
            if constexpr (WPR == 2) {
                *(uint2 *)(sQl + r * KS + c0) = make_uint2(oq[0], oq[WPR - 1]);
                *(uint2 *)(sKl + r * KS + c0) = make_uint2(ol[0], ol[WPR - 1]);
                *(uint2 *)(sKr + r * KS + c0) = make_uint2(orr[0], orr[WPR - 1]);
            } else {
                *(uint32_t *)(sQl + r * KS + c0) = oq[0];
                *(uint32_t *)(sKl + r * KS + c0) = ol[0];
                *(uint32_t *)(sKr + r * KS + c0) = orr[0];
            }
        }
        for (int i = tid; i < kC; i += kThreads) sDb[i] = 0.f;
    }
    lds_barrier();

    // ---- stage 1: KK (fp32, for the inverse) and A_qk --------------------------------
    float *sKK = (float *)sT;  // [64][68]
    for (int idx = tid; idx < kC * CS / 8; idx += kThreads) ((uint4 *)sA)[idx] = make_uint4(0u, 0u, 0u, 0u);
    {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        bf16x8 fkl[NT / 2], fql[NT / 2];  // K<-, Q<- rows R0.. (K = DK)
        load_a<false, DK>(fkl, sKl, KS, R0, 0, DK, lane);
        load_a<false, DK>(fql, sQl, KS, R0, 0, DK, lane);
        for (int tj = 0; tj < 4; ++tj) {
            f32x4 kk = z, aq = z;
            if (tj <= wave) {
                kk = mma_b<true, DK>(fkl, sKr, KS, 16 * tj, 0, DK, z, lane);
                aq = mma_b<true, DK>(fql, sKr, KS, 16 * tj, 0, DK, z, lane);
            }
            const int row = R0 + r16, col = 16 * tj + 4 * g4;
            *(float4 *)(sKK + row * 68 + col) = make_float4(col < row ? kk[0] : 0.f, col + 1 < row ? kk[1] : 0.f,
                                                         col + 2 < row ? kk[2] : 0.f, col + 3 < row ? kk[3] : 0.f);
            store4(sAqk + row * CS + col, col <= row ? aq[0] : 0.f, col + 1 <= row ? aq[1] : 0.f,
                   col + 2 <= row ? aq[2] : 0.f, col + 3 <= row ? aq[3] : 0.f);
        }
    }
    lds_barrier();

    // ---- stage 2: At = (I + L)^-1, L = Diag(beta) KK, blocked ----------------------------
    // (a) wave w inverts the diagonal 16x16 block w by forward substitution (fp32; four
    //     lanes per column, lane part s keeps x_k for k = s mod 4, quad sums complete the
    //     rows; x_k = 0 for k < j and KK is zero on and above the diagonal: no masks);
    //     every thread also writes L in bf16 for the off-diagonal products;
    // (b) [A 0; C B]^-1 = [A^-1 0; -B^-1 C A^-1 B^-1] for the 32x32 blocks (16x16x16
    //     MFMA, waves 0 and 2), then (c) for the whole 64x64 (16x16x32 MFMA, all waves).
    uint16_t *sL = (uint16_t *)(sT + kC * 68 * 4);  // bf16 [64][CS]: L, strictly lower
    uint16_t *sTm = sL + kC * CS;                     // bf16 [64][CS]: the products' middle factor
    {
        const int jl = lane >> 2, s = lane & 3, j = R0 + jl;
        float xs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int u = 0; u < (i + 3) / 4; ++u) acc += sKK[(R0 + i) * 68 + R0 + 4 * u + s] * xs[u];
            acc += dpp<kDppXor1>(acc);
            acc += dpp<kDppXor2>(acc);
            const float xi = (i == jl ? 1.f : 0.f) - sBeta[R0 + i] * acc;
            if (s == (i & 3)) xs[i >> 2] = xi;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) sA[(R0 + 4 * u + s) * CS + j] = __builtin_bit_cast(uint16_t, (__bf16)xs[u]);
        for (int idx = tid; idx < kC * kC / 8; idx += kThreads) {  // eight columns per piece
            const int i = idx >> 3, k8 = 8 * (idx & 7);
            const float bi = sBeta[i];
            const float4 a = *(const float4 *)(sKK + i * 68 + k8), b = *(const float4 *)(sKK + i * 68 + k8 + 4);
            *(uint4 *)(sL + i * CS + k8) = make_uint4(pack_bf16x2(bi * a.x, bi * a.y), pack_bf16x2(bi * a.z, bi * a.w),
                                                      pack_bf16x2(bi * b.x, bi * b.y), pack_bf16x2(bi * b.z, bi * b.w));
        }
    }
    lds_barrier();
    if (wave == 0 || wave == 2) {
        // blocks rows 16..31 x cols 0..15 (wave 0) and rows 48..63 x cols 32..47 (wave 2)
        const int o = wave == 0 ? 0 : 32;
        const int r = lane & 15, g = lane >> 4;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        // T = L[o+16..][o..o+15] A[o..][o..]
        f32x4 t = mfma16(frag4_tr(sA + o, o, CS, 0, lane), frag4(sL + o, o + 16 + r, CS, 4 * g), z);
        store4(sTm + (o + 16 + r) * CS + o + 4 * g, t[0], t[1], t[2], t[3]);
        asm volatile("" ::: "memory");
        // C-block of the inverse = -A[o+16..][o+16..] T  (same wave: the LDS writes above
        // are seen by its reads below)
        t = mfma16(frag4_tr(sTm + o, o + 16, CS, 0, lane), frag4(sA + o + 16, o + 16 + r, CS, 4 * g), z);
        store4(sA + (o + 16 + r) * CS + o + 4 * g, -t[0], -t[1], -t[2], -t[3]);
    }
    lds_barrier();
    {
        // rows 32..63 x cols 0..31: T = L[32..][0..31] A[0..31][0..31], then -A[32..][32..] T
        const int m0 = 32 + 16 * (wave >> 1), n0 = 16 * (wave & 1);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 t = mma_tile<false, false, kC>(sL, CS, sA, CS, m0, n0, 0, 32, z, lane);
        store4(sTm + (m0 + r16) * CS + n0 + 4 * g4, t[0], t[1], t[2], t[3]);
        lds_barrier();
        const f32x4 c = mma_tile<false, false, kC>(sA + 32, CS, sTm + 32 * CS, CS, m0, n0, 0, 32, z, lane);
        lds_barrier();  // every wave has read its A and T operands
        store4(sA + (m0 + r16) * CS + n0 + 4 * g4, -c[0], -c[1], -c[2], -c[3]);
    }
    lds_barrier();
    for (int idx = tid; idx < kC * kC / 8; idx += kThreads) {  // eight columns per piece
        const int i = idx >> 3, j8 = 8 * (idx & 7);
        const uint4 a = *(const uint4 *)(sA + i * CS + j8);
        const float4 b0 = *(const float4 *)(sBeta + j8), b1 = *(const float4 *)(sBeta + j8 + 4);
        *(uint4 *)(sAb + i * CS + j8) =
            make_uint4(pack_bf16x2(bf16_lo(a.x) * b0.x, bf16_hi(a.x) * b0.y), pack_bf16x2(bf16_lo(a.y) * b0.z, bf16_hi(a.y) * b0.w),
                       pack_bf16x2(bf16_lo(a.z) * b1.x, bf16_hi(a.z) * b1.y), pack_bf16x2(bf16_lo(a.w) * b1.z, bf16_hi(a.w) * b1.w));
    }
    lds_barrier();

    // ---- stage 3: W = Ab K<- ---------------------------------------------------------
    {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const int k1 = R0 + 16 <= 32 ? 32 : 64;  // Ab is lower triangular
        bf16x8 fab[2];
        load_a<false, kC>(fab, sAb, CS, R0, 0, k1, lane);
        for (int tn = 0; tn < NT; ++tn) {
            const f32x4 w = mma_b<false, kC>(fab, sKl, KS, 16 * tn, 0, k1, z, lane);
            store4(sW + (R0 + r16) * KS + 16 * tn + 4 * g4, w[0], w[1], w[2], w[3]);
        }
    }
    lds_barrier();

    // ---- stage 4: the dv tiles ---------------------------------------------------------
    f32x4 aQ[NT], aW[NT], aKg[NT], aA[4], aY[4];
    {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NT; ++t) aQ[t] = aW[t] = aKg[t] = z;
#pragma unroll
        for (int t = 0; t < 4; ++t) aA[t] = aY[t] = z;
    }
    // sum over dv of S_p * dSg for this thread's 8 columns 8 (tid % (DK / 8)) + 0..7 (the
    // same columns for every piece it stores)
    float gpart[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int lo_k = R0 >= 32 ? 32 : 0;  // At^T / A_qk^T rows R0..: contraction over j >= R0
    for (int j0 = 0; j0 < DV; j0 += 32) {
        // the tile's loads were issued one tile earlier (the first at the kernel's start);
        // into LDS, dS scaled by gamma_C per column
        {
#pragma unroll
            for (int i = 0; i < kSPT; ++i) {
                const int idx = tid + kThreads * i, r = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
                const uint32_t w4[4] = {pf.d[i].x, pf.d[i].y, pf.d[i].z, pf.d[i].w};
                const uint32_t s4[4] = {pf.s[i].x, pf.s[i].y, pf.s[i].z, pf.s[i].w};
                uint32_t o4[4], p4[4];
                // the eight columns' gamma_C and 2^n, two vector reads each
                const float4 ga = *(const float4 *)(sGam + c8), gb = *(const float4 *)(sGam + c8 + 4);
                const float4 fa = *(const float4 *)(sSpf + c8), fb = *(const float4 *)(sSpf + c8 + 4);
                const float gm[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
                const float sf[8] = {fa.x, fa.y, fa.z, fa.w, fb.x, fb.y, fb.z, fb.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float d0 = bf16_lo(w4[e]) * gm[2 * e], d1 = bf16_hi(w4[e]) * gm[2 * e + 1];
                    const float s0 = bf16_lo(s4[e]) * sf[2 * e], s1 = bf16_hi(s4[e]) * sf[2 * e + 1];
                    o4[e] = pack_bf16x2(d0, d1);
                    p4[e] = pack_bf16x2(s0, s1);
                    gpart[2 * e] += s0 * d0;
                    gpart[2 * e + 1] += s1 * d1;
                }
                *(uint4 *)(sSp + r * KS + c8) = make_uint4(p4[0], p4[1], p4[2], p4[3]);
                *(uint4 *)(sdS + r * KS + c8) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
            }
            const int r = tid >> 2, c8 = 8 * (tid & 3);
            const uint32_t keep = 0u - (uint32_t)(r < m);
            *(uint4 *)(sV + r * VS + c8) = make_uint4(pf.v.x & keep, pf.v.y & keep, pf.v.z & keep, pf.v.w & keep);
            *(uint4 *)(sdO + r * VS + c8) = make_uint4(pf.o.x & keep, pf.o.y & keep, pf.o.z & keep, pf.o.w & keep);
        }
        if (j0 + 32 < DV) issue(J, j0 + 32);
        else if (Nx.ok) issue(Nx, 0);  // the next job's first tile
        lds_barrier();
        // V_new = Ab V - W S_p^T and dV_new = K-> dSg^T + A_qk^T dO, rows R0..R0+15
        {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const int k1 = R0 + 16 <= 32 ? 32 : 64;
            // each product's A fragments (rows R0..) read once for both 16-column tiles
            f32x4 u[2], dv[2];
            {
                bf16x8 fa[2];
                load_a<false, kC>(fa, sAb, CS, R0, 0, k1, lane);
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) u[tn] = mma_b<false, kC>(fa, sV, VS, 16 * tn, 0, k1, z, lane);
            }
            {
                bf16x8 fa[NT / 2];
                load_a<false, DK>(fa, sW, KS, R0, 0, DK, lane);
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) {
                    const f32x4 ws = mma_b<true, DK>(fa, sSp, KS, 16 * tn, 0, DK, z, lane);
                    store4(sVn + (R0 + r16) * VS + 16 * tn + 4 * g4, u[tn][0] - ws[0], u[tn][1] - ws[1],
                           u[tn][2] - ws[2], u[tn][3] - ws[3]);
                }
                load_a<false, DK>(fa, sKr, KS, R0, 0, DK, lane);
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) dv[tn] = mma_b<true, DK>(fa, sdS, KS, 16 * tn, 0, DK, z, lane);
            }
            {
                bf16x8 fa[2];
                load_a<true, kC>(fa, sAqk, CS, R0, lo_k, kC, lane);
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) {
                    dv[tn] = mma_b<false, kC>(fa, sdO, VS, 16 * tn, lo_k, kC, dv[tn], lane);
                    store4(sdVn + (R0 + r16) * VS + 16 * tn + 4 * g4, dv[tn][0], dv[tn][1], dv[tn][2], dv[tn][3]);
                }
            }
        }
        lds_barrier();
        {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const int row = R0 + r16;
            const float br = sBeta[row];
            // dV = Diag(beta) At^T dV_new
            bf16x8 fat[2];
            load_a<true, kC>(fat, sA, CS, R0, lo_k, kC, lane);
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) {
                const f32x4 d = mma_b<false, kC>(fat, sdVn, VS, 16 * tn, lo_k, kC, z, lane);
                if (row < m) {
                    uint2 o;
                    o.x = pack_bf16x2(br * d[0], br * d[1]);
                    o.y = pack_bf16x2(br * d[2], br * d[3]);
                    *(uint2 *)(p.dv + ((size_t)(tok0 + row) * H + h) * DV + j0 + 16 * tn + 4 * g4) = o;
                }
            }
            // contraction over this dv tile: dQ<- += dO S_p, dW += dV_new S_p, dKg += V_new dSg
            const bf16x8 fdo = frag(sdO, R0 + r16, VS, 8 * g4);
            const bf16x8 fdv = frag(sdVn, R0 + r16, VS, 8 * g4);
            const bf16x8 fvn = frag(sVn, R0 + r16, VS, 8 * g4);
#pragma unroll
            for (int tn = 0; tn < NT; ++tn) {
                const bf16x8 fs = frag_tr(sSp, 0, KS, 16 * tn, lane);
                const bf16x8 fd = frag_tr(sdS, 0, KS, 16 * tn, lane);
                aQ[tn] = mfma(fs, fdo, aQ[tn]);
                aW[tn] = mfma(fs, fdv, aW[tn]);
                aKg[tn] = mfma(fd, fvn, aKg[tn]);
            }
            // dA += dO V_new^T (lower tiles), Y += dV_new V^T
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                if (tj <= wave) aA[tj] = mfma(frag(sVn, 16 * tj + r16, VS, 8 * g4), fdo, aA[tj]);
                aY[tj] = mfma(frag(sV, 16 * tj + r16, VS, 8 * g4), fdv, aY[tj]);
            }
        }
        lds_barrier();  // the tile buffers are reloaded
    }

    // ---- stage 5: dW, dA, Y, Z, dXt, dbeta --------------------------------------------
    uint16_t *sdW = sW;
    uint16_t *sdA = (uint16_t *)(sT + L::tdA), *sY = (uint16_t *)(sT + L::tY);
    uint16_t *sZ = (uint16_t *)(sT + L::tZ), *sdXm = sY;
    {
        const int row = R0 + r16;
#pragma unroll
        for (int tn = 0; tn < NT; ++tn)
            store4(sdW + row * KS + 16 * tn + 4 * g4, -aW[tn][0], -aW[tn][1], -aW[tn][2], -aW[tn][3]);
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            float d[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) d[e] = (16 * tj + 4 * g4 + e <= row) ? aA[tj][e] : 0.f;
            store4(sdA + row * CS + 16 * tj + 4 * g4, d[0], d[1], d[2], d[3]);
        }
        // lanes l, l + DK/8, ... of a wave hold the same columns: sum them first
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = gpart[e];
#pragma unroll
            for (int off = DK / 8; off < 64; off <<= 1) x += __shfl_xor(x, off);
            if (lane < DK / 8) sDg[wave * DK + 8 * lane + e] = x;  // this wave's slot
        }
    }
    lds_barrier();
    {
        const int row = R0 + r16;
        bf16x8 fdw[NT / 2];
        load_a<false, DK>(fdw, sdW, KS, R0, 0, DK, lane);
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            aY[tj] = mma_b<true, DK>(fdw, sKl, KS, 16 * tj, 0, DK, aY[tj], lane);
            store4(sY + row * CS + 16 * tj + 4 * g4, aY[tj][0], aY[tj][1], aY[tj][2], aY[tj][3]);
        }
    }
    lds_barrier();
    {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const int row = R0 + r16;
        bf16x8 fat[2];
        load_a<true, kC>(fat, sA, CS, R0, lo_k, kC, lane);
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            const f32x4 zt = mma_b<false, kC>(fat, sY, CS, 16 * tj, lo_k, kC, z, lane);
            store4(sZ + row * CS + 16 * tj + 4 * g4, zt[0], zt[1], zt[2], zt[3]);
            if (tj == wave && (r16 >> 2) == g4) sDb[row] = zt[r16 & 3];  // diag(Z)
        }
    }
    lds_barrier();
    {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const int row = R0 + r16;
        const float br = sBeta[row];
        float db2 = 0.f;
        bf16x8 fz[2], fkl[NT / 2];  // Z, K<- rows R0..
        load_a<false, kC>(fz, sZ, CS, R0, 0, kC, lane);
        load_a<false, DK>(fkl, sKl, KS, R0, 0, DK, lane);
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            f32x4 dx = z;
            if (tj <= wave) {
                dx = mma_b<true, kC>(fz, sAb, CS, 16 * tj, 0, kC, z, lane);
                const f32x4 kk = mma_b<true, DK>(fkl, sKr, KS, 16 * tj, 0, DK, z, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int col = 16 * tj + 4 * g4 + e;
                    dx[e] = col < row ? -dx[e] : 0.f;  // dXt, strictly lower
                    db2 += dx[e] * kk[e];
                }
            }
            store4(sdXm + row * CS + 16 * tj + 4 * g4, br * dx[0], br * dx[1], br * dx[2], br * dx[3]);
        }
        db2 += __shfl_xor(db2, 16);
        db2 += __shfl_xor(db2, 32);
        // (sdXm overwrites Y: every wave finished reading Y, for Z, before the barrier
        // above; diag(Z) went into sDb before it too)
        if (g4 == 0) sDb[row] += db2;
    }
    lds_barrier();

    // ---- stage 6: dK<-, dK->, dQ<- ------------------------------------------------------
    f32x4 gKl[NT], gKr[NT], gQl[NT];
    // dg of this lane's row and columns: dQ<- Q<- + dK<- K<- - dK-> K->, each operand the
    // bf16 value the products above used.  Every pair (r, c) of a Gram product then enters
    // the row-r and row-c terms as the same product of the same rounded numbers, so the
    // pairs inside a suffix cancel exactly in the suffix sums below, as they do in exact
    // arithmetic (with the operands rebuilt from q, k and e^g, both copies differ by the
    // bf16 rounding of the operands, and those residues swamp dlog alpha wherever the gate
    // decays fast enough to make it small).
    float dgl[NT][4];
    const bool ok_row = R0 + r16 < m;
    const size_t th_row = (size_t)(tok0 + (ok_row ? R0 + r16 : 0)) * H + h;
    {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const int row = R0 + r16;
        const float br = sBeta[row];
        float dgp[NT][4];
        // one product at a time, its row block's A fragments read once for all NT tiles
        {
            bf16x8 fat[2], fdx[2], fda[2];  // At^T, dXm and dA rows R0..
            load_a<true, kC>(fat, sA, CS, R0, lo_k, kC, lane);
            load_a<false, kC>(fdx, sdXm, CS, R0, 0, kC, lane);
            load_a<false, kC>(fda, sdA, CS, R0, 0, kC, lane);
#pragma unroll
            for (int tn = 0; tn < NT; ++tn) {
                f32x4 a = mma_b<false, kC>(fat, sdW, KS, 16 * tn, lo_k, kC, z, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] *= br;
                // dK<- = (Diag(beta) At^T dW) + dXm K->, dQ<- = dO S_p + dA K->: one K-> tile
                gKl[tn] = a;
                gQl[tn] = aQ[tn];
                mma_b2<false, kC>(fdx, fda, sKr, KS, 16 * tn, 0, kC, gKl[tn], gQl[tn], lane);
            }
        }
        {
            bf16x8 fda[2], fdx[2];  // dA^T and dXm^T rows R0..
            load_a<true, kC>(fda, sdA, CS, R0, lo_k, kC, lane);
            load_a<true, kC>(fdx, sdXm, CS, R0, lo_k, kC, lane);
#pragma unroll
            for (int tn = 0; tn < NT; ++tn) {
                const f32x4 b = mma_b<false, kC>(fda, sQl, KS, 16 * tn, lo_k, kC, aKg[tn], lane);
                gKr[tn] = mma_b<false, kC>(fdx, sKl, KS, 16 * tn, lo_k, kC, b, lane);
            }
        }
#pragma unroll
        for (int tn = 0; tn < NT; ++tn) {
            // last-row term: sum over rows of K-> dKg, per column
            const uint2 kr = *(const uint2 *)(sKr + row * KS + 16 * tn + 4 * g4);
            const uint2 ql = *(const uint2 *)(sQl + row * KS + 16 * tn + 4 * g4);
            const uint2 kl = *(const uint2 *)(sKl + row * KS + 16 * tn + 4 * g4);
            const float vr[4] = {bf16_lo(kr.x), bf16_hi(kr.x), bf16_lo(kr.y), bf16_hi(kr.y)};
            const float vq[4] = {bf16_lo(ql.x), bf16_hi(ql.x), bf16_lo(ql.y), bf16_hi(ql.y)};
            const float vl[4] = {bf16_lo(kl.x), bf16_hi(kl.x), bf16_lo(kl.y), bf16_hi(kl.y)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dgp[tn][e] = vr[e] * aKg[tn][e];
                dgl[tn][e] = gQl[tn][e] * vq[e] + gKl[tn][e] * vl[e] - gKr[tn][e] * vr[e];
            }
        }
#pragma unroll
        for (int tn = 0; tn < NT; ++tn) {
            float s4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) s4[e] = group_sum<16>(dgp[tn][e]);
            if (r16 == 0) *(float4 *)(sDg + (4 + wave) * DK + 16 * tn + 4 * g4) = make_float4(s4[0], s4[1], s4[2], s4[3]);
        }
    }
    lds_barrier();  // the operand arrays are free: Gamma goes over them

    // ---- stage 7: chain rule through Gamma, suffix sums ------------------------------
    float *sGm = (float *)(smem + L::oQl);  // fp32 [64][DK] Gamma
    float *sDl = (float *)sT;               // fp32 [64][DK] dg
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < CPT; ++e) sGm[(8 * rg + i) * DK + c0 + e] = g[i][e];
    lds_barrier();
    {
        const int row = R0 + r16;
        const bool ok = ok_row;
        const size_t th = th_row;
#pragma unroll
        for (int tn = 0; tn < NT; ++tn) {
            const int col = 16 * tn + 4 * g4;
            float dq4[4], dk4[4];
            const float4 g4v = *(const float4 *)(sGm + row * DK + col);
            const float gr[4] = {g4v.x, g4v.y, g4v.z, g4v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float gv = gr[e] * kLog2e;
                const float G = exp2_fast(gv), iG = exp2_fast(-gv);
                dq4[e] = gQl[tn][e] * G;
                dk4[e] = gKl[tn][e] * G + gKr[tn][e] * iG;
            }
            if (ok) {
                uint2 o;
                o.x = pack_bf16x2(dq4[0], dq4[1]);
                o.y = pack_bf16x2(dq4[2], dq4[3]);
                *(uint2 *)(p.dq + th * DK + col) = o;
                o.x = pack_bf16x2(dk4[0], dk4[1]);
                o.y = pack_bf16x2(dk4[2], dk4[3]);
                *(uint2 *)(p.dk + th * DK + col) = o;
            }
            *(float4 *)(sDl + row * DK + col) = make_float4(dgl[tn][0], dgl[tn][1], dgl[tn][2], dgl[tn][3]);
        }
        if (tid < kC && tid < m) p.dbeta[(size_t)(tok0 + tid) * H + h] = sDb[tid];
    }
    if (Nx.ok) load_in(Nx);  // the next job's q, k, log alpha, beta
    lds_barrier();
    if (GATE == kGateChannel) {
        // suffix sums over the 64 rows, four columns per thread: kThreads / (DK / 4) parts
        // of rows, part totals through LDS, then each part walks its rows backwards
        // (at most 8 parts: sGp holds 8 rows of DK)
        constexpr int NP = kThreads / (DK / 4) < 8 ? kThreads / (DK / 4) : 8, RP = kC / NP;
        const int col = 4 * (tid % (DK / 4)), part = tid / (DK / 4);
        const bool act = part < NP;
        if (act) {
            float4 ps = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int r = part * RP; r < (part + 1) * RP; ++r) {
                const float4 x = *(const float4 *)(sDl + r * DK + col);
                ps.x += x.x; ps.y += x.y; ps.z += x.z; ps.w += x.w;
            }
            *(float4 *)(sGp + part * DK + col) = ps;
        }
        lds_barrier();
        if (act) {
            // the last-row term: each wave's two parts, then the waves in order
            auto slot = [&](int w) {
                const float4 a = *(const float4 *)(sDg + w * DK + col), b = *(const float4 *)(sDg + (4 + w) * DK + col);
                return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
            };
            float4 acc = slot(0);
            for (int w = 1; w < 4; ++w) {
                const float4 x = slot(w);
                acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
            }
            for (int p2 = part + 1; p2 < NP; ++p2) {
                const float4 x = *(const float4 *)(sGp + p2 * DK + col);
                acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
            }
#pragma unroll
            for (int r = (part + 1) * RP - 1; r >= part * RP; --r) {
                const float4 x = *(const float4 *)(sDl + r * DK + col);
                acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
                if (r < m) *(float4 *)(p.dla + ((size_t)(tok0 + r) * H + h) * DK + col) = acc;
            }
        }
    } else if (GATE == kGateHead) {
        // row sums (four threads per row), the last-row term on row 63, then a suffix
        // scan over the rows in wave 0
        {
            const int row = tid >> 2, q = tid & 3;
            float s = 0.f;
            for (int col = q; col < DK; col += 4) s += sDl[row * DK + col];
            if (row == kC - 1)
                for (int col = q; col < DK; col += 4)
                    s += (((sDg[col] + sDg[4 * DK + col]) + (sDg[DK + col] + sDg[5 * DK + col])) +
                          (sDg[2 * DK + col] + sDg[6 * DK + col])) + (sDg[3 * DK + col] + sDg[7 * DK + col]);
            s += dpp<kDppXor1>(s);
            s += dpp<kDppXor2>(s);
            if (q == 0) sGp[row] = s;
        }
        lds_barrier();
        if (wave == 0) {
            float x = sGp[lane];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_down(x, off, 64);
                if (lane + off < 64) x += y;
            }
            if (lane < m) p.dla[(size_t)(tok0 + lane) * H + h] = x;
        }
    }
    lds_barrier();  // the next job overwrites LDS
    J = Nx;
    }
}

// ---------------------------------------------------------------------------------
// Per-chunk gradients of the gated DPLR form ("Diagonal Plus Low Rank" notes,
// section 3), with the write term scaled by beta (V' = Diag(beta) V):
//   F = I + (B<- A->^T strictly lower), E = F^-1, W = E B<-, BK = B<- K->^T strictly lower,
//   A_qk = Q<- K->^T, A_qa = Q<- A->^T (both on and below the diagonal),
//   N = -E BK V' - W S_p^T,  S_n = (S_p + V'^T K-> + N^T A->) Diag(gamma_C)
// and, with dSg = dS_n Diag(gamma_C):
//   dN = A-> dSg^T + A_qa^T dO,     dV'1 = K-> dSg^T + A_qk^T dO
//   dV' = dV'1 - (E BK)^T dN,       dV = Diag(beta) dV',  dbeta = rowsum(dV' V)
//   dW = -dN S_p,  Yc = dN V'^T,    dE = -Yc BK^T + dW B<-^T,  dF = -E^T dE E^T (strictly lower)
//   X = E^T Yc (strictly lower),    dOV = dO V'^T, dON = dO N^T (on and below the diagonal)
//   dQ<- = dO S_p + dOV K-> + dON A->
//   dB<- = E^T dW - X K-> + dF A->
//   dK-> = V' dSg + dOV^T Q<- - X^T B<-
//   dA-> = N dSg + dON^T Q<- + dF^T B<-
//   dg = dQ<- Q<- + dB<- B<- - dK-> K-> - dA-> A->, plus on the last row
//        sum_i S_n dS_n = sum_i S_p dSg + sum_r K-> (V' dSg) + sum_r A-> (N dSg)
// (the notes print dW with S_[t] and leave the state terms out of dK->, dA->; the
// forward definitions fix both).  V' is never stored: beta scales the fragments of V
// where they are read, and E BK is kept unscaled.
// ---------------------------------------------------------------------------------
template <int DK>
struct BwdDpSmem {
    static constexpr int KS = DK + 8, CS = kC + 8, VS = 32;
    static constexpr int QK = kC * KS * 2, CC = kC * CS * 2;
    static constexpr int oKr = 0;            // K->
    static constexpr int oAr = oKr + QK;     // A->
    static constexpr int oW = oAr + QK;      // W, then dW; before W: the inverse's temporaries
    static constexpr int oEBK = oW + QK;     // E BK (unscaled); then dON
    static constexpr int oQB = oEBK + CC;    // Q<-, B<-; during the dv loop the tile buffers
    static constexpr int oE = oQB + 2 * QK;  // E
    static constexpr int oBK = oE + CC;      // BK; then dE, then X
    static constexpr int oAqk = oBK + CC;    // A_qk; then Yc, Z, dF
    static constexpr int oAqa = oAqk + CC;   // A_qa; then dOV
    //   dv tile: S_p [32][KS], dSg [32][KS], V, dO, N, dN [64][VS]; over Q<-, B<- when it
    //   fits there (dk = 128), else in a region of its own
    static constexpr int tSp = 0, tdS = tSp + 32 * KS * 2, tV = tdS + 32 * KS * 2;
    static constexpr int tdO = tV + kC * VS * 2, tN = tdO + kC * VS * 2, tdN = tN + kC * VS * 2;
    static constexpr int tEnd = tdN + kC * VS * 2;
    //   the inverse: diagonal blocks of F fp32 [64][20], L, middle factor; over W and E BK
    //   when they fit there, else in a region of its own
    static constexpr int iKd = 0, iL = kC * 20 * 4, iTm = iL + CC, iEnd = iTm + CC;
    static constexpr bool kTileOverQB = tEnd <= 2 * QK, kInvOverW = iEnd <= QK + CC;
    static constexpr int oExtra = oAqa + CC;
    static constexpr int oTile = kTileOverQB ? oQB : oExtra;
    static constexpr int oInv = kInvOverW ? oW : oExtra + (kTileOverQB ? 0 : tEnd);
    static constexpr int oBeta = oExtra + (kTileOverQB ? 0 : tEnd) + (kInvOverW ? 0 : iEnd);
    static constexpr int oGam = oBeta + kC * 4;
    static constexpr int oGp = oGam + DK * 4;
    static constexpr int oDb = oGp + 8 * DK * 4;
    static constexpr int oDg = oDb + kC * 4;      // fp32 [8][DK] last-row term of dg, as above
    static constexpr int oSpf = oDg + 8 * DK * 4;
    static constexpr int bytes = oSpf + DK * 4;
    static_assert(kC * DK * 4 <= 2 * QK, "Gamma / dg fit over K->, A-> and over Q<-, B<-");
    static_assert(bytes <= 160 * 1024, "LDS");
};

template <int DK, int GATE>
__global__ __launch_bounds__(kThreads, 1) void kda_bwd_post_dplr_kernel(BwdParams p) {
    using L = BwdDpSmem<DK>;
    constexpr int KS = L::KS, CS = L::CS, VS = L::VS;
    constexpr int NT = DK / 16, CPT = DK / 32, WPR = CPT / 2;
    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    uint16_t *sKr = (uint16_t *)(smem + L::oKr), *sAr = (uint16_t *)(smem + L::oAr);
    uint16_t *sW = (uint16_t *)(smem + L::oW), *sEBK = (uint16_t *)(smem + L::oEBK);
    uint16_t *sQl = (uint16_t *)(smem + L::oQB), *sBl = sQl + kC * KS;
    uint16_t *sE = (uint16_t *)(smem + L::oE), *sBK = (uint16_t *)(smem + L::oBK);
    uint16_t *sAqk = (uint16_t *)(smem + L::oAqk), *sAqa = (uint16_t *)(smem + L::oAqa);
    char *sT = smem + L::oTile;
    uint16_t *sSp = (uint16_t *)(sT + L::tSp), *sdS = (uint16_t *)(sT + L::tdS);
    uint16_t *sV = (uint16_t *)(sT + L::tV), *sdO = (uint16_t *)(sT + L::tdO);
    uint16_t *sN = (uint16_t *)(sT + L::tN), *sdN = (uint16_t *)(sT + L::tdN);
    float *sKd = (float *)(smem + L::oInv + L::iKd);
    uint16_t *sL = (uint16_t *)(smem + L::oInv + L::iL), *sTm = (uint16_t *)(smem + L::oInv + L::iTm);
    float *sBeta = (float *)(smem + L::oBeta), *sGam = (float *)(smem + L::oGam);
    float *sGp = (float *)(smem + L::oGp), *sDb = (float *)(smem + L::oDb);
    float *sDg = (float *)(smem + L::oDg);
    float *sSpf = (float *)(smem + L::oSpf);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g4 = lane >> 4;
    const int H = p.H, DV = p.dv_;
    const int job = blockIdx.x;
    const int h = job % H;
    int n = 0, c = 0;
    if (!chunk_of(p, job / H, n, c)) return;  // workgroup-uniform
    long t0, t1;
    seq_bounds(p.cu, n, p.T, p.total, t0, t1, nullptr);
    const long tok0 = t0 + (long)c * kC;
    const int m = (int)((t1 - tok0) < kC ? (t1 - tok0) : kC);
    const size_t sbase = (size_t)(job / H) * H + h;
    const int R0 = 16 * wave;
    const int lo_k = R0 >= 32 ? 32 : 0;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};

    constexpr int kSPT = 32 * DK / 8 / kThreads;
    struct Tile {
        uint4 s[kSPT], d[kSPT], v, o;
    } pf;
    auto issue = [&](int j0) {
        const uint16_t *ps = p.S + (sbase * DV + j0) * DK;
        const uint16_t *pd = p.dS + (sbase * DV + j0) * DK;
#pragma unroll
        for (int i = 0; i < kSPT; ++i) {
            const int idx = tid + kThreads * i, r = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
            pf.s[i] = *(const uint4 *)(ps + (size_t)r * DK + c8);
            pf.d[i] = *(const uint4 *)(pd + (size_t)r * DK + c8);
        }
        const int r = tid >> 2, c8 = 8 * (tid & 3);
        const size_t off = ((size_t)(tok0 + (r < m ? r : 0)) * H + h) * DV + j0 + c8;
        pf.v = *(const uint4 *)(p.v + off);
        pf.o = *(const uint4 *)(p.dO + off);
    };

    // ---- inputs: q, b, k, a of this thread's rows and channels, then log alpha (one
    // memory round trip); the first dv tile is requested after them ------------------------
    const int rg = tid >> 5, c0 = CPT * (tid & 31);
    auto load_rows = [&](const bf16 *x, uint32_t (&xw)[8][WPR]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * rg + i;
            const size_t th = (size_t)(tok0 + (r < m ? r : 0)) * H + h;
            if constexpr (WPR == 2) {
                const uint2 a2 = *(const uint2 *)(x + th * DK + c0);
                xw[i][0] = a2.x; xw[i][WPR - 1] = a2.y;
            } else {
                xw[i][0] = *(const uint32_t *)(x + th * DK + c0);
            }
        }
    };
    uint32_t iq[8][WPR], ib[8][WPR], ik[8][WPR], ia[8][WPR];
    load_rows(p.q, iq);
    load_rows(p.b, ib);
    load_rows(p.k, ik);
    load_rows(p.a, ia);
    float g[8][CPT];
    {
        float la[8][CPT];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * rg + i;
            const size_t th = (size_t)(tok0 + (r < m ? r : 0)) * H + h;
#pragma unroll
            for (int e = 0; e < CPT; ++e) la[i][e] = 0.f;
            if (GATE == kGateChannel) {
                if constexpr (CPT == 4) {
                    const float4 x = *(const float4 *)(p.la + th * DK + c0);
                    la[i][0] = x.x; la[i][CPT > 1 ? 1 : 0] = x.y;
                    la[i][CPT > 2 ? 2 : 0] = x.z; la[i][CPT > 3 ? 3 : 0] = x.w;
                } else {
                    const float2 x = *(const float2 *)(p.la + th * DK + c0);
                    la[i][0] = x.x; la[i][CPT > 1 ? 1 : 0] = x.y;
                }
            } else if (GATE == kGateHead) {
                const float x = p.la[th];
#pragma unroll
                for (int e = 0; e < CPT; ++e) la[i][e] = x;
            }
            if (r >= m)
#pragma unroll
                for (int e = 0; e < CPT; ++e) la[i][e] = 0.f;
        }
        float run[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) run[e] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                run[e] += la[i][e];
                g[i][e] = run[e];
            }
#pragma unroll
        for (int e = 0; e < CPT; ++e) sGp[rg * DK + c0 + e] = run[e];
        lds_barrier();
        g_shift_all(g, sGp + c0, rg, sSpf + c0);
    }
    flag_wide_gate(g, wave, lane, p.err);
    issue(0);
    // Q<-, B<- (scale e^g) or K->, A-> (scale e^-g) of two loaded inputs, bf16 into LDS
    auto scaled = [&](const uint32_t (&xw)[8][WPR], const uint32_t (&yw)[8][WPR], uint16_t *dx,
                      uint16_t *dy, bool up) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * rg + i;
            uint32_t ox[WPR], oy[WPR];
            const uint32_t keep = 8 * rg + i < m ? 0xffffffffu : 0u;  // rows past the end are zero
#pragma unroll
            for (int w = 0; w < WPR; ++w) {
                const float s0 = up ? g[i][2 * w] : -g[i][2 * w], s1 = up ? g[i][2 * w + 1] : -g[i][2 * w + 1];
                const float e0 = exp2_fast(s0 * kLog2e), e1 = exp2_fast(s1 * kLog2e);
                ox[w] = pack_bf16x2(bf16_lo(xw[i][w] & keep) * e0, bf16_hi(xw[i][w] & keep) * e1);
                oy[w] = pack_bf16x2(bf16_lo(yw[i][w] & keep) * e0, bf16_hi(yw[i][w] & keep) * e1);
            }
            if constexpr (WPR == 2) {
                *(uint2 *)(dx + r * KS + c0) = make_uint2(ox[0], ox[WPR - 1]);
                *(uint2 *)(dy + r * KS + c0) = make_uint2(oy[0], oy[WPR - 1]);
            } else {
                *(uint32_t *)(dx + r * KS + c0) = ox[0];
                *(uint32_t *)(dy + r * KS + c0) = oy[0];
            }
        }
    };
    scaled(iq, ib, sQl, sBl, true);
    scaled(ik, ia, sKr, sAr, false);
    if (rg == 7)
#pragma unroll
        for (int e = 0; e < CPT; ++e) sGam[c0 + e] = exp2_fast(g[7][e] * kLog2e);
    if (tid < kC) sBeta[tid] = tid < m ? p.beta[(size_t)(tok0 + tid) * H + h] : 0.f;
    for (int i = tid; i < kC; i += kThreads) sDb[i] = 0.f;
    for (int idx = tid; idx < kC * CS / 8; idx += kThreads) ((uint4 *)sE)[idx] = make_uint4(0u, 0u, 0u, 0u);
    lds_barrier();

    // ---- C x C products: F's strictly lower part (fp32 diagonal blocks, bf16 L), BK, A_qk, A_qa
    for (int tj = 0; tj < 4; ++tj) {
        f32x4 ba = z, bk = z, aq = z, aa = z;
        if (tj <= wave) {
            ba = mma_tile<false, true, DK>(sBl, KS, sAr, KS, R0, 16 * tj, 0, DK, z, lane);
            bk = mma_tile<false, true, DK>(sBl, KS, sKr, KS, R0, 16 * tj, 0, DK, z, lane);
            aq = mma_tile<false, true, DK>(sQl, KS, sKr, KS, R0, 16 * tj, 0, DK, z, lane);
            aa = mma_tile<false, true, DK>(sQl, KS, sAr, KS, R0, 16 * tj, 0, DK, z, lane);
        }
        const int row = R0 + r16;
        float vba[4], vbk[4], vaq[4], vaa[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = 16 * tj + 4 * g4 + e;
            vba[e] = col < row ? ba[e] : 0.f;
            vbk[e] = col < row ? bk[e] : 0.f;
            vaq[e] = col <= row ? aq[e] : 0.f;
            vaa[e] = col <= row ? aa[e] : 0.f;
            if (tj == wave) sKd[row * 20 + 4 * g4 + e] = vba[e];
        }
        const int o = row * CS + 16 * tj + 4 * g4;
        store4(sL + o, vba[0], vba[1], vba[2], vba[3]);
        store4(sBK + o, vbk[0], vbk[1], vbk[2], vbk[3]);
        store4(sAqk + o, vaq[0], vaq[1], vaq[2], vaq[3]);
        store4(sAqa + o, vaa[0], vaa[1], vaa[2], vaa[3]);
    }
    lds_barrier();

    // ---- E = F^-1: diagonal blocks by forward substitution, then two doubling levels ----
    {
        const int jl = lane >> 2, s4 = lane & 3, j = R0 + jl;
        float xs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int u = 0; u < (i + 3) / 4; ++u) acc += sKd[(R0 + i) * 20 + 4 * u + s4] * xs[u];
            acc += dpp<kDppXor1>(acc);
            acc += dpp<kDppXor2>(acc);
            const float xi = (i == jl ? 1.f : 0.f) - acc;
            if (s4 == (i & 3)) xs[i >> 2] = xi;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) sE[(R0 + 4 * u + s4) * CS + j] = __builtin_bit_cast(uint16_t, (__bf16)xs[u]);
    }
    lds_barrier();
    if (wave == 0 || wave == 2) {
        const int o = wave == 0 ? 0 : 32;
        f32x4 t = mfma16(frag4_tr(sE + o, o, CS, 0, lane), frag4(sL + o, o + 16 + r16, CS, 4 * g4), z);
        store4(sTm + (o + 16 + r16) * CS + o + 4 * g4, t[0], t[1], t[2], t[3]);
        asm volatile("" ::: "memory");
        t = mfma16(frag4_tr(sTm + o, o + 16, CS, 0, lane), frag4(sE + o + 16, o + 16 + r16, CS, 4 * g4), z);
        store4(sE + (o + 16 + r16) * CS + o + 4 * g4, -t[0], -t[1], -t[2], -t[3]);
    }
    lds_barrier();
    {
        const int m0 = 32 + 16 * (wave >> 1), n0 = 16 * (wave & 1);
        const f32x4 t = mma_tile<false, false, kC>(sL, CS, sE, CS, m0, n0, 0, 32, z, lane);
        store4(sTm + (m0 + r16) * CS + n0 + 4 * g4, t[0], t[1], t[2], t[3]);
        lds_barrier();
        const f32x4 cc = mma_tile<false, false, kC>(sE + 32, CS, sTm + 32 * CS, CS, m0, n0, 0, 32, z, lane);
        lds_barrier();
        store4(sE + (m0 + r16) * CS + n0 + 4 * g4, -cc[0], -cc[1], -cc[2], -cc[3]);
    }
    lds_barrier();

    // ---- W = E B<-, E BK -------------------------------------------------------------------
    {
        const int k1 = R0 + 16 <= 32 ? 32 : 64;  // E is lower triangular
        f32x4 wv[NT], eb[4];
#pragma unroll
        for (int tn = 0; tn < NT; ++tn) wv[tn] = mma_tile<false, false, kC>(sE, CS, sBl, KS, R0, 16 * tn, 0, k1, z, lane);
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) eb[tj] = mma_tile<false, false, kC>(sE, CS, sBK, CS, R0, 16 * tj, 0, k1, z, lane);
        lds_barrier();  // the inverse's temporaries under W and E BK are read
#pragma unroll
        for (int tn = 0; tn < NT; ++tn)
            store4(sW + (R0 + r16) * KS + 16 * tn + 4 * g4, wv[tn][0], wv[tn][1], wv[tn][2], wv[tn][3]);
#pragma unroll
        for (int tj = 0; tj < 4; ++tj)
            store4(sEBK + (R0 + r16) * CS + 16 * tj + 4 * g4, eb[tj][0], eb[tj][1], eb[tj][2], eb[tj][3]);
    }
    lds_barrier();  // Q<-, B<- are not read again before they are rebuilt after the dv loop

    // ---- the dv tiles (buffers over Q<-, B<-) -----------------------------------------
    f32x4 aQ[NT], aW[NT], aKs[NT], aAs[NT], aOV[4], aON[4], aY[4];
#pragma unroll
    for (int t = 0; t < NT; ++t) aQ[t] = aW[t] = aKs[t] = aAs[t] = z;
#pragma unroll
    for (int t = 0; t < 4; ++t) aOV[t] = aON[t] = aY[t] = z;
    float gpart[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float dbp = 0.f;  // rowsum of dV' V for this lane's row and columns
    const float brow = sBeta[R0 + r16];
    // beta of the 8 rows 8(lane/16) + k0 + 0..7 (the contraction index of a transposed
    // fragment over the chunk's rows), to scale V into V' where it is read
    auto bscale8 = [&](bf16x8 f, int k0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (__bf16)((float)f[i] * sBeta[k0 + 8 * g4 + i]);
        return f;
    };
    auto bscale = [&](bf16x8 f, float bs) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (__bf16)((float)f[i] * bs);
        return f;
    };
    for (int j0 = 0; j0 < DV; j0 += 32) {
        {
#pragma unroll
            for (int i = 0; i < kSPT; ++i) {
                const int idx = tid + kThreads * i, r = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
                const uint32_t w4[4] = {pf.d[i].x, pf.d[i].y, pf.d[i].z, pf.d[i].w};
                const uint32_t s4[4] = {pf.s[i].x, pf.s[i].y, pf.s[i].z, pf.s[i].w};
                uint32_t o4[4], p4[4];
                // the eight columns' gamma_C and 2^n, two vector reads each
                const float4 ga = *(const float4 *)(sGam + c8), gb = *(const float4 *)(sGam + c8 + 4);
                const float4 fa = *(const float4 *)(sSpf + c8), fb = *(const float4 *)(sSpf + c8 + 4);
                const float gm[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
                const float sf[8] = {fa.x, fa.y, fa.z, fa.w, fb.x, fb.y, fb.z, fb.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float d0 = bf16_lo(w4[e]) * gm[2 * e], d1 = bf16_hi(w4[e]) * gm[2 * e + 1];
                    const float s0 = bf16_lo(s4[e]) * sf[2 * e], s1 = bf16_hi(s4[e]) * sf[2 * e + 1];
                    o4[e] = pack_bf16x2(d0, d1);
                    p4[e] = pack_bf16x2(s0, s1);
                    gpart[2 * e] += s0 * d0;
                    gpart[2 * e + 1] += s1 * d1;
                }
                *(uint4 *)(sSp + r * KS + c8) = make_uint4(p4[0], p4[1], p4[2], p4[3]);
                *(uint4 *)(sdS + r * KS + c8) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
            }
            const int r = tid >> 2, c8 = 8 * (tid & 3);
            const uint32_t keep = 0u - (uint32_t)(r < m);
            *(uint4 *)(sV + r * VS + c8) = make_uint4(pf.v.x & keep, pf.v.y & keep, pf.v.z & keep, pf.v.w & keep);
            *(uint4 *)(sdO + r * VS + c8) = make_uint4(pf.o.x & keep, pf.o.y & keep, pf.o.z & keep, pf.o.w & keep);
        }
        if (j0 + 32 < DV) issue(j0 + 32);
        lds_barrier();
        // N = -(E BK) V' - W S_p^T,  dN = A-> dSg^T + A_qa^T dO
        {
            const int k1 = R0 + 16 <= 32 ? 32 : 64;
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) {
                const int n0 = 16 * tn;
                f32x4 cm = z;
                for (int k = 0; k < k1; k += 32)
                    cm = mfma(bscale8(frag_tr(sV, k, VS, n0, lane), k), frag(sEBK, R0 + r16, CS, k + 8 * g4), cm);
                const f32x4 ws = mma_tile<false, true, DK>(sW, KS, sSp, KS, R0, n0, 0, DK, z, lane);
                f32x4 dn = mma_tile<false, true, DK>(sAr, KS, sdS, KS, R0, n0, 0, DK, z, lane);
                dn = mma_tile<true, false, kC>(sAqa, CS, sdO, VS, R0, n0, lo_k, kC, dn, lane);
                store4(sN + (R0 + r16) * VS + n0 + 4 * g4, -cm[0] - ws[0], -cm[1] - ws[1], -cm[2] - ws[2], -cm[3] - ws[3]);
                store4(sdN + (R0 + r16) * VS + n0 + 4 * g4, dn[0], dn[1], dn[2], dn[3]);
            }
        }
        lds_barrier();
        {
            const int row = R0 + r16;
            // dV' = K-> dSg^T + A_qk^T dO - (E BK)^T dN; dV = Diag(beta) dV'; dbeta += dV' . V
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) {
                const int n0 = 16 * tn;
                f32x4 d = mma_tile<false, true, DK>(sKr, KS, sdS, KS, R0, n0, 0, DK, z, lane);
                d = mma_tile<true, false, kC>(sAqk, CS, sdO, VS, R0, n0, lo_k, kC, d, lane);
                const f32x4 e2 = mma_tile<true, false, kC>(sEBK, CS, sdN, VS, R0, n0, lo_k, kC, z, lane);
                const uint2 vw = *(const uint2 *)(sV + row * VS + n0 + 4 * g4);
                const float vv[4] = {bf16_lo(vw.x), bf16_hi(vw.x), bf16_lo(vw.y), bf16_hi(vw.y)};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    d[e] -= e2[e];
                    dbp += d[e] * vv[e];
                }
                if (row < m) {
                    uint2 o;
                    o.x = pack_bf16x2(brow * d[0], brow * d[1]);
                    o.y = pack_bf16x2(brow * d[2], brow * d[3]);
                    *(uint2 *)(p.dv + ((size_t)(tok0 + row) * H + h) * DV + j0 + n0 + 4 * g4) = o;
                }
            }
            // contractions over the tile: dQ<- += dO S_p, dW += dN S_p, dK->s += V' dSg, dA->s += N dSg
            const bf16x8 fdo = frag(sdO, row, VS, 8 * g4);
            const bf16x8 fdn = frag(sdN, row, VS, 8 * g4);
            const bf16x8 fvp = bscale(frag(sV, row, VS, 8 * g4), brow);
            const bf16x8 fn = frag(sN, row, VS, 8 * g4);
#pragma unroll
            for (int tn = 0; tn < NT; ++tn) {
                const bf16x8 fs = frag_tr(sSp, 0, KS, 16 * tn, lane);
                const bf16x8 fd = frag_tr(sdS, 0, KS, 16 * tn, lane);
                aQ[tn] = mfma(fs, fdo, aQ[tn]);
                aW[tn] = mfma(fs, fdn, aW[tn]);
                aKs[tn] = mfma(fd, fvp, aKs[tn]);
                aAs[tn] = mfma(fd, fn, aAs[tn]);
            }
            // dOV += dO V'^T, dON += dO N^T (lower tiles); Yc += dN V'^T
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                const bf16x8 fv = bscale(frag(sV, 16 * tj + r16, VS, 8 * g4), sBeta[16 * tj + r16]);
                if (tj <= wave) {
                    aOV[tj] = mfma(fv, fdo, aOV[tj]);
                    aON[tj] = mfma(frag(sN, 16 * tj + r16, VS, 8 * g4), fdo, aON[tj]);
                }
                aY[tj] = mfma(fv, fdn, aY[tj]);
            }
        }
        lds_barrier();
    }

    // ---- after the dv loop: dW, dOV, dON, Yc to LDS; Q<-, B<- rebuilt ---------------------
    uint16_t *sdW = sW, *sOV = sAqa, *sON = sEBK, *sY = sAqk;
    {
        const int row = R0 + r16;
#pragma unroll
        for (int tn = 0; tn < NT; ++tn)
            store4(sdW + row * KS + 16 * tn + 4 * g4, -aW[tn][0], -aW[tn][1], -aW[tn][2], -aW[tn][3]);
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            float ov[4], on[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool lo = 16 * tj + 4 * g4 + e <= row;
                ov[e] = lo ? aOV[tj][e] : 0.f;
                on[e] = lo ? aON[tj][e] : 0.f;
            }
            const int o = row * CS + 16 * tj + 4 * g4;
            store4(sOV + o, ov[0], ov[1], ov[2], ov[3]);
            store4(sON + o, on[0], on[1], on[2], on[3]);
            store4(sY + o, aY[tj][0], aY[tj][1], aY[tj][2], aY[tj][3]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = gpart[e];
#pragma unroll
            for (int off = DK / 8; off < 64; off <<= 1) x += __shfl_xor(x, off);
            if (lane < DK / 8) sDg[wave * DK + 8 * lane + e] = x;  // this wave's slot
        }
        dbp += __shfl_xor(dbp, 16);
        dbp += __shfl_xor(dbp, 32);
        if (g4 == 0) sDb[row] = dbp;
    }
    load_rows(p.q, iq);  // Q<-, B<- again, over the dv-tile buffers
    load_rows(p.b, ib);
    scaled(iq, ib, sQl, sBl, true);
    lds_barrier();
    // dE = -Yc BK^T + dW B<-^T;  X = E^T Yc (strictly lower)
    f32x4 vdE[4], vX[4];
    {
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            f32x4 d = mma_tile<false, true, kC>(sY, CS, sBK, CS, R0, 16 * tj, 0, kC, z, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) d[e] = -d[e];
            vdE[tj] = mma_tile<false, true, DK>(sdW, KS, sBl, KS, R0, 16 * tj, 0, DK, d, lane);
            vX[tj] = mma_tile<true, false, kC>(sE, CS, sY, CS, R0, 16 * tj, lo_k, kC, z, lane);
        }
    }
    lds_barrier();  // Yc and BK are read
    uint16_t *sdE = sBK;
    {
        const int row = R0 + r16;
#pragma unroll
        for (int tj = 0; tj < 4; ++tj)
            store4(sdE + row * CS + 16 * tj + 4 * g4, vdE[tj][0], vdE[tj][1], vdE[tj][2], vdE[tj][3]);
    }
    lds_barrier();
    // Z = E^T dE
    f32x4 vZ[4];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) vZ[tj] = mma_tile<true, false, kC>(sE, CS, sdE, CS, R0, 16 * tj, lo_k, kC, z, lane);
    lds_barrier();  // dE is read
    uint16_t *sZ = sAqk, *sX = sBK;
    {
        const int row = R0 + r16;
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            float xv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[e] = 16 * tj + 4 * g4 + e < row ? vX[tj][e] : 0.f;
            const int o = row * CS + 16 * tj + 4 * g4;
            store4(sZ + o, vZ[tj][0], vZ[tj][1], vZ[tj][2], vZ[tj][3]);
            store4(sX + o, xv[0], xv[1], xv[2], xv[3]);
        }
    }
    lds_barrier();
    // dF = -Z E^T (strictly lower)
    f32x4 vF[4];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
        vF[tj] = z;
        if (tj <= wave) vF[tj] = mma_tile<false, true, kC>(sZ, CS, sE, CS, R0, 16 * tj, 0, kC, z, lane);
    }
    lds_barrier();  // Z is read
    uint16_t *sdF = sAqk;
    {
        const int row = R0 + r16;
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            float fv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) fv[e] = 16 * tj + 4 * g4 + e < row ? -vF[tj][e] : 0.f;
            store4(sdF + row * CS + 16 * tj + 4 * g4, fv[0], fv[1], fv[2], fv[3]);
        }
    }
    lds_barrier();

    // ---- final products -------------------------------------------------------------------
    const bool ok_row = R0 + r16 < m;
    const size_t th_row = (size_t)(tok0 + (ok_row ? R0 + r16 : 0)) * H + h;
    f32x4 gQ[NT], gB[NT], gK[NT], gA[NT];
    // dg of this lane's row and columns, dQ<- Q<- + dB<- B<- - dK-> K-> - dA-> A->, from
    // the bf16 operands the products used, so that the pairs of every Gram product cancel
    // exactly inside the suffix sums (as in the KDA kernel)
    float dgl[NT][4];
    {
        const int row = R0 + r16;
        float dgp[NT][4];
#pragma unroll
        for (int tn = 0; tn < NT; ++tn) {
            const int n0 = 16 * tn;
            f32x4 q2 = mma_tile<false, false, kC>(sOV, CS, sKr, KS, R0, n0, 0, kC, aQ[tn], lane);
            gQ[tn] = mma_tile<false, false, kC>(sON, CS, sAr, KS, R0, n0, 0, kC, q2, lane);
            f32x4 b2 = mma_tile<true, false, kC>(sE, CS, sdW, KS, R0, n0, lo_k, kC, z, lane);
            const f32x4 xk2 = mma_tile<false, false, kC>(sX, CS, sKr, KS, R0, n0, 0, kC, z, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) b2[e] -= xk2[e];
            gB[tn] = mma_tile<false, false, kC>(sdF, CS, sAr, KS, R0, n0, 0, kC, b2, lane);
            f32x4 k2 = mma_tile<true, false, kC>(sOV, CS, sQl, KS, R0, n0, lo_k, kC, aKs[tn], lane);
            const f32x4 xb2 = mma_tile<true, false, kC>(sX, CS, sBl, KS, R0, n0, lo_k, kC, z, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) k2[e] -= xb2[e];
            gK[tn] = k2;
            f32x4 a2 = mma_tile<true, false, kC>(sON, CS, sQl, KS, R0, n0, lo_k, kC, aAs[tn], lane);
            gA[tn] = mma_tile<true, false, kC>(sdF, CS, sBl, KS, R0, n0, lo_k, kC, a2, lane);
            // last-row term: sum over rows of K-> (V' dSg) + A-> (N dSg)
            const uint2 kr = *(const uint2 *)(sKr + row * KS + n0 + 4 * g4);
            const uint2 ar = *(const uint2 *)(sAr + row * KS + n0 + 4 * g4);
            const uint2 ql = *(const uint2 *)(sQl + row * KS + n0 + 4 * g4);
            const uint2 bl = *(const uint2 *)(sBl + row * KS + n0 + 4 * g4);
            const float vk[4] = {bf16_lo(kr.x), bf16_hi(kr.x), bf16_lo(kr.y), bf16_hi(kr.y)};
            const float va[4] = {bf16_lo(ar.x), bf16_hi(ar.x), bf16_lo(ar.y), bf16_hi(ar.y)};
            const float vq[4] = {bf16_lo(ql.x), bf16_hi(ql.x), bf16_lo(ql.y), bf16_hi(ql.y)};
            const float vb[4] = {bf16_lo(bl.x), bf16_hi(bl.x), bf16_lo(bl.y), bf16_hi(bl.y)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dgp[tn][e] = vk[e] * aKs[tn][e] + va[e] * aAs[tn][e];
                dgl[tn][e] = gQ[tn][e] * vq[e] + gB[tn][e] * vb[e] - gK[tn][e] * vk[e] - gA[tn][e] * va[e];
            }
        }
#pragma unroll
        for (int tn = 0; tn < NT; ++tn) {
            float s4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) s4[e] = group_sum<16>(dgp[tn][e]);
            if (r16 == 0) *(float4 *)(sDg + (4 + wave) * DK + 16 * tn + 4 * g4) = make_float4(s4[0], s4[1], s4[2], s4[3]);
        }
    }
    lds_barrier();  // the operand arrays are free: Gamma over K->, A->, dg over Q<-, B<-

    // ---- chain rule through Gamma, suffix sums -------------------------------------------
    float *sGm = (float *)(smem + L::oKr);
    float *sDl = (float *)(smem + L::oQB);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < CPT; ++e) sGm[(8 * rg + i) * DK + c0 + e] = g[i][e];
    lds_barrier();
    {
        const int row = R0 + r16;
#pragma unroll
        for (int tn = 0; tn < NT; ++tn) {
            const int col = 16 * tn + 4 * g4;
            float oq[4], ok4[4], oa[4], ob[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float gv = sGm[row * DK + col + e] * kLog2e;
                const float G = exp2_fast(gv), iG = exp2_fast(-gv);
                oq[e] = gQ[tn][e] * G;
                ob[e] = gB[tn][e] * G;
                ok4[e] = gK[tn][e] * iG;
                oa[e] = gA[tn][e] * iG;
            }
            if (ok_row) {
                const size_t o = th_row * DK + col;
                uint2 w;
                w.x = pack_bf16x2(oq[0], oq[1]); w.y = pack_bf16x2(oq[2], oq[3]);
                *(uint2 *)(p.dq + o) = w;
                w.x = pack_bf16x2(ok4[0], ok4[1]); w.y = pack_bf16x2(ok4[2], ok4[3]);
                *(uint2 *)(p.dk + o) = w;
                w.x = pack_bf16x2(oa[0], oa[1]); w.y = pack_bf16x2(oa[2], oa[3]);
                *(uint2 *)(p.da + o) = w;
                w.x = pack_bf16x2(ob[0], ob[1]); w.y = pack_bf16x2(ob[2], ob[3]);
                *(uint2 *)(p.db + o) = w;
            }
            *(float4 *)(sDl + row * DK + col) = make_float4(dgl[tn][0], dgl[tn][1], dgl[tn][2], dgl[tn][3]);
        }
        if (tid < kC && tid < m) p.dbeta[(size_t)(tok0 + tid) * H + h] = sDb[tid];
    }
    lds_barrier();
    if (GATE == kGateChannel) {
        // suffix sums over the 64 rows, four columns per thread: kThreads / (DK / 4) parts
        // of rows, part totals through LDS, then each part walks its rows backwards
        // (at most 8 parts: sGp holds 8 rows of DK)
        constexpr int NP = kThreads / (DK / 4) < 8 ? kThreads / (DK / 4) : 8, RP = kC / NP;
        const int col = 4 * (tid % (DK / 4)), part = tid / (DK / 4);
        const bool act = part < NP;
        if (act) {
            float4 ps = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int r = part * RP; r < (part + 1) * RP; ++r) {
                const float4 x = *(const float4 *)(sDl + r * DK + col);
                ps.x += x.x; ps.y += x.y; ps.z += x.z; ps.w += x.w;
            }
            *(float4 *)(sGp + part * DK + col) = ps;
        }
        lds_barrier();
        if (act) {
            // the last-row term: each wave's two parts, then the waves in order
            auto slot = [&](int w) {
                const float4 a = *(const float4 *)(sDg + w * DK + col), b = *(const float4 *)(sDg + (4 + w) * DK + col);
                return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
            };
            float4 acc = slot(0);
            for (int w = 1; w < 4; ++w) {
                const float4 x = slot(w);
                acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
            }
            for (int p2 = part + 1; p2 < NP; ++p2) {
                const float4 x = *(const float4 *)(sGp + p2 * DK + col);
                acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
            }
#pragma unroll
            for (int r = (part + 1) * RP - 1; r >= part * RP; --r) {
                const float4 x = *(const float4 *)(sDl + r * DK + col);
                acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
                if (r < m) *(float4 *)(p.dla + ((size_t)(tok0 + r) * H + h) * DK + col) = acc;
            }
        }
    } else if (GATE == kGateHead) {
        {
            const int row = tid >> 2, q4 = tid & 3;
            float sacc = 0.f;
            for (int col = q4; col < DK; col += 4) sacc += sDl[row * DK + col];
            if (row == kC - 1)
                for (int col = q4; col < DK; col += 4)
                    sacc += (((sDg[col] + sDg[4 * DK + col]) + (sDg[DK + col] + sDg[5 * DK + col])) +
                             (sDg[2 * DK + col] + sDg[6 * DK + col])) + (sDg[3 * DK + col] + sDg[7 * DK + col]);
            sacc += dpp<kDppXor1>(sacc);
            sacc += dpp<kDppXor2>(sacc);
            if (q4 == 0) sGp[row] = sacc;
        }
        lds_barrier();
        if (wave == 0) {
            float x = sGp[lane];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_down(x, off, 64);
                if (lane + off < 64) x += y;
            }
            if (lane < m) p.dla[(size_t)(tok0 + lane) * H + h] = x;
        }
    }
}

}  // namespace
}  // namespace gdr
