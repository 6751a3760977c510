// Fused chunkwise forward for the KDA family (a = k, b = beta k) with bf16
// inputs, on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
//
// One workgroup (8 waves) per (sequence, head, 32-wide dv tile).  The state
// tile S[dv 32][dk] lives in fp32 MFMA accumulators for the whole sequence; a
// bf16 copy in LDS feeds the products.  Per chunk of 64 tokens, following the
// KDA chunk form ("Kimi Delta Attention backward" notes, forward recap):
//
//   1. g = in-chunk inclusive prefix sum of log alpha (per channel or per head)
//      Q<- = Q e^g, K<- = K e^g, K-> = K e^-g, K^ = K e^(g_C - g)  -> LDS (bf16)
//   2. G = K<- K->^T and A_qk = Q<- K->^T on the lower 16x16 tiles (MFMA);
//      L = Diag(beta)(G, strictly lower), A_qk masked to the lower triangle
//   3. At = (I + L)^-1 by blocks ("DeltaNet" notes, section 4.2): the four
//      16x16 diagonal blocks by forward substitution, then the off-diagonal
//      blocks with the two-block form [A11 0; A21 A22]^-1 =
//      [A11^-1 0; -A22^-1 A21 A11^-1 A22^-1], first at 32 then at 64 rows
//   4. W = At Diag(beta) K<- and U = At Diag(beta) V (MFMA)
//   5. serial in the state: V_new = U - W S^T, O = Q<- S^T + A_qk V_new,
//      S = S Diag(gamma_C) + V_new^T K^   (all MFMA)
//
// Operand layout of the 16x16x32 MFMA as used here: lane l feeds A[l%16][8*(l/16)+0..7]
// and B[8*(l/16)+0..7][l%16] (eight contiguous bf16 along the contraction), and
// receives D[4*(l/16)+0..3][l%16].  Every product is arranged so both operands
// are read as 16-byte rows of an LDS array that is contiguous along the
// contraction index; arrays contracted over chunk rows are stored transposed.
#include "gdr_common.h"

namespace gdr {
namespace {

constexpr int kC = 64;        // chunk size
constexpr int kDVT = 32;      // dv columns per workgroup
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCS = kC + 8;   // bf16 row stride of [*][64] arrays (16 B pad)
constexpr int kXS = kC + 1;   // fp32 row stride of the 64x64 inverse
constexpr int kTS = 33;       // fp32 row stride of the inverse's temporaries

struct KdaParams {
    const bf16 *q, *k, *v;
    const float *la, *beta, *S0;
    bf16 *O;
    float *Sf;
    const int32_t *cu;
    int *err;
    long total;
    int H, T, dv, n_tiles;
};

template <int DK>
struct Smem {
    static constexpr int KS = DK + 8;  // bf16 row stride of [*][DK] arrays
    static constexpr int oKl = 0;                          // K<-  [64][KS]; later W
    static constexpr int oKr = oKl + kC * KS * 2;          // K->  [64][KS]
    static constexpr int oQl = oKr + kC * KS * 2;          // Q<-  [64][KS]
    static constexpr int oKlT = oQl + kC * KS * 2;         // K<-^T [DK][kCS]
    static constexpr int oKhT = oKlT + DK * kCS * 2;       // K^^T  [DK][kCS]
    static constexpr int oVT = oKhT + DK * kCS * 2;        // V^T   [32][kCS]
    static constexpr int oAb = oVT + kDVT * kCS * 2;       // At Diag(beta) [64][kCS]
    static constexpr int oAqk = oAb + kC * kCS * 2;        // A_qk [64][kCS]
    static constexpr int oS = oAqk + kC * kCS * 2;         // S bf16 [32][KS]
    static constexpr int oVnT = oS + kDVT * KS * 2;        // V_new^T [32][kCS]
    static constexpr int oX = oVnT + kDVT * kCS * 2;       // fp32 [64][kXS]
    static constexpr int oTmp = oX + kC * kXS * 4;         // fp32 [32][kTS]
    static constexpr int oBeta = oTmp + 32 * kTS * 4;      // fp32 [64]
    static constexpr int oGC = oBeta + kC * 4;             // fp32 [DK]
    static constexpr int oRow = oGC + DK * 4;              // fp32 [3][64] (head gate)
    static constexpr int bytes = oRow + 3 * kC * 4;
    static_assert(bytes <= 160 * 1024, "LDS budget");
    static_assert(oKr % 16 == 0 && oQl % 16 == 0 && oKlT % 16 == 0 && oKhT % 16 == 0 &&
                      oVT % 16 == 0 && oAb % 16 == 0 && oAqk % 16 == 0 && oS % 16 == 0 &&
                      oVnT % 16 == 0 && oX % 16 == 0,
                  "16-byte aligned operand arrays");
};

__device__ __forceinline__ bf16x8 frag(const uint16_t *base, int row, int stride, int col) {
    return *(const bf16x8 *)(base + row * stride + col);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void store4(uint16_t *dst, float x0, float x1, float x2, float x3) {
    uint2 w;
    w.x = pack_bf16x2(x0, x1);
    w.y = pack_bf16x2(x2, x3);
    *(uint2 *)dst = w;
}

template <int DK, int GATE>
__global__ __launch_bounds__(kThreads) void kda_mfma_kernel(KdaParams p) {
    using L = Smem<DK>;
    constexpr int KS = L::KS;
    constexpr int NCB = DK / 4;            // 4-channel blocks in the gate stage
    constexpr int NRB = kThreads / NCB;    // row blocks in the gate stage
    constexpr int RPT = kC / NRB;          // rows per thread in the gate stage
    constexpr int NST = (DK / 16) * 2 / kWaves;  // state tiles per wave
    static_assert(RPT == 2 || RPT == 4, "gate-stage layout");
    static_assert(NST >= 1, "state tiling");

    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    uint16_t *sKl = (uint16_t *)(smem + L::oKl);
    uint16_t *sW = sKl;
    uint16_t *sKr = (uint16_t *)(smem + L::oKr);
    uint16_t *sQl = (uint16_t *)(smem + L::oQl);
    uint16_t *sKlT = (uint16_t *)(smem + L::oKlT);
    uint16_t *sKhT = (uint16_t *)(smem + L::oKhT);
    uint16_t *sVT = (uint16_t *)(smem + L::oVT);
    uint16_t *sAb = (uint16_t *)(smem + L::oAb);
    uint16_t *sAqk = (uint16_t *)(smem + L::oAqk);
    uint16_t *sS = (uint16_t *)(smem + L::oS);
    uint16_t *sVnT = (uint16_t *)(smem + L::oVnT);
    float *sX = (float *)(smem + L::oX);
    float *sTmp = (float *)(smem + L::oTmp);
    float *sBeta = (float *)(smem + L::oBeta);
    float *sGC = (float *)(smem + L::oGC);
    float *sRow = (float *)(smem + L::oRow);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;   // row (A) / column (B, D) index within a tile
    const int lg = lane >> 4;    // 8-wide contraction group (A, B) / 4-row group (D)

    const int H = p.H, DV = p.dv;
    const int lin = xcd_linear_index(blockIdx.x, gridDim.x);
    const int tile = lin % p.n_tiles;
    const int h = (lin / p.n_tiles) % H;
    const int n = lin / (p.n_tiles * H);
    const int j0 = tile * kDVT;
    long t0, t1;
    seq_bounds(p.cu, n, p.T, p.total, t0, t1, p.err);

    // ---- state tiles: this wave owns S^T blocks (dk block sib[i], dv block sjb[i])
    int sib[NST], sjb[NST];
    f32x4 Sacc[NST];
#pragma unroll
    for (int i = 0; i < NST; ++i) {
        const int t = wave * NST + i;
        sib[i] = t >> 1;
        sjb[i] = t & 1;
        const int dvr = 16 * sjb[i] + l16;          // dv row of S
        const int dkc = 16 * sib[i] + 4 * lg;       // first of 4 dk columns
        if (p.S0) {
            const float4 s4 = *(const float4 *)(p.S0 + (((size_t)n * H + h) * DV + j0 + dvr) * DK + dkc);
            Sacc[i] = f32x4{s4.x, s4.y, s4.z, s4.w};
        } else {
            Sacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        store4(sS + dvr * KS + dkc, Sacc[i][0], Sacc[i][1], Sacc[i][2], Sacc[i][3]);
    }
    // Upper tiles of A_qk inside the 32-wide contraction blocks stay zero.
    for (int idx = tid; idx < 2 * 256; idx += kThreads) {
        const int blk = idx >> 8, e = idx & 255;
        const int r = (blk ? 32 : 0) + (e >> 4), c = (blk ? 48 : 16) + (e & 15);
        sAqk[r * kCS + c] = 0;
    }

    // gate-stage thread layout: 4 channels x RPT rows
    const int gcb = tid % NCB, grb = tid / NCB;
    const int gc0 = 4 * gcb, gr0 = RPT * grb;
    // value-tile loader layout: one row, 4 dv columns
    const int vr = tid >> 3, vj = 4 * (tid & 7);
    // serial-stage tile of this wave: chunk rows block, dv block
    const int vib = wave >> 1, vjb = wave & 1;

    for (long c0 = t0; c0 < t1; c0 += kC) {
        const int m = (int)((t1 - c0) < kC ? (t1 - c0) : kC);

        // ================= 1. gate prefix sums and scaled operands ===========
        float kf[RPT][4], qf[RPT][4], g[RPT][4];
        {
            float run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int rr = 0; rr < RPT; ++rr) {
                const int r = gr0 + rr;
                const size_t tok = (size_t)(c0 + r) * H + h;
                if (r < m) {
                    const uint2 kw = *(const uint2 *)(p.k + tok * DK + gc0);
                    const uint2 qw = *(const uint2 *)(p.q + tok * DK + gc0);
                    kf[rr][0] = bf16_lo(kw.x); kf[rr][1] = bf16_hi(kw.x);
                    kf[rr][2] = bf16_lo(kw.y); kf[rr][3] = bf16_hi(kw.y);
                    qf[rr][0] = bf16_lo(qw.x); qf[rr][1] = bf16_hi(qw.x);
                    qf[rr][2] = bf16_lo(qw.y); qf[rr][3] = bf16_hi(qw.y);
                    if (GATE == kGateChannel) {
                        const float4 a4 = *(const float4 *)(p.la + tok * DK + gc0);
                        run[0] += a4.x; run[1] += a4.y; run[2] += a4.z; run[3] += a4.w;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) kf[rr][e] = qf[rr][e] = 0.f;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) g[rr][e] = run[e];
            }
            if (GATE == kGateChannel)
                *(float4 *)(sX + grb * DK + gc0) = make_float4(run[0], run[1], run[2], run[3]);
            if (GATE == kGateHead && tid < 64) {
                // inclusive scan of the per-row head gate over the 64 lanes of wave 0
                float x = tid < m ? p.la[(size_t)(c0 + tid) * H + h] : 0.f;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float y = __shfl_up(x, off, 64);
                    if (tid >= off) x += y;
                }
                const float gcv = __shfl(x, 63, 64);
                sRow[tid] = expf(x);
                sRow[64 + tid] = expf(-x);
                sRow[128 + tid] = expf(gcv - x);
                for (int c = tid; c < DK; c += 64) sGC[c] = expf(gcv);
            }
            if (tid < kC) sBeta[tid] = tid < m ? p.beta[(size_t)(c0 + tid) * H + h] : 0.f;
            // value tile, stored transposed: sVT[dv][chunk row]
            {
                float vv[4] = {0.f, 0.f, 0.f, 0.f};
                if (vr < m) {
                    const uint2 w = *(const uint2 *)(p.v + ((size_t)(c0 + vr) * H + h) * DV + j0 + vj);
                    vv[0] = bf16_lo(w.x); vv[1] = bf16_hi(w.x); vv[2] = bf16_lo(w.y); vv[3] = bf16_hi(w.y);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sVT[(vj + e) * kCS + vr] = __builtin_bit_cast(uint16_t, __float2bfloat16(vv[e]));
            }
        }
        __syncthreads();
        {
            float eg[RPT][4], eig[RPT][4], eh[RPT][4];
            if (GATE == kGateChannel) {
                float carry[4] = {0.f, 0.f, 0.f, 0.f}, gcv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    const float4 t4 = *(const float4 *)(sX + rb * DK + gc0);
                    const float tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        gcv[e] += tv[e];
                        if (rb < grb) carry[e] += tv[e];
                    }
                }
#pragma unroll
                for (int rr = 0; rr < RPT; ++rr)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float gg = g[rr][e] + carry[e];
                        eg[rr][e] = __expf(gg);
                        eig[rr][e] = __expf(-gg);
                        eh[rr][e] = __expf(gcv[e] - gg);
                    }
                if (grb == 0)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sGC[gc0 + e] = __expf(gcv[e]);
            } else if (GATE == kGateHead) {
#pragma unroll
                for (int rr = 0; rr < RPT; ++rr) {
                    const int r = gr0 + rr;
                    const float a0 = sRow[r], a1 = sRow[64 + r], a2 = sRow[128 + r];
#pragma unroll
                    for (int e = 0; e < 4; ++e) { eg[rr][e] = a0; eig[rr][e] = a1; eh[rr][e] = a2; }
                }
            } else {
#pragma unroll
                for (int rr = 0; rr < RPT; ++rr)
#pragma unroll
                    for (int e = 0; e < 4; ++e) eg[rr][e] = eig[rr][e] = eh[rr][e] = 1.f;
                if (grb == 0)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sGC[gc0 + e] = 1.f;
            }
            float kl[RPT][4], kh[RPT][4];
#pragma unroll
            for (int rr = 0; rr < RPT; ++rr) {
                const int r = gr0 + rr;
                float kr[4], ql[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kl[rr][e] = kf[rr][e] * eg[rr][e];
                    kr[e] = kf[rr][e] * eig[rr][e];
                    ql[e] = qf[rr][e] * eg[rr][e];
                    kh[rr][e] = kf[rr][e] * eh[rr][e];
                }
                store4(sKl + r * KS + gc0, kl[rr][0], kl[rr][1], kl[rr][2], kl[rr][3]);
                store4(sKr + r * KS + gc0, kr[0], kr[1], kr[2], kr[3]);
                store4(sQl + r * KS + gc0, ql[0], ql[1], ql[2], ql[3]);
            }
            // transposed copies: RPT consecutive chunk rows of one channel
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint16_t *pl = sKlT + (gc0 + e) * kCS + gr0;
                uint16_t *ph = sKhT + (gc0 + e) * kCS + gr0;
                if (RPT == 4) {
                    store4(pl, kl[0][e], kl[1][e], kl[2][e], kl[3][e]);
                    store4(ph, kh[0][e], kh[1][e], kh[2][e], kh[3][e]);
                } else {
                    *(uint32_t *)pl = pack_bf16x2(kl[0][e], kl[1][e]);
                    *(uint32_t *)ph = pack_bf16x2(kh[0][e], kh[1][e]);
                }
            }
        }
        __syncthreads();

        // ================= 2. G = K<- K->^T and A_qk = Q<- K->^T ==============
        for (int job = wave; job < 20; job += kWaves) {
            const int tri = job % 10;
            const int ib = tri >= 6 ? 3 : (tri >= 3 ? 2 : (tri >= 1 ? 1 : 0));
            const int jb = tri - ib * (ib + 1) / 2;
            const bool isA = job >= 10;
            const uint16_t *src = isA ? sQl : sKl;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
                acc = mfma(frag(src, 16 * ib + l16, KS, 32 * kk + 8 * lg),
                           frag(sKr, 16 * jb + l16, KS, 32 * kk + 8 * lg), acc);
            const int c = 16 * jb + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * ib + 4 * lg + e;
                if (isA)
                    sAqk[r * kCS + c] = __builtin_bit_cast(uint16_t, __float2bfloat16(c <= r ? acc[e] : 0.f));
                else
                    sX[r * kXS + c] = c < r ? sBeta[r] * acc[e] : 0.f;
            }
        }
        __syncthreads();

        // ================= 3. At = (I + L)^-1 ===================================
        if (wave == 0) {
            // diagonal 16x16 blocks: lane -> (block, column), forward substitution
            const int blk = lane >> 4, col = lane & 15, o = 16 * blk;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) s += sX[(o + r) * kXS + o + i] * x[i];
                x[r] = r < col ? 0.f : (r == col ? 1.f : -s);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (r >= col) sX[(o + r) * kXS + o + col] = x[r];
        }
        __syncthreads();
        {
            // 32-row level: X10 = -X11 (L10 X00) for the pairs (0,1) and (2,3)
            const int which = tid >> 8, e = tid & 255, rr = e >> 4, cc = e & 15;
            const int o = 32 * which;
            float s = 0.f;
            for (int i = cc; i < 16; ++i) s += sX[(o + 16 + rr) * kXS + o + i] * sX[(o + i) * kXS + o + cc];
            sTmp[which * 16 * 17 + rr * 17 + cc] = s;
            __syncthreads();
            float s2 = 0.f;
            for (int i = 0; i <= rr; ++i)
                s2 += sX[(o + 16 + rr) * kXS + o + 16 + i] * sTmp[which * 16 * 17 + i * 17 + cc];
            sX[(o + 16 + rr) * kXS + o + cc] = -s2;
        }
        __syncthreads();
        {
            // 64-row level: X[32:64, 0:32] = -X[32:64, 32:64] (L[32:64, 0:32] X[0:32, 0:32])
            float tv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int o = tid + u * kThreads, rr = o >> 5, cc = o & 31;
                float s = 0.f;
                for (int i = cc; i < 32; ++i) s += sX[(32 + rr) * kXS + i] * sX[i * kXS + cc];
                tv[u] = s;
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int o = tid + u * kThreads;
                sTmp[(o >> 5) * kTS + (o & 31)] = tv[u];
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int o = tid + u * kThreads, rr = o >> 5, cc = o & 31;
                float s = 0.f;
                for (int i = 0; i <= rr; ++i) s += sX[(32 + rr) * kXS + 32 + i] * sTmp[i * kTS + cc];
                tv[u] = -s;
            }
            // all reads of L[32:64, 0:32] finished before the barrier above
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int o = tid + u * kThreads;
                sX[(32 + (o >> 5)) * kXS + (o & 31)] = tv[u];
            }
        }
        __syncthreads();
        // At Diag(beta) -> bf16, zero above the diagonal
        for (int idx = tid; idx < kC * kC / 2; idx += kThreads) {
            const int r = idx >> 5, c = 2 * (idx & 31);
            const float x0 = c <= r ? sX[r * kXS + c] * sBeta[c] : 0.f;
            const float x1 = c + 1 <= r ? sX[r * kXS + c + 1] * sBeta[c + 1] : 0.f;
            *(uint32_t *)(sAb + r * kCS + c) = pack_bf16x2(x0, x1);
        }
        __syncthreads();

        // ================= 4. W = At Diag(beta) K<-,  U = At Diag(beta) V =====
        for (int t = wave; t < (DK / 16) * 4; t += kWaves) {
            const int ib = t >> 2, jb = t & 3;  // dk block, chunk-row block
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma(frag(sKlT, 16 * ib + l16, kCS, 8 * lg), frag(sAb, 16 * jb + l16, kCS, 8 * lg), acc);
            if (jb >= 2)
                acc = mfma(frag(sKlT, 16 * ib + l16, kCS, 32 + 8 * lg),
                           frag(sAb, 16 * jb + l16, kCS, 32 + 8 * lg), acc);
            // lane holds W[chunk 16jb + l16][dk 16ib + 4lg + 0..3]
            store4(sW + (16 * jb + l16) * KS + 16 * ib + 4 * lg, acc[0], acc[1], acc[2], acc[3]);
        }
        f32x4 U = {0.f, 0.f, 0.f, 0.f};
        U = mfma(frag(sAb, 16 * vib + l16, kCS, 8 * lg), frag(sVT, 16 * vjb + l16, kCS, 8 * lg), U);
        if (vib >= 2)
            U = mfma(frag(sAb, 16 * vib + l16, kCS, 32 + 8 * lg),
                     frag(sVT, 16 * vjb + l16, kCS, 32 + 8 * lg), U);
        __syncthreads();

        // ================= 5. serial part ======================================
        f32x4 P = {0.f, 0.f, 0.f, 0.f}, Oa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            const bf16x8 bs = frag(sS, 16 * vjb + l16, KS, 32 * kk + 8 * lg);
            P = mfma(frag(sW, 16 * vib + l16, KS, 32 * kk + 8 * lg), bs, P);
            Oa = mfma(frag(sQl, 16 * vib + l16, KS, 32 * kk + 8 * lg), bs, Oa);
        }
        // V_new[chunk 16vib + 4lg + e][dv 16vjb + l16] -> transposed store
        store4(sVnT + (16 * vjb + l16) * kCS + 16 * vib + 4 * lg, U[0] - P[0], U[1] - P[1],
               U[2] - P[2], U[3] - P[3]);
        __syncthreads();
        Oa = mfma(frag(sAqk, 16 * vib + l16, kCS, 8 * lg), frag(sVnT, 16 * vjb + l16, kCS, 8 * lg), Oa);
        if (vib >= 2)
            Oa = mfma(frag(sAqk, 16 * vib + l16, kCS, 32 + 8 * lg),
                      frag(sVnT, 16 * vjb + l16, kCS, 32 + 8 * lg), Oa);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * vib + 4 * lg + e;
            if (r < m) p.O[((size_t)(c0 + r) * H + h) * DV + j0 + 16 * vjb + l16] = __float2bfloat16(Oa[e]);
        }
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int dkr = 16 * sib[i] + 4 * lg;
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[i][e] *= sGC[dkr + e];
            Sacc[i] = mfma(frag(sKhT, 16 * sib[i] + l16, kCS, 8 * lg), frag(sVnT, 16 * sjb[i] + l16, kCS, 8 * lg), Sacc[i]);
            Sacc[i] = mfma(frag(sKhT, 16 * sib[i] + l16, kCS, 32 + 8 * lg),
                           frag(sVnT, 16 * sjb[i] + l16, kCS, 32 + 8 * lg), Sacc[i]);
        }
        // all reads of the old bf16 state happened before the barrier above
#pragma unroll
        for (int i = 0; i < NST; ++i)
            store4(sS + (16 * sjb[i] + l16) * KS + 16 * sib[i] + 4 * lg, Sacc[i][0], Sacc[i][1],
                   Sacc[i][2], Sacc[i][3]);
        __syncthreads();
    }

    if (p.Sf) {
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int dvr = 16 * sjb[i] + l16, dkc = 16 * sib[i] + 4 * lg;
            *(float4 *)(p.Sf + (((size_t)n * H + h) * DV + j0 + dvr) * DK + dkc) =
                make_float4(Sacc[i][0], Sacc[i][1], Sacc[i][2], Sacc[i][3]);
        }
    }
}

template <int DK>
int launch_dk(const KdaParams &kp, int grid, int gate, hipStream_t s) {
    if (gate == kGateChannel)
        hipLaunchKernelGGL((kda_mfma_kernel<DK, kGateChannel>), dim3(grid), dim3(kThreads), 0, s, kp);
    else if (gate == kGateHead)
        hipLaunchKernelGGL((kda_mfma_kernel<DK, kGateHead>), dim3(grid), dim3(kThreads), 0, s, kp);
    else
        hipLaunchKernelGGL((kda_mfma_kernel<DK, kGateNone>), dim3(grid), dim3(kThreads), 0, s, kp);
    return (int)hipGetLastError();
}

}  // namespace

bool kda_mfma_supported(const FwdArgs &a) {
    return a.dtype == 1 && a.a == nullptr && a.b == nullptr && a.C == kC &&
           (a.dk == 64 || a.dk == 128) && a.dv % kDVT == 0;
}

int launch_kda_mfma(const FwdArgs &a, int n_seq_eff, hipStream_t s) {
    KdaParams kp;
    kp.q = (const bf16 *)a.q; kp.k = (const bf16 *)a.k; kp.v = (const bf16 *)a.v;
    kp.la = a.log_alpha; kp.beta = a.beta; kp.S0 = a.S0;
    kp.O = (bf16 *)a.O; kp.Sf = a.S_final; kp.cu = a.cu_seqlens;
    kp.err = (int *)a.workspace;
    kp.total = (long)a.B * a.T;
    kp.H = a.H; kp.T = a.T; kp.dv = a.dv; kp.n_tiles = a.dv / kDVT;
    const int grid = n_seq_eff * a.H * kp.n_tiles;
    if (a.dk == 128) return launch_dk<128>(kp, grid, a.gate, s);
    return launch_dk<64>(kp, grid, a.gate, s);
}

}  // namespace gdr
