// Fused chunkwise forward for the KDA family (a = k, b = beta k) with bf16
// inputs, on gfx950 matrix cores (fp32 accumulate).
//
// One workgroup (8 waves) per (sequence, head, 32-wide dv tile).  The state
// tile S[dv 32][dk] lives in fp32 MFMA accumulators for the whole sequence; a
// bf16 copy in LDS feeds the products.  Per chunk of 64 tokens, following the
// KDA chunk form ("Kimi Delta Attention backward" notes, forward recap):
//
//   gate  g = in-chunk inclusive prefix sum of log alpha (per channel or head);
//         Q<- = Q e^g, K<- = K e^g, K-> = K e^-g, K^ = K e^(g_C - g) -> LDS (bf16)
//   gram  L = Diag(beta)(K<- K->^T, strictly lower) (fp32) and
//         A_qk = Q<- K->^T on and below the diagonal (bf16), bf16 MFMA
//   inv   At = (I + L)^-1 by 16x16 blocks ("DeltaNet" notes, section 4.2):
//         diagonal blocks by forward substitution, then the two-block form
//         [A11 0; A21 A22]^-1 = [A11^-1 0; -A22^-1 A21 A11^-1  A22^-1]
//         at 32 rows and at 64 rows, with fp32 MFMA
//   wy    W = At Diag(beta) K<-,  U = At Diag(beta) V
//   state V_new = U - W S^T,  O = Q<- S^T + A_qk V_new,
//         S = S Diag(gamma_C) + V_new^T K^
//
// MFMA operand layout (v_mfma_f32_16x16x32_bf16): lane l feeds A[l%16][8(l/16)+0..7]
// and B[8(l/16)+0..7][l%16] and receives D[4(l/16)+0..3][l%16].  Operands that
// are contiguous along the contraction are read as 16-byte rows; operands whose
// rows run along the contraction (a contraction over chunk rows of a row-major
// array) are read with the LDS transpose read, so every LDS array is stored
// row-major only.  Products are oriented so that each lane's four outputs are
// contiguous in the array they are stored to.
//
// The inputs of chunk t+1 are loaded into registers while chunk t is computed.
#include "gdr_common.h"

namespace gdr {
namespace {

constexpr int kC = 64;        // chunk size
constexpr int kDVT = 32;      // dv columns per workgroup
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCS = kC + 8;   // bf16 row stride of [*][64] arrays
constexpr int kLS = kC + 4;   // fp32 row stride of the 64x64 inverse (16-byte rows)
constexpr int kTS = 33;       // fp32 row stride of the inverse's temporaries
constexpr int kVS = kDVT + 8; // bf16 row stride of the value tile
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

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
    static constexpr int KS = DK + 8;                      // bf16 row stride of [*][DK] arrays
    static constexpr int oKl = 0;                          // K<-  [64][KS]
    static constexpr int oKr = oKl + kC * KS * 2;          // K->  [64][KS]; W after the gram
    static constexpr int oQl = oKr + kC * KS * 2;          // Q<-  [64][KS]
    static constexpr int oKh = oQl + kC * KS * 2;          // K^   [64][KS]
    static constexpr int oV = oKh + kC * KS * 2;           // V    [64][kVS]
    static constexpr int oL = oV + kC * kVS * 2;           // fp32 [64][kLS]: totals, L, At
    static constexpr int oT = oL + kC * kLS * 4;           // fp32 [32][kTS] temporaries
    static constexpr int oAb = oT + 32 * kTS * 4;          // At Diag(beta) bf16 [64][kCS]
    static constexpr int oAqk = oAb + kC * kCS * 2;        // A_qk bf16 [64][kCS]
    static constexpr int oS = oAqk + kC * kCS * 2;         // S bf16 [32][KS]
    static constexpr int oVnT = oS + kDVT * KS * 2;        // V_new^T bf16 [32][kCS]
    static constexpr int oBeta = oVnT + kDVT * kCS * 2;    // fp32 [64]
    static constexpr int oGC = oBeta + kC * 4;             // fp32 [DK] gamma_C
    static constexpr int oRow = oGC + DK * 4;              // fp32 [3][64] (head gate)
    static constexpr int bytes = oRow + 3 * kC * 4;
    static_assert(bytes <= 160 * 1024, "LDS budget");
    static_assert(oKr % 16 == 0 && oQl % 16 == 0 && oKh % 16 == 0 && oV % 16 == 0 &&
                      oL % 16 == 0 && oT % 16 == 0 && oAb % 16 == 0 && oAqk % 16 == 0 &&
                      oS % 16 == 0 && oVnT % 16 == 0 && oBeta % 16 == 0 && oGC % 16 == 0,
                  "16-byte aligned arrays");
};

// A-operand (or B-operand) fragment whose 8 contraction elements are contiguous.
__device__ __forceinline__ bf16x8 frag(const uint16_t *base, int row, int stride, int col) {
    return *(const bf16x8 *)(base + row * stride + col);
}

// Fragment of a row-major array whose rows run along the contraction: lane l gets
// column col0 + l%16 at rows k0 + 8(l/16) + 0..7.  Each 16-lane group issues two
// transpose reads; source lane s of a group points at row (k0 + 8G + s/4 [+4]),
// columns col0 + 4(s%4) .. +3, and the hardware hands lane p element p%4 of source
// lanes 4e + p/4, i.e. column col0 + p, rows +e.
__device__ __forceinline__ bf16x8 frag_tr(const uint16_t *base, int k0, int stride, int col0,
                                          int lane) {
    const int G = lane >> 4, s = lane & 15;
    const uint16_t *p = base + (k0 + 8 * G + (s >> 2)) * stride + col0 + 4 * (s & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + 4 * stride));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 16x16x4: lane l feeds A[l%16][l/16] and B[l/16][l%16].
__device__ __forceinline__ f32x4 mfma32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void store4(uint16_t *dst, float x0, float x1, float x2, float x3) {
    uint2 w;
    w.x = pack_bf16x2(x0, x1);
    w.y = pack_bf16x2(x2, x3);
    *(uint2 *)dst = w;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DK, int GATE>
__global__ __launch_bounds__(kThreads) void kda_mfma_kernel(KdaParams p) {
    using L = Smem<DK>;
    constexpr int KS = L::KS;
    constexpr int NCB = DK / 4;                  // 4-channel blocks in the gate stage
    constexpr int NRB = kThreads / NCB;          // row blocks in the gate stage
    constexpr int RPT = kC / NRB;                // rows per thread in the gate stage
    constexpr int NST = (DK / 16) * 2 / kWaves;  // state tiles per wave
    constexpr int NWT = (DK / 16) * 4 / kWaves;  // W tiles per wave
    static_assert(RPT == 2 || RPT == 4, "gate-stage layout");
    static_assert(NST >= 1 && NWT >= 1, "tiling");

    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    uint16_t *sKl = (uint16_t *)(smem + L::oKl);
    uint16_t *sKr = (uint16_t *)(smem + L::oKr);
    uint16_t *sW = sKr;  // K-> is dead once the gram is formed
    uint16_t *sQl = (uint16_t *)(smem + L::oQl);
    uint16_t *sKh = (uint16_t *)(smem + L::oKh);
    uint16_t *sV = (uint16_t *)(smem + L::oV);
    float *sL = (float *)(smem + L::oL);
    float *sTot = sL;    // gate-stage partial sums, before L is formed
    float *sT = (float *)(smem + L::oT);
    uint16_t *sAb = (uint16_t *)(smem + L::oAb);
    uint16_t *sAqk = (uint16_t *)(smem + L::oAqk);
    uint16_t *sS = (uint16_t *)(smem + L::oS);
    uint16_t *sVnT = (uint16_t *)(smem + L::oVnT);
    float *sBeta = (float *)(smem + L::oBeta);
    float *sGC = (float *)(smem + L::oGC);
    float *sRow = (float *)(smem + L::oRow);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int lg = lane >> 4;

    const int H = p.H, DV = p.dv;
    const int lin = xcd_linear_index(blockIdx.x, gridDim.x);
    const int tile = lin % p.n_tiles;
    const int h = (lin / p.n_tiles) % H;
    const int n = lin / (p.n_tiles * H);
    const int j0 = tile * kDVT;
    long t0, t1;
    seq_bounds(p.cu, n, p.T, p.total, t0, t1, p.err);

    // ---- state: this wave owns S^T tiles (dk block sib[i], dv block sjb[i]) -------
    int sib[NST], sjb[NST];
    f32x4 Sacc[NST];
#pragma unroll
    for (int i = 0; i < NST; ++i) {
        const int t = wave * NST + i;
        sib[i] = t >> 1;
        sjb[i] = t & 1;
        const int dvr = 16 * sjb[i] + l16, dkc = 16 * sib[i] + 4 * lg;
        if (p.S0) {
            const float4 s4 = *(const float4 *)(p.S0 + (((size_t)n * H + h) * DV + j0 + dvr) * DK + dkc);
            Sacc[i] = f32x4{s4.x, s4.y, s4.z, s4.w};
        } else {
            Sacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        store4(sS + dvr * KS + dkc, Sacc[i][0], Sacc[i][1], Sacc[i][2], Sacc[i][3]);
    }
    // A_qk tiles above the diagonal inside the used 32-wide contraction blocks stay zero.
    for (int idx = tid; idx < 2 * 256; idx += kThreads) {
        const int blk = idx >> 8, e = idx & 255;
        sAqk[((blk ? 32 : 0) + (e >> 4)) * kCS + (blk ? 48 : 16) + (e & 15)] = 0;
    }

    // ---- register prefetch of one chunk's inputs ----------------------------------
    const int gcb = tid % NCB, grb = tid / NCB;
    const int gc0 = 4 * gcb, gr0 = RPT * grb;
    const int vr = tid >> 3, vj = 4 * (tid & 7);
    uint2 pk[RPT], pq[RPT], pv;
    float4 pla[RPT];
    float pbeta = 0.f, plah = 0.f;
    auto prefetch = [&](long c) {
        const int mc = (int)((t1 - c) < kC ? (t1 - c) : kC);
#pragma unroll
        for (int rr = 0; rr < RPT; ++rr) {
            const int r = gr0 + rr < mc ? gr0 + rr : mc - 1;
            const size_t base = ((size_t)(c + r) * H + h) * DK + gc0;
            pk[rr] = *(const uint2 *)(p.k + base);
            pq[rr] = *(const uint2 *)(p.q + base);
            if (GATE == kGateChannel) pla[rr] = *(const float4 *)(p.la + base);
        }
        const int rv = vr < mc ? vr : mc - 1;
        pv = *(const uint2 *)(p.v + ((size_t)(c + rv) * H + h) * DV + j0 + vj);
        if (tid < kC) {
            const int rb = tid < mc ? tid : mc - 1;
            pbeta = p.beta[(size_t)(c + rb) * H + h];
            if (GATE == kGateHead) plah = p.la[(size_t)(c + rb) * H + h];
        }
    };
    if (t0 < t1) prefetch(t0);

    // serial-stage tiles of this wave
    const int vib = wave >> 1, vjb = wave & 1;  // V_new / U: chunk-row block, dv block
    const int ocb = wave >> 1, odb = wave & 1;  // O^T: chunk-row block, dv block

    for (long c0 = t0; c0 < t1; c0 += kC) {
        const int m = (int)((t1 - c0) < kC ? (t1 - c0) : kC);

        // ============ gate, part 1: local prefix sums, beta, values ===================
        float kf[RPT][4], qf[RPT][4], g[RPT][4];
        {
            float run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int rr = 0; rr < RPT; ++rr) {
                const bool ok = gr0 + rr < m;
                kf[rr][0] = bf16_lo(pk[rr].x); kf[rr][1] = bf16_hi(pk[rr].x);
                kf[rr][2] = bf16_lo(pk[rr].y); kf[rr][3] = bf16_hi(pk[rr].y);
                qf[rr][0] = bf16_lo(pq[rr].x); qf[rr][1] = bf16_hi(pq[rr].x);
                qf[rr][2] = bf16_lo(pq[rr].y); qf[rr][3] = bf16_hi(pq[rr].y);
                if (GATE == kGateChannel && ok) {
                    run[0] += pla[rr].x * kLog2e; run[1] += pla[rr].y * kLog2e;
                    run[2] += pla[rr].z * kLog2e; run[3] += pla[rr].w * kLog2e;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (!ok) kf[rr][e] = qf[rr][e] = 0.f;
                    g[rr][e] = run[e];
                }
            }
            if (GATE == kGateChannel)
                *(float4 *)(sTot + grb * DK + gc0) = make_float4(run[0], run[1], run[2], run[3]);
            if (GATE == kGateHead && wave == 0) {
                float x = lane < m ? plah * kLog2e : 0.f;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float y = __shfl_up(x, off, 64);
                    if (lane >= off) x += y;
                }
                const float gc = __shfl(x, 63, 64);
                sRow[lane] = exp2_fast(x);
                sRow[64 + lane] = exp2_fast(-x);
                if (lane == 0) sRow[128] = exp2_fast(gc);
            }
            if (tid < kC) sBeta[tid] = tid < m ? pbeta : 0.f;
            *(uint2 *)(sV + vr * kVS + vj) = vr < m ? pv : make_uint2(0u, 0u);
        }
        lds_barrier();
        // ============ gate, part 2: scaled operands ===================================
        {
            float eg[RPT][4], eig[RPT][4], egc[4];
            if (GATE == kGateChannel) {
                float carry[4] = {0.f, 0.f, 0.f, 0.f}, gcv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    const float4 t4 = *(const float4 *)(sTot + rb * DK + gc0);
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
                        eg[rr][e] = exp2_fast(gg);
                        eig[rr][e] = exp2_fast(-gg);
                    }
#pragma unroll
                for (int e = 0; e < 4; ++e) egc[e] = exp2_fast(gcv[e]);
                if (grb == 0)
                    *(float4 *)(sGC + gc0) = make_float4(egc[0], egc[1], egc[2], egc[3]);
            } else if (GATE == kGateHead) {
#pragma unroll
                for (int rr = 0; rr < RPT; ++rr) {
                    const float a0 = sRow[gr0 + rr], a1 = sRow[64 + gr0 + rr];
#pragma unroll
                    for (int e = 0; e < 4; ++e) { eg[rr][e] = a0; eig[rr][e] = a1; }
                }
                const float ec = sRow[128];
#pragma unroll
                for (int e = 0; e < 4; ++e) egc[e] = ec;
                if (grb == 0) *(float4 *)(sGC + gc0) = make_float4(ec, ec, ec, ec);
            } else {
#pragma unroll
                for (int rr = 0; rr < RPT; ++rr)
#pragma unroll
                    for (int e = 0; e < 4; ++e) eg[rr][e] = eig[rr][e] = 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) egc[e] = 1.f;
                if (grb == 0) *(float4 *)(sGC + gc0) = make_float4(1.f, 1.f, 1.f, 1.f);
            }
#pragma unroll
            for (int rr = 0; rr < RPT; ++rr) {
                const int r = gr0 + rr;
                float kl[4], kr[4], ql[4], kh[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kl[e] = kf[rr][e] * eg[rr][e];
                    kr[e] = kf[rr][e] * eig[rr][e];
                    ql[e] = qf[rr][e] * eg[rr][e];
                    kh[e] = kr[e] * egc[e];
                }
                store4(sKl + r * KS + gc0, kl[0], kl[1], kl[2], kl[3]);
                store4(sKr + r * KS + gc0, kr[0], kr[1], kr[2], kr[3]);
                store4(sQl + r * KS + gc0, ql[0], ql[1], ql[2], ql[3]);
                store4(sKh + r * KS + gc0, kh[0], kh[1], kh[2], kh[3]);
            }
        }
        if (c0 + kC < t1) prefetch(c0 + kC);
        lds_barrier();

        // ============ gram: L = Diag(beta) K<- K->^T (strictly lower), A_qk ===========
        // Tile (rb, cb), cb <= rb, computed transposed (D[c][r]) so each lane holds
        // four consecutive columns of one row.
        for (int job = wave; job < 10; job += kWaves) {
            const int rb = job >= 6 ? 3 : (job >= 3 ? 2 : (job >= 1 ? 1 : 0));
            const int cb = job - rb * (rb + 1) / 2;
            f32x4 gacc = {0.f, 0.f, 0.f, 0.f}, aacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const bf16x8 a = frag(sKr, 16 * cb + l16, KS, 32 * kk + 8 * lg);
                gacc = mfma(a, frag(sKl, 16 * rb + l16, KS, 32 * kk + 8 * lg), gacc);
                aacc = mfma(a, frag(sQl, 16 * rb + l16, KS, 32 * kk + 8 * lg), aacc);
            }
            const int r = 16 * rb + l16, c = 16 * cb + 4 * lg;
            const float br = sBeta[r];
            float gl[4], al[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gl[e] = c + e < r ? br * gacc[e] : 0.f;
                al[e] = c + e <= r ? aacc[e] : 0.f;
            }
            *(float4 *)(sL + r * kLS + c) = make_float4(gl[0], gl[1], gl[2], gl[3]);
            store4(sAqk + r * kCS + c, al[0], al[1], al[2], al[3]);
        }
        lds_barrier();

        // ============ inverse, diagonal 16x16 blocks (wave 0) ==========================
        if (wave == 0) {
            const int o = 16 * lg, col = l16;  // block lg, column col
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int i4 = 0; i4 < (r + 3) / 4; ++i4) {
                    const float4 Lv = *(const float4 *)(sL + (o + r) * kLS + o + 4 * i4);
                    const float lv[4] = {Lv.x, Lv.y, Lv.z, Lv.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * i4 + e;
                        if (i < r) {
                            if (e & 1) s1 += lv[e] * x[i];
                            else s0 += lv[e] * x[i];
                        }
                    }
                }
                x[r] = r < col ? 0.f : (r == col ? 1.f : -(s0 + s1));
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (r >= col) sL[(o + r) * kLS + o + col] = x[r];
        }
        lds_barrier();
        // ============ inverse, 32-row level: X[p+1][p] = -X[p+1][p+1] L[p+1][p] X[p][p] ==
        if (wave < 2) {
            const int q0 = 32 * wave;  // rows/cols of block p = 2*wave
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                t = mfma32(sL[(q0 + 16 + l16) * kLS + q0 + 4 * s + lg],
                           sL[(q0 + 4 * s + lg) * kLS + q0 + l16], t);
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[wave * 16 * 17 + (4 * lg + e) * 17 + l16] = t[e];
        }
        lds_barrier();
        if (wave < 2) {
            const int q0 = 32 * wave;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                x = mfma32(sL[(q0 + 16 + l16) * kLS + q0 + 16 + 4 * s + lg],
                           sT[wave * 16 * 17 + (4 * s + lg) * 17 + l16], x);
#pragma unroll
            for (int e = 0; e < 4; ++e) sL[(q0 + 16 + 4 * lg + e) * kLS + q0 + l16] = -x[e];
        }
        lds_barrier();
        // ============ inverse, 64-row level: X_BA = -X_BB (L_BA X_AA) ==================
        if (wave < 4) {
            const int ti = wave >> 1, tj = wave & 1;
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            for (int kb = tj; kb < 2; ++kb)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    t = mfma32(sL[(32 + 16 * ti + l16) * kLS + 16 * kb + 4 * s + lg],
                               sL[(16 * kb + 4 * s + lg) * kLS + 16 * tj + l16], t);
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * ti + 4 * lg + e) * kTS + 16 * tj + l16] = t[e];
        }
        lds_barrier();
        if (wave < 4) {
            const int ti = wave >> 1, tj = wave & 1;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            for (int kb = 0; kb <= ti; ++kb)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    x = mfma32(sL[(32 + 16 * ti + l16) * kLS + 32 + 16 * kb + 4 * s + lg],
                               sT[(16 * kb + 4 * s + lg) * kTS + 16 * tj + l16], x);
#pragma unroll
            for (int e = 0; e < 4; ++e) sL[(32 + 16 * ti + 4 * lg + e) * kLS + 16 * tj + l16] = -x[e];
        }
        lds_barrier();
        // At Diag(beta) -> bf16 (zero above the diagonal)
        {
            const int r = tid >> 3, c = 8 * (tid & 7);
            const float4 x0 = *(const float4 *)(sL + r * kLS + c);
            const float4 x1 = *(const float4 *)(sL + r * kLS + c + 4);
            const float4 b0 = *(const float4 *)(sBeta + c);
            const float4 b1 = *(const float4 *)(sBeta + c + 4);
            const float xv[8] = {x0.x * b0.x, x0.y * b0.y, x0.z * b0.z, x0.w * b0.w,
                                 x1.x * b1.x, x1.y * b1.y, x1.z * b1.z, x1.w * b1.w};
            uint4 w;
            w.x = pack_bf16x2(c + 0 <= r ? xv[0] : 0.f, c + 1 <= r ? xv[1] : 0.f);
            w.y = pack_bf16x2(c + 2 <= r ? xv[2] : 0.f, c + 3 <= r ? xv[3] : 0.f);
            w.z = pack_bf16x2(c + 4 <= r ? xv[4] : 0.f, c + 5 <= r ? xv[5] : 0.f);
            w.w = pack_bf16x2(c + 6 <= r ? xv[6] : 0.f, c + 7 <= r ? xv[7] : 0.f);
            *(uint4 *)(sAb + r * kCS + c) = w;
        }
        lds_barrier();

        // ============ WY factors and the state-independent part of O ==================
        // W^T tile (dk block ib, chunk block jb) = K<-^T (At Diag(beta))^T
#pragma unroll
        for (int i = 0; i < NWT; ++i) {
            const int t = wave * NWT + i, ib = t >> 2, jb = t & 3;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma(frag_tr(sKl, 0, KS, 16 * ib, lane), frag(sAb, 16 * jb + l16, kCS, 8 * lg), acc);
            if (jb >= 2)
                acc = mfma(frag_tr(sKl, 32, KS, 16 * ib, lane),
                           frag(sAb, 16 * jb + l16, kCS, 32 + 8 * lg), acc);
            store4(sW + (16 * jb + l16) * KS + 16 * ib + 4 * lg, acc[0], acc[1], acc[2], acc[3]);
        }
        f32x4 U = {0.f, 0.f, 0.f, 0.f};
        U = mfma(frag(sAb, 16 * vib + l16, kCS, 8 * lg), frag_tr(sV, 0, kVS, 16 * vjb, lane), U);
        if (vib >= 2)
            U = mfma(frag(sAb, 16 * vib + l16, kCS, 32 + 8 * lg), frag_tr(sV, 32, kVS, 16 * vjb, lane), U);
        // O^T tile (dv block odb, chunk block ocb): S Q<-^T
        f32x4 Ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
            Ot = mfma(frag(sS, 16 * odb + l16, KS, 32 * kk + 8 * lg),
                      frag(sQl, 16 * ocb + l16, KS, 32 * kk + 8 * lg), Ot);
        lds_barrier();

        // ============ V_new = U - W S^T =================================================
        {
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
                P = mfma(frag(sW, 16 * vib + l16, KS, 32 * kk + 8 * lg),
                         frag(sS, 16 * vjb + l16, KS, 32 * kk + 8 * lg), P);
            store4(sVnT + (16 * vjb + l16) * kCS + 16 * vib + 4 * lg, U[0] - P[0], U[1] - P[1],
                   U[2] - P[2], U[3] - P[3]);
        }
        lds_barrier();

        // ============ O += A_qk V_new ;  S = S Diag(gamma_C) + V_new^T K^ ==============
        Ot = mfma(frag(sVnT, 16 * odb + l16, kCS, 8 * lg), frag(sAqk, 16 * ocb + l16, kCS, 8 * lg), Ot);
        if (ocb >= 2)
            Ot = mfma(frag(sVnT, 16 * odb + l16, kCS, 32 + 8 * lg),
                      frag(sAqk, 16 * ocb + l16, kCS, 32 + 8 * lg), Ot);
        {
            const int r = 16 * ocb + l16;
            if (r < m) {
                uint2 w;
                w.x = pack_bf16x2(Ot[0], Ot[1]);
                w.y = pack_bf16x2(Ot[2], Ot[3]);
                *(uint2 *)(p.O + ((size_t)(c0 + r) * H + h) * DV + j0 + 16 * odb + 4 * lg) = w;
            }
        }
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const float4 gc = *(const float4 *)(sGC + 16 * sib[i] + 4 * lg);
            Sacc[i][0] *= gc.x; Sacc[i][1] *= gc.y; Sacc[i][2] *= gc.z; Sacc[i][3] *= gc.w;
            Sacc[i] = mfma(frag_tr(sKh, 0, KS, 16 * sib[i], lane),
                           frag(sVnT, 16 * sjb[i] + l16, kCS, 8 * lg), Sacc[i]);
            Sacc[i] = mfma(frag_tr(sKh, 32, KS, 16 * sib[i], lane),
                           frag(sVnT, 16 * sjb[i] + l16, kCS, 32 + 8 * lg), Sacc[i]);
        }
        // The old bf16 state was last read before the barrier above.
#pragma unroll
        for (int i = 0; i < NST; ++i)
            store4(sS + (16 * sjb[i] + l16) * KS + 16 * sib[i] + 4 * lg, Sacc[i][0], Sacc[i][1],
                   Sacc[i][2], Sacc[i][3]);
        // No barrier here: the next chunk's first writes (totals, beta, values) touch
        // nothing read above, and its second stage starts after a barrier.
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
