// Fused chunkwise forward for the KDA family (a = k, b = beta k) with bf16
// inputs, on gfx950 matrix cores (fp32 accumulate).
//
// One workgroup (8 waves) per (sequence, head, 32-wide dv tile).  The state
// tile S[dv 32][dk] lives in fp32 MFMA accumulators for the whole sequence; a
// bf16 copy in LDS feeds the products.  Per chunk of 64 tokens, following the
// KDA chunk form ("Kimi Delta Attention backward" notes, forward recap):
//
//   gate  g = in-chunk inclusive prefix sum of log alpha (per channel or head);
//         Q<- = Q e^g, K<- = K e^g, K-> = K e^-g            -> LDS (bf16)
//   gram  L = Diag(beta)(K<- K->^T, strictly lower) (fp32) and
//         A_qk = Q<- K->^T on and below the diagonal (bf16)
//   inv   At = (I + L)^-1 by 16x16 blocks ("DeltaNet" notes, section 4.2):
//         the four diagonal blocks by forward substitution (fp32), then the
//         two-block form [A11 0; A21 A22]^-1 = [A11^-1 0; -A22^-1 A21 A11^-1  A22^-1]
//         at 32 rows and at 64 rows, with bf16 MFMA products
//   wy    W = At Diag(beta) K<-,  U = At Diag(beta) V
//   state V_new = U - W S^T,  O = Q<- S^T + A_qk V_new,
//         S = (S + V_new^T K->) Diag(gamma_C)        (gamma_C = e^(g at the last row))
//
// The last line is the pages' S Diag(gamma_C) + V_new^T K-> Diag(gamma_C) with the
// gate applied once to the fp32 accumulator.
//
// MFMA operand layout (v_mfma_f32_16x16x32_bf16): lane l feeds A[l%16][8(l/16)+0..7]
// and B[8(l/16)+0..7][l%16] and receives D[4(l/16)+0..3][l%16] (the 16x16x16 form
// feeds 4 contraction elements per lane, A[l%16][4(l/16)+0..3]).  Operands that are
// contiguous along the contraction are read as 16-byte rows; operands whose rows
// run along the contraction (a contraction over chunk rows of a row-major array)
// are read with the LDS transpose read, so every LDS operand array is row-major.
// Products are oriented so that each lane's four outputs are contiguous where
// they are stored.
//
// The inputs of chunk t+1 are loaded into registers while chunk t is computed,
// and every barrier orders LDS traffic only (see lds_barrier).
#include "gdr_mfma.h"

namespace gdr {
namespace {

constexpr int kC = 64;        // chunk size
constexpr int kDVT = 32;      // dv columns per workgroup
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRPW = kC / kWaves;  // gate-stage rows per wave
constexpr int kCS = kC + 8;   // bf16 row stride of [*][64] arrays
constexpr int kLS = kC + 4;   // fp32 row stride of the 64x64 inverse (16-byte rows)
constexpr int kTS = 33;       // fp32 row stride of the 32x32 temporary
constexpr int kVS = kDVT + 8; // bf16 row stride of the value tile
constexpr float kLog2e = 1.4426950408889634f;

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
    static constexpr int oKr = oKl + kC * KS * 2;          // K->  2 x [64][KS] (chunk parity)
    static constexpr int oQl = oKr + 2 * kC * KS * 2;      // Q<-  [64][KS]
    static constexpr int oW = oQl + kC * KS * 2;           // W    [64][KS]
    static constexpr int oV = oW + kC * KS * 2;            // V    [64][kVS]
    static constexpr int oL = oV + kC * kVS * 2;           // fp32 [64][kLS]: L, then At
    static constexpr int oT = oL + kC * kLS * 4;           // fp32 [32][kTS]
    static constexpr int oTot = oT + 32 * kTS * 4;         // fp32 [8][DK] gate partial sums
    static constexpr int oAb = oTot + kWaves * DK * 4;     // At Diag(beta) bf16 [64][kCS]
    static constexpr int oAqk = oAb + kC * kCS * 2;        // A_qk bf16 [64][kCS]
    static constexpr int oS = oAqk + kC * kCS * 2;         // S bf16 [32][KS]
    static constexpr int oVnT = oS + kDVT * KS * 2;        // V_new^T bf16 [32][kCS]
    static constexpr int oBeta = oVnT + kDVT * kCS * 2;    // fp32 [64]
    static constexpr int oGC = oBeta + kC * 4;             // fp32 [DK] gamma_C
    static constexpr int oRow = oGC + DK * 4;              // fp32 [3][64] (head gate)
    static constexpr int bytes = oRow + 3 * kC * 4;
    static_assert(bytes <= 160 * 1024, "LDS budget");
    static_assert(oKr % 16 == 0 && oQl % 16 == 0 && oW % 16 == 0 && oV % 16 == 0 &&
                      oL % 16 == 0 && oT % 16 == 0 && oTot % 16 == 0 && oAb % 16 == 0 &&
                      oAqk % 16 == 0 && oS % 16 == 0 && oVnT % 16 == 0 && oBeta % 16 == 0 &&
                      oGC % 16 == 0,
                  "16-byte aligned arrays");
};

template <int DK, int GATE>
__global__ __launch_bounds__(kThreads) void kda_mfma_kernel(KdaParams p) {
    using L = Smem<DK>;
    constexpr int KS = L::KS;
    constexpr int CPL = DK / 64;     // gate-stage channels per lane
    constexpr int GRW = kC / 4;      // gate-stage rows per gate wave (waves 4..7)
    constexpr int NSW = DK / 32;     // waves owning a 32x32 S^T tile (dk block)
    constexpr int NWT = (DK / 32) * 2;  // 32x32 W^T tiles
    static_assert(CPL == 1 || CPL == 2, "gate-stage layout");
    static_assert(NSW <= 4 && NWT <= kWaves, "tiling");

    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    uint16_t *sKl = (uint16_t *)(smem + L::oKl);
    uint16_t *sKr0 = (uint16_t *)(smem + L::oKr);
    uint16_t *sQl = (uint16_t *)(smem + L::oQl);
    uint16_t *sW = (uint16_t *)(smem + L::oW);
    uint16_t *sV = (uint16_t *)(smem + L::oV);
    float *sL = (float *)(smem + L::oL);
    float *sT = (float *)(smem + L::oT);
    float *sTot = (float *)(smem + L::oTot);
    uint16_t *sAb = (uint16_t *)(smem + L::oAb);
    uint16_t *sAqk = (uint16_t *)(smem + L::oAqk);
    uint16_t *sS = (uint16_t *)(smem + L::oS);
    uint16_t *sVnT = (uint16_t *)(smem + L::oVnT);
    float *sBeta = (float *)(smem + L::oBeta);
    float *sGC = (float *)(smem + L::oGC);
    float *sRow = (float *)(smem + L::oRow);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int l16 = lane & 15, lg = lane >> 4;
    const int l32 = lane & 31, lh = lane >> 5;

    const int H = p.H, DV = p.dv;
    const int lin = xcd_linear_index(blockIdx.x, gridDim.x);
    const int tile = lin % p.n_tiles;
    const int h = (lin / p.n_tiles) % H;
    const int n = lin / (p.n_tiles * H);
    const int j0 = tile * kDVT;
    long t0, t1;
    seq_bounds(p.cu, n, p.T, p.total, t0, t1, p.err);

    // ---- state: wave w < NSW owns the 32x32 tile S^T[dk 32w..32w+31][dv 0..31];
    //      register 4q+e holds S[dv l32][dk 32w + 8q + 4lh + e] -------------------------
    // ST is the state tile in waves 0..NSW-1 and the output tile in waves 6-7.
    f32x16 ST = {};
    if (wave < NSW) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int dk = 32 * wave + 8 * q + 4 * lh;
            float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
            if (p.S0) s4 = *(const float4 *)(p.S0 + (((size_t)n * H + h) * DV + j0 + l32) * DK + dk);
            ST[4 * q + 0] = s4.x; ST[4 * q + 1] = s4.y; ST[4 * q + 2] = s4.z; ST[4 * q + 3] = s4.w;
            store4(sS + l32 * KS + dk, s4.x, s4.y, s4.z, s4.w);
        }
    }
    // Tiles above the diagonal inside the 32-wide contraction blocks that the products
    // read, (rows 0-15, cols 16-31) and (rows 32-47, cols 48-63), stay zero: in A_qk
    // for O, and in the fp32 inverse for its 32-wide level-2 products.
    for (int idx = tid; idx < 2 * 256; idx += kThreads) {
        const int blk = idx >> 8, e = idx & 255;
        const int r = (blk ? 32 : 0) + (e >> 4), c = (blk ? 48 : 16) + (e & 15);
        sAqk[r * kCS + c] = 0;
        sL[r * kLS + c] = 0.f;
    }

    // ---- the gate stage runs one chunk ahead in waves 4..7 ---------------------------
    // Gate wave gw = wave - 4 owns chunk rows 16gw..16gw+15; lane l owns channels
    // CPL*l..+CPL-1.  Inputs are loaded into registers a chunk before they are used,
    // and the scaled operands are kept in registers (packed bf16 pairs) until the
    // LDS arrays of the current chunk are free.  Rows at or beyond the end of the
    // sequence are zero (an exact identity step), so nothing below needs masking.
    const bool gwave = wave >= 4;
    const int gw = wave - 4;
    const int gc0 = CPL * lane;
    const int vr = tid >> 3, vj = 4 * (tid & 7);  // value-tile loader: one row, 4 columns
    const uint32_t rstride = (uint32_t)(H * DK);   // elements between consecutive tokens
    uint32_t pk[GRW], pq[GRW], skl[GRW];
    float2 pla[GRW];
    float plah = 0.f, gcarry[CPL], segc[CPL];
    uint2 pv;
    float pbeta = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) gcarry[e] = 0.f, segc[e] = 1.f;

    auto gate_load = [&](long c) {  // gate waves
        long mcl = t1 - c;
        const int mc = (int)(mcl < 0 ? 0 : (mcl < kC ? mcl : kC));
        const size_t cbase = ((size_t)c * H + h) * DK;
        const char *kc = (const char *)(p.k + cbase), *qc = (const char *)(p.q + cbase);
        const char *lc = (const char *)(p.la + cbase);
        const uint32_t lo2 = 2u * gc0, lo4 = 4u * gc0;  // lane offsets (bytes)
#pragma unroll
        for (int rr = 0; rr < GRW; ++rr) {
            const int r = GRW * gw + rr;
            if (r < mc) {
                // wave-uniform row offset: the address is an SGPR base plus lo2 / lo4
                const uint32_t ro = __builtin_amdgcn_readfirstlane((uint32_t)r * rstride * 2u);
                const char *kr = kc + ro, *qr = qc + ro, *lr = lc + 2u * ro;
                if (CPL == 2) {
                    pk[rr] = *(const uint32_t *)(kr + lo2);
                    pq[rr] = *(const uint32_t *)(qr + lo2);
                    if (GATE == kGateChannel) pla[rr] = *(const float2 *)(lr + lo4);
                } else {
                    pk[rr] = *(const uint16_t *)(kr + lo2);
                    pq[rr] = *(const uint16_t *)(qr + lo2);
                    if (GATE == kGateChannel) pla[rr] = make_float2(*(const float *)(lr + lo4), 0.f);
                }
            } else {
                pk[rr] = pq[rr] = 0u;
                pla[rr] = make_float2(0.f, 0.f);
            }
        }
        if (GATE == kGateHead && gw == 0)
            plah = lane < mc ? p.la[(size_t)(c + lane) * H + h] : 0.f;
    };
    auto vb_load = [&](long c) {  // all threads
        long mcl = t1 - c;
        const int mc = (int)(mcl < 0 ? 0 : (mcl < kC ? mcl : kC));
        pv = vr < mc ? *(const uint2 *)(p.v + ((size_t)(c + vr) * H + h) * DV + j0 + vj)
                     : make_uint2(0u, 0u);
        if (tid < kC) pbeta = tid < mc ? p.beta[(size_t)(c + tid) * H + h] : 0.f;
    };
    // part 1: prefix sums inside the wave's 16 rows (log2 domain, kept in pla);
    // wave totals to LDS; for the head gate, gate wave 0 scans the 64 row gates.
    auto gate_part1 = [&]() {
        if (GATE == kGateChannel) {
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int rr = 0; rr < GRW; ++rr) {
                r0 += pla[rr].x * kLog2e;
                r1 += pla[rr].y * kLog2e;
                pla[rr] = make_float2(r0, r1);
            }
            if (CPL == 2) *(float2 *)(sTot + gw * DK + gc0) = make_float2(r0, r1);
            else sTot[gw * DK + gc0] = r0;
        }
        if (GATE == kGateHead && gw == 0) {
            float x = plah * kLog2e;
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
    };
    // part 2: scaled operands of rows [rr0, rr1) of this gate wave, into registers.
    auto gate_part2 = [&](int rr0, int rr1, uint16_t *dKr) {
        if (rr0 == 0) {
            if (GATE == kGateChannel) {
#pragma unroll
                for (int e = 0; e < CPL; ++e) gcarry[e] = 0.f;
                for (int w2 = 0; w2 < gw; ++w2) {  // wave-uniform trip count
                    if (CPL == 2) {
                        const float2 t2 = *(const float2 *)(sTot + w2 * DK + gc0);
                        gcarry[0] += t2.x;
                        gcarry[CPL - 1] += t2.y;
                    } else {
                        gcarry[0] += sTot[w2 * DK + gc0];
                    }
                }
                if (gw == 3) {
                    segc[0] = exp2_fast(gcarry[0] + pla[GRW - 1].x);
                    if (CPL == 2) segc[CPL - 1] = exp2_fast(gcarry[CPL - 1] + pla[GRW - 1].y);
                }
            } else if (GATE == kGateHead) {
#pragma unroll
                for (int e = 0; e < CPL; ++e) segc[e] = sRow[128];
            }
        }
#pragma unroll
        for (int rr = rr0; rr < rr1; ++rr) {
            float kv[CPL], qv[CPL], eg[CPL], eig[CPL];
            kv[0] = bf16_lo(pk[rr]);
            qv[0] = bf16_lo(pq[rr]);
            if (CPL == 2) {
                kv[CPL - 1] = bf16_hi(pk[rr]);
                qv[CPL - 1] = bf16_hi(pq[rr]);
            }
            const float gpre[2] = {pla[rr].x, pla[rr].y};
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                if (GATE == kGateChannel) {
                    const float gg = gpre[e] + gcarry[e];
                    eg[e] = exp2_fast(gg);
                    eig[e] = exp2_fast(-gg);
                } else if (GATE == kGateHead) {
                    eg[e] = sRow[GRW * gw + rr];
                    eig[e] = sRow[64 + GRW * gw + rr];
                } else {
                    eg[e] = eig[e] = 1.f;
                }
            }
            // K<- is staged in registers (the current chunk still reads it); K-> goes
            // to the other parity buffer and Q<- to its (already consumed) array.
            const int r = GRW * gw + rr;
            if (CPL == 2) {
                skl[rr] = pack_bf16x2(kv[0] * eg[0], kv[CPL - 1] * eg[CPL - 1]);
                *(uint32_t *)(dKr + r * KS + gc0) = pack_bf16x2(kv[0] * eig[0], kv[CPL - 1] * eig[CPL - 1]);
                *(uint32_t *)(sQl + r * KS + gc0) = pack_bf16x2(qv[0] * eg[0], qv[CPL - 1] * eg[CPL - 1]);
            } else {
                skl[rr] = __builtin_bit_cast(uint16_t, __float2bfloat16(kv[0] * eg[0]));
                dKr[r * KS + gc0] = __builtin_bit_cast(uint16_t, __float2bfloat16(kv[0] * eig[0]));
                sQl[r * KS + gc0] = __builtin_bit_cast(uint16_t, __float2bfloat16(qv[0] * eg[0]));
            }
        }
    };
    auto gate_store = [&]() {  // gate waves
#pragma unroll
        for (int rr = 0; rr < GRW; ++rr) {
            const int r = GRW * gw + rr;
            if (CPL == 2) *(uint32_t *)(sKl + r * KS + gc0) = skl[rr];
            else sKl[r * KS + gc0] = (uint16_t)skl[rr];
        }
        if (gw == 3) {
            if (CPL == 2) *(float2 *)(sGC + gc0) = make_float2(segc[0], segc[CPL - 1]);
            else sGC[gc0] = segc[0];
        }
    };

    // prologue: the first chunk's gate stage
    if (gwave) { gate_load(t0); gate_part1(); }
    vb_load(t0);
    lds_barrier();
    if (gwave) { gate_part2(0, GRW, sKr0); gate_load(t0 + kC); }

    for (long c0 = t0; c0 < t1; c0 += kC) {
        const int m = (int)((t1 - c0) < kC ? (t1 - c0) : kC);
        const int par = (int)(((c0 - t0) / kC) & 1);
        uint16_t *sKr = sKr0 + par * kC * KS;          // K-> of this chunk
        uint16_t *sKrN = sKr0 + (par ^ 1) * kC * KS;   // K-> of the next chunk

        // ====== 1. staged gate outputs, beta and values of this chunk -> LDS ==========
        if (gwave) gate_store();
        if (tid < kC) sBeta[tid] = pbeta;
        *(uint2 *)(sV + vr * kVS + vj) = pv;
        vb_load(c0 + kC);
        lds_barrier();

        // ====== 2. gram (waves 0-5) and O^T = S Q<-^T (waves 6-7) =====================
        // Gram: 32x32 tiles (RB, CB) in {(0,0), (1,0), (1,1)}; waves 2j, 2j+1 form tile j
        // of L and of A_qk, computed transposed (D[c][r]) so a lane holds four
        // consecutive columns of one row.  The diagonal tiles also write the zeros
        // above the diagonal.
        if (wave < 6) {
            const int job = wave >> 1, RB = job >= 1 ? 1 : 0, CB = job == 2 ? 1 : 0;
            const bool isA = wave & 1;
            const uint16_t *src = isA ? sQl : sKl;
            bf16x8 fa[DK / 16], fb[DK / 16];
#pragma unroll
            for (int s16 = 0; s16 < DK / 16; ++s16) {
                fa[s16] = frag(sKr, 32 * CB + l32, KS, 16 * s16 + 8 * lh);
                fb[s16] = frag(src, 32 * RB + l32, KS, 16 * s16 + 8 * lh);
            }
            f32x16 acc = {};
#pragma unroll
            for (int s16 = 0; s16 < DK / 16; ++s16) acc = mfma32x32(fa[s16], fb[s16], acc);
            const int r = 32 * RB + l32;
            const float br = sBeta[r];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = 32 * CB + 8 * q + 4 * lh;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = acc[4 * q + e];
                    v[e] = isA ? (c + e <= r ? x : 0.f) : (c + e < r ? br * x : 0.f);
                }
                if (isA) store4(sAqk + r * kCS + c, v[0], v[1], v[2], v[3]);
                else *(float4 *)(sL + r * kLS + c) = make_float4(v[0], v[1], v[2], v[3]);
            }
        } else {
            // O^T tile (dv 0..31, chunk rows 32cbk..32cbk+31): A = S rows, B = Q<- rows
            const int cbk = wave - 6;
            ST = f32x16{};
            bf16x8 fs[DK / 16], fq[DK / 16];
#pragma unroll
            for (int s16 = 0; s16 < DK / 16; ++s16) {
                fs[s16] = frag(sS, l32, KS, 16 * s16 + 8 * lh);
                fq[s16] = frag(sQl, 32 * cbk + l32, KS, 16 * s16 + 8 * lh);
            }
#pragma unroll
            for (int s16 = 0; s16 < DK / 16; ++s16) ST = mfma32x32(fs[s16], fq[s16], ST);
        }
        lds_barrier();

        // ====== 3. inverse: diagonal 16x16 blocks (wave 0) | gate, part 1 (next chunk) ==
        // Lane (block lg, column l16): x_r = [r == col] - sum_{i<r} L[r][i] x_i, which
        // leaves x_r = 0 for r < col without any masking.
        if (wave == 0) {
            const int o = 16 * lg;
            float x[16];
            float4 cur[4], nxt[4];
            cur[0] = *(const float4 *)(sL + (o + 1) * kLS + o);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (r + 1 < 16) {
#pragma unroll
                    for (int i4 = 0; i4 < (r + 4) / 4; ++i4)
                        nxt[i4] = *(const float4 *)(sL + (o + r + 1) * kLS + o + 4 * i4);
                }
                float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i4 = 0; i4 < (r + 3) / 4; ++i4) {
                    const float lv[4] = {cur[i4].x, cur[i4].y, cur[i4].z, cur[i4].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * i4 + e < r) ps[e] += lv[e] * x[4 * i4 + e];
                }
                x[r] = (r == l16 ? 1.f : 0.f) - ((ps[0] + ps[1]) + (ps[2] + ps[3]));
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) cur[i4] = nxt[i4];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sL[(o + r) * kLS + o + l16] = x[r];
        }
        if (gwave) gate_part1();
        lds_barrier();

        // ====== 4. inverse 32-row level (waves 0,1) | gate part 2, first half ===========
        //   X[p+1][p] = -X[p+1][p+1] (L[p+1][p] X[p][p])
        if (wave < 2) {
            const int a0 = 32 * wave, a1 = a0 + 16;
            const float4 la4 = *(const float4 *)(sL + (a1 + l16) * kLS + a0 + 4 * lg);
            const bf16x4 fL = to_bf16x4(la4.x, la4.y, la4.z, la4.w);
            const bf16x4 fX = to_bf16x4(sL[(a0 + 4 * lg + 0) * kLS + a0 + l16], sL[(a0 + 4 * lg + 1) * kLS + a0 + l16],
                                        sL[(a0 + 4 * lg + 2) * kLS + a0 + l16], sL[(a0 + 4 * lg + 3) * kLS + a0 + l16]);
            const f32x4 t = mfma16(fL, fX, f32x4{0.f, 0.f, 0.f, 0.f});  // t[e] = T[4lg+e][l16]
            const float4 xa = *(const float4 *)(sL + (a1 + l16) * kLS + a1 + 4 * lg);
            const f32x4 x = mfma16(to_bf16x4(xa.x, xa.y, xa.z, xa.w), to_bf16x4(t[0], t[1], t[2], t[3]),
                                   f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e) sL[(a1 + 4 * lg + e) * kLS + a0 + l16] = -x[e];
        }
        if (gwave) gate_part2(0, GRW / 2, sKrN);
        lds_barrier();

        // ====== 5. inverse 64-row level, T2 = L_BA X_AA (waves 0-3) | gate part 2 ======
        // Tile (ti, tj) of the 32x32 lower-left block; the contraction runs over 32 with
        // the zero tiles above the diagonal filling the unused half.
        const int ti = (wave >> 1) & 1, tj = wave & 1;
        if (wave < 4) {
            const float4 l0 = *(const float4 *)(sL + (32 + 16 * ti + l16) * kLS + 8 * lg);
            const float4 l1 = *(const float4 *)(sL + (32 + 16 * ti + l16) * kLS + 8 * lg + 4);
            float xb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) xb[e] = sL[(8 * lg + e) * kLS + 16 * tj + l16];
            const f32x4 t = mfma(to_bf16x8(l0, l1),
                                 to_bf16x8(make_float4(xb[0], xb[1], xb[2], xb[3]),
                                           make_float4(xb[4], xb[5], xb[6], xb[7])),
                                 f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * ti + 4 * lg + e) * kTS + 16 * tj + l16] = t[e];
        }
        if (gwave) gate_part2(GRW / 2, GRW, sKrN);
        lds_barrier();
        // ====== 6. inverse 64-row level, X_BA = -X_BB T2 (waves 0-3) ===================
        if (wave < 4) {
            const float4 x0 = *(const float4 *)(sL + (32 + 16 * ti + l16) * kLS + 32 + 8 * lg);
            const float4 x1 = *(const float4 *)(sL + (32 + 16 * ti + l16) * kLS + 32 + 8 * lg + 4);
            float tb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) tb[e] = sT[(8 * lg + e) * kTS + 16 * tj + l16];
            const f32x4 x = mfma(to_bf16x8(x0, x1),
                                 to_bf16x8(make_float4(tb[0], tb[1], tb[2], tb[3]),
                                           make_float4(tb[4], tb[5], tb[6], tb[7])),
                                 f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e) sL[(32 + 16 * ti + 4 * lg + e) * kLS + 16 * tj + l16] = -x[e];
        }
        lds_barrier();
        // ====== 7. At Diag(beta) -> bf16 (zero above the diagonal) =======================
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

        // Inputs of the chunk after next: issued here, first used in stage 3 of the next
        // chunk, so the loads have most of a chunk to arrive.
        if (gwave) gate_load(c0 + 2 * kC);

        // ====== 8. W = At Diag(beta) K<- (32x32 W^T tiles), U = At Diag(beta) V ==========
        if (wave < NWT) {
            const int ib = wave >> 1, jb = wave & 1;  // dk block, chunk-row block
            f32x16 acc = {};
#pragma unroll
            for (int s16 = 0; s16 < 4; ++s16)
                if (s16 < 2 * (jb + 1))  // wave-uniform: At is lower triangular
                    acc = mfma32x32(frag_tr32(sKl, 16 * s16, KS, 32 * ib, lane),
                                    frag(sAb, 32 * jb + l32, kCS, 16 * s16 + 8 * lh), acc);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                store4(sW + (32 * jb + l32) * KS + 32 * ib + 8 * q + 4 * lh, acc[4 * q + 0],
                       acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
        }
        const int vib = wave >> 1, vjb = wave & 1;  // 16x16 U / V_new tile
        f32x4 U = mfma(frag(sAb, 16 * vib + l16, kCS, 8 * lg), frag_tr(sV, 0, kVS, 16 * vjb, lane),
                       f32x4{0.f, 0.f, 0.f, 0.f});
        if (vib >= 2)
            U = mfma(frag(sAb, 16 * vib + l16, kCS, 32 + 8 * lg), frag_tr(sV, 32, kVS, 16 * vjb, lane), U);
        lds_barrier();

        // ====== 9. V_new = U - W S^T ======================================================
        {
            bf16x8 fw[DK / 32], fs[DK / 32];
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                fw[kk] = frag(sW, 16 * vib + l16, KS, 32 * kk + 8 * lg);
                fs[kk] = frag(sS, 16 * vjb + l16, KS, 32 * kk + 8 * lg);
            }
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) P = mfma(fw[kk], fs[kk], P);
            store4(sVnT + (16 * vjb + l16) * kCS + 16 * vib + 4 * lg, U[0] - P[0], U[1] - P[1],
                   U[2] - P[2], U[3] - P[3]);
        }
        lds_barrier();

        // ====== 10. O += A_qk V_new (waves 6-7);  S = (S + V_new^T K->) Diag(gamma_C) ====
        if (wave >= 6) {
            const int cbk = wave - 6;
#pragma unroll
            for (int s16 = 0; s16 < 4; ++s16)
                if (s16 < 2 * (cbk + 1))  // wave-uniform: A_qk is lower triangular
                    ST = mfma32x32(frag(sVnT, l32, kCS, 16 * s16 + 8 * lh),
                                   frag(sAqk, 32 * cbk + l32, kCS, 16 * s16 + 8 * lh), ST);
            const int r = 32 * cbk + l32;
            if (r < m) {
                bf16 *orow = p.O + ((size_t)(c0 + r) * H + h) * DV + j0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint2 w;
                    w.x = pack_bf16x2(ST[4 * q + 0], ST[4 * q + 1]);
                    w.y = pack_bf16x2(ST[4 * q + 2], ST[4 * q + 3]);
                    *(uint2 *)(orow + 8 * q + 4 * lh) = w;
                }
            }
        }
        if (wave < NSW) {
#pragma unroll
            for (int s16 = 0; s16 < 4; ++s16)
                ST = mfma32x32(frag_tr32(sKr, 16 * s16, KS, 32 * wave, lane),
                                 frag(sVnT, l32, kCS, 16 * s16 + 8 * lh), ST);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int dk = 32 * wave + 8 * q + 4 * lh;
                const float4 gc = *(const float4 *)(sGC + dk);
                ST[4 * q + 0] *= gc.x; ST[4 * q + 1] *= gc.y;
                ST[4 * q + 2] *= gc.z; ST[4 * q + 3] *= gc.w;
                store4(sS + l32 * KS + dk, ST[4 * q + 0], ST[4 * q + 1], ST[4 * q + 2],
                       ST[4 * q + 3]);
            }
        }
        lds_barrier();
    }

    if (p.Sf && wave < NSW) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int dk = 32 * wave + 8 * q + 4 * lh;
            *(float4 *)(p.Sf + (((size_t)n * H + h) * DV + j0 + l32) * DK + dk) =
                make_float4(ST[4 * q + 0], ST[4 * q + 1], ST[4 * q + 2], ST[4 * q + 3]);
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
