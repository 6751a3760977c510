// Chunkwise forward for the KDA family (a = k, b = beta k) with bf16 inputs, as two
// kernels on gfx950 matrix cores (fp32 accumulate).
//
// Per chunk of 64 tokens the KDA chunk form ("Kimi Delta Attention backward" notes,
// forward recap) splits into work that does not depend on the state and a short
// serial remainder:
//
//   kda_prep_kernel   one workgroup per (chunk, head), every chunk at once
//     g      in-chunk inclusive prefix sum of log alpha (per channel or head)
//     Q<- = Q e^g, K<- = K e^g, K-> = K e^-g, K^ = K e^(g_C - g), gamma_C = e^g_C
//     L      = Diag(beta)(K<- K->^T strictly lower),  A_qk = Q<- K->^T on and below
//              the diagonal
//     At     = (I + L)^-1 by 16x16 blocks ("DeltaNet" notes, section 4.2): diagonal
//              blocks by forward substitution, then the two-block form
//              [A 0; C B]^-1 = [A^-1 0; -B^-1 C A^-1  B^-1] at 32 and 64 rows
//     Ab     = At Diag(beta),  Ao = A_qk Ab
//     W'     = -Ab K<-,  Q~ = Q<- - Ao K<-
//   kda_state_kernel  one workgroup per (sequence, head, 32-wide dv tile), serial
//                     over the sequence's chunks, state tile in registers
//     V_new  = Ab V + W' S^T                 (= U - W S^T)
//     O      = Ao V + Q~ S^T                 (= Q<- S^T + A_qk V_new)
//     S      = S Diag(gamma_C) + V_new^T K^  (= (S + V_new^T K->) Diag(gamma_C))
//
// The two right-hand forms of O are equal because A_qk V_new = A_qk Ab V - A_qk Ab
// K<- S^T; with them the output no longer waits for V_new, and the serial kernel's
// chain per chunk is two products.
//
// With distinct a, b (the gated DPLR form, "Diagonal Plus Low Rank" notes, section 2,
// matrix form, write term scaled by beta) the same two kernels run with DP set:
//   prep   A-> = A e^-g, B<- = B e^g, A^ = A e^(g_C - g), K^b = Diag(beta) K^
//          E   = (I + (B<- A->^T strictly lower))^-1        (same blocked inverse)
//          Ec' = -E (B<- K->^T strictly lower) Diag(beta),  W' = -E B<-
//          Ao' = A_qk Diag(beta) + (Q<- A->^T on and below the diagonal) Ec'
//          Q~  = Q<- + (Q<- A->^T ...) W'
//   state  N = Ec' V + W' S^T,  O = Ao' V + Q~ S^T,  S = S Diag(gamma_C) + N^T A^ + V^T K^b
// which expands the pages' N = C - W S^T, O = Q<- S^T + (Q<- K->^T)V' + (Q<- A->^T)N and
// S = (S + V'^T K-> + N^T A->) Diag(gamma_C), with V' = Diag(beta) V.  The prep kernel hands its results over in the
// operand order of v_mfma_f32_32x32x16_bf16, so the state kernel loads them straight
// into registers with whole-wave contiguous loads.
//
// Two variants around these:
//   - a chunk whose gate falls by more than 2^96 in a channel (K-> would leave the float
//     range) is flagged by the prep kernel and redone by its SUB instantiation, which
//     forms L and A_qk by 16-row sub-chunks in the log domain ("Gated Linear Attention"
//     notes, section 5.3) and shares everything after them;
//   - with few (sequence, head) chains the serial pass is cut into runs joined through
//     the affine map of each run, S_end = S_start P + R (seg_combine_kernel between two
//     launches of the state kernel), so that more CUs work at once.
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "gdr_mfma.h"
#include "gdr_split_common.h"

namespace gdr {
namespace {

constexpr int kC = 64;         // chunk size
constexpr int kC2 = 128;       // chunk size of the 128-token path (two halves of kC)
constexpr int kDVT = 32;       // dv columns per state workgroup
constexpr int kThreads = 256;  // 4 waves, both kernels
constexpr int kCS = kC + 8;    // bf16 row stride of [*][64] arrays
constexpr int kDS = 20;        // fp32 row stride of the 16x16 diagonal blocks
constexpr int kTS = 32 + 8;    // bf16 row stride of the 32x32 level temporary
constexpr int kVS = kDVT + 8;  // bf16 row stride of the value tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One (chunk, head) block of the workspace.  A "fragment tile" of 32 rows and K
// contraction columns is stored as K/16 steps x 64 lanes x 16 bytes; lane l of
// step s holds row l%32, columns 16s + 8(l/32) + 0..7 -- the A-operand registers of
// v_mfma_f32_32x32x16_bf16, so one wave-wide load of a step is one contiguous KiB.
// With DP (distinct a, b) the slots hold the DPLR counterparts named after the slash.
template <int DK, bool DP = false>
struct Blk {
    static constexpr int oW = 0;                // W' = -Ab K<- / -E B<-: row tiles 0-31, 32-63, K = DK
    static constexpr int oQ = oW + 128 * DK;    // Q~ = Q<- - Ao K<- / Q<- + Aqa W': same
    static constexpr int oK = oQ + 128 * DK;    // K^ / A^ transposed: tiles of dk rows 32w.., K = 64 tokens
    static constexpr int oAb = oK + 128 * DK;   // Ab / Ec': 32x32 tiles (0,0), (1,0), (1,1), K = 32
    static constexpr int oAo = oAb + 6144;      // Ao / Ao': same tiles
    static constexpr int oG = oAo + 6144;       // gamma_C [DK] fp32
    static constexpr int oKb = oG + 4 * DK;     // DP only: Diag(beta) K^ transposed, as oK
    static constexpr int bytes = oKb + (DP ? 128 * DK : 0);
    static_assert(bytes % 256 == 0, "block alignment");
};

// One (128-token chunk, head) block of the C = 128 path (KDA form, dk = 128), in the
// same fragment order: 4 row tiles of W'' and Q~'', K^'' tiles of dk rows with K = 128
// tokens, and the 10 lower 32x32 tiles of Ab'' and Ao'' (tile (rt, ct) at index
// rt (rt + 1) / 2 + ct, K = 32 each).  Rows 0-63 are those of the first 64-token half;
// the second half's rows are re-expressed against the state entering the whole chunk.
template <int DK>
struct Blk128 {
    static constexpr int oW = 0;                 // W'': row tiles 0-3, K = DK
    static constexpr int oQ = oW + 256 * DK;     // Q~'': same
    static constexpr int oK = oQ + 256 * DK;     // K^'' transposed: DK/32 tiles, K = 128 tokens
    static constexpr int oAb = oK + 256 * DK;    // Ab'': 10 tiles
    static constexpr int oAo = oAb + 10 * 2048;  // Ao'': 10 tiles
    static constexpr int oG = oAo + 10 * 2048;   // gamma of the whole chunk [DK] fp32
    static constexpr int bytes = (oG + 4 * DK + 255) / 256 * 256;
};

struct SplitParams {
    const bf16 *q, *k, *v;
    const bf16 *a, *b;  // DPLR low-rank vectors, or NULL (a = k, b = beta k)
    const float *la, *beta, *S0;
    bf16 *O;
    float *Sf;
    const int32_t *cu;
    int32_t *coff;   // first chunk of each packed sequence (with cu_seqlens), else NULL
    int32_t *order;  // packed sequences, longest first (with cu_seqlens), else NULL
    int *err;
    char *blk;      // (chunk, head) blocks
    uint16_t *states;  // state kernel modes 1, 2: bf16 [chunk][head][dv][dk], the state entering each step
    int fblk;  // state kernel mode 2: byte stride of the forward blocks it reads
    long total;
    int H, T, dv, n_seq, n_tiles;
    int C;           // chunk size (always kC here)
    int nc;          // chunks per sequence (fixed-length batch)
    int max_chunks;  // blocks per head in the workspace
    // Segmented state pass (seg_n >= 3; 0 otherwise): each (sequence, head) chain is cut
    // into seg_n runs of chunks.  The map a run applies to the state is affine,
    // S_end = S_start P + R, so phase 1 runs run 0 as usual (its end state is the start
    // of run 1) next to runs 1 .. seg_n-2 from a zero state (R) and from the identity
    // with zero values (P); seg_combine_kernel chains the maps into the start states;
    // phase 2 runs 1 .. seg_n-1 from those with the output.
    int seg_n, seg_phase;
    float *seg_ws;  // fp32 per chain: start states of runs 1..n-1, then R and P of runs 1..n-2
    // Per (chunk, head) job: 1 when the chunk's gate range is too wide for the scaled
    // operands (see kSubGateRange); such jobs are redone by the log-domain prep variant.
    // NULL: not recorded.
    int *sub;
};

// ---------------------------------------------------------------------------------
// Prep kernel
// ---------------------------------------------------------------------------------
template <int DK, bool DP, bool SUB = false>
struct PrepSmem {
    static constexpr int KS = DK + 8;                   // bf16 row stride of [64][DK] arrays
    static constexpr int CCB = kC * kCS * 2;            // bytes of one bf16 [64][kCS] array
    static constexpr int oKl = 0;                       // K<- (DP: B<-)
    static constexpr int oKr = oKl + kC * KS * 2;       // K->, then W'
    static constexpr int oQl = oKr + kC * KS * 2;       // Q<-, then Q~
    static constexpr int oAr = oQl + kC * KS * 2;       // DP only: A->
    static constexpr int oX = oAr + (DP ? kC * KS * 2 : 0);  // L off the diagonal blocks -> At -> Ab (DP: -> E)
    static constexpr int oAqk = oX + CCB;               // A_qk -> Ao (DP: A_qk Diag(beta) -> Ao')
    static constexpr int oBK = oAqk + CCB;              // DP only: B<- K->^T strictly lower, Diag(beta)
    static constexpr int oAqa = oBK + (DP ? CCB : 0);   // DP only: Q<- A->^T on and below the diagonal
    static constexpr int oEc = oAqa + (DP ? CCB : 0);   // DP only: Ec'
    static constexpr int nCC = DP ? 5 : 2;              // [64][kCS] arrays from oX, cleared per job
    static constexpr int oLd = oX + nCC * CCB;          // fp32 4 x [16][kDS]: diagonal blocks of L -> of At
    static constexpr int oT = oLd + 4 * 16 * kDS * 4;   // bf16 [32][kTS]
    static constexpr int oTot = oLd;                    // fp32 [8][DK] gate partial sums (before oLd is used)
    static constexpr int oBeta = oT + 32 * kTS * 2;     // fp32 [64]
    static constexpr int oG = oBeta + kC * 4;           // fp32 [65]: head-gate prefix sums and total
    // SUB only: the gate, fp32 [64][GS] (log2), whose space then holds the bf16 operands
    // of the off-diagonal Gram tiles ([128][KS]: GS = KS makes the two the same size),
    // and the gate of the first row of each 16-row tile, fp32 [4][DK]
    static constexpr int GS = KS;
    static constexpr int oGf = oG + 80 * 4;
    static constexpr int oGref = oGf + (SUB ? kC * GS * 4 : 0);
    static constexpr int oWide = oGref + (SUB ? 4 * DK * 4 : 0);  // SUB only: int [4]
    static constexpr int bytes = oWide + (SUB ? 16 : 0);
    static_assert(8 * DK * 4 <= oBeta - oLd, "gate partial sums fit");
    static_assert(DP || SUB || bytes <= 80 * 1024, "two workgroups per CU");
    static_assert(bytes <= 160 * 1024, "one workgroup per CU");
};

// Gate ranges of the scaled operands (log2 units, any channel).  Up to kSubGateRange the
// operands K e^-g stay in the bf16/fp32 exponent range; up to twice that the prep refers
// the gate of a channel to the middle of the chunk (sh below); a chunk whose gate falls
// further is redone by the SUB variant.
constexpr float kSubGateRange = 96.f;
// In the SUB variant a diagonal 16x16 tile whose gate falls by at most this much goes on
// MFMA with columns y_c 2^(g_s - g_c) (at most 2^64); a wider one is formed element-wise.
constexpr float kSubTileRange = 64.f;

template <int DK, int GATE, bool DP, bool CLIP, bool SUB = false, bool PAIR = false>
__global__ __launch_bounds__(kThreads, DP || SUB ? 1 : 2) void kda_prep_kernel(SplitParams p) {
    using L = PrepSmem<DK, DP, SUB>;
    using Bk = Blk<DK, DP>;
    // PAIR: chunks of 128 tokens.  Each job runs the 64-token code on the two halves in
    // turn and merges them into one Blk128 block (see the end of the job loop).
    using B2 = Blk128<DK>;
    static_assert(!PAIR || (!DP && !SUB && DK == 128), "the 128-token path covers the KDA form at dk = 128");
    constexpr int kBlkBytes = PAIR ? B2::bytes : Bk::bytes;
    constexpr int KS = L::KS;
    constexpr int CPT = DK / 32;  // gate stage: channels per thread
    constexpr int WPR = CPT / 2;  // 32-bit words of bf16 per row per thread
    // The gate is summed per (row, channel) in registers for a channel gate, and for
    // every gate when it is clipped (the clip bound differs from row to row).
    constexpr bool kRowGate = GATE == kGateChannel || CLIP;

    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    uint16_t *sKl = (uint16_t *)(smem + L::oKl);
    uint16_t *sKr = (uint16_t *)(smem + L::oKr);
    uint16_t *sQl = (uint16_t *)(smem + L::oQl);
    uint16_t *sX = (uint16_t *)(smem + L::oX);
    uint16_t *sAqk = (uint16_t *)(smem + L::oAqk);
    uint16_t *sAr = (uint16_t *)(smem + L::oAr);
    uint16_t *sBK = (uint16_t *)(smem + L::oBK);
    uint16_t *sAqa = (uint16_t *)(smem + L::oAqa);
    uint16_t *sEc = (uint16_t *)(smem + L::oEc);
    float *sLd = (float *)(smem + L::oLd);
    uint16_t *sT = (uint16_t *)(smem + L::oT);
    float *sTot = (float *)(smem + L::oTot);
    float *sBeta = (float *)(smem + L::oBeta);
    float *sG = (float *)(smem + L::oG);
    float *sGf = (float *)(smem + L::oGf);      // SUB only
    float *sGref = (float *)(smem + L::oGref);  // SUB only
    uint16_t *sVar = (uint16_t *)sGf;           // SUB only, after the diagonal tiles
    int *sWide = (int *)(smem + L::oWide);      // SUB only

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int H = p.H;
    const int njobs = H * p.max_chunks;
    const int rg = tid >> 5, cg = tid & 31, c0 = CPT * cg;

    // The workgroup is persistent: it walks jobs (chunk j, head h), job g = j H + h,
    // with stride gridDim.x.  The raw inputs of the next job are loaded while the
    // current one is processed (from the moment its own inputs have been consumed).
    struct Job {
        int g, m;
        long tok0;
        bool ok;
        int half;  // PAIR: which 64-token half of the 128-token chunk g
    };
    auto decode = [&](int g, int half = 0) {
        Job J;
        J.g = g;
        J.tok0 = 0;
        J.m = 1;
        J.half = half;
        int n = 0, c = 0;
        J.ok = g < njobs && chunk_of(p, g / H, n, c);
        if (J.ok) {
            long t0, t1;
            seq_bounds(p.cu, n, p.T, p.total, t0, t1, nullptr);
            if constexpr (PAIR) {
                const long base = t0 + (long)c * kC2;
                const int m2 = (int)((t1 - base) < kC2 ? (t1 - base) : kC2);  // >= 1
                J.m = half ? (m2 > kC ? m2 - kC : 0) : (m2 < kC ? m2 : kC);
                // an empty second half reads (and zeroes) rows of the first
                J.tok0 = half && J.m > 0 ? base + kC : base;
            } else {
                J.tok0 = t0 + (long)c * kC;
                J.m = (int)((t1 - J.tok0) < kC ? (t1 - J.tok0) : kC);  // >= 1
            }
        }
        return J;
    };

    // Thread (rg, cg) owns rows 8rg..8rg+7, channels CPT*cg..+CPT-1.  Every load is
    // issued unconditionally (rows past the end of the sequence re-read its last row)
    // so that all of them are in flight at once; those rows are zeroed when consumed,
    // which makes them exact identity steps.
    uint32_t kw[8][WPR], qw[8][WPR], aw[8][WPR], bw[8][WPR];
    float lw[8][CPT];
    float beta_r = 0.f, lah = 0.f;
    auto issue = [&](const Job &J) {
        const int h = J.g % H;
        const size_t rs = (size_t)H * DK;
        const bf16 *kb = p.k + ((size_t)J.tok0 * H + h) * DK + c0;
        const bf16 *qb = p.q + ((size_t)J.tok0 * H + h) * DK + c0;
        const float *lb = p.la + ((size_t)J.tok0 * H + h) * DK + c0;
        const bf16 *ab = DP ? p.a + ((size_t)J.tok0 * H + h) * DK + c0 : nullptr;
        const bf16 *bb = DP ? p.b + ((size_t)J.tok0 * H + h) * DK + c0 : nullptr;
        const int last = J.m > 0 ? J.m - 1 : 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * rg + i, rr = r < J.m ? r : last;
            if constexpr (WPR == 2) {
                const uint2 xk = *(const uint2 *)(kb + rr * rs), xq = *(const uint2 *)(qb + rr * rs);
                kw[i][0] = xk.x; kw[i][WPR - 1] = xk.y;
                qw[i][0] = xq.x; qw[i][WPR - 1] = xq.y;
                if constexpr (DP) {
                    const uint2 xa = *(const uint2 *)(ab + rr * rs), xb = *(const uint2 *)(bb + rr * rs);
                    aw[i][0] = xa.x; aw[i][WPR - 1] = xa.y;
                    bw[i][0] = xb.x; bw[i][WPR - 1] = xb.y;
                }
            } else {
                kw[i][0] = *(const uint32_t *)(kb + rr * rs);
                qw[i][0] = *(const uint32_t *)(qb + rr * rs);
                if constexpr (DP) {
                    aw[i][0] = *(const uint32_t *)(ab + rr * rs);
                    bw[i][0] = *(const uint32_t *)(bb + rr * rs);
                }
            }
            if constexpr (GATE == kGateChannel) {
                if constexpr (CPT == 4) {
                    const float4 x = *(const float4 *)(lb + rr * rs);
                    lw[i][0] = x.x; lw[i][1] = x.y; lw[i][2] = x.z; lw[i][3] = x.w;
                } else {
                    const float2 x = *(const float2 *)(lb + rr * rs);
                    lw[i][0] = x.x; lw[i][1] = x.y;
                }
            } else if constexpr (CLIP && GATE == kGateHead) {
                lw[i][0] = p.la[(size_t)(J.tok0 + rr) * H + h];
            }
        }
        const int rb0 = tid < kC ? (tid < J.m ? tid : last) : 0;
        beta_r = p.beta[(size_t)(J.tok0 + rb0) * H + h];
        if (GATE == kGateHead && !CLIP) lah = p.la[(size_t)(J.tok0 + (lane < J.m ? lane : last)) * H + h];
    };

    // DPLR after the inverse (E in sX as bf16, unit diagonal, zero above it):
    //   stage 1  Ec' = -E BK' (wave ti: row block ti),  W' = -E B<- (into the K-> array)
    //   stage 2  Ao' = A_qk' + Aqa Ec' (in place),      Q~ = Q<- + Aqa W' (in place)
    // where BK' = (B<- K->^T strictly lower) Diag(beta), A_qk' = (Q<- K->^T) Diag(beta)
    // and Aqa = Q<- A->^T, both on and below the diagonal.
    auto dplr_products = [&]() {
        int tidv = threadIdx.x;
        asm volatile("" : "+v"(tidv));
        const int lane = tidv & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tidv >> 6);
        const int l16 = lane & 15, lg = lane >> 4;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        {
            const int ti = wave;
            const bf16x8 e0 = frag(sX, 16 * ti + l16, kCS, 8 * lg);
            const bf16x8 e1 = frag(sX, 16 * ti + l16, kCS, 32 + 8 * lg);
            for (int tj = 0; tj <= ti; ++tj) {  // wave-uniform
                f32x4 d = mfma(frag_tr(sBK, 0, kCS, 16 * tj, lane), e0, zero);
                d = mfma(frag_tr(sBK, 32, kCS, 16 * tj, lane), e1, d);
                store4(sEc + (16 * ti + l16) * kCS + 16 * tj + 4 * lg, -d[0], -d[1], -d[2], -d[3]);
            }
        }
        {
            bf16x8 fe[4][2];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int s = 0; s < 2; ++s) fe[ti][s] = frag(sX, 16 * ti + l16, kCS, 32 * s + 8 * lg);
#pragma unroll
            for (int tt = 0; tt < DK / 64; ++tt) {
                const int tn = wave * (DK / 64) + tt;
                const bf16x8 b0 = frag_tr(sKl, 0, KS, 16 * tn, lane);
                const bf16x8 b1 = frag_tr(sKl, 32, KS, 16 * tn, lane);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    f32x4 w = mfma(b0, fe[ti][0], zero);
                    w = mfma(b1, fe[ti][1], w);
                    store4(sKr + (16 * ti + l16) * KS + 16 * tn + 4 * lg, -w[0], -w[1], -w[2], -w[3]);
                }
            }
        }
        lds_barrier();
        {
            const int ti = wave;
            const bf16x8 a0 = frag(sAqa, 16 * ti + l16, kCS, 8 * lg);
            const bf16x8 a1 = frag(sAqa, 16 * ti + l16, kCS, 32 + 8 * lg);
            for (int tj = 0; tj <= ti; ++tj) {  // wave-uniform
                uint16_t *dst = sAqk + (16 * ti + l16) * kCS + 16 * tj + 4 * lg;
                const uint2 o = *(const uint2 *)dst;
                f32x4 d = {bf16_lo(o.x), bf16_hi(o.x), bf16_lo(o.y), bf16_hi(o.y)};
                d = mfma(frag_tr(sEc, 0, kCS, 16 * tj, lane), a0, d);
                d = mfma(frag_tr(sEc, 32, kCS, 16 * tj, lane), a1, d);
                store4(dst, d[0], d[1], d[2], d[3]);
            }
        }
        {
            bf16x8 fa[4][2];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int s = 0; s < 2; ++s) fa[ti][s] = frag(sAqa, 16 * ti + l16, kCS, 32 * s + 8 * lg);
#pragma unroll
            for (int tt = 0; tt < DK / 64; ++tt) {
                const int tn = wave * (DK / 64) + tt;
                const bf16x8 w0 = frag_tr(sKr, 0, KS, 16 * tn, lane);
                const bf16x8 w1 = frag_tr(sKr, 32, KS, 16 * tn, lane);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    f32x4 o = mfma(w0, fa[ti][0], zero);
                    o = mfma(w1, fa[ti][1], o);
                    const int r = 16 * ti + l16, cc = 16 * tn + 4 * lg;
                    const uint2 qv = *(const uint2 *)(sQl + r * KS + cc);
                    store4(sQl + r * KS + cc, bf16_lo(qv.x) + o[0], bf16_hi(qv.x) + o[1],
                           bf16_lo(qv.y) + o[2], bf16_hi(qv.y) + o[3]);
                }
            }
        }
        lds_barrier();
    };

    // SUB: this workgroup's next flagged job at or after g (stride gridDim.x), 64
    // candidates per round trip; njobs when there is none.
    auto next_job = [&](int g) {
        if constexpr (SUB) {
            while (g < njobs) {  // workgroup-uniform
                const long gi = (long)g + (long)lane * gridDim.x;
                const int f = gi < njobs ? p.sub[gi] : 0;
                const unsigned long long b = __builtin_amdgcn_ballot_w64(f != 0);
                if (b) return g + (int)__builtin_ctzll(b) * (int)gridDim.x;
                g += 64 * (int)gridDim.x;
            }
            return njobs;
        } else {
            return g;
        }
    };

    Job cur = decode(next_job(blockIdx.x));
    if (cur.ok) issue(cur);
    // PAIR: the first half's K^ (before its scaling by the second half's gamma) and its
    // gamma, carried to the merge; the second half's gamma
    float kha[CPT][8], gama[CPT], gamb[CPT];
    while (cur.ok) {  // workgroup-uniform
        // Thread-index values are re-derived from an opaque copy each job: otherwise the
        // compiler hoists every per-lane LDS address of the body out of the loop and
        // keeps them all live, which costs more registers than the body itself.
        int tidv = threadIdx.x;
        asm volatile("" : "+v"(tidv));
        const int tid = tidv;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int l16 = lane & 15, lg = lane >> 4;
        const int rg = tid >> 5, cg = tid & 31, c0 = CPT * cg;
        const int m = cur.m;
        char *bp = p.blk + (size_t)cur.g * kBlkBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (8 * rg + i >= m) {
#pragma unroll
                for (int w = 0; w < WPR; ++w) kw[i][w] = qw[i][w] = aw[i][w] = bw[i][w] = 0u;
#pragma unroll
                for (int e = 0; e < CPT; ++e) lw[i][e] = 0.f;
            }
        }
        if (tid < kC) sBeta[tid] = tid < m ? beta_r : 0.f;
        if (GATE == kGateHead && !CLIP && wave == 0) {
            float x = lane < m ? lah * kLog2e : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            sG[lane] = x;
            if (lane == 63) sG[64] = x;
        }
        // The products read whole 32-wide contraction blocks of X and A_qk, so everything
        // not written below (above the diagonal) must be zero.
        for (int i = tid; i < L::nCC * L::CCB / 16; i += kThreads)
            ((uint4 *)(smem + L::oX))[i] = make_uint4(0u, 0u, 0u, 0u);

        // ---- spectral clip bound per row: log2 (1 / ||I - b a^T||_2) ----------------------
        // Per row |a|^2, |b|^2 and a.b (without a, b: a = k, b = beta k, so |k|^2 alone),
        // summed over this thread's channels and then over the 32 lanes of the row group
        // by a reduce-scatter: three exchange steps each halve the rows a lane keeps
        // (lane bit 3 picks rows 0-3 or 4-7, then bit 2, then bit 1), two full steps finish
        // the sums, and lane l ends with row (l >> 1) & 7.  Its bound is then read back
        // from lane 2 i of the half-wave for each row i.
        float lc[8];
        if constexpr (CLIP) {
            if constexpr (!DP) lds_barrier();  // sBeta of this job
            constexpr int Q = DP ? 3 : 1;
            float sq[8 * Q];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float s0 = 0.f, s1 = 0.f, s2 = 0.f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) {
                    if constexpr (DP) {
                        const float a0 = bf16_lo(aw[i][w]), a1 = bf16_hi(aw[i][w]);
                        const float b0 = bf16_lo(bw[i][w]), b1 = bf16_hi(bw[i][w]);
                        s0 += a0 * a0 + a1 * a1;
                        s1 += b0 * b0 + b1 * b1;
                        s2 += a0 * b0 + a1 * b1;
                    } else {
                        const float k0 = bf16_lo(kw[i][w]), k1 = bf16_hi(kw[i][w]);
                        s0 += k0 * k0 + k1 * k1;
                    }
                }
                sq[Q * i] = s0;
                if constexpr (DP) {
                    sq[Q * i + 1] = s1;
                    sq[Q * i + 2] = s2;
                }
            }
            const int l = lane & 31;
            auto half_step = [&](auto ctrl, int n, bool hi) {
#pragma unroll
                for (int v = 0; v < 4 * Q; ++v) {
                    if (v < n) {
                        const float keep = hi ? sq[v + n] : sq[v], send = hi ? sq[v] : sq[v + n];
                        sq[v] = keep + dpp<decltype(ctrl)::value>(send);
                    }
                }
            };
            half_step(std::integral_constant<int, kDppMirror>(), 4 * Q, (l >> 3) & 1);      // partner 15 - l
            half_step(std::integral_constant<int, kDppHalfMirror>(), 2 * Q, (l >> 2) & 1);  // partner l ^ 7
            half_step(std::integral_constant<int, kDppXor2>(), Q, (l >> 1) & 1);            // partner l ^ 2
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                sq[q] += dpp<kDppXor1>(sq[q]);
                sq[q] += swizzle_xor16(sq[q]);
            }
            float mine;
            if constexpr (DP) {
                mine = clip_bound(sq[0], sq[1], sq[2], 1.f);
            } else {
                const float br = sBeta[8 * rg + ((l >> 1) & 7)];
                mine = clip_bound(sq[0], br * br * sq[0], br * sq[0], 1.f);
            }
            const int mb = __float_as_int(mine);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float lo = __int_as_float(__builtin_amdgcn_readlane(mb, 2 * i));
                const float hi = __int_as_float(__builtin_amdgcn_readlane(mb, 32 + 2 * i));
                lc[i] = lane < 32 ? lo : hi;
            }
        }

        // ---- gate: prefix sums (log2 domain) -------------------------------------------
        float g[8][CPT], gC[CPT];
        if (kRowGate) {
            float run[CPT];
#pragma unroll
            for (int e = 0; e < CPT; ++e) run[e] = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < CPT; ++e) {
                    float x = GATE == kGateChannel ? lw[i][e] * kLog2e
                                                   : (GATE == kGateHead ? lw[i][0] * kLog2e : 0.f);
                    if (CLIP) x = fminf(x, lc[i]);
                    run[e] += x;
                    g[i][e] = run[e];
                }
#pragma unroll
            for (int e = 0; e < CPT; ++e) sTot[rg * DK + c0 + e] = run[e];
        }
        lds_barrier();
        if (kRowGate) {
            float carry[CPT], tot[CPT];
#pragma unroll
            for (int e = 0; e < CPT; ++e) carry[e] = tot[e] = 0.f;
#pragma unroll
            for (int r2 = 0; r2 < 8; ++r2)
#pragma unroll
                for (int e = 0; e < CPT; ++e) {
                    const float t = sTot[r2 * DK + c0 + e];
                    tot[e] += t;
                    carry[e] += r2 < rg ? t : 0.f;
                }
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                gC[e] = tot[e];
#pragma unroll
                for (int i = 0; i < 8; ++i) g[i][e] += carry[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                gC[e] = GATE == kGateHead ? sG[64] : 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) g[i][e] = GATE == kGateHead ? sG[8 * rg + i] : 0.f;
            }
        }
        if constexpr (PAIR) {
            // no log-domain variant on this path: a half whose gate falls beyond the shifted
            // operands' range (below) makes the call's result invalid (error bit 2)
            if (wave == 0) {
                bool wide = false;
#pragma unroll
                for (int e = 0; e < CPT; ++e) wide = wide || !(gC[e] >= -2.f * kSubGateRange);
                if (__builtin_amdgcn_ballot_w64(wide) != 0 && lane == 0) atomicOr(p.err, 2);
            }
        } else if constexpr (!SUB) {
            // wave 0 holds gamma_C of every channel: flag the chunk for the SUB variant when
            // it falls beyond what the shifted operands below cover
            if (p.sub && wave == 0) {
                bool wide = false;
#pragma unroll
                for (int e = 0; e < CPT; ++e) wide = wide || !(gC[e] >= -2.f * kSubGateRange);
                const bool any = __builtin_amdgcn_ballot_w64(wide) != 0;
                if (lane == 0) p.sub[cur.g] = any ? 1 : 0;
            }
        }

        // Gate reference of the Gram operands.  A channel whose gate falls by more than
        // 2^kSubGateRange within the chunk would take K-> = K e^-g out of range; its operands
        // are formed with the gate referred to sh = round(g_C / 2) (a power of two) instead,
        // K<-' = K e^(g - sh), K->' = K e^(sh - g), Q<-' = Q e^(g - sh), so every factor stays
        // within 2^(|g_C| / 2) either way and a chunk may fall by up to 2^(2 kSubGateRange).
        // Their products (the Gram and A_qk) are unchanged; K<- and Q<- (DP: B<- and Q<-)
        // are multiplied back by 2^sh in LDS before the stages that need them (exact in bf16),
        // so the block holds the same quantities either way.  Other channels: sh = 0.
        float sh[CPT];
        [[maybe_unused]] bool shifted = false;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            sh[e] = !SUB && gC[e] < -kSubGateRange ? rintf(0.5f * gC[e]) : 0.f;
            shifted = shifted || sh[e] != 0.f;
        }

        // ---- scaled operands: Q<-, K<-, K-> to LDS; K^ and gamma_C to the block ---------
        // (DP: Q<-, B<-, K->, A-> to LDS; A^, Diag(beta) K^ and gamma_C to the block)
        {
            float kh[CPT][8], kb[CPT][8], gam[CPT];
#pragma unroll
            for (int e = 0; e < CPT; ++e) gam[e] = GATE == kGateNone && !CLIP ? 1.f : exp2_fast(gC[e]);
            // e^(g_C - g) = e^(sh - g) e^(g_C - sh): one exp2 per channel, and neither factor
            // leaves the range (sh = 0: gamma_C itself)
            float gsh[CPT];
#pragma unroll
            for (int e = 0; e < CPT; ++e) gsh[e] = sh[e] != 0.f ? exp2_fast(gC[e] - sh[e]) : gam[e];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * rg + i;
                const float br = DP ? sBeta[r] : 0.f;
                float kv[CPT], qv[CPT], av[CPT], bv[CPT], a[CPT], b[CPT], cq[CPT], ar[CPT];
#pragma unroll
                for (int w = 0; w < WPR; ++w) {
                    kv[2 * w] = bf16_lo(kw[i][w]); kv[2 * w + 1] = bf16_hi(kw[i][w]);
                    qv[2 * w] = bf16_lo(qw[i][w]); qv[2 * w + 1] = bf16_hi(qw[i][w]);
                    if constexpr (DP) {
                        av[2 * w] = bf16_lo(aw[i][w]); av[2 * w + 1] = bf16_hi(aw[i][w]);
                        bv[2 * w] = bf16_lo(bw[i][w]); bv[2 * w + 1] = bf16_hi(bw[i][w]);
                    }
                }
#pragma unroll
                for (int e = 0; e < CPT; ++e) {
                    if constexpr (SUB) {
                        // raw rows for the log-domain Gram (Q<- and B<- are formed after it);
                        // e^(g_C - g) directly, since e^-g may overflow here
                        const float egc = exp2_fast(gC[e] - g[i][e]);
                        a[e] = DP ? bv[e] : kv[e] * exp2_fast(g[i][e]);
                        b[e] = kv[e];
                        cq[e] = qv[e];
                        kh[e][i] = (DP ? av[e] : kv[e]) * egc;
                        if constexpr (DP) {
                            ar[e] = av[e];
                            kb[e][i] = br * kv[e] * egc;
                        }
                        sGf[r * L::GS + c0 + e] = g[i][e];
                        if ((r & 15) == 0) sGref[(r >> 4) * DK + c0 + e] = g[i][e];
                    } else {
                        const float gs = g[i][e] - sh[e];  // (sh = 0: g itself)
                        const float eg = GATE == kGateNone && !CLIP ? 1.f : exp2_fast(gs);
                        const float eig = GATE == kGateNone && !CLIP ? 1.f : exp2_fast(-gs);
                        const float egc = eig * gsh[e];  // e^(g_C - g)
                        a[e] = (DP ? bv[e] : kv[e]) * eg;
                        b[e] = kv[e] * eig;
                        cq[e] = qv[e] * eg;
                        kh[e][i] = (DP ? av[e] : kv[e]) * egc;
                        if constexpr (DP) {
                            ar[e] = av[e] * eig;
                            kb[e][i] = br * kv[e] * egc;
                        }
                    }
                }
                uint32_t wa[WPR], wb[WPR], wq[WPR], wr[WPR];
#pragma unroll
                for (int w = 0; w < WPR; ++w) {
                    wa[w] = pack_bf16x2(a[2 * w], a[2 * w + 1]);
                    wb[w] = pack_bf16x2(b[2 * w], b[2 * w + 1]);
                    wq[w] = pack_bf16x2(cq[2 * w], cq[2 * w + 1]);
                    if constexpr (DP) wr[w] = pack_bf16x2(ar[2 * w], ar[2 * w + 1]);
                }
                if constexpr (WPR == 2) {
                    *(uint2 *)(sKl + r * KS + c0) = make_uint2(wa[0], wa[1]);
                    *(uint2 *)(sKr + r * KS + c0) = make_uint2(wb[0], wb[1]);
                    *(uint2 *)(sQl + r * KS + c0) = make_uint2(wq[0], wq[1]);
                    if constexpr (DP) *(uint2 *)(sAr + r * KS + c0) = make_uint2(wr[0], wr[1]);
                } else {
                    *(uint32_t *)(sKl + r * KS + c0) = wa[0];
                    *(uint32_t *)(sKr + r * KS + c0) = wb[0];
                    *(uint32_t *)(sQl + r * KS + c0) = wq[0];
                    if constexpr (DP) *(uint32_t *)(sAr + r * KS + c0) = wr[0];
                }
            }
            // K^ transposed: channel cc is row cc%32 of fragment tile cc/32; this thread's
            // 8 rows are one 16-byte piece (step rg/2, lane half rg%2).  PAIR: the first
            // half's waits in registers for the second half's gamma; the second half's
            // takes steps 4-7 of the 8 the 128-token tiles have.
            if (PAIR && cur.half == 0) {
#pragma unroll
                for (int e = 0; e < CPT; ++e) {
                    gama[e] = gam[e];
#pragma unroll
                    for (int i = 0; i < 8; ++i) kha[e][i] = kh[e][i];
                }
            } else {
#pragma unroll
                for (int e = 0; e < CPT; ++e) {
                    const int cc = c0 + e;
                    const int pc = PAIR ? (cc >> 5) * 8 * 64 + (4 + (rg >> 1)) * 64 + (cc & 31) + 32 * (rg & 1)
                                        : (cc >> 5) * 4 * 64 + (rg >> 1) * 64 + (cc & 31) + 32 * (rg & 1);
                    uint4 w;
                    w.x = pack_bf16x2(kh[e][0], kh[e][1]);
                    w.y = pack_bf16x2(kh[e][2], kh[e][3]);
                    w.z = pack_bf16x2(kh[e][4], kh[e][5]);
                    w.w = pack_bf16x2(kh[e][6], kh[e][7]);
                    ((uint4 *)(bp + (PAIR ? B2::oK : Bk::oK)))[pc] = w;
                    if constexpr (DP) {
                        w.x = pack_bf16x2(kb[e][0], kb[e][1]);
                        w.y = pack_bf16x2(kb[e][2], kb[e][3]);
                        w.z = pack_bf16x2(kb[e][4], kb[e][5]);
                        w.w = pack_bf16x2(kb[e][6], kb[e][7]);
                        ((uint4 *)(bp + Bk::oKb))[pc] = w;
                    }
                }
            }
            if (PAIR && cur.half == 1) {
#pragma unroll
                for (int e = 0; e < CPT; ++e) gamb[e] = gam[e];
            }
            if (rg == 0 && !(PAIR && cur.half == 0)) {
#pragma unroll
                for (int e = 0; e < CPT; ++e)
                    ((float *)(bp + (PAIR ? B2::oG : Bk::oG)))[c0 + e] = PAIR ? gama[e] * gam[e] : gam[e];
            }
        }
        // this job's raw inputs are consumed: the next job's start loading (PAIR: the
        // second half of this chunk, then the next chunk)
        const Job nxt = PAIR && cur.half == 0 ? decode(cur.g, 1) : decode(next_job(cur.g + gridDim.x));
        if (nxt.ok) issue(nxt);
        lds_barrier();

        // ---- L and A_qk: the 10 lower-triangle 16x16 tiles of each (20 jobs) -----------
        // (DP: B<- A->^T, B<- K->^T, Q<- K->^T, Q<- A->^T; 40 jobs.)
        // Computed transposed, D[c][r] = K->[c] . (K<- or Q<-)[r], so that each lane holds
        // four consecutive columns of one row.
        if constexpr (SUB) {
            // Log-domain Gram by 16-row sub-chunks (GLA notes, section 5.3): no operand
            // carries e^-g, so nothing overflows however far the gate falls.  Tile (ti, tj)
            // takes the gate referred to the first row s of tile ti: rows x_r 2^(g_r - g_s)
            // (at most 1), columns y_c 2^(g_s - g_c) (at most 1 for tj < ti; for the
            // diagonal tile at most 2^(g_s - g_(s+15)), which is bounded by kSubTileRange
            // there) on MFMA.  A diagonal tile whose gate falls further is formed
            // element-wise in fp32, x_r . (y_c 2^(g_r - g_c)) with the exponent formed as
            // a difference (the notes' form for diagonal sub-chunks), by the wave that owns
            // its rows: ten lower 4x4 blocks of pairs on four lanes each (a quarter of the
            // channels per lane), six upper blocks written as zeros.
            constexpr int NP = DP ? 4 : 2;  // products: DP: BA, BK, QK, QA; else KK, QK
            // results of one output row of four pairs (r, cb..cb+3), as the fast path
            // stores them: L (DP: B<- A->^T) strictly lower, x beta_r (not for DP) ...
            auto put = [&](const float (&acc)[NP][4], int r, int cb, bool diag) {
                const float4 bc = *(const float4 *)(sBeta + cb);
                const float bcv[4] = {bc.x, bc.y, bc.z, bc.w};
                const float br = DP ? 1.f : sBeta[r];
                float lv[4], av[4], bkv[4], qav[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = cb + j;
                    lv[j] = c < r ? br * acc[0][j] : 0.f;
                    if constexpr (DP) {
                        bkv[j] = c < r ? bcv[j] * acc[1][j] : 0.f;  // B<- K->^T Diag(beta)
                        av[j] = c <= r ? bcv[j] * acc[2][j] : 0.f;  // Q<- K->^T Diag(beta)
                        qav[j] = c <= r ? acc[3][j] : 0.f;          // Q<- A->^T
                    } else {
                        av[j] = c <= r ? acc[1][j] : 0.f;           // A_qk
                    }
                }
                if (diag) *(float4 *)(sLd + r * kDS + (cb & 15)) = make_float4(lv[0], lv[1], lv[2], lv[3]);
                else store4(sX + r * kCS + cb, lv[0], lv[1], lv[2], lv[3]);
                store4(sAqk + r * kCS + cb, av[0], av[1], av[2], av[3]);
                if constexpr (DP) {
                    store4(sBK + r * kCS + cb, bkv[0], bkv[1], bkv[2], bkv[3]);
                    store4(sAqa + r * kCS + cb, qav[0], qav[1], qav[2], qav[3]);
                }
            };
            // rows x (DP: b, else k) and q; columns k (DP: and a), all raw
            const uint16_t *rx = DP ? sKl : sKr;
            // does the gate of this wave's tile fall further than kSubTileRange? (lanes
            // 32-63 hold the tile's last row; sGref its first)
            bool wide_t = false;
#pragma unroll
            for (int e = 0; e < CPT; ++e) wide_t = wide_t || !(sGref[wave * DK + c0 + e] - g[7][e] <= kSubTileRange);
            wide_t = __builtin_amdgcn_ballot_w64(wide_t && lane >= 32) != 0;
            if (lane == 0) sWide[wave] = wide_t ? 1 : 0;
            if (wide_t && lane < 40) {
                const int qd = lane & 3, t = wave, lb = lane >> 2;
                const int u = lb >= 6 ? 3 : (lb >= 3 ? 2 : (lb >= 1 ? 1 : 0));
                const int v = lb - u * (u + 1) / 2;
                const int r0 = 16 * t + 4 * u, cb = 16 * t + 4 * v;
                float acc[NP][4][4];
#pragma unroll
                for (int pp = 0; pp < NP; ++pp)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[pp][i][j] = 0.f;
                for (int d = qd * (DK / 4); d < (qd + 1) * (DK / 4); d += 4) {
                    float gr[4][4], gc[4][4], xr[4][4], qr[4][4], kc[4][4], ac[4][4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float4 a4 = *(const float4 *)(sGf + (r0 + i) * L::GS + d);
                        const float4 b4 = *(const float4 *)(sGf + (cb + i) * L::GS + d);
                        gr[i][0] = a4.x; gr[i][1] = a4.y; gr[i][2] = a4.z; gr[i][3] = a4.w;
                        gc[i][0] = b4.x; gc[i][1] = b4.y; gc[i][2] = b4.z; gc[i][3] = b4.w;
                        const uint2 x2 = *(const uint2 *)(rx + (r0 + i) * KS + d);
                        const uint2 q2 = *(const uint2 *)(sQl + (r0 + i) * KS + d);
                        const uint2 k2 = *(const uint2 *)(sKr + (cb + i) * KS + d);
                        xr[i][0] = bf16_lo(x2.x); xr[i][1] = bf16_hi(x2.x); xr[i][2] = bf16_lo(x2.y); xr[i][3] = bf16_hi(x2.y);
                        qr[i][0] = bf16_lo(q2.x); qr[i][1] = bf16_hi(q2.x); qr[i][2] = bf16_lo(q2.y); qr[i][3] = bf16_hi(q2.y);
                        kc[i][0] = bf16_lo(k2.x); kc[i][1] = bf16_hi(k2.x); kc[i][2] = bf16_lo(k2.y); kc[i][3] = bf16_hi(k2.y);
                        if constexpr (DP) {
                            const uint2 a2 = *(const uint2 *)(sAr + (cb + i) * KS + d);
                            ac[i][0] = bf16_lo(a2.x); ac[i][1] = bf16_hi(a2.x); ac[i][2] = bf16_lo(a2.y); ac[i][3] = bf16_hi(a2.y);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                // pairs above the diagonal are discarded: keep them finite
                                const float x = exp2_fast(fminf(gr[i][e] - gc[j][e], 0.f));
                                const float xk = kc[j][e] * x;
                                if constexpr (DP) {
                                    const float xa = ac[j][e] * x;
                                    acc[0][i][j] += xr[i][e] * xa;
                                    acc[1][i][j] += xr[i][e] * xk;
                                    acc[2][i][j] += qr[i][e] * xk;
                                    acc[3][i][j] += qr[i][e] * xa;
                                } else {
                                    acc[0][i][j] += xr[i][e] * xk;
                                    acc[1][i][j] += qr[i][e] * xk;
                                }
                            }
                }
#pragma unroll
                for (int pp = 0; pp < NP; ++pp)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            acc[pp][i][j] += dpp<kDppXor1>(acc[pp][i][j]);
                            acc[pp][i][j] += dpp<kDppXor2>(acc[pp][i][j]);
                        }
                if (qd == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float row[NP][4];
#pragma unroll
                        for (int pp = 0; pp < NP; ++pp)
#pragma unroll
                            for (int j = 0; j < 4; ++j) row[pp][j] = acc[pp][i][j];
                        put(row, r0 + i, cb, true);
                    }
                }
            } else if (wide_t && lane < 46) {
                const int t = wave, k6 = lane - 40;
                const int u = k6 < 3 ? 0 : (k6 < 5 ? 1 : 2);
                const int v = u == 0 ? k6 + 1 : (u == 1 ? k6 - 1 : 3);
                float zero[NP][4];
#pragma unroll
                for (int pp = 0; pp < NP; ++pp)
#pragma unroll
                    for (int j = 0; j < 4; ++j) zero[pp][j] = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) put(zero, 16 * t + 4 * u + i, 16 * t + 4 * v, true);
            }
            lds_barrier();  // the gate array is free: the operands below go over it

            // scratch rows (bf16, stride KS): columns k' at 0..47 (DP: a' at 48..95), rows x'
            // at 96..111, q' at 112..127; the diagonal tile's columns at 0..15 (a' 48..63)
            for (int ti = 0; ti < 4; ++ti) {
                if (ti > 0 && rg < 2 * ti + 2) {  // owners of rows 0 .. 16 ti + 15
                    const int s0 = 16 * ti;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int r = 8 * rg + i;
                        float f[CPT];
#pragma unroll
                        for (int e = 0; e < CPT; ++e) {
                            const float gs = sGref[ti * DK + c0 + e];
                            f[e] = exp2_fast(r >= s0 ? g[i][e] - gs : gs - g[i][e]);
                        }
#pragma unroll
                        for (int w = 0; w < WPR; ++w) {
                            if (r >= s0) {
                                const uint32_t xw = *(const uint32_t *)(rx + r * KS + c0 + 2 * w);
                                const uint32_t qw2 = *(const uint32_t *)(sQl + r * KS + c0 + 2 * w);
                                *(uint32_t *)(sVar + (96 + r - s0) * KS + c0 + 2 * w) =
                                    pack_bf16x2(bf16_lo(xw) * f[2 * w], bf16_hi(xw) * f[2 * w + 1]);
                                *(uint32_t *)(sVar + (112 + r - s0) * KS + c0 + 2 * w) =
                                    pack_bf16x2(bf16_lo(qw2) * f[2 * w], bf16_hi(qw2) * f[2 * w + 1]);
                            } else {
                                const uint32_t kw2 = *(const uint32_t *)(sKr + r * KS + c0 + 2 * w);
                                *(uint32_t *)(sVar + r * KS + c0 + 2 * w) =
                                    pack_bf16x2(bf16_lo(kw2) * f[2 * w], bf16_hi(kw2) * f[2 * w + 1]);
                                if constexpr (DP) {
                                    const uint32_t aw2 = *(const uint32_t *)(sAr + r * KS + c0 + 2 * w);
                                    *(uint32_t *)(sVar + (48 + r) * KS + c0 + 2 * w) =
                                        pack_bf16x2(bf16_lo(aw2) * f[2 * w], bf16_hi(aw2) * f[2 * w + 1]);
                                }
                            }
                        }
                    }
                }
                lds_barrier();
                // tiles (ti, tj < ti) of each product, one 16x16 tile per wave and turn,
                // computed transposed like the fast path
                for (int jb = wave; jb < NP * ti; jb += 4) {
                    const int pr = jb / ti, tj = jb - pr * ti;
                    const bool qrow = DP ? pr >= 2 : pr == 1;
                    const bool acol = DP && (pr == 0 || pr == 3);
                    const uint16_t *src = sVar + (qrow ? 112 : 96) * KS;
                    const uint16_t *col = sVar + (acol ? 48 : 0) * KS;
                    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < DK / 32; ++s)
                        d = mfma(frag(col, 16 * tj + l16, KS, 32 * s + 8 * lg), frag(src, l16, KS, 32 * s + 8 * lg), d);
                    const int r = 16 * ti + l16, cb = 16 * tj + 4 * lg;
                    if (DP && pr > 0) {
                        const float4 be = pr < 3 ? *(const float4 *)(sBeta + cb) : make_float4(1.f, 1.f, 1.f, 1.f);
                        uint16_t *dst = pr == 1 ? sBK : (pr == 2 ? sAqk : sAqa);
                        store4(dst + r * kCS + cb, be.x * d[0], be.y * d[1], be.z * d[2], be.w * d[3]);
                    } else if (!DP && pr == 1) {
                        store4(sAqk + r * kCS + cb, d[0], d[1], d[2], d[3]);
                    } else {
                        const float br = DP ? 1.f : sBeta[r];
                        store4(sX + r * kCS + cb, br * d[0], br * d[1], br * d[2], br * d[3]);
                    }
                }
                if (ti > 0) lds_barrier();  // the column rows are rewritten below
                // the diagonal tile (ti, ti), unless it was formed element-wise
                const bool wide = sWide[ti] != 0;  // workgroup-uniform
                if (!wide) {
                    if (rg == 2 * ti || rg == 2 * ti + 1) {  // owners of tile ti's rows
                        const int s0 = 16 * ti;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const int r = 8 * rg + i;
                            float fc[CPT], fr[CPT];
#pragma unroll
                            for (int e = 0; e < CPT; ++e) {
                                const float gs = sGref[ti * DK + c0 + e];
                                fc[e] = exp2_fast(gs - g[i][e]);
                                fr[e] = exp2_fast(g[i][e] - gs);
                            }
#pragma unroll
                            for (int w = 0; w < WPR; ++w) {
                                const uint32_t kw2 = *(const uint32_t *)(sKr + r * KS + c0 + 2 * w);
                                *(uint32_t *)(sVar + (r - s0) * KS + c0 + 2 * w) =
                                    pack_bf16x2(bf16_lo(kw2) * fc[2 * w], bf16_hi(kw2) * fc[2 * w + 1]);
                                if constexpr (DP) {
                                    const uint32_t aw2 = *(const uint32_t *)(sAr + r * KS + c0 + 2 * w);
                                    *(uint32_t *)(sVar + (48 + r - s0) * KS + c0 + 2 * w) =
                                        pack_bf16x2(bf16_lo(aw2) * fc[2 * w], bf16_hi(aw2) * fc[2 * w + 1]);
                                }
                                if (ti == 0) {  // the rows were not built above
                                    const uint32_t xw = *(const uint32_t *)(rx + r * KS + c0 + 2 * w);
                                    const uint32_t qw2 = *(const uint32_t *)(sQl + r * KS + c0 + 2 * w);
                                    *(uint32_t *)(sVar + (96 + r - s0) * KS + c0 + 2 * w) =
                                        pack_bf16x2(bf16_lo(xw) * fr[2 * w], bf16_hi(xw) * fr[2 * w + 1]);
                                    *(uint32_t *)(sVar + (112 + r - s0) * KS + c0 + 2 * w) =
                                        pack_bf16x2(bf16_lo(qw2) * fr[2 * w], bf16_hi(qw2) * fr[2 * w + 1]);
                                }
                            }
                        }
                    }
                    lds_barrier();
                    for (int pr = wave; pr < NP; pr += 4) {
                        const bool qrow = DP ? pr >= 2 : pr == 1;
                        const bool acol = DP && (pr == 0 || pr == 3);
                        const uint16_t *src = sVar + (qrow ? 112 : 96) * KS;
                        const uint16_t *col = sVar + (acol ? 48 : 0) * KS;
                        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < DK / 32; ++s)
                            d = mfma(frag(col, l16, KS, 32 * s + 8 * lg), frag(src, l16, KS, 32 * s + 8 * lg), d);
                        const int r = 16 * ti + l16, cb = 16 * ti + 4 * lg;
                        const float4 be = *(const float4 *)(sBeta + cb);
                        const float bcv[4] = {be.x, be.y, be.z, be.w};
                        float o[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int c = cb + j;
                            const bool strict = DP ? pr < 2 : pr == 0;  // L, BA, BK: below the diagonal
                            const bool keep = strict ? c < r : c <= r;
                            const float sc = DP ? ((pr == 1 || pr == 2) ? bcv[j] : 1.f) : (pr == 0 ? sBeta[r] : 1.f);
                            o[j] = keep ? sc * d[j] : 0.f;
                        }
                        if (pr == 0) {
                            *(float4 *)(sLd + r * kDS + 4 * lg) = make_float4(o[0], o[1], o[2], o[3]);
                        } else {
                            uint16_t *dst = DP ? (pr == 1 ? sBK : (pr == 2 ? sAqk : sAqa)) : sAqk;
                            store4(dst + r * kCS + cb, o[0], o[1], o[2], o[3]);
                        }
                    }
                }
                lds_barrier();  // the scratch rows are rewritten for the next ti
            }
        } else
        for (int jb = wave; jb < (DP ? 40 : 20); jb += 4) {
            const int pr = jb / 10;  // product
            const bool isA = !DP && pr == 1;
            const int t = jb - 10 * pr;
            const int ti = t >= 6 ? 3 : (t >= 3 ? 2 : (t >= 1 ? 1 : 0));
            const int tj = t - ti * (ti + 1) / 2;
            const uint16_t *src = DP ? (pr < 2 ? sKl : sQl) : (isA ? sQl : sKl);
            const uint16_t *col = DP && (pr == 0 || pr == 3) ? sAr : sKr;
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < DK / 32; ++s)
                d = mfma(frag(col, 16 * tj + l16, KS, 32 * s + 8 * lg),
                         frag(src, 16 * ti + l16, KS, 32 * s + 8 * lg), d);
            const int r = 16 * ti + l16, cb = 16 * tj + 4 * lg;
            if (DP && pr > 0) {
                // B<- K->^T (strictly lower) and Q<- K->^T (with the diagonal) take the
                // column scaling Diag(beta) of the value they multiply; Q<- A->^T does not.
                const float4 be = pr < 3 ? *(const float4 *)(sBeta + cb) : make_float4(1.f, 1.f, 1.f, 1.f);
                const int lim = pr == 1 ? r : r + 1;  // columns below lim are kept
                uint16_t *dst = pr == 1 ? sBK : (pr == 2 ? sAqk : sAqa);
                store4(dst + r * kCS + cb, cb + 0 < lim ? be.x * d[0] : 0.f, cb + 1 < lim ? be.y * d[1] : 0.f,
                       cb + 2 < lim ? be.z * d[2] : 0.f, cb + 3 < lim ? be.w * d[3] : 0.f);
            } else if (isA) {
                store4(sAqk + r * kCS + cb, cb + 0 <= r ? d[0] : 0.f, cb + 1 <= r ? d[1] : 0.f,
                       cb + 2 <= r ? d[2] : 0.f, cb + 3 <= r ? d[3] : 0.f);
            } else {
                const float br = DP ? 1.f : sBeta[r];  // DP: E's system has no beta
                const float v0 = cb + 0 < r ? br * d[0] : 0.f, v1 = cb + 1 < r ? br * d[1] : 0.f;
                const float v2 = cb + 2 < r ? br * d[2] : 0.f, v3 = cb + 3 < r ? br * d[3] : 0.f;
                if (ti == tj) *(float4 *)(sLd + (16 * ti + l16) * kDS + 4 * lg) = make_float4(v0, v1, v2, v3);
                else store4(sX + r * kCS + cb, v0, v1, v2, v3);
            }
        }
        lds_barrier();
        if constexpr (!SUB && (GATE != kGateNone || CLIP)) {
            // shifted channels: K<-' 2^sh = K<-, Q<-' 2^sh = Q<- (DP: B<-, Q<-), now that the
            // Gram has read them; later stages read them after further barriers
            if (shifted) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 8 * rg + i;
#pragma unroll
                    for (int e = 0; e < CPT; e += 2) {
                        const int n0 = (int)sh[e], n1 = (int)sh[e + 1];
                        uint32_t *pq = (uint32_t *)(sQl + r * KS + c0 + e);
                        uint32_t *pk = (uint32_t *)(sKl + r * KS + c0 + e);
                        *pq = pack_bf16x2(__builtin_amdgcn_ldexpf(bf16_lo(*pq), n0),
                                          __builtin_amdgcn_ldexpf(bf16_hi(*pq), n1));
                        *pk = pack_bf16x2(__builtin_amdgcn_ldexpf(bf16_lo(*pk), n0),
                                          __builtin_amdgcn_ldexpf(bf16_hi(*pk), n1));
                    }
                }
            }
        }
        if constexpr (SUB) {
            // Q<- (DP: and B<-) from the raw rows, now that the Gram has read them; later
            // stages read them after further barriers
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * rg + i;
#pragma unroll
                for (int e = 0; e < CPT; e += 2) {
                    const float e0 = exp2_fast(g[i][e]), e1 = exp2_fast(g[i][e + 1]);
                    uint32_t *pq = (uint32_t *)(sQl + r * KS + c0 + e);
                    *pq = pack_bf16x2(bf16_lo(*pq) * e0, bf16_hi(*pq) * e1);
                    if constexpr (DP) {
                        uint32_t *pb = (uint32_t *)(sKl + r * KS + c0 + e);
                        *pb = pack_bf16x2(bf16_lo(*pb) * e0, bf16_hi(*pb) * e1);
                    }
                }
            }
        }

        // ---- At, diagonal blocks: forward substitution (wave 0) ------------------------
        // Lane (block lg, column l16): x_r = [r == col] - sum_{i<r} L[r][i] x_i, which
        // leaves x_r = 0 for r < col without any masking.
        if (wave == 0) {
            const float *Lb = sLd + 16 * lg * kDS;
            float x[16];
            float4 cur[4], nxt[4];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (r + 1 < 16) {
#pragma unroll
                    for (int i4 = 0; i4 < (r + 4) / 4; ++i4) nxt[i4] = *(const float4 *)(Lb + (r + 1) * kDS + 4 * i4);
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
            for (int r = 0; r < 16; ++r) {
                sLd[(16 * lg + r) * kDS + l16] = x[r];
                sX[(16 * lg + r) * kCS + 16 * lg + l16] = __builtin_bit_cast(uint16_t, (__bf16)x[r]);
            }
        }
        lds_barrier();

        // ---- At, 32-row level (waves 0, 1): X_BA = -X_BB (L_BA X_AA) --------------------
        if (wave < 2) {
            const int a0 = 32 * wave, a1 = a0 + 16;
            const bf16x4 fL = *(const bf16x4 *)(sX + (a1 + l16) * kCS + a0 + 4 * lg);
            bf16x4 fXa;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                fXa[e] = __builtin_bit_cast(__bf16, sX[(a0 + 4 * lg + e) * kCS + a0 + l16]);
            const f32x4 t = mfma16(fL, fXa, f32x4{0.f, 0.f, 0.f, 0.f});  // t[e] = T[4lg+e][l16]
            const bf16x4 fXb = *(const bf16x4 *)(sX + (a1 + l16) * kCS + a1 + 4 * lg);
            const f32x4 x = mfma16(fXb, to_bf16x4(t[0], t[1], t[2], t[3]), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sX[(a1 + 4 * lg + e) * kCS + a0 + l16] = __builtin_bit_cast(uint16_t, (__bf16)(-x[e]));
        }
        lds_barrier();

        // ---- At, 64-row level (waves 0-3, one 16x16 tile each) -------------------------
        {
            const int ti = wave >> 1, tj = wave & 1;
            const f32x4 t = mfma(frag(sX, 32 + 16 * ti + l16, kCS, 8 * lg), frag_tr(sX, 0, kCS, 16 * tj, lane),
                                 f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sT[(16 * ti + 4 * lg + e) * kTS + 16 * tj + l16] = __builtin_bit_cast(uint16_t, (__bf16)t[e]);
            lds_barrier();
            const f32x4 x = mfma(frag(sX, 32 + 16 * ti + l16, kCS, 32 + 8 * lg), frag_tr(sT, 0, kTS, 16 * tj, lane),
                                 f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sX[(32 + 16 * ti + 4 * lg + e) * kCS + 16 * tj + l16] = __builtin_bit_cast(uint16_t, (__bf16)(-x[e]));
        }
        lds_barrier();

        if constexpr (DP) {
            dplr_products();
        } else {
        // ---- Ab = At Diag(beta), in place (diagonal blocks from the fp32 copy) ---------
        // Thread: row r, 16 columns from cb.  Both sources are read and one is selected,
        // so that the lanes of a wave do not diverge.
        {
            const int r = tid >> 2, cbk = tid & 3, cb = 16 * cbk, b = r >> 4;
            const uint4 x0 = *(const uint4 *)(sX + r * kCS + cb), x1 = *(const uint4 *)(sX + r * kCS + cb + 8);
            const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const float *dr = sLd + (16 * b + (r & 15)) * kDS;
            const bool diag = cbk == b;
            uint32_t w[8];
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const float4 d = *(const float4 *)(dr + 4 * i4);
                const float4 be = *(const float4 *)(sBeta + cb + 4 * i4);
                const float dv[4] = {d.x, d.y, d.z, d.w}, bv[4] = {be.x, be.y, be.z, be.w};
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * i4 + e, ca = cb + i;
                    const uint32_t word = xw[i >> 1];
                    const float a = diag ? dv[e] : ((i & 1) ? bf16_hi(word) : bf16_lo(word));
                    x[e] = ca <= r ? a * bv[e] : 0.f;
                }
                w[2 * i4] = pack_bf16x2(x[0], x[1]);
                w[2 * i4 + 1] = pack_bf16x2(x[2], x[3]);
            }
            *(uint4 *)(sX + r * kCS + cb) = make_uint4(w[0], w[1], w[2], w[3]);
            *(uint4 *)(sX + r * kCS + cb + 8) = make_uint4(w[4], w[5], w[6], w[7]);
        }
        lds_barrier();

        // ---- Ao = A_qk Ab, in place: wave ti owns 16-row block ti ----------------------
        {
            const int ti = wave;
            const bf16x8 b0 = frag(sAqk, 16 * ti + l16, kCS, 8 * lg);
            const bf16x8 b1 = frag(sAqk, 16 * ti + l16, kCS, 32 + 8 * lg);
            for (int tj = 0; tj <= ti; ++tj) {  // wave-uniform
                f32x4 d = mfma(frag_tr(sX, 0, kCS, 16 * tj, lane), b0, f32x4{0.f, 0.f, 0.f, 0.f});
                d = mfma(frag_tr(sX, 32, kCS, 16 * tj, lane), b1, d);
                store4(sAqk + (16 * ti + l16) * kCS + 16 * tj + 4 * lg, d[0], d[1], d[2], d[3]);
            }
        }
        lds_barrier();

        // ---- W' = -Ab K<- (into the K-> array), Q~ = Q<- - Ao K<- (in place) ------------
        {
            bf16x8 fab[4][2], fao[4][2];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    fab[ti][s] = frag(sX, 16 * ti + l16, kCS, 32 * s + 8 * lg);
                    fao[ti][s] = frag(sAqk, 16 * ti + l16, kCS, 32 * s + 8 * lg);
                }
#pragma unroll
            for (int tt = 0; tt < DK / 64; ++tt) {
                const int tn = wave * (DK / 64) + tt;
                const bf16x8 k0 = frag_tr(sKl, 0, KS, 16 * tn, lane);
                const bf16x8 k1 = frag_tr(sKl, 32, KS, 16 * tn, lane);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    f32x4 w = mfma(k0, fab[ti][0], f32x4{0.f, 0.f, 0.f, 0.f});
                    w = mfma(k1, fab[ti][1], w);
                    f32x4 o = mfma(k0, fao[ti][0], f32x4{0.f, 0.f, 0.f, 0.f});
                    o = mfma(k1, fao[ti][1], o);
                    const int r = 16 * ti + l16, cc = 16 * tn + 4 * lg;
                    store4(sKr + r * KS + cc, -w[0], -w[1], -w[2], -w[3]);
                    const uint2 qv = *(const uint2 *)(sQl + r * KS + cc);
                    store4(sQl + r * KS + cc, bf16_lo(qv.x) - o[0], bf16_hi(qv.x) - o[1],
                           bf16_lo(qv.y) - o[2], bf16_hi(qv.y) - o[3]);
                }
            }
        }
        lds_barrier();
        }

        // ---- fragment tiles out: W', Q~ (2 row tiles x DK/16 steps), Ab, Ao (3 tiles) ---
        // (PAIR, first half: the same tiles are rows 0-63 of the 128-token block)
        constexpr int NPW = 2 * (DK / 16) * 64;
        if (!PAIR || cur.half == 0) {
            for (int pc = tid; pc < NPW; pc += kThreads) {
                const int t = pc / ((DK / 16) * 64), s = (pc >> 6) % (DK / 16), ln = pc & 63;
                const int r = 32 * t + (ln & 31), cc = 16 * s + 8 * (ln >> 5);
                ((uint4 *)(bp + (PAIR ? B2::oW : Bk::oW)))[pc] = *(const uint4 *)(sKr + r * KS + cc);
                ((uint4 *)(bp + (PAIR ? B2::oQ : Bk::oQ)))[pc] = *(const uint4 *)(sQl + r * KS + cc);
            }
            for (int pc = tid; pc < 3 * 128; pc += kThreads) {
                const int tau = pc >> 7, s = (pc >> 6) & 1, ln = pc & 63;
                const int r = (tau ? 32 : 0) + (ln & 31), cc = (tau == 2 ? 32 : 0) + 16 * s + 8 * (ln >> 5);
                ((uint4 *)(bp + (PAIR ? B2::oAb : Bk::oAb)))[pc] = *(const uint4 *)((DP ? sEc : sX) + r * kCS + cc);
                ((uint4 *)(bp + (PAIR ? B2::oAo : Bk::oAo)))[pc] = *(const uint4 *)(sAqk + r * kCS + cc);
            }
        } else if constexpr (PAIR) {
            // ---- merge of the two halves into one 128-token chunk --------------------------
            // With a, b the halves, the state entering b is S_a = S Diag(gamma_a) + V_a^T K^_a
            // (V_a = Ab_a V + W'_a S^T), so b's rows against the state entering the chunk are
            //   V_b = [M Ab_a, Ab_b] V + (W'_b Diag(gamma_a) + M W'_a) S^T,     M = W'_b K^_a^T
            //   O_b = [N Ab_a, Ao_b] V + (Q~_b Diag(gamma_a) + N W'_a) S^T,     N = Q~_b K^_a^T
            // and the chunk's state update is S Diag(gamma_a gamma_b) + V_a^T (K^_a Diag(gamma_b))
            // + V_b^T K^_b: the WY factors of the 128-token chunk, built from those of its
            // 64-token sub-chunks (secondary chunking, "Gated Linear Attention" notes,
            // section 5.3).  W'_b, Q~_b, Ab_b, Ao_b are in LDS; W'_a and Ab_a are read back
            // from the first half's tiles of this block; K^_a is in registers.
            //
            // (1) Ab_b, Ao_b -> tiles (2,2), (3,2), (3,3) of Ab'', Ao''
            for (int pc = tid; pc < 3 * 128; pc += kThreads) {
                const int tau = pc >> 7, s = (pc >> 6) & 1, ln = pc & 63;
                const int r = (tau ? 32 : 0) + (ln & 31), cc = (tau == 2 ? 32 : 0) + 16 * s + 8 * (ln >> 5);
                const int dt = tau == 0 ? 5 : (tau == 1 ? 8 : 9);
                ((uint4 *)(bp + B2::oAb))[dt * 128 + (pc & 127)] = *(const uint4 *)(sX + r * kCS + cc);
                ((uint4 *)(bp + B2::oAo))[dt * 128 + (pc & 127)] = *(const uint4 *)(sAqk + r * kCS + cc);
            }
            // (2) K^_a as rows [64 tokens][KS] over K<- (free since W'_b, Q~_b were formed);
            //     gamma_a over the gate scratch
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * rg + i;
                uint32_t wk[WPR];
#pragma unroll
                for (int w = 0; w < WPR; ++w) wk[w] = pack_bf16x2(kha[2 * w][i], kha[2 * w + 1][i]);
                if constexpr (WPR == 2) *(uint2 *)(sKl + r * KS + c0) = make_uint2(wk[0], wk[WPR - 1]);
                else *(uint32_t *)(sKl + r * KS + c0) = wk[0];
            }
            if (rg == 0) {
#pragma unroll
                for (int e = 0; e < CPT; ++e) sTot[c0 + e] = gama[e];
            }
            __syncthreads();  // also completes the first half's stores, which are read back below
            // (3) M -> X array, N -> A_qk array (64 x 64 each; transposed products as for the
            //     Gram, so that each lane holds four consecutive columns of one row)
            for (int jb = wave; jb < 32; jb += 4) {
                const int pr = jb >> 4, t = jb & 15, ti = t >> 2, tj = t & 3;
                const uint16_t *src = pr ? sQl : sKr;
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < DK / 32; ++s)
                    d = mfma(frag(sKl, 16 * tj + l16, KS, 32 * s + 8 * lg), frag(src, 16 * ti + l16, KS, 32 * s + 8 * lg), d);
                store4((pr ? sAqk : sX) + (16 * ti + l16) * kCS + 16 * tj + 4 * lg, d[0], d[1], d[2], d[3]);
            }
            lds_barrier();
            // (4) W'_a, row-major over K<- (from the first half's fragment tiles)
            for (int pc = tid; pc < NPW; pc += kThreads) {
                const int t = pc / ((DK / 16) * 64), s = (pc >> 6) % (DK / 16), ln = pc & 63;
                const int r = 32 * t + (ln & 31), cc = 16 * s + 8 * (ln >> 5);
                *(uint4 *)(sKl + r * KS + cc) = ((const uint4 *)(bp + B2::oW))[pc];
            }
            lds_barrier();
            //     W''_b = W'_b Diag(gamma_a) + M W'_a, Q~''_b = Q~_b Diag(gamma_a) + N W'_a, in place
            {
                bf16x8 fm[4][2], fn[4][2];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        fm[ti][s] = frag(sX, 16 * ti + l16, kCS, 32 * s + 8 * lg);
                        fn[ti][s] = frag(sAqk, 16 * ti + l16, kCS, 32 * s + 8 * lg);
                    }
#pragma unroll
                for (int tt = 0; tt < DK / 64; ++tt) {
                    const int tn = wave * (DK / 64) + tt;
                    const bf16x8 w0 = frag_tr(sKl, 0, KS, 16 * tn, lane);
                    const bf16x8 w1 = frag_tr(sKl, 32, KS, 16 * tn, lane);
                    const float4 ga = *(const float4 *)(sTot + 16 * tn + 4 * lg);
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) {
                        const int r = 16 * ti + l16, cc = 16 * tn + 4 * lg;
                        const uint2 wv = *(const uint2 *)(sKr + r * KS + cc);
                        const uint2 qv = *(const uint2 *)(sQl + r * KS + cc);
                        f32x4 w = {bf16_lo(wv.x) * ga.x, bf16_hi(wv.x) * ga.y, bf16_lo(wv.y) * ga.z, bf16_hi(wv.y) * ga.w};
                        f32x4 o = {bf16_lo(qv.x) * ga.x, bf16_hi(qv.x) * ga.y, bf16_lo(qv.y) * ga.z, bf16_hi(qv.y) * ga.w};
                        w = mfma(w0, fm[ti][0], w);
                        w = mfma(w1, fm[ti][1], w);
                        o = mfma(w0, fn[ti][0], o);
                        o = mfma(w1, fn[ti][1], o);
                        store4(sKr + r * KS + cc, w[0], w[1], w[2], w[3]);
                        store4(sQl + r * KS + cc, o[0], o[1], o[2], o[3]);
                    }
                }
            }
            lds_barrier();
            // (5) W''_b, Q~''_b -> row tiles 2, 3; Ab_a, row-major over K<- (zero where the
            //     tiles are: rows 0-31, columns 32-63)
            for (int pc = tid; pc < NPW; pc += kThreads) {
                const int t = pc / ((DK / 16) * 64), s = (pc >> 6) % (DK / 16), ln = pc & 63;
                const int r = 32 * t + (ln & 31), cc = 16 * s + 8 * (ln >> 5);
                ((uint4 *)(bp + B2::oW))[NPW + pc] = *(const uint4 *)(sKr + r * KS + cc);
                ((uint4 *)(bp + B2::oQ))[NPW + pc] = *(const uint4 *)(sQl + r * KS + cc);
            }
            for (int pc = tid; pc < 3 * 128; pc += kThreads) {
                const int tau = pc >> 7, s = (pc >> 6) & 1, ln = pc & 63;
                const int r = (tau ? 32 : 0) + (ln & 31), cc = (tau == 2 ? 32 : 0) + 16 * s + 8 * (ln >> 5);
                *(uint4 *)(sKl + r * kCS + cc) = ((const uint4 *)(bp + B2::oAb))[pc];
            }
            for (int i = tid; i < 128; i += kThreads)
                *(uint4 *)(sKl + (i >> 2) * kCS + 32 + 8 * (i & 3)) = make_uint4(0u, 0u, 0u, 0u);
            lds_barrier();
            //     M Ab_a, N Ab_a: wave w owns rows 16w..16w+15, four 16-column tiles
            f32x4 vm[4], vn[4];
            {
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const bf16x8 m0 = frag(sX, 16 * wave + l16, kCS, 8 * lg), m1 = frag(sX, 16 * wave + l16, kCS, 32 + 8 * lg);
                const bf16x8 n0 = frag(sAqk, 16 * wave + l16, kCS, 8 * lg), n1 = frag(sAqk, 16 * wave + l16, kCS, 32 + 8 * lg);
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) {
                    const bf16x8 a0 = frag_tr(sKl, 0, kCS, 16 * tn, lane), a1 = frag_tr(sKl, 32, kCS, 16 * tn, lane);
                    vm[tn] = mfma(a1, m1, mfma(a0, m0, zero));
                    vn[tn] = mfma(a1, n1, mfma(a0, n0, zero));
                }
            }
            lds_barrier();  // M, N are read
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) {
                const int o = (16 * wave + l16) * kCS + 16 * tn + 4 * lg;
                store4(sX + o, vm[tn][0], vm[tn][1], vm[tn][2], vm[tn][3]);
                store4(sAqk + o, vn[tn][0], vn[tn][1], vn[tn][2], vn[tn][3]);
            }
            lds_barrier();
            // (6) M Ab_a, N Ab_a -> tiles (2,0), (2,1), (3,0), (3,1) of Ab'', Ao'';
            //     K^_a Diag(gamma_b) -> steps 0-3 of the K^'' tiles
            for (int pc = tid; pc < 4 * 128; pc += kThreads) {
                const int tq = pc >> 7, s = (pc >> 6) & 1, ln = pc & 63;
                const int r = 32 * (tq >> 1) + (ln & 31), cc = 32 * (tq & 1) + 16 * s + 8 * (ln >> 5);
                const int dt = (tq >> 1) ? 6 + (tq & 1) : 3 + (tq & 1);
                ((uint4 *)(bp + B2::oAb))[dt * 128 + (pc & 127)] = *(const uint4 *)(sX + r * kCS + cc);
                ((uint4 *)(bp + B2::oAo))[dt * 128 + (pc & 127)] = *(const uint4 *)(sAqk + r * kCS + cc);
            }
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                const int cc = c0 + e;
                const int pc = (cc >> 5) * 8 * 64 + (rg >> 1) * 64 + (cc & 31) + 32 * (rg & 1);
                const float gb = gamb[e];
                uint4 w;
                w.x = pack_bf16x2(kha[e][0] * gb, kha[e][1] * gb);
                w.y = pack_bf16x2(kha[e][2] * gb, kha[e][3] * gb);
                w.z = pack_bf16x2(kha[e][4] * gb, kha[e][5] * gb);
                w.w = pack_bf16x2(kha[e][6] * gb, kha[e][7] * gb);
                ((uint4 *)(bp + B2::oK))[pc] = w;
            }
        }
        lds_barrier();  // every LDS array is free for the next job
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------------
// State kernel
// ---------------------------------------------------------------------------------
template <int DK>
struct StateSmem {
    static constexpr int KS = DK + 8;
    static constexpr int oS = 0;                   // S bf16 [32 dv][KS]
    static constexpr int oV = oS + kDVT * KS * 2;  // V bf16 [64][kVS]
    static constexpr int oVn = oV + kC * kVS * 2;  // V_new^T bf16 [32 dv][kCS]
    static constexpr int oO = oVn + kDVT * kCS * 2;  // output staging, 2 x bf16 [32][kVS]
    static constexpr int oG = oO + 2 * 32 * kVS * 2;  // gamma_C, 2 x fp32 [DK] (chunk parity)
    static constexpr int bytes = oG + 2 * DK * 4;
    // The reverse pass reads the forward blocks and transposes their operands here: K^ as
    // K^T row-major [DK][kCS]; W' and Q~ row-major [64 tokens][KS], two of each (chunk
    // parity: they are read after the step's second barrier).
    static constexpr int oRt = bytes;
    static constexpr int oRw = oRt + DK * kCS * 2;
    static constexpr int oRq = oRw + 2 * kC * KS * 2;
    static constexpr int bytes_rev = oRq + 2 * kC * KS * 2;
};

// Operands of one chunk for one wave, loaded one or two chunks ahead (DEPTH).
template <int DK>
struct Pre {
    uint4 P[DK / 16];  // W' (waves 0, 1) or Q~ (waves 2, 3): this wave's 32 rows
    uint4 A[4];        // Ab or Ao tiles of those rows (2 steps for rows 0-31, 4 for 32-63)
    uint4 K[4];        // K^ (DPLR: A^) tile of dk rows 32w.. (waves w < DK/32)
    uint4 Kb[4];       // DPLR only: Diag(beta) K^ tile of the same rows
    uint4 V;           // one 16-byte piece of the value tile
    float4 G;          // wave 0, lanes 0..DK/4-1: gamma_C[4 lane..+3]
};
// Fewest loads any wave issues per chunk (rows 0-31 take two A steps; waves past
// DK/32 take no K^ tile); waiting until at most this many are in flight therefore
// completes every load of the chunk before, whatever the wave.
template <int DK, bool DP>
constexpr int kMinLoadsPerChunk = DK / 16 + 2 + (DK / 32 >= 4 ? (DP ? 8 : 4) : 0) + 1;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

// vmcnt(N) alone (expcnt and lgkmcnt left at their maxima), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// Chunks whose operands are in flight ahead of the one being computed: two, in three
// rotating register sets (one workgroup per CU); or one, in two sets, which fits 256
// registers so that two workgroups share a CU and one's first loads and last stores
// overlap the other's steps (for passes with more workgroups than CUs).
constexpr int kDepth = 2;

// Modes of the state kernel.  Forward: the forward pass.  SaveStates: the forward
// recurrence without the output, writing the state that enters each chunk (bf16)
// to p.states.  Reverse (DP set): the chunks in reverse order on the forward blocks
// (byte stride p.fblk), no output and no Ab V term, writing the state entering each
// step to p.states: with K^ (DPLR: A^) in place of W', W'^T in place of the K^ tile
// and Q~^T in place of K^b, all three transposed in LDS, and dO as the value tile,
// this is the backward state pass dS <- dS Diag(gamma_C) + (K^ dS^T)^T W' + dO^T Q~.
// kForwardSave: the forward pass that also stores the states (both of the first two)
constexpr int kForward = 0, kSaveStates = 1, kReverse = 2, kForwardSave = 3;

template <int DK, bool DP, int MODE = kForward, int DEPTH = kDepth>
__global__ __launch_bounds__(kThreads, DEPTH == 1 ? 2 : 1) void kda_state_kernel(SplitParams p) {
    using L = StateSmem<DK>;
    using Bk = Blk<DK, DP>;
    constexpr int KS = L::KS;
    constexpr int NSW = DK / 32;  // waves owning a 32x32 S^T tile
    constexpr bool kOut = MODE == kForward || MODE == kForwardSave;  // writes O
    // The reverse pass runs on the forward blocks: it loads what the forward loads (no
    // K^b) and takes the transposes it needs from LDS.
    constexpr bool kRev = MODE == kReverse;
    constexpr bool kLoadKb = DP && !kRev;

    __shared__ __attribute__((aligned(16))) char smem[kRev ? L::bytes_rev : L::bytes];
    uint16_t *sS = (uint16_t *)(smem + L::oS);
    uint16_t *sV = (uint16_t *)(smem + L::oV);
    uint16_t *sVn = (uint16_t *)(smem + L::oVn);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, lh = lane >> 5;
    const int H = p.H, DV = p.dv;
    // Workgroups go to the 8 XCDs round-robin by block index.  A group is the workgroups
    // that read the same chunk operands (the n_tiles dv tiles of a (sequence, head)
    // chain, or of one run of it), so they are kept on one XCD (one L2); groups, longest
    // sequence first, are dealt to the XCDs in turn so that every XCD gets an equal share
    // of the long ones.  The grid is padded to a multiple of 8 groups; the padding exits
    // at once.
    const int runs = p.seg_n > 1 ? p.seg_n - 1 : 1;  // groups per chain
    const int tpg = p.seg_phase == 1 ? p.n_tiles + NSW : p.n_tiles;  // workgroups per group
    const int pos = blockIdx.x >> 3;
    const int grp = (pos / tpg) * 8 + (blockIdx.x & 7);
    if (grp >= p.n_seq * H * runs) return;
    const int tile = pos % tpg;
    const int chain = grp / runs;
    const int h = chain % H;
    const int rank = chain / H;
    const int n = p.order ? p.order[rank] : rank;
    long t0, t1;
    seq_bounds(p.cu, n, p.T, p.total, t0, t1, nullptr);
    int nck = (int)((t1 - t0 + kC - 1) / kC);
    long cbase;
    if (p.coff) {
        cbase = p.coff[n];
        const long room = p.max_chunks - cbase;  // only short of nck for malformed offsets
        nck = (int)(room < 0 ? 0 : (room < nck ? room : nck));
    } else {
        cbase = (long)n * p.nc;
    }

    // What this workgroup computes: its rows j0.. of a state-like matrix, where it starts
    // (s_in rows, the identity, or zero), where its end state goes, and whether the values
    // are read and the output and per-step states are written.
    int j0 = tile * kDVT;
    const float *s_in = p.S0 ? p.S0 + ((size_t)n * H + h) * DV * DK : nullptr;
    float *s_out = p.Sf ? p.Sf + ((size_t)n * H + h) * DV * DK : nullptr;
    bool ident = false, vzero = false, emit = true;
    if (p.seg_n > 1) {
        const int G = p.seg_n;
        const int g = grp % runs + (p.seg_phase == 1 ? 0 : 1);  // run of this group
        const size_t mat = (size_t)DV * DK;
        float *ws = p.seg_ws + ((size_t)n * H + h) * ((size_t)(2 * G - 3) * mat + (size_t)(G - 2) * DK * DK);
        float *start = ws;                          // start state of run g at start + (g-1) mat
        float *R = ws + (size_t)(G - 1) * mat;      // R of run g at R + (g-1) mat
        float *P = ws + (size_t)(2 * G - 3) * mat;  // P of run g at P + (g-1) DK DK
        if (p.seg_phase == 1) {
            if (g == 0) {
                if (tile >= p.n_tiles) return;
                s_out = start;  // run 0 as usual; its end is the start of run 1
            } else if (tile < p.n_tiles) {
                s_in = nullptr;  // R: from zero
                s_out = R + (size_t)(g - 1) * mat;
                emit = false;
            } else {
                j0 = (tile - p.n_tiles) * kDVT;  // P: rows of the dk x dk map, from I
                s_in = nullptr;
                s_out = P + (size_t)(g - 1) * DK * DK;
                ident = vzero = true;
                emit = false;
            }
        } else {
            s_in = start + (size_t)(g - 1) * mat;
            if (g < G - 1) s_out = nullptr;
        }
        // chunks of run g (counted from the end in reverse mode)
        const int len = (nck + G - 1) / G;
        const int a0 = g * len < nck ? g * len : nck, a1 = (g + 1) * len < nck ? (g + 1) * len : nck;
        const int lo = MODE == kReverse ? nck - a1 : a0;
        cbase += lo;
        t0 += (long)lo * kC;
        nck = a1 - a0;
    }
    const int jv = vzero ? 0 : j0;  // dv column of the value loads (any, when unused)

    const int rt = wave & 1;      // 32-row tile of the chunk
    const bool vw = wave < 2;     // V_new waves (W', Ab); waves 2, 3: output (Q~, Ao)
    // chunk of the sequence that step c works on
    auto cid = [&](int c) { return MODE == kReverse ? nck - 1 - c : c; };
    uint16_t *sO = (uint16_t *)(smem + L::oO) + (wave & 1) * 32 * kVS;

    // state: wave w < NSW holds S^T[dk 32w..+31][dv 0..31]; register 4q+e is
    // S[dv l32][dk 32w + 8q + 4lh + e]
    f32x16 ST = {};
    if (wave < NSW) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int dk = 32 * wave + 8 * q + 4 * lh;
            float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
            if (s_in) s4 = *(const float4 *)(s_in + (size_t)(j0 + l32) * DK + dk);
            if (ident) {
                const int r = j0 + l32;
                s4 = make_float4(r == dk ? 1.f : 0.f, r == dk + 1 ? 1.f : 0.f, r == dk + 2 ? 1.f : 0.f,
                                 r == dk + 3 ? 1.f : 0.f);
            }
            ST[4 * q + 0] = s4.x; ST[4 * q + 1] = s4.y; ST[4 * q + 2] = s4.z; ST[4 * q + 3] = s4.w;
            store4(sS + l32 * KS + dk, s4.x, s4.y, s4.z, s4.w);
        }
    }

    const int vr = tid >> 2, vc = 8 * (tid & 3);
    // Loads of one chunk in two batches: the W'/Q~ tile first, the rest later in the
    // step, so that the memory pipeline is fed while the wave computes.
    const size_t bstride = kRev ? (size_t)p.fblk : (size_t)Bk::bytes;
    auto load_p = [&](Pre<DK> &x, int c) {
        const char *bp = p.blk + ((size_t)(cbase + cid(c)) * H + h) * bstride;
        const uint4 *pw = (const uint4 *)(bp + (vw ? Bk::oW : Bk::oQ)) + rt * (DK / 16) * 64 + lane;
#pragma unroll
        for (int s = 0; s < DK / 16; ++s) x.P[s] = pw[s * 64];
    };
    auto load_rest = [&](Pre<DK> &x, int c) {
        const char *bp = p.blk + ((size_t)(cbase + cid(c)) * H + h) * bstride;
        const uint4 *pa = (const uint4 *)(bp + (vw ? Bk::oAb : Bk::oAo)) + rt * 128 + lane;
        x.A[0] = pa[0];
        x.A[1] = pa[64];
        if (rt) {
            x.A[2] = pa[128];
            x.A[3] = pa[192];
        }
        if (wave < NSW) {
            const uint4 *pk = (const uint4 *)(bp + Bk::oK) + wave * 256 + lane;
#pragma unroll
            for (int s = 0; s < 4; ++s) x.K[s] = pk[s * 64];
            if constexpr (kLoadKb) {
                const uint4 *pkb = (const uint4 *)(bp + Bk::oKb) + wave * 256 + lane;
#pragma unroll
                for (int s = 0; s < 4; ++s) x.Kb[s] = pkb[s * 64];
            }
        }
        const long tok = t0 + (long)cid(c) * kC + vr;
        x.V = *(const uint4 *)(p.v + ((size_t)(tok < t1 ? tok : t1 - 1) * H + h) * DV + jv + vc);
        if (wave == 0 && lane < DK / 4) x.G = ((const float4 *)(bp + Bk::oG))[lane];
    };

    // Output rows of the previous chunk, staged in LDS by this wave: 16 rows x 64 bytes
    // per store instruction.
    auto store_out = [&](int c) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 16 * i + (lane >> 2), q4 = lane & 3;
            const long tok = t0 + (long)c * kC + 32 * rt + r;
            const uint4 o = *(const uint4 *)(sO + r * kVS + 8 * q4);
            if (tok < t1 && emit) *(uint4 *)(p.O + ((size_t)tok * H + h) * DV + j0 + 8 * q4) = o;
        }
    };

    auto step = [&](int c, Pre<DK> &x, Pre<DK> &nx) {
        wait_vmcnt<(DEPTH - 1) * kMinLoadsPerChunk<DK, kLoadKb>>();  // operands of chunk c have arrived
        float *sG = (float *)(smem + L::oG) + (c & 1) * DK;
        if (wave == 0 && lane < DK / 4) ((float4 *)sG)[lane] = x.G;
        {
            // rows past the end of the sequence are zero (branch-free: a lane mask)
            const uint32_t keep = 0u - (uint32_t)(t0 + (long)cid(c) * kC + vr < t1 && !vzero);
            *(uint4 *)(sV + vr * kVS + vc) = make_uint4(x.V.x & keep, x.V.y & keep, x.V.z & keep, x.V.w & keep);
        }
        if (kOut && !vw && c > 0) store_out(c - 1);
        const int cn = c + DEPTH < nck ? c + DEPTH : nck - 1;
        load_p(nx, cn);
        // reverse pass: this chunk's K^ tiles (as K^T) and W', Q~ rows, row-major in LDS
        uint16_t *sRt = kRev ? (uint16_t *)(smem + L::oRt) : nullptr;
        const uint16_t *sRw = kRev ? (const uint16_t *)(smem + L::oRw) + (c & 1) * kC * KS : nullptr;
        const uint16_t *sRq = kRev ? (const uint16_t *)(smem + L::oRq) + (c & 1) * kC * KS : nullptr;
        if constexpr (kRev) {
            // (through registers: as a plain copy the compiler would keep the operand sets
            // in scratch memory)
            auto put = [](uint16_t *d, uint4 u) {
                asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
                *(uint4 *)d = u;
            };
            if (wave < NSW) {
#pragma unroll
                for (int s = 0; s < 4; ++s) put(sRt + (32 * wave + l32) * kCS + 16 * s + 8 * lh, x.K[s]);
            }
            uint16_t *sR = (uint16_t *)(vw ? sRw : sRq);
#pragma unroll
            for (int s = 0; s < DK / 16; ++s) put(sR + (32 * rt + l32) * KS + 16 * s + 8 * lh, x.P[s]);
        }
        lds_barrier();  // value tile, gamma_C and S of chunk c visible (reverse: and its operands)
        if (MODE != kForward && emit) {  // kSaveStates, kReverse, kForwardSave
            // the state entering this step, bf16, 16 bytes per thread and pass
            uint16_t *dst = p.states + (((size_t)(cbase + cid(c)) * H + h) * DV + j0) * DK;
#pragma unroll
            for (int i = 0; i < kDVT * DK / 8 / kThreads; ++i) {
                const int idx = tid + kThreads * i, r = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
                *(uint4 *)(dst + (size_t)r * DK + c8) = *(const uint4 *)(sS + r * KS + c8);
            }
        }

        // LDS operands are all read before the products so that their latency overlaps.
        bf16x8 fv[4], fs[DK / 16];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i < 2 || rt || DP) fv[i] = frag_tr32(sV, 16 * i, kVS, 0, lane);
#pragma unroll
        for (int s = 0; s < DK / 16; ++s) fs[s] = frag(sS, l32, KS, 16 * s + 8 * lh);
        // reverse: the row tile of K^ (natural layout) in place of W'
        bf16x8 fp[DK / 16];
#pragma unroll
        for (int s = 0; s < DK / 16; ++s)
            fp[s] = kRev ? frag_tr32(sRt, 16 * s, kCS, 32 * rt, lane) : as_bf16x8(x.P[s]);
        f32x16 acc = {};
        if (vw) {
            // V_new = Ab V + W' S^T; register 4q+e is V_new[row 32rt + 8q + 4lh + e][dv l32]
            if constexpr (MODE != kReverse) {
                acc = mfma32x32(as_bf16x8(x.A[0]), fv[0], acc);
                acc = mfma32x32(as_bf16x8(x.A[1]), fv[1], acc);
                if (rt) {
                    acc = mfma32x32(as_bf16x8(x.A[2]), fv[2], acc);
                    acc = mfma32x32(as_bf16x8(x.A[3]), fv[3], acc);
                }
            }
#pragma unroll
            for (int s = 0; s < DK / 16; ++s) acc = mfma32x32(fp[s], fs[s], acc);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                store4(sVn + l32 * kCS + 32 * rt + 8 * q + 4 * lh, acc[4 * q + 0], acc[4 * q + 1],
                       acc[4 * q + 2], acc[4 * q + 3]);
        } else if constexpr (kOut) {
            // O^T = V^T Ao^T + S Q~^T (operands swapped); register 4q+e is
            // O[row 32rt + l32][dv 8q + 4lh + e]
            acc = mfma32x32(fv[0], as_bf16x8(x.A[0]), acc);
            acc = mfma32x32(fv[1], as_bf16x8(x.A[1]), acc);
            if (rt) {
                acc = mfma32x32(fv[2], as_bf16x8(x.A[2]), acc);
                acc = mfma32x32(fv[3], as_bf16x8(x.A[3]), acc);
            }
#pragma unroll
            for (int s = 0; s < DK / 16; ++s) acc = mfma32x32(fs[s], as_bf16x8(x.P[s]), acc);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                store4(sO + l32 * kVS + 8 * q + 4 * lh, acc[4 * q + 0], acc[4 * q + 1],
                       acc[4 * q + 2], acc[4 * q + 3]);
        }
        load_rest(nx, cn);
        lds_barrier();  // V_new^T visible

        // S <- S Diag(gamma_C) + V_new^T K^ (transposed: S^T tile = K^T-tile V_new)
        // (DP: + N^T A^ + V^T Diag(beta) K^)
        if (wave < NSW) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 g = *(const float4 *)(sG + 32 * wave + 8 * q + 4 * lh);
                ST[4 * q + 0] *= g.x; ST[4 * q + 1] *= g.y;
                ST[4 * q + 2] *= g.z; ST[4 * q + 3] *= g.w;
            }
            // reverse: W'^T and Q~^T tiles of dk rows 32w.. in place of the K^ and K^b tiles
            bf16x8 fk[4], fb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                fk[s] = kRev ? frag_tr32(sRw, 16 * s, KS, 32 * wave, lane) : as_bf16x8(x.K[s]);
                if constexpr (DP) fb[s] = kRev ? frag_tr32(sRq, 16 * s, KS, 32 * wave, lane) : as_bf16x8(x.Kb[s]);
            }
            bf16x8 fn[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) fn[s] = frag(sVn, l32, kCS, 16 * s + 8 * lh);
#pragma unroll
            for (int s = 0; s < 4; ++s) ST = mfma32x32(fk[s], fn[s], ST);
            if constexpr (DP) {  // + V^T Diag(beta) K^
#pragma unroll
                for (int s = 0; s < 4; ++s) ST = mfma32x32(fb[s], fv[s], ST);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                store4(sS + l32 * KS + 32 * wave + 8 * q + 4 * lh, ST[4 * q + 0], ST[4 * q + 1],
                       ST[4 * q + 2], ST[4 * q + 3]);
        }
    };

    if (nck > 0) {
        Pre<DK> buf[DEPTH + 1];
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            load_p(buf[u], u < nck ? u : nck - 1);
            load_rest(buf[u], u < nck ? u : nck - 1);
            asm volatile("" ::: "memory");  // keep the chunks' loads in chunk order
        }
        // Whole rounds of steps (one per operand set), then the tail: every path through
        // this code runs the steps in order with nothing skipped, so the compiler's count
        // of memory operations in flight stays exact and the waits above are the only ones.
        int c = 0;
        if constexpr (DEPTH == 2) {
            for (; c + 3 <= nck; c += 3) {
                step(c, buf[0], buf[2]);
                step(c + 1, buf[1], buf[0]);
                step(c + 2, buf[2], buf[1]);
            }
            if (c < nck) {
                step(c, buf[0], buf[2]);
                if (c + 1 < nck) step(c + 1, buf[1], buf[0]);
            }
        } else {
            static_assert(DEPTH == 1, "one or two chunks ahead");
            for (; c + 2 <= nck; c += 2) {
                step(c, buf[0], buf[1]);
                step(c + 1, buf[1], buf[0]);
            }
            if (c < nck) step(c, buf[0], buf[1]);
        }
        if (kOut && !vw) store_out(nck - 1);
    }

    if (s_out && wave < NSW) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int dk = 32 * wave + 8 * q + 4 * lh;
            *(float4 *)(s_out + (size_t)(j0 + l32) * DK + dk) =
                make_float4(ST[4 * q + 0], ST[4 * q + 1], ST[4 * q + 2], ST[4 * q + 3]);
        }
    }
}

// ---------------------------------------------------------------------------------
// State kernel for chunks of 128 tokens (KDA form, dk = 128, forward pass): one
// workgroup of 8 waves per (sequence, head, 32-wide dv tile), serial over the chunks.
//   waves 0-3 (w)      V_new rows 32w..+31 = Ab'' V + W'' S^T, then the S^T rows 32w..+31
//                      of dk: S <- S Diag(gamma) + V_new^T K^''
//   waves 4-7 (w - 4)  O rows 32(w-4)..+31 = Ao'' V + Q~'' S^T
// A chunk's rows, row tiles, value tile and gamma are loaded one chunk ahead (a step is
// twice as long as at C = 64); the K^'' tile, read only after the V_new products, is
// loaded at the start of its own step.
// ---------------------------------------------------------------------------------
constexpr int kThreads2 = 512;          // 8 waves
constexpr int kC2S = kC2 + 8;           // bf16 row stride of [*][128] arrays
struct State128Smem {
    static constexpr int KS = 128 + 8;
    static constexpr int oS = 0;                       // S bf16 [32 dv][KS]
    static constexpr int oV = oS + kDVT * KS * 2;      // V bf16 [128][kVS]
    static constexpr int oVn = oV + kC2 * kVS * 2;     // V_new^T bf16 [32 dv][kC2S]
    static constexpr int oO = oVn + kDVT * kC2S * 2;   // output staging, 4 x bf16 [32][kVS]
    static constexpr int oG = oO + 4 * 32 * kVS * 2;   // gamma, 2 x fp32 [128] (chunk parity)
    static constexpr int bytes = oG + 2 * 128 * 4;
};

struct Pre128 {
    uint4 P[8];  // W'' (waves 0-3) or Q~'' (waves 4-7): this wave's 32 rows, K = 128
    uint4 A[8];  // Ab'' or Ao'' tiles (r, 0..r) of row tile r: 2 (r + 1) steps
    uint4 V;     // one 16-byte piece of the value tile
    float4 G;    // wave 0, lanes 0..31: gamma[4 lane..+3]
};

// vmcnt(N) with N chosen at run time among the counts a row tile can leave in flight.
__device__ __forceinline__ void wait_vmcnt_rows(int rt) {
    switch (rt) {  // wave-uniform
        case 0: wait_vmcnt<8 + 2 + 1>(); break;
        case 1: wait_vmcnt<8 + 4 + 1>(); break;
        case 2: wait_vmcnt<8 + 6 + 1>(); break;
        default: wait_vmcnt<8 + 8 + 1>(); break;
    }
}

__global__ __launch_bounds__(kThreads2) void kda_state128_kernel(SplitParams p) {
    constexpr int DK = 128;
    using L = State128Smem;
    using Bk = Blk128<DK>;
    constexpr int KS = L::KS;

    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    uint16_t *sS = (uint16_t *)(smem + L::oS);
    uint16_t *sV = (uint16_t *)(smem + L::oV);
    uint16_t *sVn = (uint16_t *)(smem + L::oVn);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, lh = lane >> 5;
    const int H = p.H, DV = p.dv;
    // XCD-aware placement as in kda_state_kernel: the dv tiles of a chain on one XCD,
    // chains (longest packed sequence first) dealt to the XCDs in turn.
    const int tpg = p.n_tiles;
    const int pos = blockIdx.x >> 3;
    const int chain = (pos / tpg) * 8 + (blockIdx.x & 7);
    if (chain >= p.n_seq * H) return;
    const int j0 = (pos % tpg) * kDVT;
    const int h = chain % H;
    const int rank = chain / H;
    const int n = p.order ? p.order[rank] : rank;
    long t0, t1;
    seq_bounds(p.cu, n, p.T, p.total, t0, t1, nullptr);
    int nck = (int)((t1 - t0 + kC2 - 1) / kC2);
    long cbase;
    if (p.coff) {
        cbase = p.coff[n];
        const long room = p.max_chunks - cbase;  // only short of nck for malformed offsets
        nck = (int)(room < 0 ? 0 : (room < nck ? room : nck));
    } else {
        cbase = (long)n * p.nc;
    }
    const float *s_in = p.S0 ? p.S0 + ((size_t)n * H + h) * DV * DK : nullptr;
    float *s_out = p.Sf ? p.Sf + ((size_t)n * H + h) * DV * DK : nullptr;

    const bool vw = wave < 4;  // V_new and state waves; waves 4-7: output
    const int rt = wave & 3;   // 32-row tile of the chunk
    uint16_t *sO = (uint16_t *)(smem + L::oO) + rt * 32 * kVS;

    // state (waves 0-3): wave w holds S^T[dk 32w..+31][dv 0..31]; register 4q+e is
    // S[dv l32][dk 32w + 8q + 4lh + e]
    f32x16 ST = {};
    if (vw) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int dk = 32 * rt + 8 * q + 4 * lh;
            float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
            if (s_in) s4 = *(const float4 *)(s_in + (size_t)(j0 + l32) * DK + dk);
            ST[4 * q + 0] = s4.x; ST[4 * q + 1] = s4.y; ST[4 * q + 2] = s4.z; ST[4 * q + 3] = s4.w;
            store4(sS + l32 * KS + dk, s4.x, s4.y, s4.z, s4.w);
        }
    }

    const int vr = tid >> 2, vc = 8 * (tid & 3);  // value tile: token vr, columns vc..vc+7
    const int na = 2 * (rt + 1);                  // A steps of this row tile
    auto load = [&](Pre128 &x, int c) {
        const char *bp = p.blk + ((size_t)(cbase + c) * H + h) * Bk::bytes;
        const uint4 *pw = (const uint4 *)(bp + (vw ? Bk::oW : Bk::oQ)) + rt * (DK / 16) * 64 + lane;
#pragma unroll
        for (int s = 0; s < DK / 16; ++s) x.P[s] = pw[s * 64];
        // tiles (rt, 0..rt) are consecutive: index rt (rt + 1) / 2 + ct, two steps each
        const uint4 *pa = (const uint4 *)(bp + (vw ? Bk::oAb : Bk::oAo)) + (rt * (rt + 1) / 2) * 128 + lane;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < na) x.A[i] = pa[i * 64];
        const long tok = t0 + (long)c * kC2 + vr;
        x.V = *(const uint4 *)(p.v + ((size_t)(tok < t1 ? tok : t1 - 1) * H + h) * DV + j0 + vc);
        if (wave == 0 && lane < DK / 4) x.G = ((const float4 *)(bp + Bk::oG))[lane];
    };
    uint4 K[8];  // K^'' tile of dk rows 32w.. (waves 0-3), chunk of the current step
    auto load_k = [&](int c) {
        const char *bp = p.blk + ((size_t)(cbase + c) * H + h) * Bk::bytes;
        const uint4 *pk = (const uint4 *)(bp + Bk::oK) + rt * 512 + lane;
#pragma unroll
        for (int s = 0; s < 8; ++s) K[s] = pk[s * 64];
    };

    auto store_out = [&](int c) {  // output rows of chunk c, staged by this O wave
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 16 * i + (lane >> 2), q4 = lane & 3;
            const long tok = t0 + (long)c * kC2 + 32 * rt + r;
            const uint4 o = *(const uint4 *)(sO + r * kVS + 8 * q4);
            if (tok < t1) *(uint4 *)(p.O + ((size_t)tok * H + h) * DV + j0 + 8 * q4) = o;
        }
    };

    auto step = [&](int c, Pre128 &x, Pre128 &nx) {
        wait_vmcnt<0>();  // chunk c's operands have arrived (issued one step ago)
        if (vw) load_k(c);
        float *sG = (float *)(smem + L::oG) + (c & 1) * 128;
        if (wave == 0 && lane < DK / 4) ((float4 *)sG)[lane] = x.G;
        {
            const uint32_t keep = 0u - (uint32_t)(t0 + (long)c * kC2 + vr < t1);
            *(uint4 *)(sV + vr * kVS + vc) = make_uint4(x.V.x & keep, x.V.y & keep, x.V.z & keep, x.V.w & keep);
        }
        if (!vw && c > 0) store_out(c - 1);
        load(nx, c + 1 < nck ? c + 1 : nck - 1);
        lds_barrier();  // value tile, gamma and S of chunk c visible

        f32x16 acc = {};
        if (vw) {
            // V_new rows 32rt.. = Ab'' V + W'' S^T; register 4q+e is V_new[32rt + 8q + 4lh + e][dv l32]
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (i < na) acc = mfma32x32(as_bf16x8(x.A[i]), frag_tr32(sV, 16 * i, kVS, 0, lane), acc);
#pragma unroll
            for (int s = 0; s < DK / 16; ++s)
                acc = mfma32x32(as_bf16x8(x.P[s]), frag(sS, l32, KS, 16 * s + 8 * lh), acc);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                store4(sVn + l32 * kC2S + 32 * rt + 8 * q + 4 * lh, acc[4 * q + 0], acc[4 * q + 1],
                       acc[4 * q + 2], acc[4 * q + 3]);
        } else {
            // O^T = V^T Ao''^T + S Q~''^T; register 4q+e is O[row 32rt + l32][dv 8q + 4lh + e]
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (i < na) acc = mfma32x32(frag_tr32(sV, 16 * i, kVS, 0, lane), as_bf16x8(x.A[i]), acc);
#pragma unroll
            for (int s = 0; s < DK / 16; ++s)
                acc = mfma32x32(frag(sS, l32, KS, 16 * s + 8 * lh), as_bf16x8(x.P[s]), acc);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                store4(sO + l32 * kVS + 8 * q + 4 * lh, acc[4 * q + 0], acc[4 * q + 1], acc[4 * q + 2],
                       acc[4 * q + 3]);
        }
        lds_barrier();  // V_new^T visible; every read of S is done

        if (vw) {
            // S <- S Diag(gamma) + V_new^T K^'' (transposed: S^T tile = K^''^T-tile V_new)
            wait_vmcnt_rows(rt);  // this step's K^'' tile has arrived (the next chunk's loads may not)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 g = *(const float4 *)(sG + 32 * rt + 8 * q + 4 * lh);
                ST[4 * q + 0] *= g.x; ST[4 * q + 1] *= g.y;
                ST[4 * q + 2] *= g.z; ST[4 * q + 3] *= g.w;
            }
#pragma unroll
            for (int s = 0; s < 8; ++s)
                ST = mfma32x32(as_bf16x8(K[s]), frag(sVn, l32, kC2S, 16 * s + 8 * lh), ST);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                store4(sS + l32 * KS + 32 * rt + 8 * q + 4 * lh, ST[4 * q + 0], ST[4 * q + 1],
                       ST[4 * q + 2], ST[4 * q + 3]);
        }
    };

    if (nck > 0) {
        Pre128 buf[2];
        load(buf[0], 0);
        int c = 0;
        for (; c + 2 <= nck; c += 2) {
            step(c, buf[0], buf[1]);
            step(c + 1, buf[1], buf[0]);
        }
        if (c < nck) step(c, buf[0], buf[1]);
        if (!vw) store_out(nck - 1);
    }

    if (s_out && vw) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int dk = 32 * rt + 8 * q + 4 * lh;
            *(float4 *)(s_out + (size_t)(j0 + l32) * DK + dk) =
                make_float4(ST[4 * q + 0], ST[4 * q + 1], ST[4 * q + 2], ST[4 * q + 3]);
        }
    }
}

// Start state of run g + 1 of a segmented state pass: S_start(g+1) = S_start(g) P_g + R_g
// (fp32), one workgroup per (chain, 32 rows of dv, 32 columns of dk); launched for
// g = 1 .. seg_n-2 in turn.
template <int DK>
__global__ __launch_bounds__(kThreads) void seg_combine_kernel(SplitParams p, int g) {
    constexpr int XS = DK + 4, PS = 32 + 4;  // padded LDS rows
    __shared__ __attribute__((aligned(16))) float sX[kDVT * XS];
    __shared__ __attribute__((aligned(16))) float sP[DK * PS];
    const int tid = threadIdx.x;
    const int G = p.seg_n, DV = p.dv;
    const int per_chain = p.n_tiles * (DK / 32);
    const int chain = blockIdx.x / per_chain, rem = blockIdx.x % per_chain;
    const int j0 = (rem / (DK / 32)) * kDVT, k0 = (rem % (DK / 32)) * 32;
    if (chain >= p.n_seq * p.H) return;
    const size_t mat = (size_t)DV * DK;
    float *start = p.seg_ws + (size_t)chain * ((size_t)(2 * G - 3) * mat + (size_t)(G - 2) * DK * DK);
    const float *Xg = start + (size_t)(g - 1) * mat;
    const float *Rg = start + (size_t)(G - 1) * mat + (size_t)(g - 1) * mat;
    const float *Pg = start + (size_t)(2 * G - 3) * mat + (size_t)(g - 1) * DK * DK;
    for (int i = tid; i < kDVT * DK / 4; i += kThreads) {
        const int row = i / (DK / 4), c4 = 4 * (i % (DK / 4));
        *(float4 *)(sX + row * XS + c4) = *(const float4 *)(Xg + (size_t)(j0 + row) * DK + c4);
    }
    for (int i = tid; i < DK * 8; i += kThreads) {
        const int row = i >> 3, c4 = 4 * (i & 7);
        *(float4 *)(sP + row * PS + c4) = *(const float4 *)(Pg + (size_t)row * DK + k0 + c4);
    }
    __syncthreads();
    const int r = tid >> 3, c = 4 * (tid & 7);
    float4 acc = *(const float4 *)(Rg + (size_t)(j0 + r) * DK + k0 + c);
    for (int k = 0; k < DK; ++k) {
        const float x = sX[r * XS + k];
        const float4 y = *(const float4 *)(sP + k * PS + c);
        acc.x += x * y.x; acc.y += x * y.y; acc.z += x * y.z; acc.w += x * y.w;
    }
    *(float4 *)(start + (size_t)g * mat + (size_t)(j0 + r) * DK + k0 + c) = acc;
}

// Compute units of the current device (cached per device).
int compute_units() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Runs per chain for a segmented state pass, or 0 for the plain pass.  A segmented pass
// takes about 2/G of the plain pass's serial steps; it is used when the plain pass
// leaves most CUs idle (its first phase, chains x (G-1) x (dv + dk) / 32 workgroups,
// must fit on the device at once) and the chains are long enough to amortise the two
// extra launches.  GDR_SEGMENTS=0 in the environment turns it off (the workspace is
// sized for it either way).
constexpr int kSegMinChunks = 8, kSegMaxRuns = 8;
int seg_runs(int chains, int dk, int dv, long chunks_per_chain, bool honour_env) {
    if (honour_env) {
        const char *e = std::getenv("GDR_SEGMENTS");
        if (e && e[0] == '0' && e[1] == 0) return 0;
    }
    const long per_group = dv / kDVT + dk / 32;
    long G = 1 + compute_units() / ((long)chains * per_group);
    if (chunks_per_chain / kSegMinChunks < G) G = chunks_per_chain / kSegMinChunks;
    if (G > kSegMaxRuns) G = kSegMaxRuns;
    return G >= 3 ? (int)G : 0;
}

// Longest chain in chunks (packed sequences: at most the whole token axis).
long chunks_per_chain(const FwdArgs &a) { return (a.T + kC - 1) / kC; }

// The segmented-pass area follows the other workspace contents (256-byte aligned).
size_t seg_offset(size_t total) { return (total + 255) / 256 * 256; }

size_t seg_bytes(int chains, int dk, int dv, int runs) {
    if (runs < 3) return 0;
    return (size_t)chains * ((size_t)(2 * runs - 3) * dv * dk + (size_t)(runs - 2) * dk * dk) * 4;
}

// One state pass: plain, or segmented (phase 1, the map combination, phase 2).
template <int DK, bool DP, int MODE>
void run_state(SplitParams sp, int runs, hipStream_t s) {
    const long chains = (long)sp.n_seq * sp.H;
    if (runs < 3) {
        sp.seg_n = sp.seg_phase = 0;
        const dim3 grid((unsigned)(((chains + 7) / 8) * 8 * sp.n_tiles));
        // (the state-keeping forward spills in the smaller register budget at dk = 128)
        if constexpr (!DP && (MODE == kForward || MODE == kSaveStates)) {
            if (chains * sp.n_tiles > compute_units()) {  // more than one round of workgroups
                hipLaunchKernelGGL((kda_state_kernel<DK, DP, MODE, 1>), grid, dim3(kThreads), 0, s, sp);
                return;
            }
        }
        hipLaunchKernelGGL((kda_state_kernel<DK, DP, MODE>), grid, dim3(kThreads), 0, s, sp);
        return;
    }
    const long groups = chains * (runs - 1);
    sp.seg_n = runs;
    sp.seg_phase = 1;
    hipLaunchKernelGGL((kda_state_kernel<DK, DP, MODE>), dim3((unsigned)(((groups + 7) / 8) * 8 * (sp.n_tiles + DK / 32))),
                       dim3(kThreads), 0, s, sp);
    for (int g = 1; g <= runs - 2; ++g)
        hipLaunchKernelGGL((seg_combine_kernel<DK>), dim3((unsigned)(chains * sp.n_tiles * (DK / 32))),
                           dim3(kThreads), 0, s, sp, g);
    sp.seg_phase = 2;
    hipLaunchKernelGGL((kda_state_kernel<DK, DP, MODE>), dim3((unsigned)(((groups + 7) / 8) * 8 * sp.n_tiles)),
                       dim3(kThreads), 0, s, sp);
}

int blk_bytes(int dk, bool dp) {
    if (dp) return dk == 128 ? Blk<128, true>::bytes : Blk<64, true>::bytes;
    return dk == 128 ? Blk<128>::bytes : Blk<64>::bytes;
}

}  // namespace
}  // namespace gdr

#include "gdr_kda_bwd.h"

namespace gdr {
namespace {

// Forward-pass view of the backward arguments (for the shared sizing and planning).
FwdArgs fwd_view(const BwdArgs &b) {
    FwdArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = b.q; a.k = b.k; a.v = b.v; a.a = b.a; a.b = b.b;
    a.log_alpha = b.log_alpha; a.beta = b.beta; a.S0 = b.S0;
    a.cu_seqlens = b.cu_seqlens;
    a.n_seq = b.n_seq; a.B = b.B; a.H = b.H; a.T = b.T; a.dk = b.dk; a.dv = b.dv; a.C = b.C;
    a.dtype = b.dtype; a.gate = b.gate;
    return a;
}

// Backward workspace: [header][packed-sequence plan][forward blocks][log-domain job
// flags (gated forms)][S_p states][dS_n states][segmented-pass area], the states bf16
// [chunk][head][dv][dk].  Everything up to the flags sits where the forward workspace
// has it, so that a forward call's workspace can stand in for the first kernel; the
// reverse pass reads the forward blocks too.
struct BwdLayout {
    SplitLayout fw;
    size_t sub_off, s_off, ds_off, seg_off, total;
    bool sub;
    int runs;  // of the segmented state passes (0: plain)
};

BwdLayout bwd_layout(const BwdArgs &b, int N) {
    BwdLayout L;
    const FwdArgs a = fwd_view(b);
    L.fw = split_layout(a, N, blk_bytes(b.dk, b.a != nullptr));
    const size_t nblk = (size_t)b.H * L.fw.max_chunks;
    L.sub = b.gate != kGateNone;
    L.sub_off = seg_offset(L.fw.total);
    L.s_off = seg_offset(L.sub_off + (L.sub ? nblk * 4 : 0));
    L.ds_off = L.s_off + nblk * b.dv * b.dk * 2;
    L.seg_off = seg_offset(L.ds_off + nblk * b.dv * b.dk * 2);
    L.runs = seg_runs(N * b.H, b.dk, b.dv, chunks_per_chain(a), false);
    L.total = L.seg_off + seg_bytes(N * b.H, b.dk, b.dv, L.runs);  // shared by both passes
    return L;
}

}  // namespace

bool kda_split_supported(const FwdArgs &a) {
    if (a.dtype != 1 || (a.a == nullptr) != (a.b == nullptr) || a.dv % kDVT != 0) return false;
    if (a.C == kC2)  // 128-token chunks: the KDA form at dk = 128, forward only
        return a.a == nullptr && a.dk == 128 && !a.keep_states;
    return a.C == kC && (a.dk == 64 || a.dk == 128);
}

// Forward workspace: the split layout, then the per-job flags of the log-domain prep
// (gated forms only), then the segmented-pass area.
struct KdaWs {
    SplitLayout lay;
    size_t sub_off, seg_off, total;
    bool sub;
    int runs;
};
KdaWs kda_ws(const FwdArgs &a, int n_seq_eff) {
    KdaWs w;
    if (a.C == kC2) {  // blocks of 128-token chunks; no log-domain flags, plain state pass
        w.lay = split_layout(a, n_seq_eff, Blk128<128>::bytes);
        w.sub = false;
        w.sub_off = w.seg_off = w.total = seg_offset(w.lay.total);
        w.runs = 0;
        return w;
    }
    w.lay = split_layout(a, n_seq_eff, blk_bytes(a.dk, a.a != nullptr));
    w.sub = a.gate != kGateNone || a.clip;
    w.sub_off = seg_offset(w.lay.total);
    w.seg_off = seg_offset(w.sub_off + (w.sub ? (size_t)a.H * w.lay.max_chunks * 4 : 0));
    const int chains = n_seq_eff * a.H;
    w.runs = seg_runs(chains, a.dk, a.dv, chunks_per_chain(a), false);
    w.total = w.seg_off + seg_bytes(chains, a.dk, a.dv, w.runs);
    return w;
}

size_t kda_split_workspace_bytes(const FwdArgs &a, int n_seq_eff) { return kda_ws(a, n_seq_eff).total; }

BwdArgs bwd_view(const FwdArgs &a) {
    BwdArgs b;
    std::memset(&b, 0, sizeof(b));
    b.q = a.q; b.k = a.k; b.v = a.v; b.a = a.a; b.b = a.b;
    b.log_alpha = a.log_alpha; b.beta = a.beta; b.S0 = a.S0;
    b.cu_seqlens = a.cu_seqlens;
    b.n_seq = a.n_seq; b.B = a.B; b.H = a.H; b.T = a.T; b.dk = a.dk; b.dv = a.dv; b.C = a.C;
    b.dtype = a.dtype; b.gate = a.gate;
    return b;
}

int launch_kda_split(const FwdArgs &a, int n_seq_eff, hipStream_t s) {
    const bool varlen = a.cu_seqlens != nullptr;
    const KdaWs kw = kda_ws(a, n_seq_eff);
    const SplitLayout lay = kw.lay;
    const int max_chunks = lay.max_chunks;
    SplitParams sp;
    std::memset(&sp, 0, sizeof(sp));
    sp.q = (const bf16 *)a.q; sp.k = (const bf16 *)a.k; sp.v = (const bf16 *)a.v;
    sp.a = (const bf16 *)a.a; sp.b = (const bf16 *)a.b;
    const bool dp = a.a != nullptr;
    sp.la = a.log_alpha; sp.beta = a.beta; sp.S0 = a.S0;
    sp.O = (bf16 *)a.O; sp.Sf = a.S_final; sp.cu = a.cu_seqlens;
    char *ws = (char *)a.workspace;
    sp.err = a.err ? a.err : (int *)ws;
    sp.coff = varlen ? (int32_t *)(ws + lay.coff_off) : nullptr;
    sp.order = varlen ? sp.coff + n_seq_eff + 1 : nullptr;
    sp.blk = ws + lay.blk_off;
    sp.total = (long)a.B * a.T;
    sp.H = a.H; sp.T = a.T; sp.dv = a.dv; sp.n_seq = n_seq_eff; sp.n_tiles = a.dv / kDVT;
    sp.nc = lay.nc; sp.max_chunks = max_chunks; sp.C = a.C;
    sp.seg_ws = (float *)(ws + kw.seg_off);
    sp.sub = kw.sub ? (int *)(ws + kw.sub_off) : nullptr;
    int runs = kw.runs ? seg_runs(n_seq_eff * a.H, a.dk, a.dv, chunks_per_chain(a), true) : 0;
    if (a.keep_states) {
        // the backward's layout: the same header, plan, blocks and flags, then the states
        // entering each chunk where gdr_chunk_bwd reads them, and its segmented-pass area
        const BwdLayout bl = bwd_layout(bwd_view(a), n_seq_eff);
        sp.states = (uint16_t *)(ws + bl.s_off);
        sp.seg_ws = (float *)(ws + bl.seg_off);
        runs = bl.runs ? seg_runs(n_seq_eff * a.H, a.dk, a.dv, chunks_per_chain(a), true) : 0;
    }

    if (varlen) hipLaunchKernelGGL((chunk_plan_kernel<SplitParams>), dim3(1), dim3(kPlanThreads), 0, s, sp);
    // persistent prep workgroups: two per CU (one with a, b: their LDS allows no more)
    const long njobs = (long)a.H * max_chunks;
    if (a.C == kC2) {
        // 128-token chunks: the prep merges each chunk's two halves, then the 128-row pass
        const dim3 grid((unsigned)(njobs < 2L * compute_units() ? njobs : 2L * compute_units()));
#define GDR_PREP2(G, CL) hipLaunchKernelGGL((kda_prep_kernel<128, G, false, CL, false, true>), grid, dim3(kThreads), 0, s, sp)
        if (a.clip) {
            if (a.gate == kGateChannel) GDR_PREP2(kGateChannel, true);
            else if (a.gate == kGateHead) GDR_PREP2(kGateHead, true);
            else GDR_PREP2(kGateNone, true);
        } else {
            if (a.gate == kGateChannel) GDR_PREP2(kGateChannel, false);
            else if (a.gate == kGateHead) GDR_PREP2(kGateHead, false);
            else GDR_PREP2(kGateNone, false);
        }
#undef GDR_PREP2
        const long chains = (long)n_seq_eff * a.H;
        hipLaunchKernelGGL(kda_state128_kernel, dim3((unsigned)(((chains + 7) / 8) * 8 * sp.n_tiles)),
                           dim3(kThreads2), 0, s, sp);
        return (int)hipGetLastError();
    }
    const long slots = (dp ? 1L : 2L) * compute_units();
    const dim3 grid_prep((unsigned)(njobs < slots ? njobs : slots));
    const long cus = compute_units();
    const dim3 grid_sub((unsigned)(njobs < cus ? njobs : cus));
    // the log-domain variant redoes the jobs the first pass flagged (usually none)
#define GDR_PREP(DK, G, D, CL)                                                                    \
    do {                                                                                          \
        hipLaunchKernelGGL((kda_prep_kernel<DK, G, D, CL>), grid_prep, dim3(kThreads), 0, s, sp); \
        if (sp.sub)                                                                               \
            hipLaunchKernelGGL((kda_prep_kernel<DK, G, D, CL, true>), grid_sub, dim3(kThreads), 0, s, sp); \
    } while (0)
#define GDR_GATES(DK, D, CL)                                 \
    do {                                                     \
        if (a.gate == kGateChannel) GDR_PREP(DK, kGateChannel, D, CL); \
        else if (a.gate == kGateHead) GDR_PREP(DK, kGateHead, D, CL);  \
        else GDR_PREP(DK, kGateNone, D, CL);                 \
    } while (0)
#define GDR_PATH(DK, D)                                                                     \
    do {                                                                                    \
        if (a.clip) GDR_GATES(DK, D, true);                                                 \
        else GDR_GATES(DK, D, false);                                                       \
        if (a.keep_states) run_state<DK, D, kForwardSave>(sp, runs, s);                     \
        else run_state<DK, D, kForward>(sp, runs, s);                                       \
    } while (0)
    if (a.dk == 128) {
        if (dp) GDR_PATH(128, true);
        else GDR_PATH(128, false);
    } else {
        if (dp) GDR_PATH(64, true);
        else GDR_PATH(64, false);
    }
#undef GDR_PATH
#undef GDR_GATES
#undef GDR_PREP
    return (int)hipGetLastError();
}

}  // namespace gdr

namespace gdr {

bool kda_bwd_supported(const BwdArgs &a) {
    return a.dtype == 1 && a.C == kC && (a.dk == 64 || a.dk == 128) && a.dv % kDVT == 0 &&
           a.dv <= 256 && a.gate >= kGateNone && a.gate <= kGateChannel;
}

size_t kda_bwd_workspace_bytes(const BwdArgs &a, int n_seq_eff) { return bwd_layout(a, n_seq_eff).total; }

int launch_kda_bwd(const BwdArgs &b, int n_seq_eff, hipStream_t s) {
    const bool varlen = b.cu_seqlens != nullptr;
    const BwdLayout lay = bwd_layout(b, n_seq_eff);
    const int max_chunks = lay.fw.max_chunks;
    char *ws = (char *)b.workspace;
    SplitParams sp;
    std::memset(&sp, 0, sizeof(sp));
    sp.q = (const bf16 *)b.q; sp.k = (const bf16 *)b.k; sp.v = (const bf16 *)b.v;
    sp.a = (const bf16 *)b.a; sp.b = (const bf16 *)b.b;
    sp.la = b.log_alpha; sp.beta = b.beta; sp.S0 = b.S0; sp.cu = b.cu_seqlens;
    sp.err = (int *)ws;
    sp.coff = varlen ? (int32_t *)(ws + lay.fw.coff_off) : nullptr;
    sp.order = varlen ? sp.coff + n_seq_eff + 1 : nullptr;
    sp.blk = ws + lay.fw.blk_off;
    sp.states = (uint16_t *)(ws + lay.s_off);
    sp.total = (long)b.B * b.T;
    sp.H = b.H; sp.T = b.T; sp.dv = b.dv; sp.n_seq = n_seq_eff; sp.n_tiles = b.dv / kDVT;
    sp.nc = lay.fw.nc; sp.max_chunks = max_chunks; sp.C = kC;
    sp.seg_ws = (float *)(ws + lay.seg_off);
    sp.sub = lay.sub ? (int *)(ws + lay.sub_off) : nullptr;
    const int runs = lay.runs ? seg_runs(n_seq_eff * b.H, b.dk, b.dv, chunks_per_chain(fwd_view(b)), true) : 0;
    // the reverse pass: the forward blocks, dO as the value tile, dS_final in, dS0 out
    SplitParams rp = sp;
    rp.fblk = blk_bytes(b.dk, b.a != nullptr);
    rp.v = (const bf16 *)b.dO;
    rp.S0 = b.dS_final;
    rp.Sf = b.grad_S0;
    rp.states = (uint16_t *)(ws + lay.ds_off);
    rp.sub = nullptr;
    BwdParams bp;
    std::memset(&bp, 0, sizeof(bp));
    bp.q = (const bf16 *)b.q; bp.k = (const bf16 *)b.k; bp.v = (const bf16 *)b.v;
    bp.dO = (const bf16 *)b.dO; bp.la = b.log_alpha; bp.beta = b.beta;
    bp.a = (const bf16 *)b.a; bp.b = (const bf16 *)b.b;
    bp.da = (bf16 *)b.grad_a; bp.db = (bf16 *)b.grad_b;
    bp.S = (const uint16_t *)(ws + lay.s_off); bp.dS = (const uint16_t *)(ws + lay.ds_off);
    bp.dq = (bf16 *)b.grad_q; bp.dk = (bf16 *)b.grad_k; bp.dv = (bf16 *)b.grad_v;
    bp.dla = b.grad_la; bp.dbeta = b.grad_beta;
    bp.cu = b.cu_seqlens; bp.coff = sp.coff; bp.total = sp.total; bp.err = (int *)ws;
    bp.H = b.H; bp.T = b.T; bp.dv_ = b.dv; bp.n_seq = n_seq_eff; bp.nc = lay.fw.nc;
    bp.max_chunks = max_chunks; bp.C = kC;

    if (varlen) hipLaunchKernelGGL((chunk_plan_kernel<SplitParams>), dim3(1), dim3(kPlanThreads), 0, s, sp);
    const long njobs = (long)b.H * max_chunks;
    const bool dp = b.a != nullptr;
    const long slots = (dp ? 1L : 2L) * compute_units();  // resident prep workgroups per CU
    const dim3 grid_prep((unsigned)(njobs < slots ? njobs : slots));
    const dim3 grid_jobs((unsigned)njobs);
    // the KDA gradient kernel is persistent: one workgroup per CU (its LDS allows no more)
    const long cus = compute_units();
    const dim3 grid_sub((unsigned)(njobs < cus ? njobs : cus));
    const dim3 grid_post(dp ? grid_jobs : dim3((unsigned)(njobs < cus ? njobs : cus)));
#define GDR_BWD(DK, G, D, POST)                                                                    \
    do {                                                                                           \
        if (!b.reuse_fwd) { /* else the forward left its blocks in the workspace */             \
            hipLaunchKernelGGL((kda_prep_kernel<DK, G, D, false>), grid_prep, dim3(kThreads), 0, s, sp); \
            if (sp.sub)                                                                            \
                hipLaunchKernelGGL((kda_prep_kernel<DK, G, D, false, true>), grid_sub, dim3(kThreads), 0, s, sp); \
        }                                                                                          \
        if (!b.reuse_states) run_state<DK, D, kSaveStates>(sp, runs, s);                          \
        run_state<DK, true, kReverse>(rp, runs, s); /* on the forward blocks */                    \
        hipLaunchKernelGGL((POST<DK, G>), grid_post, dim3(kThreads), 0, s, bp);                   \
    } while (0)
#define GDR_BWD_GATES(DK, D, POST)                                        \
    do {                                                                  \
        if (b.gate == kGateChannel) GDR_BWD(DK, kGateChannel, D, POST);   \
        else if (b.gate == kGateHead) GDR_BWD(DK, kGateHead, D, POST);    \
        else GDR_BWD(DK, kGateNone, D, POST);                             \
    } while (0)
    if (dp) {
        if (b.dk == 128) GDR_BWD_GATES(128, true, kda_bwd_post_dplr_kernel);
        else GDR_BWD_GATES(64, true, kda_bwd_post_dplr_kernel);
    } else {
        if (b.dk == 128) GDR_BWD_GATES(128, false, kda_bwd_post_kernel);
        else GDR_BWD_GATES(64, false, kda_bwd_post_kernel);
    }
#undef GDR_BWD_GATES
#undef GDR_BWD
    return (int)hipGetLastError();
}

}  // namespace gdr
