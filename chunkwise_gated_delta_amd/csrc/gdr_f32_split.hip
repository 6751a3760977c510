// Chunkwise forward with fp32 arithmetic throughout, as two kernels.
//
// Serves fp32 inputs (where bf16 matrix-core products would not meet fp32
// accuracy) at C = 16, 32 or 64, and bf16 DPLR inputs at C = 16 or 32.  The
// algebra is the one the bf16 matrix-core path uses (see gdr_kda_split.hip): per
// chunk the state-independent factors are formed in parallel over all chunks,
// and a serial kernel per (sequence, head, 32-wide dv tile) applies them.
//
//   f32_prep_kernel   one workgroup per (chunk, head)
//     g  = in-chunk inclusive prefix sum of log alpha; Q<- = Q e^g, K<- = K e^g,
//          K-> = K e^-g, K^ = K e^(g_C - g), gamma_C = e^g_C
//     KDA form ("Kimi Delta Attention backward" notes, forward recap):
//       At = (I + Diag(beta)(K<- K->^T strictly lower))^-1,  Ab = At Diag(beta)
//       Ao = A_qk Ab,  W' = -Ab K<-,  Q~ = Q<- - Ao K<-
//     gated DPLR form ("Diagonal Plus Low Rank" notes, section 2, matrix form, write
//     term scaled by beta), with A-> = A e^-g, B<- = B e^g, A^ = A e^(g_C - g):
//       E = (I + (B<- A->^T strictly lower))^-1,  Ec' = -E (B<- K->^T strictly lower) Diag(beta)
//       W' = -E B<-,  Ao' = A_qk Diag(beta) + (Q<- A->^T) Ec',  Q~ = Q<- + (Q<- A->^T) W'
//   f32_state_kernel  serial over the chunks of one sequence
//     V_new = Ab V + W' S^T,  O = Ao V + Q~ S^T,  S = S Diag(gamma_C) + V_new^T K^
//     (DPLR: N = Ec' V + W' S^T, O = Ao' V + Q~ S^T, S = S Diag(gamma_C) + N^T A^ + V^T Diag(beta) K^)
//
// The prep kernel holds its operands in LDS in 64-channel blocks of dk (the C x C
// products accumulate over the blocks), so dk = 128 fits for every form.  The unit
// lower-triangular inverse is forward substitution, one column per thread with the
// column in registers ("DeltaNet" notes, section 4.2, solved column by column).
// Padding rows of a partial chunk carry q = k = v = a = b = 0, beta = 0 and log
// alpha = 0, which makes them identity steps.
#include "gdr_split_common.h"

namespace gdr {
namespace {

constexpr int kFT = 256;       // threads per workgroup, both kernels
constexpr float kF32GateRange = 80.f;  // natural log
constexpr int kDB = 64;        // dk channels per operand block of the prep kernel
constexpr int kOS = kDB + 1;   // row stride (floats) of [C][kDB] operand arrays
constexpr int kFDVT = 32;      // dv columns per state workgroup
constexpr int kMaxDK = 128;
constexpr float kLn2 = 0.6931471805599453f;

struct F32Params {
    const void *q, *k, *v, *a, *b;  // a, b: DPLR low-rank vectors, or NULL
    const float *la, *beta, *S0;
    void *O;
    float *Sf;
    const int32_t *cu;
    int32_t *coff, *order;  // packed sequences (with cu_seqlens), else NULL
    int *err;
    float *blk;  // (chunk, head) blocks of bf floats
    long total;
    int H, T, dk, dv, n_seq, n_tiles, C, gate;
    int clip;  // spectral clipping of the gate: alpha <- min(alpha, 1 / ||I - b a^T||_2)
    int nc, max_chunks, bf;
};

// One (chunk, head) block, in floats.
struct F32Blk {
    int oW, oQ, oK, oKb, oAb, oAo, oG, floats;
};
__host__ __device__ inline F32Blk f32_blk(int C, int dk, bool dp) {
    F32Blk b;
    b.oW = 0;                      // W' [C][dk]
    b.oQ = C * dk;                 // Q~ [C][dk]
    b.oK = 2 * C * dk;             // K^ (DPLR: A^) [C][dk]
    b.oKb = 3 * C * dk;            // DPLR: Diag(beta) K^ [C][dk]
    b.oAb = (dp ? 4 : 3) * C * dk; // Ab (DPLR: Ec') [C][C]
    b.oAo = b.oAb + C * C;         // Ao (DPLR: Ao') [C][C]
    b.oG = b.oAo + C * C;          // gamma_C [dk]
    b.floats = (b.oG + dk + 63) / 64 * 64;
    return b;
}

template <int C, bool DP>
struct F32PrepSmem {  // offsets in floats
    static constexpr int CS = C + 4;                  // row stride of [C][C] arrays
    static constexpr int oQl = 0;                     // Q<-            [C][kOS]
    static constexpr int oKl = oQl + C * kOS;         // K<- (DP: B<-)
    static constexpr int oKr = oKl + C * kOS;         // K->; DP: then W'
    static constexpr int oAr = oKr + C * kOS;         // DP: A->
    static constexpr int oL = oAr + (DP ? C * kOS : 0);  // L -> At -> Ab (DP: B<-A->^T -> E)
    static constexpr int oAqk = oL + C * CS;          // A_qk -> Ao (DP: A_qk Diag(beta) -> Ao')
    static constexpr int oBK = oAqk + C * CS;         // DP: B<-K->^T Diag(beta), strictly lower
    static constexpr int oAqa = oBK + (DP ? C * CS : 0);  // DP: Q<-A->^T with the diagonal
    static constexpr int oEc = oAqa + (DP ? C * CS : 0);  // DP: Ec'
    static constexpr int oBeta = oEc + (DP ? C * CS : 0);
    static constexpr int oTot = oBeta + C;            // gate partial sums [4][kDB]
    static constexpr int oGh = oTot + 4 * kDB;        // head gate prefix sums [C]
    static constexpr int oClip = oGh + C;             // clip bound -ln rho per row [C]
    static constexpr int floats = oClip + C;
    static_assert(floats * 4 <= 160 * 1024, "LDS");
};

template <typename Tin, int C, bool DP>
__global__ __launch_bounds__(kFT) void f32_prep_kernel(F32Params p) {
    using L = F32PrepSmem<C, DP>;
    constexpr int CS = L::CS;
    constexpr int RPG = C / 4;  // rows per row group in the staging
    constexpr int TR = C / 16;  // rows (and C x C columns) per thread tile
    __shared__ __attribute__((aligned(16))) float smem[L::floats];
    float *sQl = smem + L::oQl, *sKl = smem + L::oKl, *sKr = smem + L::oKr, *sAr = smem + L::oAr;
    float *sL = smem + L::oL, *sAqk = smem + L::oAqk, *sBK = smem + L::oBK, *sAqa = smem + L::oAqa;
    float *sEc = smem + L::oEc, *sBeta = smem + L::oBeta, *sTot = smem + L::oTot, *sGh = smem + L::oGh;
    float *sClip = smem + L::oClip;

    const Tin *q = (const Tin *)p.q, *k = (const Tin *)p.k, *a = (const Tin *)p.a, *b = (const Tin *)p.b;
    const int tid = threadIdx.x, H = p.H, dk = p.dk;
    const int g = blockIdx.x, h = g % H;
    int n = 0, c = 0;
    if (!chunk_of(p, g / H, n, c)) return;  // workgroup-uniform
    long t0, t1;
    seq_bounds(p.cu, n, p.T, p.total, t0, t1, nullptr);
    const long tok0 = t0 + (long)c * C;
    const int m = (int)((t1 - tok0) < C ? (t1 - tok0) : C);
    const F32Blk B = f32_blk(C, dk, DP);
    float *bp = p.blk + (size_t)g * p.bf;

    if (tid < C) sBeta[tid] = tid < m ? p.beta[(size_t)(tok0 + tid) * H + h] : 0.f;
    if (p.clip) {  // workgroup-uniform
        // Spectral clip bound per row, -ln ||I - b a^T||_2, from |a|^2, |b|^2 and a.b
        // (without a, b: a = k, b = beta k), kFT / C threads per row.
        constexpr int TPR = kFT / C;
        const int r = tid / TPR, j = tid % TPR;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f;
        if (r < m) {
            const size_t base = ((size_t)(tok0 + r) * H + h) * dk;
            for (int d = j; d < dk; d += TPR) {
                if (DP) {
                    const float av = ld(a, base + d), bv = ld(b, base + d);
                    s0 += av * av;
                    s1 += bv * bv;
                    s2 += av * bv;
                } else {
                    const float kv = ld(k, base + d);
                    s0 += kv * kv;
                }
            }
        }
        s0 = group_sum<TPR>(s0);
        s1 = group_sum<TPR>(s1);
        s2 = group_sum<TPR>(s2);
        if (j == 0) {
            const float br = r < m ? p.beta[(size_t)(tok0 + r) * H + h] : 0.f;
            sClip[r] = DP ? clip_bound(s0, s1, s2, kLn2) : clip_bound(s0, br * br * s0, br * s0, kLn2);
        }
        lds_barrier();
    }
    // A clipped gate without a gate input is one value per row, like a head gate.
    const bool head_scan = p.gate == kGateHead || (p.clip && p.gate == kGateNone);
    if (head_scan && tid < 64) {
        float x = tid < m && tid < C && p.gate == kGateHead ? p.la[(size_t)(tok0 + tid) * H + h] : 0.f;
        if (p.clip && tid < C) x = fminf(x, sClip[tid]);
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (tid >= off) x += y;
        }
        if (tid < C) sGh[tid] = x;
    }
    lds_barrier();

    // Operands of channel block db into LDS: thread (channel d, row group rg).  With
    // `first`, also K->, A-> and the block's K^ / A^ / Diag(beta) K^ / gamma_C.
    auto stage = [&](int db, bool first) {
        const int d = tid & (kDB - 1), rg = tid >> 6, col = db * kDB + d;
        float qv[RPG], kv[RPG], av[RPG], bv[RPG], gv[RPG];
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
            const int r = rg * RPG + i;
            const bool ok = r < m;
            const size_t e = ((size_t)(tok0 + (ok ? r : 0)) * H + h) * dk + col;
            qv[i] = ok ? ld(q, e) : 0.f;
            kv[i] = ok ? ld(k, e) : 0.f;
            av[i] = DP && ok ? ld(a, e) : 0.f;
            bv[i] = DP && ok ? ld(b, e) : 0.f;
            if (p.gate == kGateChannel) {
                float x = ok ? p.la[e] : 0.f;
                if (p.clip) x = fminf(x, sClip[r]);
                run += x;
            }
            gv[i] = run;
        }
        float gC = 0.f;
        if (p.gate == kGateChannel) {
            sTot[rg * kDB + d] = run;
            lds_barrier();
            float carry = 0.f;
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) {
                const float t = sTot[r2 * kDB + d];
                gC += t;
                carry += r2 < rg ? t : 0.f;
            }
#pragma unroll
            for (int i = 0; i < RPG; ++i) gv[i] += carry;
        } else if (head_scan) {
            gC = sGh[C - 1];
#pragma unroll
            for (int i = 0; i < RPG; ++i) gv[i] = sGh[rg * RPG + i];
        }
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
            const int r = rg * RPG + i;
            const float eg = expf(gv[i]), eig = expf(-gv[i]);
            sQl[r * kOS + d] = qv[i] * eg;
            sKl[r * kOS + d] = (DP ? bv[i] : kv[i]) * eg;
            if (first) {
                const float egc = expf(gC - gv[i]);
                sKr[r * kOS + d] = kv[i] * eig;
                if (DP) sAr[r * kOS + d] = av[i] * eig;
                bp[B.oK + r * dk + col] = (DP ? av[i] : kv[i]) * egc;
                if (DP) bp[B.oKb + r * dk + col] = sBeta[r] * kv[i] * egc;
            }
        }
        if (first && rg == 0) {
            bp[B.oG + col] = expf(gC);
            // e^-g leaves the float range once a channel falls by e^80 inside the chunk:
            // such a chunk's result is not valid, which the error word reports (bit 2)
            if (!(gC >= -kF32GateRange)) atomicOr(p.err, 2);
        }
        lds_barrier();
    };

    // C x C products accumulate over the channel blocks; thread tile rows R0.., cols I0..
    const int tr = tid >> 4, tc = tid & 15, R0 = TR * tr, I0 = TR * tc;
    float accL[TR][TR] = {}, accQ[TR][TR] = {}, accB[TR][TR] = {}, accA[TR][TR] = {};
    const int nb = dk / kDB;
    for (int db = 0; db < nb; ++db) {
        stage(db, true);
        if (I0 <= R0 + TR - 1) {  // tile reaches the lower triangle
            for (int d = 0; d < kDB; ++d) {
                float ra[TR], rq[TR], ck[TR], ca[TR];
#pragma unroll
                for (int x = 0; x < TR; ++x) {
                    ra[x] = sKl[(R0 + x) * kOS + d];
                    rq[x] = sQl[(R0 + x) * kOS + d];
                    ck[x] = sKr[(I0 + x) * kOS + d];
                    ca[x] = DP ? sAr[(I0 + x) * kOS + d] : 0.f;
                }
#pragma unroll
                for (int x = 0; x < TR; ++x)
#pragma unroll
                    for (int y = 0; y < TR; ++y) {
                        accL[x][y] += ra[x] * (DP ? ca[y] : ck[y]);
                        accQ[x][y] += rq[x] * ck[y];
                        if (DP) {
                            accB[x][y] += ra[x] * ck[y];
                            accA[x][y] += rq[x] * ca[y];
                        }
                    }
            }
        }
        lds_barrier();
    }
#pragma unroll
    for (int x = 0; x < TR; ++x)
#pragma unroll
        for (int y = 0; y < TR; ++y) {
            const int r = R0 + x, i = I0 + y;
            if (DP) {
                sL[r * CS + i] = i < r ? accL[x][y] : 0.f;
                sBK[r * CS + i] = i < r ? accB[x][y] * sBeta[i] : 0.f;
                sAqk[r * CS + i] = i <= r ? accQ[x][y] * sBeta[i] : 0.f;
                sAqa[r * CS + i] = i <= r ? accA[x][y] : 0.f;
            } else {
                sL[r * CS + i] = i < r ? sBeta[r] * accL[x][y] : 0.f;
                sAqk[r * CS + i] = i <= r ? accQ[x][y] : 0.f;
            }
        }
    lds_barrier();

    // (I + L)^-1: thread c solves column c, x_r = [r == c] - sum_{i<r} L[r][i] x_i
    // (x_r = 0 above the diagonal follows without masking).
    {
        float x[C];
        if (tid < C) {
#pragma unroll
            for (int r = 0; r < C; ++r) {
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) {
                    if (i & 1) s1 += sL[r * CS + i] * x[i];
                    else s0 += sL[r * CS + i] * x[i];
                }
                x[r] = (r == tid ? 1.f : 0.f) - (s0 + s1);
            }
        }
        lds_barrier();
        if (tid < C) {
#pragma unroll
            for (int r = 0; r < C; ++r) sL[r * CS + tid] = x[r];
        }
        lds_barrier();
    }

    // C x C x C products on thread tiles: acc = sum_k A[R0+x][k] Bm[k][I0+y]
    auto mm = [&](const float *A, const float *Bm, float (&acc)[TR][TR]) {
        for (int kk = 0; kk < C; ++kk) {
            float ar[TR], bc[TR];
#pragma unroll
            for (int x = 0; x < TR; ++x) {
                ar[x] = A[(R0 + x) * CS + kk];
                bc[x] = Bm[kk * CS + I0 + x];
            }
#pragma unroll
            for (int x = 0; x < TR; ++x)
#pragma unroll
                for (int y = 0; y < TR; ++y) acc[x][y] += ar[x] * bc[y];
        }
    };
    if (DP) {
        float acc[TR][TR] = {};
        mm(sL, sBK, acc);  // E BK'
#pragma unroll
        for (int x = 0; x < TR; ++x)
#pragma unroll
            for (int y = 0; y < TR; ++y) sEc[(R0 + x) * CS + I0 + y] = -acc[x][y];
        lds_barrier();
        float acc2[TR][TR];
#pragma unroll
        for (int x = 0; x < TR; ++x)
#pragma unroll
            for (int y = 0; y < TR; ++y) acc2[x][y] = sAqk[(R0 + x) * CS + I0 + y];
        mm(sAqa, sEc, acc2);  // Ao' = A_qk' + Aqa Ec' (each thread rewrites only its own tile)
#pragma unroll
        for (int x = 0; x < TR; ++x)
#pragma unroll
            for (int y = 0; y < TR; ++y) sAqk[(R0 + x) * CS + I0 + y] = acc2[x][y];
        lds_barrier();
    } else {
        for (int idx = tid; idx < C * C; idx += kFT) {  // Ab = At Diag(beta)
            const int r = idx / C, i = idx % C;
            sL[r * CS + i] *= sBeta[i];
        }
        lds_barrier();
        float acc[TR][TR] = {};
        mm(sAqk, sL, acc);  // Ao = A_qk Ab
        lds_barrier();
#pragma unroll
        for (int x = 0; x < TR; ++x)
#pragma unroll
            for (int y = 0; y < TR; ++y) sAqk[(R0 + x) * CS + I0 + y] = acc[x][y];
        lds_barrier();
    }
    for (int idx = tid; idx < C * C; idx += kFT) {
        const int r = idx / C, i = idx % C;
        bp[B.oAb + idx] = (DP ? sEc : sL)[r * CS + i];
        bp[B.oAo + idx] = sAqk[r * CS + i];
    }

    // W' and Q~, one channel block at a time (the last block staged is still in LDS).
    // Thread tile: rows TR*tr + x, channels 4*tc + y.
    for (int db = nb - 1; db >= 0; --db) {
        if (db != nb - 1) stage(db, false);
        float w[TR][4] = {};
        for (int kk = 0; kk < C; ++kk) {
            float kr[4];
#pragma unroll
            for (int y = 0; y < 4; ++y) kr[y] = sKl[kk * kOS + 4 * tc + y];
#pragma unroll
            for (int x = 0; x < TR; ++x) {
                const float e = sL[(R0 + x) * CS + kk];
#pragma unroll
                for (int y = 0; y < 4; ++y) w[x][y] += e * kr[y];
            }
        }
#pragma unroll
        for (int x = 0; x < TR; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                const int r = R0 + x, col = db * kDB + 4 * tc + y;
                bp[B.oW + r * dk + col] = -w[x][y];
                if (DP) sKr[r * kOS + 4 * tc + y] = -w[x][y];
            }
        if (DP) lds_barrier();
        float o[TR][4] = {};
        const float *Am = DP ? sAqa : sAqk;  // Q~ = Q<- + Aqa W'  |  Q<- - Ao K<-
        const float *Bm = DP ? sKr : sKl;
        for (int kk = 0; kk < C; ++kk) {
            float br[4];
#pragma unroll
            for (int y = 0; y < 4; ++y) br[y] = Bm[kk * kOS + 4 * tc + y];
#pragma unroll
            for (int x = 0; x < TR; ++x) {
                const float e = Am[(R0 + x) * CS + kk];
#pragma unroll
                for (int y = 0; y < 4; ++y) o[x][y] += e * br[y];
            }
        }
#pragma unroll
        for (int x = 0; x < TR; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                const int r = R0 + x, cc = 4 * tc + y;
                const float ql = sQl[r * kOS + cc];
                bp[B.oQ + r * dk + db * kDB + cc] = DP ? ql + o[x][y] : ql - o[x][y];
            }
        lds_barrier();
    }
}

template <typename Tin, int C, bool DP>
__global__ __launch_bounds__(kFT) void f32_state_kernel(F32Params p) {
    constexpr int VS = kFDVT + 4;      // row stride of [*][32] tiles
    constexpr int TPR = kFT / C;       // phase 1: threads per chunk row
    constexpr int JW = kFDVT / TPR;    // phase 1: dv columns per thread
    __shared__ __attribute__((aligned(16))) float sST[kMaxDK * VS];  // S^T [dk][32]
    __shared__ __attribute__((aligned(16))) float sV[C * VS];
    __shared__ __attribute__((aligned(16))) float sVn[C * VS];
    __shared__ float sGam[kMaxDK];

    const Tin *v = (const Tin *)p.v;
    Tin *O = (Tin *)p.O;
    const int tid = threadIdx.x, H = p.H, dk = p.dk, DV = p.dv;
    const int lin = blockIdx.x;
    const int tile = lin % p.n_tiles;
    const int h = (lin / p.n_tiles) % H;
    const int rank = lin / (p.n_tiles * H);
    const int n = p.order ? p.order[rank] : rank;
    const int j0 = tile * kFDVT;
    long t0, t1;
    seq_bounds(p.cu, n, p.T, p.total, t0, t1, nullptr);
    int nck = (int)((t1 - t0 + C - 1) / C);
    long cbase;
    if (p.coff) {
        cbase = p.coff[n];
        const long room = p.max_chunks - cbase;  // only short of nck for malformed offsets
        nck = (int)(room < 0 ? 0 : (room < nck ? room : nck));
    } else {
        cbase = (long)n * p.nc;
    }
    const F32Blk B = f32_blk(C, dk, DP);

    for (int idx = tid; idx < dk * kFDVT; idx += kFT) {
        const int j = idx / dk, d = idx % dk;
        sST[d * VS + j] = p.S0 ? p.S0[(((size_t)n * H + h) * DV + j0 + j) * dk + d] : 0.f;
    }

    const int r1 = tid / TPR, jc = JW * (tid % TPR);  // phase 1
    constexpr int kJS = 8;  // phase 2: dv columns per item (channel d, columns js..js+7)
    for (int c = 0; c < nck; ++c) {
        const float *bp = p.blk + ((size_t)(cbase + c) * H + h) * p.bf;
        const long tc0 = t0 + (long)c * C;
        const int m = (int)((t1 - tc0) < C ? (t1 - tc0) : C);
        for (int idx = tid; idx < C * kFDVT; idx += kFT) {
            const int r = idx / kFDVT, j = idx % kFDVT;
            sV[r * VS + j] = r < m ? ld(v, ((size_t)(tc0 + r) * H + h) * DV + j0 + j) : 0.f;
        }
        for (int d = tid; d < dk; d += kFT) sGam[d] = bp[B.oG + d];
        lds_barrier();

        // V_new (N) and O rows: row r1, columns jc..jc+JW-1
        {
            // Operand rows are read in batches of kBU float4 per matrix, all loads of a
            // batch in flight together (the rows come from L2 or HBM).
            float vn[JW] = {}, o[JW] = {};
            const float4 *ab = (const float4 *)(bp + B.oAb + r1 * C);
            const float4 *ao = (const float4 *)(bp + B.oAo + r1 * C);
            constexpr int kBU = C / 4 < 8 ? C / 4 : 8;
            for (int i0 = 0; i0 < C / 4; i0 += kBU) {
                float4 xa[kBU], xo[kBU];
#pragma unroll
                for (int u = 0; u < kBU; ++u) {
                    xa[u] = ab[i0 + u];
                    xo[u] = ao[i0 + u];
                }
#pragma unroll
                for (int u = 0; u < kBU; ++u) {
                    const float xv[4] = {xa[u].x, xa[u].y, xa[u].z, xa[u].w};
                    const float yv[4] = {xo[u].x, xo[u].y, xo[u].z, xo[u].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int jj = 0; jj < JW; ++jj) {
                            const float vv = sV[(4 * (i0 + u) + e) * VS + jc + jj];
                            vn[jj] += xv[e] * vv;
                            o[jj] += yv[e] * vv;
                        }
                }
            }
            const float4 *wr = (const float4 *)(bp + B.oW + (size_t)r1 * dk);
            const float4 *qr = (const float4 *)(bp + B.oQ + (size_t)r1 * dk);
            for (int d0 = 0; d0 < dk / 4; d0 += 8) {
                float4 xw[8], xq[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    xw[u] = wr[d0 + u];
                    xq[u] = qr[d0 + u];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float xv[4] = {xw[u].x, xw[u].y, xw[u].z, xw[u].w};
                    const float yv[4] = {xq[u].x, xq[u].y, xq[u].z, xq[u].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int jj = 0; jj < JW; ++jj) {
                            const float s = sST[(4 * (d0 + u) + e) * VS + jc + jj];
                            vn[jj] += xv[e] * s;
                            o[jj] += yv[e] * s;
                        }
                }
            }
#pragma unroll
            for (int jj = 0; jj < JW; ++jj) sVn[r1 * VS + jc + jj] = vn[jj];
            if (r1 < m) {
#pragma unroll
                for (int jj = 0; jj < JW; ++jj) st(O, ((size_t)(tc0 + r1) * H + h) * DV + j0 + jc + jj, o[jj]);
            }
        }
        lds_barrier();

        // S^T[d][js..] = gamma_C S^T + K^^T V_new (+ (Diag(beta) K^)^T V), items of one
        // channel and 8 dv columns (1 per thread at dk = 64, 2 at dk = 128)
        for (int it = tid; it < dk * (kFDVT / kJS); it += kFT) {
            const int d2 = it % dk, js = kJS * (it / dk);
            float acc[kJS];
            const float gm = sGam[d2];
#pragma unroll
            for (int jj = 0; jj < kJS; ++jj) acc[jj] = gm * sST[d2 * VS + js + jj];
            for (int r0 = 0; r0 < C; r0 += 16) {
                float kh[16], kb[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    kh[u] = bp[B.oK + (size_t)(r0 + u) * dk + d2];
                    kb[u] = DP ? bp[B.oKb + (size_t)(r0 + u) * dk + d2] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 16; ++u)
#pragma unroll
                    for (int jj = 0; jj < kJS; ++jj) {
                        acc[jj] += kh[u] * sVn[(r0 + u) * VS + js + jj];
                        if (DP) acc[jj] += kb[u] * sV[(r0 + u) * VS + js + jj];
                    }
            }
#pragma unroll
            for (int jj = 0; jj < kJS; ++jj) sST[d2 * VS + js + jj] = acc[jj];
        }
        lds_barrier();
    }

    if (p.Sf) {
        for (int idx = tid; idx < dk * kFDVT; idx += kFT) {
            const int j = idx / dk, d = idx % dk;
            p.Sf[(((size_t)n * H + h) * DV + j0 + j) * dk + d] = sST[d * VS + j];
        }
    }
}

// At dk = 64 the whole fp32 block of a chunk fits in LDS next to the state: the staged
// variant copies each chunk's block (rows padded by 4 floats) and value tile into LDS
// and loads the next chunk's into registers while it computes, so a chunk costs one
// memory latency hidden behind the previous chunk instead of several exposed ones.
template <int C, bool DP, int DVT>
struct F32StagedSmem {  // offsets in floats; dk = 64
    static constexpr int RS = 64 + 4;                  // row stride of [C][dk] matrices
    static constexpr int CS = C + 4;                   // row stride of [C][C] matrices
    static constexpr int VS = DVT + 4;                 // row stride of [*][DVT] tiles
    static constexpr int oW = 0;
    static constexpr int oQ = oW + C * RS;
    static constexpr int oK = oQ + C * RS;
    static constexpr int oKb = oK + C * RS;            // DP only
    static constexpr int oAb = oKb + (DP ? C * RS : 0);
    static constexpr int oAo = oAb + C * CS;
    static constexpr int oG = oAo + C * CS;
    static constexpr int oDump = oG + 64;              // 4 floats: target of the padding copies
    static constexpr int oST = oDump + 4;              // S^T [64][VS]
    static constexpr int oV = oST + 64 * VS;           // V [C][VS]
    static constexpr int oVn = oV + C * VS;            // V_new (N) [C][VS]
    static constexpr int floats = oVn + C * VS;
    static_assert(floats * 4 <= 160 * 1024, "LDS");
};

// DVT (dv columns per workgroup) is 32, or 8 for problems too small to fill the GPU.
template <typename Tin, int C, bool DP, int DVT>
__global__ __launch_bounds__(kFT) void f32_state_staged_kernel(F32Params p) {
    using L = F32StagedSmem<C, DP, DVT>;
    constexpr int DK = 64;
    constexpr int VS = L::VS;
    constexpr int TPR = kFT / C < DVT ? kFT / C : DVT;  // phase 1: threads per chunk row
    constexpr int JW = DVT / TPR;                       // phase 1: dv columns per thread
    constexpr int NT1 = C * TPR;                        // phase 1: busy threads
    constexpr int kJS = DVT < 8 ? DVT : 8;              // phase 2: dv columns per item
    constexpr int NT2 = DK * (DVT / kJS);               // phase 2: items (<= threads)
    static_assert(NT1 <= kFT && NT2 <= kFT, "one item per thread");
    constexpr int NB4 = ((DP ? 4 : 3) * C * DK + 2 * C * C + DK) / 4;  // float4 of a block's data
    constexpr int NPF = (NB4 + kFT - 1) / kFT;                          // per thread
    constexpr int NPV = (C * DVT + kFT - 1) / kFT;                      // value elements per thread
    __shared__ __attribute__((aligned(16))) float smem[L::floats];
    float *sST = smem + L::oST, *sV = smem + L::oV, *sVn = smem + L::oVn;

    const Tin *v = (const Tin *)p.v;
    Tin *O = (Tin *)p.O;
    const int tid = threadIdx.x, H = p.H, DV = p.dv;
    const int lin = blockIdx.x;
    const int tile = lin % p.n_tiles;
    const int h = (lin / p.n_tiles) % H;
    const int rank = lin / (p.n_tiles * H);
    const int n = p.order ? p.order[rank] : rank;
    const int j0 = tile * DVT;
    long t0, t1;
    seq_bounds(p.cu, n, p.T, p.total, t0, t1, nullptr);
    int nck = (int)((t1 - t0 + C - 1) / C);
    long cbase;
    if (p.coff) {
        cbase = p.coff[n];
        const long room = p.max_chunks - cbase;
        nck = (int)(room < 0 ? 0 : (room < nck ? room : nck));
    } else {
        cbase = (long)n * p.nc;
    }

    for (int idx = tid; idx < DK * DVT; idx += kFT) {
        const int j = idx / DK, d = idx % DK;
        sST[d * VS + j] = p.S0 ? p.S0[(((size_t)n * H + h) * DV + j0 + j) * DK + d] : 0.f;
    }

    // LDS position of the block's float4 number e4 (block order: W', Q~, K^, [K^b],
    // Ab, Ao, gamma_C; each matrix row-major, rows padded in LDS).
    // Float4 numbers past the block's data go to a dump slot, so every thread stores
    // the same number of values with no branch.
    auto lds_pos = [&](int e4) __attribute__((always_inline)) {
        const int e = 4 * e4;
        constexpr int nm = DP ? 4 : 3;
        const int f = e - nm * C * DK;
        const int pm = L::oW + (e / DK) * L::RS + e % DK;  // the [C][dk] matrices are stacked
        const int pc = L::oAb + (f / C) * L::CS + f % C;    // so are the two [C][C] ones
        const int pg = L::oG + (f - 2 * C * C);
        return e4 >= NB4 ? L::oDump : (f < 0 ? pm : (f < 2 * C * C ? pc : pg));
    };
    // Loads of chunk c's block and value tile into registers (native vector type: HIP's
    // float4 class is copied through memory, which would put these registers in scratch).
#define GDR_F32_FETCH(c)                                                                            \
    do {                                                                                            \
        const f32x4 *bp_ = (const f32x4 *)(p.blk + ((size_t)(cbase + (c)) * H + h) * p.bf);         \
        _Pragma("unroll") for (int u = 0; u < NPF; ++u) {                                           \
            const int e4 = tid + kFT * u;                                                           \
            pf[u] = bp_[e4 < NB4 ? e4 : 0];                                                         \
        }                                                                                           \
        const long tc0_ = t0 + (long)(c) * C;                                                       \
        _Pragma("unroll") for (int u = 0; u < NPV; ++u) {                                           \
            const int idx = (tid + kFT * u) % (C * DVT), r = idx / DVT, j = idx % DVT;              \
            const long tok = tc0_ + r < t1 ? tc0_ + r : t1 - 1;                                     \
            pv[u] = ld(v, ((size_t)tok * H + h) * DV + j0 + j);                                     \
        }                                                                                           \
    } while (0)
    f32x4 pf[NPF];
    float pv[NPV];
    if (nck > 0) GDR_F32_FETCH(0);

    const int r1 = tid / TPR, jc = JW * (tid % TPR);  // phase 1
    for (int c = 0; c < nck; ++c) {
        const long tc0 = t0 + (long)c * C;
        const int m = (int)((t1 - tc0) < C ? (t1 - tc0) : C);
#pragma unroll
        for (int u = 0; u < NPF; ++u) *(f32x4 *)(smem + lds_pos(tid + kFT * u)) = pf[u];
#pragma unroll
        for (int u = 0; u < NPV; ++u) {
            const int idx = tid + kFT * u, r = (idx % (C * DVT)) / DVT, j = idx % DVT;
            if (idx < C * DVT) sV[r * VS + j] = r < m ? pv[u] : 0.f;
        }
        lds_barrier();  // chunk c in LDS; S^T of chunk c visible
        if (c + 1 < nck) GDR_F32_FETCH(c + 1);

        // V_new (N) and O rows: row r1, columns jc..jc+JW-1
        if (tid < NT1) {
            float vn[JW] = {}, o[JW] = {};
            const float *ab = smem + L::oAb + r1 * L::CS, *ao = smem + L::oAo + r1 * L::CS;
#pragma unroll 4
            for (int i4 = 0; i4 < C / 4; ++i4) {
                const float4 x = *(const float4 *)(ab + 4 * i4), y = *(const float4 *)(ao + 4 * i4);
                const float xv[4] = {x.x, x.y, x.z, x.w}, yv[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int jj = 0; jj < JW; ++jj) {
                        const float vv = sV[(4 * i4 + e) * VS + jc + jj];
                        vn[jj] += xv[e] * vv;
                        o[jj] += yv[e] * vv;
                    }
            }
            const float *wr = smem + L::oW + r1 * L::RS, *qr = smem + L::oQ + r1 * L::RS;
#pragma unroll 4
            for (int d4 = 0; d4 < DK / 4; ++d4) {
                const float4 x = *(const float4 *)(wr + 4 * d4), y = *(const float4 *)(qr + 4 * d4);
                const float xv[4] = {x.x, x.y, x.z, x.w}, yv[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int jj = 0; jj < JW; ++jj) {
                        const float s = sST[(4 * d4 + e) * VS + jc + jj];
                        vn[jj] += xv[e] * s;
                        o[jj] += yv[e] * s;
                    }
            }
#pragma unroll
            for (int jj = 0; jj < JW; ++jj) sVn[r1 * VS + jc + jj] = vn[jj];
            if (r1 < m) {
#pragma unroll
                for (int jj = 0; jj < JW; ++jj) st(O, ((size_t)(tc0 + r1) * H + h) * DV + j0 + jc + jj, o[jj]);
            }
        }
        lds_barrier();

        // S^T[d][js..] = gamma_C S^T + K^^T V_new (+ (Diag(beta) K^)^T V); one item per thread
        if (tid < NT2) {
            const int d2 = tid % DK, js = kJS * (tid / DK);
            float acc[kJS];
            const float gm = smem[L::oG + d2];
#pragma unroll
            for (int jj = 0; jj < kJS; ++jj) acc[jj] = gm * sST[d2 * VS + js + jj];
#pragma unroll 8
            for (int r = 0; r < C; ++r) {
                const float kh = smem[L::oK + r * L::RS + d2];
                const float kb = DP ? smem[L::oKb + r * L::RS + d2] : 0.f;
#pragma unroll
                for (int jj = 0; jj < kJS; ++jj) {
                    acc[jj] += kh * sVn[r * VS + js + jj];
                    if (DP) acc[jj] += kb * sV[r * VS + js + jj];
                }
            }
#pragma unroll
            for (int jj = 0; jj < kJS; ++jj) sST[d2 * VS + js + jj] = acc[jj];
        }
        lds_barrier();  // before the next chunk overwrites the block, V and V_new
    }

    if (p.Sf) {
        for (int idx = tid; idx < DK * DVT; idx += kFT) {
            const int j = idx / DK, d = idx % DK;
            p.Sf[(((size_t)n * H + h) * DV + j0 + j) * DK + d] = sST[d * VS + j];
        }
    }
#undef GDR_F32_FETCH
}

// dv columns per state workgroup at dk = 64: 8 when 32 would leave most of the GPU idle.
int f32_dvt(const FwdArgs &a, int n_seq_eff) {
    return a.dk == 64 && (long)n_seq_eff * a.H * (a.dv / kFDVT) < 64 ? 8 : kFDVT;
}

template <typename Tin, int C, bool DP>
void f32_launch(const F32Params &fp, dim3 gp, hipStream_t s, int dvt) {
    hipLaunchKernelGGL((f32_prep_kernel<Tin, C, DP>), gp, dim3(kFT), 0, s, fp);
    const dim3 gs((unsigned)(fp.n_seq * fp.H * fp.n_tiles));
    if (fp.dk == 64 && dvt == 8)
        hipLaunchKernelGGL((f32_state_staged_kernel<Tin, C, DP, 8>), gs, dim3(kFT), 0, s, fp);
    else if (fp.dk == 64)
        hipLaunchKernelGGL((f32_state_staged_kernel<Tin, C, DP, kFDVT>), gs, dim3(kFT), 0, s, fp);
    else
        hipLaunchKernelGGL((f32_state_kernel<Tin, C, DP>), gs, dim3(kFT), 0, s, fp);
}

}  // namespace

bool f32_split_supported(const FwdArgs &a) {
    const bool ab = a.a != nullptr && a.b != nullptr;
    if (a.dk != 64 && a.dk != 128) return false;
    if (a.dv % kFDVT != 0 || !(a.C == 16 || a.C == 32 || a.C == 64)) return false;
    if (a.dtype == 0) return true;
    return a.dtype == 1 && ab && a.C != 64;  // bf16 DPLR at C = 64 takes the matrix-core path
}

size_t f32_split_workspace_bytes(const FwdArgs &a, int n_seq_eff) {
    return split_layout(a, n_seq_eff, (size_t)f32_blk(a.C, a.dk, a.a != nullptr).floats * 4).total;
}

int launch_f32_split(const FwdArgs &a, int n_seq_eff, hipStream_t s) {
    const bool dp = a.a != nullptr;
    const F32Blk B = f32_blk(a.C, a.dk, dp);
    const SplitLayout lay = split_layout(a, n_seq_eff, (size_t)B.floats * 4);
    F32Params fp;
    fp.q = a.q; fp.k = a.k; fp.v = a.v; fp.a = a.a; fp.b = a.b;
    fp.la = a.log_alpha; fp.beta = a.beta; fp.S0 = a.S0;
    fp.O = a.O; fp.Sf = a.S_final; fp.cu = a.cu_seqlens;
    char *ws = (char *)a.workspace;
    fp.err = a.err ? a.err : (int *)ws;
    const bool varlen = a.cu_seqlens != nullptr;
    fp.coff = varlen ? (int32_t *)(ws + lay.coff_off) : nullptr;
    fp.order = varlen ? fp.coff + n_seq_eff + 1 : nullptr;
    fp.blk = (float *)(ws + lay.blk_off);
    fp.total = (long)a.B * a.T;
    fp.H = a.H; fp.T = a.T; fp.dk = a.dk; fp.dv = a.dv; fp.n_seq = n_seq_eff;
    const int dvt = f32_dvt(a, n_seq_eff);
    fp.n_tiles = a.dv / dvt; fp.C = a.C; fp.gate = a.gate; fp.clip = a.clip ? 1 : 0;
    fp.nc = lay.nc; fp.max_chunks = lay.max_chunks; fp.bf = B.floats;

    if (varlen) hipLaunchKernelGGL((chunk_plan_kernel<F32Params>), dim3(1), dim3(kPlanThreads), 0, s, fp);
    const dim3 gp((unsigned)((long)a.H * lay.max_chunks));
    if (a.dtype == 0) {
        if (dp) {
            if (a.C == 16) f32_launch<float, 16, true>(fp, gp, s, dvt);
            else if (a.C == 32) f32_launch<float, 32, true>(fp, gp, s, dvt);
            else f32_launch<float, 64, true>(fp, gp, s, dvt);
        } else {
            if (a.C == 16) f32_launch<float, 16, false>(fp, gp, s, dvt);
            else if (a.C == 32) f32_launch<float, 32, false>(fp, gp, s, dvt);
            else f32_launch<float, 64, false>(fp, gp, s, dvt);
        }
    } else {
        if (a.C == 16) f32_launch<bf16, 16, true>(fp, gp, s, dvt);
        else f32_launch<bf16, 32, true>(fp, gp, s, dvt);
    }
    return (int)hipGetLastError();
}

}  // namespace gdr
