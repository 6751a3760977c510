// Generic chunkwise forward with fp32 arithmetic throughout.
//
// Serves fp32 inputs (where bf16 matrix-core products would not meet fp32
// accuracy) and the gated DPLR form.  One workgroup per (sequence, head,
// 32-wide dv tile); chunks are processed in order.  Per chunk (C tokens):
//
//   g       in-chunk inclusive prefix sum of log alpha (per key channel)
//   Q<- = Q e^g,  K<- = K e^g,  K-> = K e^-g,  K^ = K e^(g_C - g)
//   KDA form ("Kimi Delta Attention backward" notes, forward recap):
//     L = Diag(beta)(K<- K->^T (strictly lower)),  At = (I + L)^-1
//     W = At Diag(beta) K<-,  U = At Diag(beta) V,  V_new = U - W S^T
//     O = Q<- S^T + (Q<- K->^T (lower incl. diagonal)) V_new
//     S = S Diag(gamma_C) + V_new^T K^
//   gated DPLR form ("Diagonal Plus Low Rank" notes, section 2, matrix form),
//   with V := Diag(beta) V:
//     E = (I + (B<- A->^T strictly lower))^-1,  W = E B<-
//     Cm = -E (B<- K->^T strictly lower) V,      N = Cm - W S^T
//     O = Q<- S^T + (Q<- K->^T lower) V + (Q<- A->^T lower) N
//     S = S Diag(gamma_C) + V^T K^ + N^T A^     (A^ = A e^(g_C - g))
//
// The unit-lower-triangular inverse is plain forward substitution, one column
// per thread ("DeltaNet" notes, section 4.2, solved column by column).  The
// dk-wide per-chunk operands live in a per-workgroup slice of the workspace;
// the C x C matrices, the state tile and the value tiles live in LDS.
// Padding rows of a partial chunk use q = k = v = a = b = 0, beta = 0 and
// log alpha = 0, which makes them identity steps.
#include "gdr_common.h"

namespace gdr {
namespace {

constexpr int kThreads = 256;
constexpr int kDVT = 32;       // dv columns per workgroup
constexpr int kMaxDK = 128;
constexpr int kScratchArrays = 7;

struct GenericParams {
    const void *q, *k, *v, *a, *b;
    const float *la, *beta, *S0;
    void *O;
    float *Sf;
    const int32_t *cu;
    float *scratch;
    int *err;
    long total;
    int n_seq, H, T, dk, dv, n_tiles, gate;
};

template <typename Tin, int C, bool DPLR>
__global__ __launch_bounds__(kThreads) void generic_kernel(GenericParams p) {
    constexpr int CP = C + 1;
    __shared__ float sG[C][CP];    // L (KDA) or B<- A->^T strictly lower (DPLR)
    __shared__ float sInv[C][CP];  // (I + sG)^-1
    __shared__ float sAqk[C][CP];  // Q<- K->^T, lower incl. diagonal
    __shared__ float sGbk[DPLR ? C : 1][CP];
    __shared__ float sAqa[DPLR ? C : 1][CP];
    __shared__ float sS[kDVT][kMaxDK];   // state tile S[dv][dk]
    __shared__ float sVb[C][kDVT];       // Diag(beta) V
    __shared__ float sU[C][kDVT];        // U (KDA) or Cm (DPLR)
    __shared__ float sN[C][kDVT];        // V_new (KDA) or N (DPLR)
    __shared__ float sBeta[C];
    __shared__ float sGC[kMaxDK];        // gamma_C = exp(g_C)

    const Tin *q = (const Tin *)p.q, *k = (const Tin *)p.k, *v = (const Tin *)p.v;
    const Tin *a = (const Tin *)p.a, *b = (const Tin *)p.b;
    Tin *O = (Tin *)p.O;
    const int tid = threadIdx.x;
    const int dk = p.dk, dv = p.dv, H = p.H;
    const int lin = xcd_linear_index(blockIdx.x, gridDim.x);
    const int tile = lin % p.n_tiles;
    const int h = (lin / p.n_tiles) % H;
    const int n = lin / (p.n_tiles * H);
    const int j0 = tile * kDVT;
    long t0, t1;
    seq_bounds(p.cu, n, p.T, p.total, t0, t1, p.err);

    float *base = p.scratch + (size_t)blockIdx.x * kScratchArrays * C * dk;
    float *Ql = base, *Kl = base + C * dk, *Kr = base + 2 * C * dk, *Kh = base + 3 * C * dk;
    float *W = base + 4 * C * dk, *Ar = base + 5 * C * dk, *Ah = base + 6 * C * dk;
    float *Bl = Kl;  // DPLR never needs K<-

    for (int idx = tid; idx < kDVT * dk; idx += kThreads) {
        const int j = idx / dk, d = idx % dk;
        sS[j][d] = p.S0 ? p.S0[(((size_t)n * H + h) * dv + j0 + j) * dk + d] : 0.f;
    }

    for (long c0 = t0; c0 < t1; c0 += C) {
        const int m = (int)((t1 - c0) < C ? (t1 - c0) : C);
        __syncthreads();
        // ---- gate prefix sums and scaled operands ------------------------
        for (int r = tid; r < C; r += kThreads)
            sBeta[r] = r < m ? p.beta[(size_t)(c0 + r) * H + h] : 0.f;
        for (int d = tid; d < dk; d += kThreads) {
            float g = 0.f;
            for (int r = 0; r < C; ++r) {
                const size_t tok = (size_t)(c0 + r) * H + h;
                if (r < m) {
                    if (p.gate == kGateChannel) g += p.la[tok * dk + d];
                    else if (p.gate == kGateHead) g += p.la[tok];
                }
                const float e = expf(g), ei = expf(-g);
                const float qv = r < m ? ld(q, tok * dk + d) : 0.f;
                const float kv = r < m ? ld(k, tok * dk + d) : 0.f;
                Ql[r * dk + d] = qv * e;
                if (!DPLR) Kl[r * dk + d] = kv * e;
                Kr[r * dk + d] = kv * ei;
                W[r * dk + d] = g;  // g_r, kept until W is formed
                if (DPLR) {
                    const float av = r < m ? ld(a, tok * dk + d) : 0.f;
                    const float bv = r < m ? ld(b, tok * dk + d) : 0.f;
                    Ar[r * dk + d] = av * ei;
                    Bl[r * dk + d] = bv * e;
                }
            }
            sGC[d] = expf(g);
            for (int r = 0; r < C; ++r) {
                const size_t tok = (size_t)(c0 + r) * H + h;
                const float dec = expf(g - W[r * dk + d]);
                const float kv = r < m ? ld(k, tok * dk + d) : 0.f;
                Kh[r * dk + d] = kv * dec;
                if (DPLR) {
                    const float av = r < m ? ld(a, tok * dk + d) : 0.f;
                    Ah[r * dk + d] = av * dec;
                }
            }
        }
        for (int idx = tid; idx < C * kDVT; idx += kThreads) {
            const int r = idx / kDVT, j = idx % kDVT;
            const float bet = r < m ? p.beta[(size_t)(c0 + r) * H + h] : 0.f;
            sVb[r][j] = r < m ? bet * ld(v, ((size_t)(c0 + r) * H + h) * dv + j0 + j) : 0.f;
        }
        __syncthreads();
        // ---- C x C products ----------------------------------------------
        for (int idx = tid; idx < C * C; idx += kThreads) {
            const int r = idx / C, i = idx % C;
            float g1 = 0.f, aqk = 0.f, gbk = 0.f, aqa = 0.f;
            if (i <= r) {
                for (int d = 0; d < dk; ++d) {
                    const float krd = Kr[i * dk + d];
                    aqk += Ql[r * dk + d] * krd;
                    if (DPLR) {
                        const float ard = Ar[i * dk + d];
                        aqa += Ql[r * dk + d] * ard;
                        if (i < r) {
                            g1 += Bl[r * dk + d] * ard;
                            gbk += Bl[r * dk + d] * krd;
                        }
                    } else if (i < r) {
                        g1 += Kl[r * dk + d] * krd;
                    }
                }
            }
            sG[r][i] = (i < r) ? (DPLR ? g1 : sBeta[r] * g1) : 0.f;
            sAqk[r][i] = aqk;
            if (DPLR) {
                sGbk[r][i] = (i < r) ? gbk : 0.f;
                sAqa[r][i] = aqa;
            }
        }
        __syncthreads();
        // ---- unit-lower-triangular inverse, one column per thread ---------
        for (int c = tid; c < C; c += kThreads) {
            for (int r = 0; r < C; ++r) {
                float x;
                if (r < c) x = 0.f;
                else if (r == c) x = 1.f;
                else {
                    float s = 0.f;
                    for (int i = c; i < r; ++i) s += sG[r][i] * sInv[i][c];
                    x = -s;
                }
                sInv[r][c] = x;
            }
        }
        __syncthreads();
        // ---- WY factors ----------------------------------------------------
        for (int idx = tid; idx < C * dk; idx += kThreads) {
            const int r = idx / dk, d = idx % dk;
            float s = 0.f;
            for (int i = 0; i <= r; ++i)
                s += sInv[r][i] * (DPLR ? Bl[i * dk + d] : sBeta[i] * Kl[i * dk + d]);
            W[r * dk + d] = s;
        }
        if (DPLR) {
            for (int idx = tid; idx < C * kDVT; idx += kThreads) {
                const int r = idx / kDVT, j = idx % kDVT;
                float s = 0.f;
                for (int l = 0; l < r; ++l) s += sGbk[r][l] * sVb[l][j];
                sN[r][j] = s;
            }
            __syncthreads();
        }
        for (int idx = tid; idx < C * kDVT; idx += kThreads) {
            const int r = idx / kDVT, j = idx % kDVT;
            float s = 0.f;
            for (int i = 0; i <= r; ++i) s += sInv[r][i] * (DPLR ? sN[i][j] : sVb[i][j]);
            sU[r][j] = DPLR ? -s : s;
        }
        __syncthreads();
        // ---- serial part: state-dependent values, output, state -----------
        for (int idx = tid; idx < C * kDVT; idx += kThreads) {
            const int r = idx / kDVT, j = idx % kDVT;
            float s = 0.f;
            for (int d = 0; d < dk; ++d) s += W[r * dk + d] * sS[j][d];
            sN[r][j] = sU[r][j] - s;
        }
        __syncthreads();
        for (int idx = tid; idx < C * kDVT; idx += kThreads) {
            const int r = idx / kDVT, j = idx % kDVT;
            if (r >= m) continue;
            float s = 0.f;
            for (int d = 0; d < dk; ++d) s += Ql[r * dk + d] * sS[j][d];
            for (int i = 0; i <= r; ++i) {
                s += sAqk[r][i] * (DPLR ? sVb[i][j] : sN[i][j]);
                if (DPLR) s += sAqa[r][i] * sN[i][j];
            }
            st(O, ((size_t)(c0 + r) * H + h) * dv + j0 + j, s);
        }
        __syncthreads();
        for (int idx = tid; idx < kDVT * dk; idx += kThreads) {
            const int j = idx / dk, d = idx % dk;
            float s = sS[j][d] * sGC[d];
            for (int r = 0; r < C; ++r) {
                s += sN[r][j] * (DPLR ? Ah[r * dk + d] : Kh[r * dk + d]);
                if (DPLR) s += sVb[r][j] * Kh[r * dk + d];
            }
            sS[j][d] = s;
        }
    }
    __syncthreads();
    if (p.Sf) {
        for (int idx = tid; idx < kDVT * dk; idx += kThreads) {
            const int j = idx / dk, d = idx % dk;
            p.Sf[(((size_t)n * H + h) * dv + j0 + j) * dk + d] = sS[j][d];
        }
    }
}

template <typename Tin, int C>
int launch_c(const GenericParams &gp, int grid, hipStream_t s, bool dplr) {
    if (dplr)
        hipLaunchKernelGGL((generic_kernel<Tin, C, true>), dim3(grid), dim3(kThreads), 0, s, gp);
    else
        hipLaunchKernelGGL((generic_kernel<Tin, C, false>), dim3(grid), dim3(kThreads), 0, s, gp);
    return (int)hipGetLastError();
}

}  // namespace

size_t generic_workspace_bytes(const FwdArgs &a, int n_seq_eff) {
    const size_t grid = (size_t)n_seq_eff * a.H * (a.dv / kDVT);
    return kWorkspaceHeader + grid * kScratchArrays * (size_t)a.C * a.dk * sizeof(float);
}

int launch_generic(const FwdArgs &a, int n_seq_eff, hipStream_t s) {
    GenericParams gp;
    gp.q = a.q; gp.k = a.k; gp.v = a.v; gp.a = a.a; gp.b = a.b;
    gp.la = a.log_alpha; gp.beta = a.beta; gp.S0 = a.S0;
    gp.O = a.O; gp.Sf = a.S_final; gp.cu = a.cu_seqlens;
    gp.err = (int *)a.workspace;
    gp.scratch = (float *)((char *)a.workspace + kWorkspaceHeader);
    gp.total = (long)a.B * a.T;
    gp.n_seq = n_seq_eff; gp.H = a.H; gp.T = a.T; gp.dk = a.dk; gp.dv = a.dv;
    gp.n_tiles = a.dv / kDVT; gp.gate = a.gate;
    const int grid = n_seq_eff * a.H * gp.n_tiles;
    const bool dplr = a.a != nullptr;
    if (a.dtype == 0) {
        if (a.C == 16) return launch_c<float, 16>(gp, grid, s, dplr);
        if (a.C == 32) return launch_c<float, 32>(gp, grid, s, dplr);
        if (a.C == 64) return launch_c<float, 64>(gp, grid, s, dplr);
    } else {
        if (a.C == 16) return launch_c<bf16, 16>(gp, grid, s, dplr);
        if (a.C == 32) return launch_c<bf16, 32>(gp, grid, s, dplr);
        if (a.C == 64) return launch_c<bf16, 64>(gp, grid, s, dplr);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace gdr
