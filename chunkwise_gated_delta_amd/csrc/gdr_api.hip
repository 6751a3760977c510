// Host side of libgdr: argument validation, workspace sizing and kernel choice
// behind the C ABI declared in include/gdr.h.
#include "../../include/gdr.h"
#include "gdr_common.h"

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace {

using gdr::FwdArgs;

bool trace_enabled() {
    static const int on = [] {
        const char *s = std::getenv("GDR_TRACE");
        return (s && s[0] == '1') ? 1 : 0;
    }();
    return on != 0;
}

size_t elem_size(int dtype) { return dtype == GDR_F32 ? 4 : 2; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range(const void *p, size_t bytes) {
    const uintptr_t a = (uintptr_t)p;
    return Range{a, a + bytes};
}

bool overlaps(Range a, Range b) { return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi; }

// Every tensor and the workspace must start on a 16-byte boundary: the kernels move
// them with 16-byte vector loads and stores.  NULL pointers pass.
bool aligned16(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (((uintptr_t)p & 15u) != 0) return false;
    return true;
}

bool shape_ok(int B, int H, int T, int dk, int dv, int n_seq, bool varlen) {
    if (B < 1 || H < 1 || T < 1 || dk < 1 || dv < 1) return false;
    if (varlen && (B != 1 || n_seq < 1)) return false;
    // elements per tensor below 2^40 (the product of four ints needs more than 64 bits)
    const __int128 elems = (__int128)B * T * H * (dk > dv ? dk : dv);
    if (elems >= ((__int128)1 << 40)) return false;
    // (sequence, head) chains below 2^27: the serial kernels number their workgroups
    // (chains x tiles x runs) in 32 bits
    return (long long)(varlen ? n_seq : B) * H < (1LL << 27);
}

int supported(int dtype, int dk, int dv, int C, bool has_ab) {
    if (dtype != GDR_F32 && dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
    if (dk != 64 && dk != 128) return GDR_ERR_UNSUPPORTED;
    if (dv % 32 != 0 || dv > 256) return GDR_ERR_UNSUPPORTED;
    if (dtype == GDR_BF16 && !has_ab)
        return (C == 64 || (C == 128 && dk == 128)) ? GDR_OK : GDR_ERR_UNSUPPORTED;
    return (C == 16 || C == 32 || C == 64) ? GDR_OK : GDR_ERR_UNSUPPORTED;
}

// The gate argument: a layout (GDR_GATE_NONE/HEAD/CHANNEL), optionally with GDR_GATE_CLIP.
bool gate_ok(int gate) {
    const int layout = gate & ~GDR_GATE_CLIP;
    return layout >= GDR_GATE_NONE && layout <= GDR_GATE_CHANNEL;
}

FwdArgs make_args(int B, int H, int T, int dk, int dv, int C, int n_seq, int dtype, int gate,
                  bool has_ab) {
    FwdArgs a;
    std::memset(&a, 0, sizeof(a));
    a.B = B; a.H = H; a.T = T; a.dk = dk; a.dv = dv; a.C = C; a.n_seq = n_seq;
    a.dtype = dtype; a.gate = gate & ~GDR_GATE_CLIP; a.clip = (gate & GDR_GATE_CLIP) != 0;
    static const char dummy = 0;
    static const int32_t dummy_cu = 0;
    if (has_ab) a.a = a.b = &dummy;
    if (n_seq > 0) a.cu_seqlens = &dummy_cu;  // marks packed sequences for the size query
    return a;
}

size_t workspace_for(const FwdArgs &a, int n_seq_eff) {
    if (gdr::kda_split_supported(a)) return gdr::kda_split_workspace_bytes(a, n_seq_eff);
    if (gdr::f32_split_supported(a)) return gdr::f32_split_workspace_bytes(a, n_seq_eff);
    return 0;
}

}  // namespace

// Scratch of gdr_chunk_fwd_noalloc: the forward's workspace in a fixed device array,
// one per GPU (each device that loads the library holds its own copy until the process
// ends).  Host code never uses the array's name as an address: the device address of
// the current device's copy comes from hipGetSymbolAddress, once per device, and is
// kept in scratch_ptr.
constexpr size_t kScratchBytes = (size_t)GDR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (NULL on failure).
void *scratch_of_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}
}  // namespace

extern "C" {

size_t gdr_chunk_fwd_workspace(int B, int H, int T, int dk, int dv, int C, int n_seq, int dtype,
                               int gate, int has_ab) {
    const bool varlen = n_seq > 0;
    if (!shape_ok(B, H, T, dk, dv, n_seq, varlen)) return 0;
    if (!gate_ok(gate)) return 0;
    if (supported(dtype, dk, dv, C, has_ab != 0) != GDR_OK) return 0;
    const FwdArgs a = make_args(B, H, T, dk, dv, C, n_seq, dtype, gate, has_ab != 0);
    return workspace_for(a, varlen ? n_seq : B);
}

namespace {
int chunk_fwd(const void *q, const void *k, const void *v, const void *a, const void *b,
              const float *log_alpha, const float *beta, const float *S0, void *O, float *S_final,
              const int32_t *cu_seqlens, int n_seq, int B, int H, int T, int dk, int dv, int C,
              int dtype, int gate, void *workspace, size_t workspace_bytes, void *stream, bool keep,
              int *err_word = nullptr, bool use_scratch = false) {
    if (!q || !k || !v || !beta || !O) return GDR_ERR_NULL;
    if ((a == nullptr) != (b == nullptr)) return GDR_ERR_NULL;
    if (!gate_ok(gate)) return GDR_ERR_SHAPE;
    const int layout = gate & ~GDR_GATE_CLIP;
    if ((layout == GDR_GATE_NONE) != (log_alpha == nullptr)) return GDR_ERR_NULL;
    const bool varlen = cu_seqlens != nullptr;
    if (!shape_ok(B, H, T, dk, dv, n_seq, varlen)) return GDR_ERR_SHAPE;
    const bool has_ab = a != nullptr;
    const int sup = supported(dtype, dk, dv, C, has_ab);
    if (sup != GDR_OK) return sup;
    if (!aligned16({q, k, v, a, b, log_alpha, beta, S0, O, S_final, cu_seqlens, workspace}) ||
        ((uintptr_t)err_word & 3u) != 0)
        return GDR_ERR_ALIGN;
    const int N = varlen ? n_seq : B;

    // Bytes of every tensor, for the alias check.
    const size_t tokens = (size_t)B * T, es = elem_size(dtype);
    const Range rq = range(q, tokens * H * dk * es), rk = range(k, tokens * H * dk * es);
    const Range rv = range(v, tokens * H * dv * es);
    const Range ra = range(a, has_ab ? tokens * H * dk * es : 0);
    const Range rb = range(b, has_ab ? tokens * H * dk * es : 0);
    const size_t la_elems =
        layout == GDR_GATE_CHANNEL ? tokens * H * dk : (layout == GDR_GATE_HEAD ? tokens * H : 0);
    const Range rla = range(log_alpha, la_elems * 4), rbeta = range(beta, tokens * H * 4);
    const size_t sbytes = (size_t)N * H * dv * dk * 4;
    const Range rs0 = range(S0, S0 ? sbytes : 0), rO = range(O, tokens * H * dv * es);
    const Range rsf = range(S_final, S_final ? sbytes : 0);
    const Range rcu = range(cu_seqlens, varlen ? (size_t)(n_seq + 1) * 4 : 0);
    const Range inputs[] = {rq, rk, rv, ra, rb, rla, rbeta, rs0, rcu};
    for (const Range &r : inputs)
        if (overlaps(rO, r)) return GDR_ERR_ALIAS;
    for (const Range &r : inputs) {
        if (&r == &inputs[7]) continue;  // S_final may be S0 exactly ...
        if (overlaps(rsf, r)) return GDR_ERR_ALIAS;
    }
    if (overlaps(rsf, rO)) return GDR_ERR_ALIAS;
    if (S0 && S_final && overlaps(rsf, rs0) && (const void *)S_final != (const void *)S0)
        return GDR_ERR_ALIAS;  // ... but not partly overlap it

    FwdArgs args = make_args(B, H, T, dk, dv, C, varlen ? n_seq : 0, dtype, gate, has_ab);
    args.q = q; args.k = k; args.v = v; args.a = a; args.b = b;
    args.log_alpha = log_alpha; args.beta = beta; args.S0 = S0;
    args.O = O; args.S_final = S_final; args.cu_seqlens = cu_seqlens;
    args.workspace = workspace; args.workspace_bytes = workspace_bytes;
    args.err = err_word;
    size_t need = workspace_for(args, N);
    if (keep) {
        // the states go where gdr_chunk_bwd reads them: its workspace layout and limits
        const gdr::BwdArgs bv = gdr::bwd_view(args);
        if (args.clip || !gdr::kda_bwd_supported(bv)) return GDR_ERR_UNSUPPORTED;
        args.keep_states = true;
        need = std::max(need, gdr::kda_bwd_workspace_bytes(bv, N));
    }
    if (use_scratch) {
        // the fixed per-GPU array stands in for the workspace (set up on first use)
        if (need > kScratchBytes) return GDR_ERR_WORKSPACE;
        workspace = scratch_of_current_device();
        if (workspace == nullptr) return GDR_ERR_HIP;
        workspace_bytes = kScratchBytes;
        args.workspace = workspace; args.workspace_bytes = workspace_bytes;
    }
    if (!workspace || workspace_bytes < need) return GDR_ERR_WORKSPACE;
    const Range rws = range(workspace, need);
    for (const Range &r : inputs)
        if (overlaps(rws, r)) return GDR_ERR_ALIAS;
    if (overlaps(rws, rO) || overlaps(rws, rsf)) return GDR_ERR_ALIAS;
    if (err_word) {
        const Range rerr = range(err_word, sizeof(int));
        for (const Range &r : inputs)
            if (overlaps(rerr, r)) return GDR_ERR_ALIAS;
        if (overlaps(rerr, rO) || overlaps(rerr, rsf) || overlaps(rerr, rws)) return GDR_ERR_ALIAS;
    }

    hipStream_t s = (hipStream_t)stream;
    const bool split = gdr::kda_split_supported(args);
    if (trace_enabled())
        std::fprintf(stderr, "[gdr] %s B=%d H=%d T=%d N=%d dk=%d dv=%d C=%d dtype=%d gate=%d clip=%d ws=%zu\n",
                     split ? "kda_split" : "f32_split", B, H, T, N, dk, dv, C, dtype, layout,
                     (int)args.clip, need);
    if (!split && !gdr::f32_split_supported(args)) return GDR_ERR_UNSUPPORTED;
    const int rc = split ? gdr::launch_kda_split(args, N, s) : gdr::launch_f32_split(args, N, s);
    return rc == 0 ? GDR_OK : GDR_ERR_HIP;
}
}  // namespace

int gdr_chunk_fwd(const void *q, const void *k, const void *v, const void *a, const void *b,
                  const float *log_alpha, const float *beta, const float *S0, void *O,
                  float *S_final, const int32_t *cu_seqlens, int n_seq, int B, int H, int T,
                  int dk, int dv, int C, int dtype, int gate, void *workspace,
                  size_t workspace_bytes, void *stream) {
    return chunk_fwd(q, k, v, a, b, log_alpha, beta, S0, O, S_final, cu_seqlens, n_seq, B, H, T,
                     dk, dv, C, dtype, gate, workspace, workspace_bytes, stream, false);
}

int gdr_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *a,
                          const void *b, const float *log_alpha, const float *beta,
                          const float *S0, void *O, float *S_final, const int32_t *cu_seqlens,
                          int n_seq, int B, int H, int T, int dk, int dv, int C, int dtype,
                          int gate, int *flags, void *stream) {
    return chunk_fwd(q, k, v, a, b, log_alpha, beta, S0, O, S_final, cu_seqlens, n_seq, B, H, T,
                     dk, dv, C, dtype, gate, nullptr, 0, stream, false, flags, true);
}

int gdr_chunk_fwd_for_bwd(const void *q, const void *k, const void *v, const void *a,
                          const void *b, const float *log_alpha, const float *beta,
                          const float *S0, void *O, float *S_final, const int32_t *cu_seqlens,
                          int n_seq, int B, int H, int T, int dk, int dv, int C, int dtype,
                          int gate, void *workspace, size_t workspace_bytes, void *stream) {
    return chunk_fwd(q, k, v, a, b, log_alpha, beta, S0, O, S_final, cu_seqlens, n_seq, B, H, T,
                     dk, dv, C, dtype, gate, workspace, workspace_bytes, stream, true);
}

size_t gdr_chunk_bwd_workspace(int B, int H, int T, int dk, int dv, int C, int n_seq, int dtype,
                               int gate, int has_ab) {
    const bool varlen = n_seq > 0;
    if (!shape_ok(B, H, T, dk, dv, n_seq, varlen)) return 0;
    gdr::BwdArgs a;
    std::memset(&a, 0, sizeof(a));
    a.B = B; a.H = H; a.T = T; a.dk = dk; a.dv = dv; a.C = C; a.n_seq = n_seq;
    a.dtype = dtype; a.gate = gate;
    static const int32_t dummy_cu = 0;
    static const char dummy = 0;
    if (varlen) a.cu_seqlens = &dummy_cu;
    if (has_ab) a.a = a.b = &dummy;
    if (!gdr::kda_bwd_supported(a)) return 0;
    return gdr::kda_bwd_workspace_bytes(a, varlen ? n_seq : B);
}

int gdr_chunk_bwd(const void *q, const void *k, const void *v, const void *a_, const void *b_,
                  const float *log_alpha, const float *beta, const float *S0, const void *dO,
                  const float *dS_final, void *dq, void *dk, void *dv, void *da, void *db,
                  float *dlog_alpha, float *dbeta, float *dS0, const int32_t *cu_seqlens,
                  int n_seq, int B, int H, int T, int dk_, int dv_, int C, int dtype, int gate,
                  int flags, void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !k || !v || !beta || !dO || !dq || !dk || !dv || !dbeta) return GDR_ERR_NULL;
    if (flags & ~(GDR_BWD_FORWARD_WORKSPACE | GDR_BWD_FORWARD_STATES)) return GDR_ERR_SHAPE;
    const bool has_ab = a_ != nullptr;
    if ((a_ == nullptr) != (b_ == nullptr)) return GDR_ERR_NULL;
    if ((da == nullptr) != !has_ab || (db == nullptr) != !has_ab) return GDR_ERR_NULL;
    if (!gate_ok(gate)) return GDR_ERR_SHAPE;
    if (gate & GDR_GATE_CLIP) return GDR_ERR_UNSUPPORTED;
    if ((gate == GDR_GATE_NONE) != (log_alpha == nullptr)) return GDR_ERR_NULL;
    if ((gate == GDR_GATE_NONE) != (dlog_alpha == nullptr)) return GDR_ERR_NULL;
    const bool varlen = cu_seqlens != nullptr;
    if (!shape_ok(B, H, T, dk_, dv_, n_seq, varlen)) return GDR_ERR_SHAPE;
    gdr::BwdArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q; a.k = k; a.v = v; a.a = a_; a.b = b_; a.dO = dO; a.log_alpha = log_alpha;
    a.beta = beta; a.S0 = S0; a.dS_final = dS_final;
    a.grad_q = dq; a.grad_k = dk; a.grad_v = dv; a.grad_a = da; a.grad_b = db;
    a.grad_la = dlog_alpha; a.grad_beta = dbeta; a.grad_S0 = dS0; a.cu_seqlens = cu_seqlens;
    a.n_seq = varlen ? n_seq : 0;
    a.B = B; a.H = H; a.T = T; a.dk = dk_; a.dv = dv_; a.C = C; a.dtype = dtype; a.gate = gate;
    a.reuse_states = (flags & GDR_BWD_FORWARD_STATES) != 0;
    a.reuse_fwd = a.reuse_states || (flags & GDR_BWD_FORWARD_WORKSPACE) != 0;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    if (!gdr::kda_bwd_supported(a)) return GDR_ERR_UNSUPPORTED;
    if (!aligned16({q, k, v, a_, b_, log_alpha, beta, S0, dO, dS_final, dq, dk, dv, da, db,
                    dlog_alpha, dbeta, dS0, cu_seqlens, workspace}))
        return GDR_ERR_ALIGN;
    const int N = varlen ? n_seq : B;

    const size_t tokens = (size_t)B * T, es = elem_size(dtype);
    const size_t la_elems = gate == GDR_GATE_CHANNEL ? tokens * H * dk_ : (gate == GDR_GATE_HEAD ? tokens * H : 0);
    const size_t sbytes = (size_t)N * H * dv_ * dk_ * 4;
    const size_t kbytes = tokens * H * dk_ * es, vbytes = tokens * H * dv_ * es;
    const Range inputs[] = {range(q, kbytes), range(k, kbytes), range(v, vbytes),
                            range(a_, has_ab ? kbytes : 0), range(b_, has_ab ? kbytes : 0),
                            range(log_alpha, la_elems * 4), range(beta, tokens * H * 4),
                            range(S0, S0 ? sbytes : 0), range(dO, vbytes),
                            range(dS_final, dS_final ? sbytes : 0),
                            range(cu_seqlens, varlen ? (size_t)(n_seq + 1) * 4 : 0)};
    const Range outputs[] = {range(dq, kbytes), range(dk, kbytes), range(dv, vbytes),
                             range(da, has_ab ? kbytes : 0), range(db, has_ab ? kbytes : 0),
                             range(dlog_alpha, la_elems * 4), range(dbeta, tokens * H * 4),
                             range(dS0, dS0 ? sbytes : 0)};
    constexpr int kOut = sizeof(outputs) / sizeof(outputs[0]);
    const size_t need = gdr::kda_bwd_workspace_bytes(a, N);
    if (!workspace || workspace_bytes < need) return GDR_ERR_WORKSPACE;
    const Range rws = range(workspace, need);
    for (int i = 0; i < kOut; ++i) {
        for (const Range &r : inputs)
            if (overlaps(outputs[i], r)) return GDR_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (overlaps(outputs[i], outputs[j])) return GDR_ERR_ALIAS;
        if (overlaps(outputs[i], rws)) return GDR_ERR_ALIAS;
    }
    for (const Range &r : inputs)
        if (overlaps(rws, r)) return GDR_ERR_ALIAS;
    if (trace_enabled())
        std::fprintf(stderr, "[gdr] %s B=%d H=%d T=%d N=%d dk=%d dv=%d gate=%d ws=%zu\n",
                     has_ab ? "dplr_bwd" : "kda_bwd", B, H, T, N, dk_, dv_, gate, need);
    const int rc = gdr::launch_kda_bwd(a, N, (hipStream_t)stream);
    return rc == 0 ? GDR_OK : GDR_ERR_HIP;
}

int gdr_workspace_error(void *workspace, void *stream) {
    if (!workspace) return GDR_ERR_NULL;
    hipStream_t s = (hipStream_t)stream;
    if (hipStreamSynchronize(s) != hipSuccess) return GDR_ERR_HIP;
    int flag = 0;
    if (hipMemcpy(&flag, workspace, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return GDR_ERR_HIP;
    if (flag != 0) {
        const int zero = 0;
        if (hipMemcpy(workspace, &zero, sizeof(int), hipMemcpyHostToDevice) != hipSuccess)
            return GDR_ERR_HIP;
    }
    return flag;
}

const char *gdr_status_string(int status) {
    switch (status) {
        case GDR_OK: return "ok";
        case GDR_ERR_NULL: return "required pointer is NULL (or only one of a, b given)";
        case GDR_ERR_SHAPE: return "size out of range or inconsistent";
        case GDR_ERR_UNSUPPORTED: return "unsupported dtype, head size or chunk size";
        case GDR_ERR_WORKSPACE: return "workspace missing or too small";
        case GDR_ERR_ALIAS: return "output overlaps an input or the workspace";
        case GDR_ERR_HIP: return "HIP launch failed";
        case GDR_ERR_ALIGN: return "a tensor or the workspace is not 16-byte aligned";
        default: return "unknown status";
    }
}

int gdr_version(void) { return 100; }

}  // extern "C"
