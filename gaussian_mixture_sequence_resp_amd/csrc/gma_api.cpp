// Host side of libgma.so: argument validation, workspace sizing and dispatch.
// Every check runs before the first HIP call, so an invalid call enqueues nothing.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "gma_internal.h"

namespace {

using gma::Args;

int check_desc(const gma_desc* d) {
    if (!d) return GMA_ERR_NULL_ARG;
    if (d->B < 0 || d->H < 0 || d->N < 0 || d->d_r < 1 || d->d_v < 1 || d->K < 1) return GMA_ERR_BAD_SHAPE;
    if (d->dtype != GMA_F32 && d->dtype != GMA_BF16) return GMA_ERR_UNSUPPORTED;
    if (d->algo != GMA_ALGO_AUTO && d->algo != GMA_ALGO_SIMT && d->algo != GMA_ALGO_MFMA) return GMA_ERR_UNSUPPORTED;
    if (d->K > GMA_MAX_K || d->d_r > GMA_MAX_DR || d->d_v > GMA_MAX_DV) return GMA_ERR_UNSUPPORTED;
    // element counts: B*H*N rows must index with int32, tensors with int64
    const int64_t rows = (int64_t)d->B * d->H * d->N;
    if ((int64_t)d->B * d->H > INT32_MAX || rows > INT32_MAX) return GMA_ERR_BAD_SHAPE;
    if (d->algo == GMA_ALGO_MFMA && d->dtype != GMA_BF16) return GMA_ERR_UNSUPPORTED;
    if (!(d->var_floor >= 0.0f) || !isfinite(d->var_floor)) return GMA_ERR_BAD_SCALAR;
    return GMA_OK;
}

// Resolve AUTO: the MFMA family for bf16 shapes it covers, SIMT otherwise.
int resolve_algo(const gma_desc& d, int causal) {
    if (d.algo == GMA_ALGO_SIMT) return GMA_ALGO_SIMT;
    if (d.algo == GMA_ALGO_MFMA) return gma::mfma_supported(d, causal) ? GMA_ALGO_MFMA : -1;
    return (d.dtype == GMA_BF16 && gma::mfma_supported(d, causal)) ? GMA_ALGO_MFMA : GMA_ALGO_SIMT;
}

size_t workspace_for(const gma_desc& d, int causal, int Nk) {
    const int algo = resolve_algo(d, causal);
    if (algo == GMA_ALGO_MFMA) return gma::mfma_workspace(d, causal, Nk);
    if (algo == GMA_ALGO_SIMT) return gma::simt_workspace(d, causal, Nk);
    return 0;
}

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// The key length of a call: N for self-mixing, n_k for the cross variant (-1 = invalid).
int key_rows(const gma_desc& d, int64_t n_k) {
    if (n_k < 0 || (int64_t)d.B * d.H * n_k > INT32_MAX) return -1;
    return (int)n_k;
}

size_t workspace_common(const gma_desc* desc, int causal, int64_t n_k) {
    if (check_desc(desc) != GMA_OK || (causal != 0 && causal != 1)) return 0;
    if ((int64_t)desc->B * desc->H * desc->N == 0) return 0;
    const int Nk = key_rows(*desc, n_k);
    if (Nk < 0) return 0;
    return workspace_for(*desc, causal, Nk);
}

}  // namespace

extern "C" {

size_t gma_workspace_size(const gma_desc* desc, int causal) {
    return workspace_common(desc, causal, desc ? desc->N : 0);
}

size_t gma_workspace_size_cross(const gma_desc* desc, int32_t n_k) { return workspace_common(desc, 0, n_k); }

static int forward_impl(const void* qr, const void* kr, const void* v, const float* mu, const float* var_raw,
                        const float* prior_logits, int causal, int64_t n_k, float eps, void* out,
                        float* gamma_out, const gma_desc* desc, void* workspace, size_t workspace_bytes,
                        void* stream, gma::Recorder* rec, const gma::ScratchSource* scratch = nullptr) {
    int st = check_desc(desc);
    if (st != GMA_OK) return st;
    const gma_desc d = *desc;
    if (causal != 0 && causal != 1) return GMA_ERR_BAD_SCALAR;
    if (!(eps >= 0.0f) || !isfinite(eps)) return GMA_ERR_BAD_SCALAR;
    const int Nk = key_rows(d, n_k);
    if (Nk < 0) return GMA_ERR_BAD_SHAPE;
    const size_t rows = (size_t)d.B * d.H * d.N;      // query and output rows
    const size_t krows = (size_t)d.B * d.H * Nk;      // key and value rows
    if (rows == 0) return GMA_OK;  // empty sequence or batch: nothing to compute
    if (!qr || !mu || !var_raw || !prior_logits || !out) return GMA_ERR_NULL_ARG;
    if (Nk > 0 && (!kr || !v)) return GMA_ERR_NULL_ARG;  // no key rows: kr and v are not read
    const size_t esz = d.dtype == GMA_F32 ? 4 : 2;
    const size_t nq = rows * d.d_r * esz, nk = krows * d.d_r * esz, nv = krows * d.d_v * esz;
    const size_t no = rows * d.d_v * esz;
    const size_t np = (size_t)d.H * d.K * d.d_r * 4, npr = (size_t)d.H * d.K * 4;
    const size_t ng = (rows + krows) * d.K * 4;
    if (misaligned(qr, 16) || misaligned(kr, 16) || misaligned(v, 16) || misaligned(out, 16))
        return GMA_ERR_ALIGN;
    if (misaligned(mu, 4) || misaligned(var_raw, 4) || misaligned(prior_logits, 4) ||
        (gamma_out && misaligned(gamma_out, 4)))
        return GMA_ERR_ALIGN;
    if (workspace && misaligned(workspace, gma::kWsAlign)) return GMA_ERR_ALIGN;
    const void* ins[6] = {qr, kr, v, mu, var_raw, prior_logits};
    const size_t ins_n[6] = {nq, nk, nv, np, np, npr};
    for (int i = 0; i < 6; ++i) {
        if (overlaps(out, no, ins[i], ins_n[i])) return GMA_ERR_ALIAS;
        if (gamma_out && overlaps(gamma_out, ng, ins[i], ins_n[i])) return GMA_ERR_ALIAS;
    }
    if (gamma_out && overlaps(out, no, gamma_out, ng)) return GMA_ERR_ALIAS;
    const int algo = resolve_algo(d, causal);
    if (algo < 0) return GMA_ERR_UNSUPPORTED;
    const size_t need = workspace_for(d, causal, Nk);
    if (scratch) {
        // the library's own scratch: every other check has passed, so this is the first HIP call
        if (need > scratch->capacity) return GMA_ERR_TOO_LARGE;
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0) {
            int sst = GMA_OK;
            workspace = scratch->get(stream, &sst);
            if (!workspace) return sst != GMA_OK ? sst : GMA_ERR_HIP;
            workspace_bytes = scratch->capacity;
        }
    }
    if (need > 0 && (!workspace || workspace_bytes < need)) return GMA_ERR_WORKSPACE;
    if (workspace && (overlaps(workspace, need, out, no) || (gamma_out && overlaps(workspace, need, gamma_out, ng))))
        return GMA_ERR_ALIAS;
    for (int i = 0; i < 6; ++i)
        if (workspace && overlaps(workspace, need, ins[i], ins_n[i])) return GMA_ERR_ALIAS;

    Args a;
    a.qr = qr;
    a.kr = kr;
    a.v = v;
    a.mu = mu;
    a.var_raw = var_raw;
    a.prior = prior_logits;
    a.causal = causal;
    a.eps = eps;
    a.out = out;
    a.gamma_out = gamma_out;
    a.state = nullptr;
    a.d = d;
    a.Nk = Nk;
    a.ws = static_cast<unsigned char*>(workspace);
    a.ws_bytes = workspace_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    a.rec = rec;
    const hipError_t e = (algo == GMA_ALGO_MFMA) ? gma::mfma_forward(a) : gma::simt_forward(a);
    return e == hipSuccess ? GMA_OK : GMA_ERR_HIP;
}

}  // extern "C"

int gma::forward_with_scratch(const void* qr, const void* kr, const void* v, const float* mu, const float* var_raw,
                              const float* prior_logits, int causal, float eps, void* out, float* gamma_out,
                              const gma_desc* desc, void* stream, const ScratchSource& scratch) {
    return forward_impl(qr, kr, v, mu, var_raw, prior_logits, causal, desc ? desc->N : 0, eps, out, gamma_out,
                        desc, nullptr, 0, stream, nullptr, &scratch);
}

extern "C" {

int gma_forward(const void* qr, const void* kr, const void* v, const float* mu, const float* var_raw,
                const float* prior_logits, int causal, float eps, void* out, float* gamma_out,
                const gma_desc* desc, void* workspace, size_t workspace_bytes, void* stream) {
    return forward_impl(qr, kr, v, mu, var_raw, prior_logits, causal, desc ? desc->N : 0, eps, out, gamma_out,
                        desc, workspace, workspace_bytes, stream, nullptr);
}

int gma_forward_cross(const void* qr, const void* kr, const void* v, const float* mu, const float* var_raw,
                      const float* prior_logits, int32_t n_k, float eps, void* out, float* gamma_out,
                      const gma_desc* desc, void* workspace, size_t workspace_bytes, void* stream) {
    return forward_impl(qr, kr, v, mu, var_raw, prior_logits, 0, n_k, eps, out, gamma_out, desc, workspace,
                        workspace_bytes, stream, nullptr);
}

static int timed(const void* qr, const void* kr, const void* v, const float* mu, const float* var_raw,
                 const float* prior_logits, int causal, int64_t n_k, float eps, void* out, float* gamma_out,
                 const gma_desc* desc, void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                 int n_events, const char** names, int* n_kernels) {
    if (n_kernels) *n_kernels = 0;
    if (n_events < 0 || (n_events > 0 && !events)) return GMA_ERR_NULL_ARG;
    gma::Recorder rec{events, n_events, names, 0};
    const int st = forward_impl(qr, kr, v, mu, var_raw, prior_logits, causal, n_k, eps, out, gamma_out, desc,
                                workspace, workspace_bytes, stream, &rec);
    if (n_kernels) *n_kernels = rec.count;
    return st;
}

int gma_forward_timed(const void* qr, const void* kr, const void* v, const float* mu, const float* var_raw,
                      const float* prior_logits, int causal, float eps, void* out, float* gamma_out,
                      const gma_desc* desc, void* workspace, size_t workspace_bytes, void* stream,
                      void* const* events, int n_events, const char** names, int* n_kernels) {
    return timed(qr, kr, v, mu, var_raw, prior_logits, causal, desc ? desc->N : 0, eps, out, gamma_out, desc,
                 workspace, workspace_bytes, stream, events, n_events, names, n_kernels);
}

int gma_forward_cross_timed(const void* qr, const void* kr, const void* v, const float* mu, const float* var_raw,
                            const float* prior_logits, int32_t n_k, float eps, void* out, float* gamma_out,
                            const gma_desc* desc, void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events, int n_events, const char** names, int* n_kernels) {
    return timed(qr, kr, v, mu, var_raw, prior_logits, 0, n_k, eps, out, gamma_out, desc, workspace,
                 workspace_bytes, stream, events, n_events, names, n_kernels);
}

// ---- causal memory (prefill) and single-token decode step

static bool memory_algo_ok(const gma_desc& d) {
    return d.algo != GMA_ALGO_MFMA || (d.dtype == GMA_BF16 && gma::mfma_memory_supported(d));
}

size_t gma_memory_workspace_size(const gma_desc* desc) {
    if (check_desc(desc) != GMA_OK || (int64_t)desc->B * desc->H == 0 || !memory_algo_ok(*desc)) return 0;
    return gma::memory_workspace(*desc);
}

int gma_memory(const void* kr, const void* v, const float* mu, const float* var_raw, const float* prior_logits,
               float* state, const gma_desc* desc, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_desc(desc);
    if (st != GMA_OK) return st;
    const gma_desc d = *desc;
    const size_t bh = (size_t)d.B * d.H;
    if (bh == 0) return GMA_OK;
    if (!mu || !var_raw || !prior_logits || !state) return GMA_ERR_NULL_ARG;
    if (d.N > 0 && (!kr || !v)) return GMA_ERR_NULL_ARG;  // no positions: kr and v are not read
    const size_t esz = d.dtype == GMA_F32 ? 4 : 2;
    const size_t nk = bh * d.N * d.d_r * esz, nv = bh * d.N * d.d_v * esz;
    const size_t np = (size_t)d.H * d.K * d.d_r * 4, npr = (size_t)d.H * d.K * 4;
    const size_t ns = bh * d.K * (d.d_v + 1) * 4;
    if (misaligned(kr, 16) || misaligned(v, 16)) return GMA_ERR_ALIGN;
    if (misaligned(mu, 4) || misaligned(var_raw, 4) || misaligned(prior_logits, 4) || misaligned(state, 4))
        return GMA_ERR_ALIGN;
    if (workspace && misaligned(workspace, gma::kWsAlign)) return GMA_ERR_ALIGN;
    if (!memory_algo_ok(d)) return GMA_ERR_UNSUPPORTED;
    const void* ins[5] = {kr, v, mu, var_raw, prior_logits};
    const size_t ins_n[5] = {nk, nv, np, np, npr};
    const size_t need = gma::memory_workspace(d);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GMA_ERR_WORKSPACE;
    if (workspace && overlaps(workspace, need, state, ns)) return GMA_ERR_ALIAS;
    for (int i = 0; i < 5; ++i)
        if (overlaps(state, ns, ins[i], ins_n[i]) || (workspace && overlaps(workspace, need, ins[i], ins_n[i])))
            return GMA_ERR_ALIAS;
    Args a;
    memset(&a, 0, sizeof(a));
    a.kr = kr;
    a.v = v;
    a.mu = mu;
    a.var_raw = var_raw;
    a.prior = prior_logits;
    a.state = state;
    a.d = d;
    a.Nk = d.N;
    a.ws = static_cast<unsigned char*>(workspace);
    a.ws_bytes = workspace_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    return gma::memory_forward(a) == hipSuccess ? GMA_OK : GMA_ERR_HIP;
}

size_t gma_decode_workspace_size(const gma_desc* desc) {
    if (check_desc(desc) != GMA_OK || desc->N != 1 || desc->algo == GMA_ALGO_MFMA) return 0;
    if ((int64_t)desc->B * desc->H == 0) return 0;
    return gma::decode_workspace(*desc);
}

int gma_decode_step(const void* qr, const void* kr, const void* v, const float* mu, const float* var_raw,
                    const float* prior_logits, float* state, float eps, void* out, const gma_desc* desc,
                    void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_desc(desc);
    if (st != GMA_OK) return st;
    const gma_desc d = *desc;
    if (d.N != 1) return GMA_ERR_BAD_SHAPE;
    if (!(eps >= 0.0f) || !isfinite(eps)) return GMA_ERR_BAD_SCALAR;
    const size_t bh = (size_t)d.B * d.H;
    if (bh == 0) return GMA_OK;
    if (!qr || !kr || !v || !mu || !var_raw || !prior_logits || !state || !out) return GMA_ERR_NULL_ARG;
    // one kernel family (a small latency-bound kernel): an explicit matrix-core request is
    // not honoured
    if (d.algo == GMA_ALGO_MFMA) return GMA_ERR_UNSUPPORTED;
    const size_t esz = d.dtype == GMA_F32 ? 4 : 2;
    const size_t nx = bh * d.d_r * esz, nv = bh * d.d_v * esz;
    const size_t np = (size_t)d.H * d.K * d.d_r * 4, npr = (size_t)d.H * d.K * 4;
    const size_t ns = bh * d.K * (d.d_v + 1) * 4;
    if (misaligned(qr, 16) || misaligned(kr, 16) || misaligned(v, 16) || misaligned(out, 16)) return GMA_ERR_ALIGN;
    if (misaligned(mu, 4) || misaligned(var_raw, 4) || misaligned(prior_logits, 4) || misaligned(state, 4))
        return GMA_ERR_ALIGN;
    if (workspace && misaligned(workspace, gma::kWsAlign)) return GMA_ERR_ALIGN;
    const void* ins[6] = {qr, kr, v, mu, var_raw, prior_logits};
    const size_t ins_n[6] = {nx, nx, nv, np, np, npr};
    for (int i = 0; i < 6; ++i)
        if (overlaps(out, nv, ins[i], ins_n[i]) || overlaps(state, ns, ins[i], ins_n[i])) return GMA_ERR_ALIAS;
    if (overlaps(out, nv, state, ns)) return GMA_ERR_ALIAS;
    const size_t need = gma::decode_workspace(d);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GMA_ERR_WORKSPACE;
    if (workspace && (overlaps(workspace, need, out, nv) || overlaps(workspace, need, state, ns))) return GMA_ERR_ALIAS;
    for (int i = 0; i < 6; ++i)
        if (workspace && overlaps(workspace, need, ins[i], ins_n[i])) return GMA_ERR_ALIAS;
    Args a;
    memset(&a, 0, sizeof(a));
    a.qr = qr;
    a.kr = kr;
    a.v = v;
    a.mu = mu;
    a.var_raw = var_raw;
    a.prior = prior_logits;
    a.eps = eps;
    a.out = out;
    a.state = state;
    a.d = d;
    a.Nk = 1;
    a.ws = static_cast<unsigned char*>(workspace);
    a.ws_bytes = workspace_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    return gma::decode_forward(a) == hipSuccess ? GMA_OK : GMA_ERR_HIP;
}

size_t gma_decode_prepared_size(const gma_desc* desc) {
    if (check_desc(desc) != GMA_OK || desc->algo == GMA_ALGO_MFMA || desc->H == 0) return 0;
    return gma::decode_prepared_bytes(*desc);
}

int gma_decode_prepare(const float* mu, const float* var_raw, const float* prior_logits, void* prepared,
                       size_t prepared_bytes, const gma_desc* desc, void* stream) {
    int st = check_desc(desc);
    if (st != GMA_OK) return st;
    const gma_desc d = *desc;
    if (d.algo == GMA_ALGO_MFMA) return GMA_ERR_UNSUPPORTED;
    if (d.H == 0) return GMA_OK;
    if (!mu || !var_raw || !prior_logits || !prepared) return GMA_ERR_NULL_ARG;
    if (misaligned(mu, 4) || misaligned(var_raw, 4) || misaligned(prior_logits, 4)) return GMA_ERR_ALIGN;
    if (misaligned(prepared, gma::kWsAlign)) return GMA_ERR_ALIGN;
    const size_t need = gma::decode_prepared_bytes(d);
    if (prepared_bytes < need) return GMA_ERR_WORKSPACE;
    const size_t np = (size_t)d.H * d.K * d.d_r * 4, npr = (size_t)d.H * d.K * 4;
    if (overlaps(prepared, need, mu, np) || overlaps(prepared, need, var_raw, np) ||
        overlaps(prepared, need, prior_logits, npr))
        return GMA_ERR_ALIAS;
    Args a;
    memset(&a, 0, sizeof(a));
    a.mu = mu;
    a.var_raw = var_raw;
    a.prior = prior_logits;
    a.d = d;
    a.ws = static_cast<unsigned char*>(prepared);
    a.ws_bytes = prepared_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    return gma::decode_prepare(a) == hipSuccess ? GMA_OK : GMA_ERR_HIP;
}

int gma_decode_step_prepared(const void* qr, const void* kr, const void* v, const void* prepared, float* state,
                             float eps, void* out, const gma_desc* desc, void* stream) {
    int st = check_desc(desc);
    if (st != GMA_OK) return st;
    const gma_desc d = *desc;
    if (d.N != 1) return GMA_ERR_BAD_SHAPE;
    if (!(eps >= 0.0f) || !isfinite(eps)) return GMA_ERR_BAD_SCALAR;
    const size_t bh = (size_t)d.B * d.H;
    if (bh == 0) return GMA_OK;
    if (!qr || !kr || !v || !prepared || !state || !out) return GMA_ERR_NULL_ARG;
    if (d.algo == GMA_ALGO_MFMA) return GMA_ERR_UNSUPPORTED;
    const size_t esz = d.dtype == GMA_F32 ? 4 : 2;
    const size_t nx = bh * d.d_r * esz, nv = bh * d.d_v * esz;
    const size_t ns = bh * d.K * (d.d_v + 1) * 4, np = gma::decode_prepared_bytes(d);
    if (misaligned(qr, 16) || misaligned(kr, 16) || misaligned(v, 16) || misaligned(out, 16)) return GMA_ERR_ALIGN;
    if (misaligned(state, 4) || misaligned(prepared, gma::kWsAlign)) return GMA_ERR_ALIGN;
    const void* ins[4] = {qr, kr, v, prepared};
    const size_t ins_n[4] = {nx, nx, nv, np};
    for (int i = 0; i < 4; ++i)
        if (overlaps(out, nv, ins[i], ins_n[i]) || overlaps(state, ns, ins[i], ins_n[i])) return GMA_ERR_ALIAS;
    if (overlaps(out, nv, state, ns)) return GMA_ERR_ALIAS;
    Args a;
    memset(&a, 0, sizeof(a));
    a.qr = qr;
    a.kr = kr;
    a.v = v;
    a.eps = eps;
    a.out = out;
    a.state = state;
    a.d = d;
    a.Nk = 1;
    a.ws = static_cast<unsigned char*>(const_cast<void*>(prepared));
    a.ws_bytes = np;
    a.stream = static_cast<hipStream_t>(stream);
    return gma::decode_prepared_forward(a, 0) == hipSuccess ? GMA_OK : GMA_ERR_HIP;
}

// ---- backward

static bool backward_algo_ok(const gma_desc& d) { return d.algo != GMA_ALGO_MFMA && gma::backward_supported(d); }

size_t gma_backward_workspace_size(const gma_desc* desc, int causal) {
    if (check_desc(desc) != GMA_OK || (causal != 0 && causal != 1)) return 0;
    if ((int64_t)desc->B * desc->H == 0 || !backward_algo_ok(*desc)) return 0;
    return gma::backward_workspace(*desc);
}

int gma_backward(const void* qr, const void* kr, const void* v, const float* mu, const float* var_raw,
                 const float* prior_logits, const void* dout, int causal, float eps, void* dqr, void* dkr, void* dv,
                 float* dmu, float* dvar_raw, float* dprior, const gma_desc* desc, void* workspace,
                 size_t workspace_bytes, void* stream) {
    int st = check_desc(desc);
    if (st != GMA_OK) return st;
    const gma_desc d = *desc;
    if (causal != 0 && causal != 1) return GMA_ERR_BAD_SCALAR;
    if (!(eps >= 0.0f) || !isfinite(eps)) return GMA_ERR_BAD_SCALAR;
    const size_t bh = (size_t)d.B * d.H;
    if (bh == 0) return GMA_OK;
    if (!mu || !var_raw || !prior_logits || !dmu || !dvar_raw || !dprior) return GMA_ERR_NULL_ARG;
    if (d.N > 0 && (!qr || !kr || !v || !dout || !dqr || !dkr || !dv)) return GMA_ERR_NULL_ARG;
    if (d.algo == GMA_ALGO_MFMA) return GMA_ERR_UNSUPPORTED;  // one kernel family so far
    if (!gma::backward_supported(d)) return GMA_ERR_UNSUPPORTED;
    const size_t esz = d.dtype == GMA_F32 ? 4 : 2;
    const size_t nx = bh * d.N * d.d_r * esz, nv = bh * d.N * d.d_v * esz;
    const size_t np = (size_t)d.H * d.K * d.d_r * 4, npr = (size_t)d.H * d.K * 4;
    if (misaligned(qr, 16) || misaligned(kr, 16) || misaligned(v, 16) || misaligned(dout, 16) ||
        misaligned(dqr, 16) || misaligned(dkr, 16) || misaligned(dv, 16))
        return GMA_ERR_ALIGN;
    if (misaligned(mu, 4) || misaligned(var_raw, 4) || misaligned(prior_logits, 4) || misaligned(dmu, 4) ||
        misaligned(dvar_raw, 4) || misaligned(dprior, 4))
        return GMA_ERR_ALIGN;
    if (workspace && misaligned(workspace, gma::kWsAlign)) return GMA_ERR_ALIGN;
    const size_t need = gma::backward_workspace(d);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GMA_ERR_WORKSPACE;
    const void* ins[7] = {qr, kr, v, mu, var_raw, prior_logits, dout};
    const size_t ins_n[7] = {nx, nx, nv, np, np, npr, nv};
    const void* outs[7] = {dqr, dkr, dv, dmu, dvar_raw, dprior, workspace};
    const size_t outs_n[7] = {nx, nx, nv, np, np, npr, need};
    for (int i = 0; i < 7; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlaps(outs[i], outs_n[i], ins[j], ins_n[j])) return GMA_ERR_ALIAS;
        for (int j = i + 1; j < 7; ++j)
            if (overlaps(outs[i], outs_n[i], outs[j], outs_n[j])) return GMA_ERR_ALIAS;
    }
    Args a;
    memset(&a, 0, sizeof(a));
    a.qr = qr;
    a.kr = kr;
    a.v = v;
    a.mu = mu;
    a.var_raw = var_raw;
    a.prior = prior_logits;
    a.causal = causal;
    a.eps = eps;
    a.d = d;
    a.Nk = d.N;
    a.ws = static_cast<unsigned char*>(workspace);
    a.ws_bytes = workspace_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    gma::BwdArgs g;
    g.dout = dout;
    g.dqr = dqr;
    g.dkr = dkr;
    g.dv = dv;
    g.dmu = dmu;
    g.dvar_raw = dvar_raw;
    g.dprior = dprior;
    return gma::backward_run(a, g) == hipSuccess ? GMA_OK : GMA_ERR_HIP;
}

// ---- responsibility statistics

static bool stats_algo_ok(const gma_desc& d) { return d.algo != GMA_ALGO_MFMA || gma::stats_on_mfma(d); }

size_t gma_stats_workspace_size(const gma_desc* desc) {
    if (check_desc(desc) != GMA_OK || (int64_t)desc->B * desc->H == 0 || !stats_algo_ok(*desc)) return 0;
    return gma::stats_workspace(*desc);
}

int gma_resp_stats(const void* x, const float* mu, const float* var_raw, const float* prior_logits, int32_t* hard,
                   int32_t* counts, float* usage, int32_t* used, float* entropy, const gma_desc* desc,
                   void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_desc(desc);
    if (st != GMA_OK) return st;
    const gma_desc d = *desc;
    const size_t bh = (size_t)d.B * d.H;
    if (bh == 0) return GMA_OK;
    if (!mu || !var_raw || !prior_logits || !counts || !usage || !used || !entropy) return GMA_ERR_NULL_ARG;
    if (d.N > 0 && !x) return GMA_ERR_NULL_ARG;  // no rows: x is not read
    const size_t esz = d.dtype == GMA_F32 ? 4 : 2;
    const size_t nx = bh * d.N * d.d_r * esz;
    const size_t np = (size_t)d.H * d.K * d.d_r * 4, npr = (size_t)d.H * d.K * 4;
    const size_t nhard = bh * d.N * 4, nhk = (size_t)d.H * d.K * 4, nh = (size_t)d.H * 4;
    if (misaligned(x, 16)) return GMA_ERR_ALIGN;
    if (misaligned(mu, 4) || misaligned(var_raw, 4) || misaligned(prior_logits, 4) || misaligned(hard, 4) ||
        misaligned(counts, 4) || misaligned(usage, 4) || misaligned(used, 4) || misaligned(entropy, 4))
        return GMA_ERR_ALIGN;
    if (workspace && misaligned(workspace, gma::kWsAlign)) return GMA_ERR_ALIGN;
    if (!stats_algo_ok(d)) return GMA_ERR_UNSUPPORTED;
    const size_t need = gma::stats_workspace(d);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GMA_ERR_WORKSPACE;
    const void* ins[4] = {x, mu, var_raw, prior_logits};
    const size_t ins_n[4] = {nx, np, np, npr};
    const void* outs[6] = {hard, counts, usage, used, entropy, workspace};
    const size_t outs_n[6] = {nhard, nhk, nhk, nh, nh, need};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 4; ++j)
            if (overlaps(outs[i], outs_n[i], ins[j], ins_n[j])) return GMA_ERR_ALIAS;
        for (int j = i + 1; j < 6; ++j)
            if (overlaps(outs[i], outs_n[i], outs[j], outs_n[j])) return GMA_ERR_ALIAS;
    }
    Args a;
    memset(&a, 0, sizeof(a));
    a.kr = x;
    a.mu = mu;
    a.var_raw = var_raw;
    a.prior = prior_logits;
    a.hard = hard;
    a.counts = counts;
    a.usage = usage;
    a.used = used;
    a.entropy = entropy;
    a.d = d;
    a.Nk = d.N;
    a.ws = static_cast<unsigned char*>(workspace);
    a.ws_bytes = workspace_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    return gma::stats_forward(a) == hipSuccess ? GMA_OK : GMA_ERR_HIP;
}

const char* gma_strerror(int status) {
    switch (status) {
        case GMA_OK: return "success";
        case GMA_ERR_NULL_ARG: return "a required pointer argument is NULL";
        case GMA_ERR_BAD_SHAPE: return "invalid shape (B, H, N must be >= 0; d_r, d_v, K >= 1; sizes too large)";
        case GMA_ERR_UNSUPPORTED: return "unsupported configuration (K, d_r, d_v above the limits, dtype or algorithm)";
        case GMA_ERR_ALIGN: return "misaligned pointer (tensors 16 B, parameters 4 B, workspace 256 B)";
        case GMA_ERR_BAD_SCALAR: return "invalid scalar (eps/var_floor must be finite and >= 0; causal 0 or 1)";
        case GMA_ERR_WORKSPACE: return "workspace missing or smaller than gma_workspace_size()";
        case GMA_ERR_ALIAS: return "an output overlaps an input, the workspace or the other output";
        case GMA_ERR_HIP: return "a HIP kernel launch failed";
        case GMA_ERR_TOO_LARGE:
            return "the call needs more scratch than gma_forward_noalloc's static buffer holds "
                   "(GMA_NOALLOC_SCRATCH_BYTES); use gma_forward with a workspace";
        default: return "unknown status";
    }
}

int gma_version(void) { return GMA_VERSION; }

}  // extern "C"
