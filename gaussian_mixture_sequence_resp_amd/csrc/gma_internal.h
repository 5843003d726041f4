// Internal interfaces of libgma.so shared by the host API and the kernel families.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gma.h"

namespace gma {

// Optional per-kernel event recording (gma_forward_timed).
struct Recorder {
    void* const* events;
    int n_events;
    const char** names;
    int count;
};

struct Args {
    const void* qr;
    const void* kr;
    const void* v;
    const float* mu;
    const float* var_raw;
    const float* prior;
    int causal;
    float eps;
    void* out;
    float* gamma_out;
    float* state;  // causal memory [B,H,K,d_v+1] (memory and decode entry points only)
    // responsibility statistics (stats entry point only)
    int* hard;       // [B,H,N] or null
    int* counts;     // [H,K]
    float* usage;    // [H,K]
    int* used;       // [H]
    float* entropy;  // [H]
    gma_desc d;    // d.N is the query (and output) length
    int Nk;        // key / value length (= d.N except in the cross variant)
    unsigned char* ws;
    size_t ws_bytes;
    hipStream_t stream;
    Recorder* rec;
};

// Bracket the next kernel launch with events when recording; no-ops otherwise.
inline void rec_begin(const Args& a, const char* name) {
    Recorder* r = a.rec;
    if (r && 2 * r->count + 1 < r->n_events) {
        (void)hipEventRecord(static_cast<hipEvent_t>(r->events[2 * r->count]), a.stream);
        if (r->names) r->names[r->count] = name;
    }
}
inline void rec_end(const Args& a) {
    Recorder* r = a.rec;
    if (!r) return;
    if (2 * r->count + 1 < r->n_events)
        (void)hipEventRecord(static_cast<hipEvent_t>(r->events[2 * r->count + 1]), a.stream);
    r->count++;
}

// Round a byte count up to the workspace region alignment.
constexpr size_t kWsAlign = 256;
inline size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// SIMT family: plain fp32 arithmetic, one thread per output element.
size_t simt_workspace(const gma_desc& d, int causal, int Nk);
hipError_t simt_forward(const Args& a);
// Responsibilities only, written as float32 Gamma_Q [B,H,N,K] then Gamma_K [B,H,Nk,K]; used for
// gamma_out by every family.
hipError_t simt_gamma(const Args& a, float* gamma, const double* lam, const double* cst, int* hard = nullptr);
// The same responsibilities in double (the backward of float32 inputs).
hipError_t simt_gamma(const Args& a, double* gamma, const double* lam, const double* cst);
// Parameter prep of the SIMT family: lam = 1/var [H,K,d_r], cst [H,K] (log prior minus half
// the log-determinant), both double.
hipError_t simt_params(const Args& a, double* lam, double* cst);
size_t simt_param_bytes(const gma_desc& d);
// Causal memory [B,H,K,d_v+1] of the d.N positions of a.kr, a.v into a.state (SIMT).
size_t simt_memory_workspace(const gma_desc& d);
hipError_t simt_memory(const Args& a);

// Causal memory (prefill) and single-token decode step (gma_decode.hip).
size_t memory_workspace(const gma_desc& d);
hipError_t memory_forward(const Args& a);
size_t decode_workspace(const gma_desc& d);
hipError_t decode_forward(const Args& a);
// Prepared parameters of the decode step (gma_decode.hip): byte size, the preparation
// (a.ws = the prepared block) and the step on them (groups <= 0: the default column groups).
size_t decode_prepared_bytes(const gma_desc& d);
hipError_t decode_prepare(const Args& a);
hipError_t decode_prepared_forward(const Args& a, int groups);

// Backward (gma_backward.hip): dout and the gradients; the inputs are those of the forward
// in Args (qr, kr, v, mu, var_raw, prior, causal, eps).
struct BwdArgs {
    const void* dout;  // [B,H,N,d_v], input dtype
    void* dqr;         // [B,H,N,d_r], input dtype
    void* dkr;
    void* dv;          // [B,H,N,d_v], input dtype
    float* dmu;        // [H,K,d_r]
    float* dvar_raw;   // [H,K,d_r]
    float* dprior;     // [H,K]
};
size_t backward_workspace(const gma_desc& d);
bool backward_supported(const gma_desc& d);
hipError_t backward_run(const Args& a, const BwdArgs& g);

// Responsibility statistics of the rows a.kr (gma_stats.hip).
size_t stats_workspace(const gma_desc& d);
hipError_t stats_forward(const Args& a);
bool stats_on_mfma(const gma_desc& d);

// Scratch that the library supplies itself (gma_forward_noalloc): `get` returns the device
// address of `capacity` bytes of scratch on the device that `stream` runs on, or nullptr
// with *status set.
struct ScratchSource {
    size_t capacity;
    void* (*get)(void* stream, int* status);
};
// gma_forward with the workspace taken from `scratch` once every argument has been checked.
int forward_with_scratch(const void* qr, const void* kr, const void* v, const float* mu, const float* var_raw,
                         const float* prior_logits, int causal, float eps, void* out, float* gamma_out,
                         const gma_desc* desc, void* stream, const ScratchSource& scratch);

// MFMA family (bf16 inputs): fused matrix-core kernels.
size_t mfma_workspace(const gma_desc& d, int causal, int Nk);
bool mfma_supported(const gma_desc& d, int causal);
hipError_t mfma_forward(const Args& a);
// Causal memory of the N key rows of a.kr, a.v into a.state (layout [B,H,K,d_v+1]): split
// partials of the bidirectional write kernel summed in split order, or, where that kernel's
// coefficient block does not fit in LDS, Gamma_K from the causal responsibilities kernel and
// sub-segment totals summed in order; used by memory_forward.
bool mfma_memory_supported(const gma_desc& d);
hipError_t mfma_memory(const Args& a);
size_t mfma_memory_workspace(const gma_desc& d);

}  // namespace gma
