// gdn_api.cpp -- the C ABI of libgdn: argument checks, workspace sizing and kernel dispatch.
//
// Every check happens on the host before anything is enqueued, so a rejected call has no effect
// on device memory.  Device memory is never read here (no synchronisation on the call path).

#include <stdint.h>

#include "gdn.h"
#include "launch.h"

namespace {

bool aligned(const void* p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

size_t dtype_bytes(gdn_dtype t) { return t == GDN_BF16 ? 2 : 4; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }

bool dtype_ok(gdn_dtype t) { return t == GDN_F32 || t == GDN_BF16; }

bool use_mfma(int dk, int dv, gdn_dtype qkv) { return gdn::chunk_mfma_supported(dk, dv, qkv); }

// Largest element count any tensor of a call may have (indices inside kernels are 64-bit, but
// per-dimension arithmetic on ints must not overflow).
bool sizes_fit(long long B, long long T, long long H, long long d) {
    const long long lim = (1LL << 40);
    return B * T < (1LL << 31) && B * T * H * d < lim;
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status status) {
    switch (status) {
        case GDN_SUCCESS: return "GDN_SUCCESS";
        case GDN_ERROR_INVALID_VALUE: return "GDN_ERROR_INVALID_VALUE";
        case GDN_ERROR_NOT_SUPPORTED: return "GDN_ERROR_NOT_SUPPORTED";
        case GDN_ERROR_WORKSPACE: return "GDN_ERROR_WORKSPACE";
        case GDN_ERROR_LAUNCH_FAILURE: return "GDN_ERROR_LAUNCH_FAILURE";
        default: break;
    }
    return "GDN_ERROR_UNKNOWN";
}

int gdn_version(void) { return 100; }

size_t gdn_chunk_fwd_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                    gdn_dtype qkv_dtype) {
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1 || N < 1 || Hv % Hk != 0) return 0;
    if (!head_dim_ok(dk) || !head_dim_ok(dv) || !dtype_ok(qkv_dtype)) return 0;
    if (!sizes_fit(B, T, Hv, dv > dk ? dv : dk) || !sizes_fit(N, 1, Hv, (long long)dk * dv)) return 0;
    if (!use_mfma(dk, dv, qkv_dtype)) return 0;
    return gdn::chunk_mfma_workspace_size(B, T, Hk, Hv, dk, dv, N);
}

size_t gdn_chunk_fwd_gated_norm_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                               gdn_dtype qkv_dtype) {
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1 || N < 1 || Hv % Hk != 0) return 0;
    if (!head_dim_ok(dk) || !head_dim_ok(dv) || !dtype_ok(qkv_dtype)) return 0;
    if (!sizes_fit(B, T, Hv, dv > dk ? dv : dk) || !sizes_fit(N, 1, Hv, (long long)dk * dv)) return 0;
    if (use_mfma(dk, dv, qkv_dtype)) return gdn::chunk_mfma_workspace_size(B, T, Hk, Hv, dk, dv, N, true);
    return align256((size_t)B * T * Hv * dv * sizeof(float));   // o, between the two passes
}

}  // extern "C"

namespace {

// The gated output norm of gdn_chunk_fwd_gated_norm (null for the plain calls).
struct FusedNorm {
    const void* z;
    const float* weight;
    float eps;
    gdn_dtype z_dtype, y_dtype;
    void* y;
};

// Shared body of gdn_chunk_fwd and its two halves: checks, then the selected stages.
// With A_log set, g and beta carry the raw projections a and b and the kernels form the gates.
// With state_indices set, initial_state and final_state are the same pool of num_slots states.
gdn_status chunk_call(const void* q, const void* k, const void* v, const void* g, const void* beta,
                      const float* A_log, const float* dt_bias, const int32_t* state_indices,
                      int num_slots, const float* initial_state, const int32_t* cu_seqlens, int B, int T, int Hk,
                      int Hv, int dk, int dv, int N, gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                      float* o, float* final_state, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, unsigned stages, int qk_l2norm = 0,
                      const FusedNorm* fn = nullptr) {
    if (!final_state) return GDN_ERROR_INVALID_VALUE;
    if (T > 0 && (!q || !k || !v || !g || !beta || (!fn && !o))) return GDN_ERROR_INVALID_VALUE;
    if (fn) {
        if (!dtype_ok(fn->z_dtype) || !dtype_ok(fn->y_dtype)) return GDN_ERROR_INVALID_VALUE;
        if (!(fn->eps >= 0.f) || fn->eps > 3.0e38f) return GDN_ERROR_INVALID_VALUE;   // also NaN
        if (T > 0 && (!fn->z || !fn->weight || !fn->y)) return GDN_ERROR_INVALID_VALUE;
        if (!aligned16(fn->z) || !aligned16(fn->weight) || !aligned16(fn->y)) return GDN_ERROR_INVALID_VALUE;
    }
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1 || N < 1 || Hv % Hk != 0) return GDN_ERROR_INVALID_VALUE;
    if (!dtype_ok(qkv_dtype) || !dtype_ok(gate_dtype)) return GDN_ERROR_INVALID_VALUE;
    if (cu_seqlens ? B != 1 : N != B) return GDN_ERROR_INVALID_VALUE;
    if (dk < 1 || dv < 1) return GDN_ERROR_INVALID_VALUE;
    if (!sizes_fit(B, T, Hv, dv > dk ? dv : dk) || !sizes_fit(N, 1, Hv, (long long)dk * dv))
        return GDN_ERROR_INVALID_VALUE;
    for (const void* p : {q, k, v, (const void*)initial_state, (const void*)o, (const void*)final_state})
        if (p && !aligned16(p)) return GDN_ERROR_INVALID_VALUE;
    for (const void* p : {g, beta})
        if (p && !aligned(p, dtype_bytes(gate_dtype))) return GDN_ERROR_INVALID_VALUE;
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return GDN_ERROR_INVALID_VALUE;
    if (A_log && (!dt_bias || !aligned(A_log, 4) || !aligned(dt_bias, 4))) return GDN_ERROR_INVALID_VALUE;
    if (state_indices && (num_slots < 1 || !aligned(state_indices, 4) ||
                          !sizes_fit(num_slots, 1, Hv, (long long)dk * dv)))
        return GDN_ERROR_INVALID_VALUE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDN_ERROR_NOT_SUPPORTED;

    gdn::ChunkArgs a{q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens,
                     state_indices, num_slots, B, T, Hk, Hv, dk, dv, N, qkv_dtype, gate_dtype, o,
                     final_state, workspace, workspace_bytes, stream, qk_l2norm};
    const size_t need = fn ? gdn_chunk_fwd_gated_norm_workspace_size(B, T, Hk, Hv, dk, dv, N, qkv_dtype)
                           : gdn_chunk_fwd_workspace_size(B, T, Hk, Hv, dk, dv, N, qkv_dtype);
    if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
        return GDN_ERROR_WORKSPACE;
    hipError_t e;
    if (use_mfma(dk, dv, qkv_dtype)) {
        if (fn) {
            a.o = nullptr;
            a.z = fn->z;
            a.norm_weight = fn->weight;
            a.eps = fn->eps;
            a.z_dtype = fn->z_dtype;
            a.y_dtype = fn->y_dtype;
            a.y = fn->y;
        }
        e = gdn::launch_chunk_mfma(a, stages);
    } else if (fn) {        // fp32 inputs: the prefill's o into the workspace, then the norm over it
        a.o = static_cast<float*>(workspace);
        e = gdn::launch_chunk_f32(a);
        if (e == hipSuccess && (long long)B * T > 0) {
            const gdn::NormArgs na{a.o, fn->z, fn->weight, fn->eps, (long long)B * T * Hv, dv, fn->z_dtype,
                                   fn->y_dtype, fn->y, stream};
            e = gdn::launch_gated_rmsnorm(na);
        }
    } else {
        e = (stages & gdn::kStageScan) ? gdn::launch_chunk_f32(a) : hipSuccess;
    }
    return e == hipSuccess ? GDN_SUCCESS : GDN_ERROR_LAUNCH_FAILURE;
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                         int B, int T, int Hk, int Hv, int dk, int dv, int N,
                         gdn_dtype qkv_dtype, gdn_dtype gate_dtype, float* o, float* final_state,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return chunk_call(q, k, v, g, beta, nullptr, nullptr, nullptr, 0, initial_state, cu_seqlens, B, T, Hk, Hv, dk, dv, N,
                      qkv_dtype, gate_dtype, o, final_state, workspace, workspace_bytes, stream,
                      gdn::kStagePrepare | gdn::kStageScan);
}

gdn_status gdn_chunk_fwd_prepare(const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, int B, int T, int Hk, int Hv, int dk,
                                 int dv, int N, gdn_dtype qkv_dtype, gdn_dtype gate_dtype, float* o,
                                 float* final_state, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    return chunk_call(q, k, v, g, beta, nullptr, nullptr, nullptr, 0, initial_state, cu_seqlens, B, T, Hk, Hv, dk, dv, N,
                      qkv_dtype, gate_dtype, o, final_state, workspace, workspace_bytes, stream,
                      gdn::kStagePrepare);
}

gdn_status gdn_chunk_fwd_scan(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, const float* initial_state,
                              const int32_t* cu_seqlens, int B, int T, int Hk, int Hv, int dk,
                              int dv, int N, gdn_dtype qkv_dtype, gdn_dtype gate_dtype, float* o,
                              float* final_state, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    return chunk_call(q, k, v, g, beta, nullptr, nullptr, nullptr, 0, initial_state, cu_seqlens, B, T, Hk, Hv, dk, dv, N,
                      qkv_dtype, gate_dtype, o, final_state, workspace, workspace_bytes, stream,
                      gdn::kStageScan);
}

}  // extern "C"

namespace {

// With state_indices set, state is a pool of num_slots states and row b uses slot state_indices[b].
gdn_status recurrent_call(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, const float* A_log, const float* dt_bias, float* state,
                          const int32_t* state_indices, int num_slots, int B, int T, int Hk, int Hv,
                          int dk, int dv, gdn_dtype qkv_dtype, gdn_dtype gate_dtype, float* o,
                          hipStream_t stream, int qk_l2norm = 0) {
    if (!q || !k || !v || !g || !beta || !state || !o) return GDN_ERROR_INVALID_VALUE;
    if (B < 1 || T < 1 || Hk < 1 || Hv < 1 || Hv % Hk != 0) return GDN_ERROR_INVALID_VALUE;
    if (!dtype_ok(qkv_dtype) || !dtype_ok(gate_dtype)) return GDN_ERROR_INVALID_VALUE;
    if (dk < 1 || dv < 1) return GDN_ERROR_INVALID_VALUE;
    if (!sizes_fit(B, T, Hv, dv > dk ? dv : dk) || !sizes_fit(B, 1, Hv, (long long)dk * dv))
        return GDN_ERROR_INVALID_VALUE;
    if (state_indices && (num_slots < 1 || !aligned(state_indices, 4) ||
                          !sizes_fit(num_slots, 1, Hv, (long long)dk * dv)))
        return GDN_ERROR_INVALID_VALUE;
    for (const void* p : {(const void*)state, (const void*)o})
        if (!aligned16(p)) return GDN_ERROR_INVALID_VALUE;
    for (const void* p : {q, k, v})
        if (!aligned(p, dtype_bytes(qkv_dtype))) return GDN_ERROR_INVALID_VALUE;
    for (const void* p : {g, beta})
        if (!aligned(p, dtype_bytes(gate_dtype))) return GDN_ERROR_INVALID_VALUE;
    if (A_log && (!dt_bias || !aligned(A_log, 4) || !aligned(dt_bias, 4))) return GDN_ERROR_INVALID_VALUE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDN_ERROR_NOT_SUPPORTED;

    const gdn::RecurrentArgs a{q, k, v, g, beta, A_log, dt_bias, state, state_indices, num_slots,
                               B, T, Hk, Hv, dk, dv, qkv_dtype, gate_dtype, o, stream, qk_l2norm};
    return gdn::launch_recurrent(a) == hipSuccess ? GDN_SUCCESS : GDN_ERROR_LAUNCH_FAILURE;
}

}  // namespace

extern "C" {

gdn_status gdn_recurrent_step(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, float* state, int B, int T, int Hk, int Hv,
                              int dk, int dv, gdn_dtype qkv_dtype, gdn_dtype gate_dtype, float* o,
                              hipStream_t stream) {
    return recurrent_call(q, k, v, g, beta, nullptr, nullptr, state, nullptr, 0, B, T, Hk, Hv, dk,
                          dv, qkv_dtype, gate_dtype, o, stream);
}

gdn_status gdn_recurrent_step_indexed(const void* q, const void* k, const void* v, const void* g,
                                      const void* beta, float* state_pool,
                                      const int32_t* state_indices, int num_slots, int B, int T,
                                      int Hk, int Hv, int dk, int dv, gdn_dtype qkv_dtype,
                                      gdn_dtype gate_dtype, float* o, hipStream_t stream) {
    if (!state_indices) return GDN_ERROR_INVALID_VALUE;
    return recurrent_call(q, k, v, g, beta, nullptr, nullptr, state_pool, state_indices, num_slots,
                          B, T, Hk, Hv, dk, dv, qkv_dtype, gate_dtype, o, stream);
}

gdn_status gdn_chunk_fwd_indexed(const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, float* state_pool, const int32_t* state_indices,
                                 int num_slots, const int32_t* cu_seqlens, int B, int T, int Hk,
                                 int Hv, int dk, int dv, int N, gdn_dtype qkv_dtype,
                                 gdn_dtype gate_dtype, float* o, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    if (!state_indices) return GDN_ERROR_INVALID_VALUE;
    return chunk_call(q, k, v, g, beta, nullptr, nullptr, state_indices, num_slots, state_pool,
                      cu_seqlens, B, T, Hk, Hv, dk, dv, N, qkv_dtype, gate_dtype, o, state_pool,
                      workspace, workspace_bytes, stream, gdn::kStagePrepare | gdn::kStageScan);
}

gdn_status gdn_recurrent_step_gating(const void* q, const void* k, const void* v, const void* a,
                                     const void* b, const float* A_log, const float* dt_bias,
                                     float* state, int B, int T, int Hk, int Hv, int dk, int dv,
                                     gdn_dtype qkv_dtype, gdn_dtype gate_dtype, float* o,
                                     hipStream_t stream) {
    if (!A_log) return GDN_ERROR_INVALID_VALUE;
    return recurrent_call(q, k, v, a, b, A_log, dt_bias, state, nullptr, 0, B, T, Hk, Hv, dk, dv,
                          qkv_dtype, gate_dtype, o, stream);
}

gdn_status gdn_chunk_fwd_gating(const void* q, const void* k, const void* v, const void* a,
                                const void* b, const float* A_log, const float* dt_bias,
                                const float* initial_state, const int32_t* cu_seqlens, int B, int T,
                                int Hk, int Hv, int dk, int dv, int N, gdn_dtype qkv_dtype,
                                gdn_dtype gate_dtype, float* o, float* final_state,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!A_log) return GDN_ERROR_INVALID_VALUE;
    return chunk_call(q, k, v, a, b, A_log, dt_bias, nullptr, 0, initial_state, cu_seqlens, B, T, Hk, Hv, dk,
                      dv, N, qkv_dtype, gate_dtype, o, final_state, workspace, workspace_bytes,
                      stream, gdn::kStagePrepare | gdn::kStageScan);
}

gdn_status gdn_gated_rmsnorm(const float* x, const void* z, const float* weight, float eps,
                             int64_t rows, int d, gdn_dtype z_dtype, gdn_dtype out_dtype, void* out,
                             hipStream_t stream) {
    if (rows < 0 || !dtype_ok(z_dtype) || !dtype_ok(out_dtype)) return GDN_ERROR_INVALID_VALUE;
    if (!(eps >= 0.f) || eps > 3.0e38f) return GDN_ERROR_INVALID_VALUE;   // also rejects NaN
    if (rows > 0 && (!x || !z || !weight || !out)) return GDN_ERROR_INVALID_VALUE;
    if (d < 1 || !sizes_fit(rows, 1, 1, d)) return GDN_ERROR_INVALID_VALUE;
    if (!aligned16(x) || !aligned16(weight) || !aligned(z, 4 * dtype_bytes(z_dtype)) ||
        !aligned(out, 4 * dtype_bytes(out_dtype)))
        return GDN_ERROR_INVALID_VALUE;
    if (!head_dim_ok(d)) return GDN_ERROR_NOT_SUPPORTED;
    const gdn::NormArgs a{x, z, weight, eps, (long long)rows, d, z_dtype, out_dtype, out, stream};
    return gdn::launch_gated_rmsnorm(a) == hipSuccess ? GDN_SUCCESS : GDN_ERROR_LAUNCH_FAILURE;
}

gdn_status gdn_causal_conv1d(const void* x, const float* weight, const float* bias,
                             void* conv_state, const int32_t* state_indices, int num_slots,
                             const int32_t* cu_seqlens, int B, int T, int C, int W, int N,
                             gdn_dtype x_dtype, int silu, void* y, hipStream_t stream) {
    if (B < 1 || T < 0 || C < 1 || N < 1 || !dtype_ok(x_dtype)) return GDN_ERROR_INVALID_VALUE;
    if (cu_seqlens ? B != 1 : N != B) return GDN_ERROR_INVALID_VALUE;
    if (C % 4 != 0 || !sizes_fit(B, T, 1, C)) return GDN_ERROR_INVALID_VALUE;
    if (W < 1 || W > 16) return GDN_ERROR_NOT_SUPPORTED;
    if (T > 0 && (!x || !weight || !y)) return GDN_ERROR_INVALID_VALUE;
    if (W == 1) {                   // no input history exists: the cache arguments are ignored
        conv_state = nullptr;
        state_indices = nullptr;
    }
    if (state_indices && (!conv_state || num_slots < 1 || !aligned(state_indices, 4) ||
                          !sizes_fit(num_slots, W, 1, C)))
        return GDN_ERROR_INVALID_VALUE;
    if (conv_state && !state_indices && !sizes_fit(N, W, 1, C)) return GDN_ERROR_INVALID_VALUE;
    const uintptr_t v4 = 4 * dtype_bytes(x_dtype);
    if (!aligned(x, v4) || !aligned(y, v4) || !aligned(conv_state, v4) || !aligned(weight, 4) ||
        !aligned16(bias) || (cu_seqlens && !aligned(cu_seqlens, 4)))
        return GDN_ERROR_INVALID_VALUE;
    const gdn::ConvArgs a{x, weight, bias, conv_state, state_indices, num_slots, cu_seqlens, B, T, C, W,
                          N, x_dtype, silu ? 1 : 0, y, stream};
    return gdn::launch_causal_conv1d(a) == hipSuccess ? GDN_SUCCESS : GDN_ERROR_LAUNCH_FAILURE;
}

gdn_status gdn_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* A_log, const float* dt_bias,
                            const float* initial_state, float* final_state,
                            const int32_t* state_indices, int num_slots, const int32_t* cu_seqlens,
                            int B, int T, int Hk, int Hv, int dk, int dv, int N, gdn_dtype qkv_dtype,
                            gdn_dtype gate_dtype, unsigned flags, float* o, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    if ((flags & ~GDN_FLAG_QK_L2NORM) || (dt_bias && !A_log)) return GDN_ERROR_INVALID_VALUE;
    if (state_indices && initial_state != final_state) return GDN_ERROR_INVALID_VALUE;
    return chunk_call(q, k, v, g, beta, A_log, dt_bias, state_indices, num_slots, initial_state,
                      cu_seqlens, B, T, Hk, Hv, dk, dv, N, qkv_dtype, gate_dtype, o, final_state,
                      workspace, workspace_bytes, stream, gdn::kStagePrepare | gdn::kStageScan,
                      (flags & GDN_FLAG_QK_L2NORM) ? 1 : 0);
}

gdn_status gdn_chunk_fwd_gated_norm(const void* q, const void* k, const void* v, const void* g,
                                    const void* beta, const float* A_log, const float* dt_bias,
                                    const float* initial_state, float* final_state,
                                    const int32_t* state_indices, int num_slots, const int32_t* cu_seqlens,
                                    const void* z, const float* weight, float eps, int B, int T, int Hk,
                                    int Hv, int dk, int dv, int N, gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                                    gdn_dtype z_dtype, gdn_dtype y_dtype, unsigned flags, void* y,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if ((flags & ~GDN_FLAG_QK_L2NORM) || (dt_bias && !A_log)) return GDN_ERROR_INVALID_VALUE;
    if (state_indices && initial_state != final_state) return GDN_ERROR_INVALID_VALUE;
    const FusedNorm fn{z, weight, eps, z_dtype, y_dtype, y};
    return chunk_call(q, k, v, g, beta, A_log, dt_bias, state_indices, num_slots, initial_state,
                      cu_seqlens, B, T, Hk, Hv, dk, dv, N, qkv_dtype, gate_dtype, nullptr, final_state,
                      workspace, workspace_bytes, stream, gdn::kStagePrepare | gdn::kStageScan,
                      (flags & GDN_FLAG_QK_L2NORM) ? 1 : 0, &fn);
}

gdn_status gdn_recurrent_step_ex(const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, const float* A_log, const float* dt_bias,
                                 float* state, const int32_t* state_indices, int num_slots, int B,
                                 int T, int Hk, int Hv, int dk, int dv, gdn_dtype qkv_dtype,
                                 gdn_dtype gate_dtype, unsigned flags, float* o, hipStream_t stream) {
    if ((flags & ~GDN_FLAG_QK_L2NORM) || (dt_bias && !A_log)) return GDN_ERROR_INVALID_VALUE;
    return recurrent_call(q, k, v, g, beta, A_log, dt_bias, state, state_indices, num_slots, B, T,
                          Hk, Hv, dk, dv, qkv_dtype, gate_dtype, o, stream,
                          (flags & GDN_FLAG_QK_L2NORM) ? 1 : 0);
}

}  // extern "C"

namespace {

// Shared body of gdn_chunk_bwd and gdn_chunk_bwd_ex: every check, then the launches.
gdn_status bwd_call(const void* q, const void* k, const void* v, const void* g, const void* beta,
                    const float* A_log, const float* dt_bias, const float* initial_state,
                    const int32_t* state_indices, int num_slots, const int32_t* cu_seqlens, const float* d_o,
                    const float* d_final, int B, int T, int Hk, int Hv, int dk, int dv, int N,
                    gdn_dtype qkv_dtype, gdn_dtype gate_dtype, unsigned flags, float* dq, float* dk_out,
                    float* dv_out, float* dg, float* dbeta, float* d_A_log, float* d_dt_bias,
                    float* d_initial, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (T > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk_out || !dv_out || !dg || !dbeta))
        return GDN_ERROR_INVALID_VALUE;
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1 || N < 1 || Hv % Hk != 0) return GDN_ERROR_INVALID_VALUE;
    if (!dtype_ok(qkv_dtype) || !dtype_ok(gate_dtype)) return GDN_ERROR_INVALID_VALUE;
    if (cu_seqlens ? B != 1 : N != B) return GDN_ERROR_INVALID_VALUE;
    if (dk < 1 || dv < 1) return GDN_ERROR_INVALID_VALUE;
    if (!sizes_fit(B, T, Hv, dv > dk ? dv : dk) || !sizes_fit(N, 1, Hv, (long long)dk * dv))
        return GDN_ERROR_INVALID_VALUE;
    if ((flags & ~GDN_FLAG_QK_L2NORM) || (dt_bias && !A_log)) return GDN_ERROR_INVALID_VALUE;
    if (A_log && (!dt_bias || !d_A_log || !d_dt_bias)) return GDN_ERROR_INVALID_VALUE;
    if (state_indices && (!initial_state || num_slots < 1 || !sizes_fit(num_slots, 1, Hv, (long long)dk * dv)))
        return GDN_ERROR_INVALID_VALUE;
    for (const void* p : {q, k})
        if (p && !aligned16(p)) return GDN_ERROR_INVALID_VALUE;
    if (state_indices && !aligned16(initial_state)) return GDN_ERROR_INVALID_VALUE;
    if (v && !aligned(v, dtype_bytes(qkv_dtype))) return GDN_ERROR_INVALID_VALUE;
    for (const void* p : {g, beta})
        if (p && !aligned(p, dtype_bytes(gate_dtype))) return GDN_ERROR_INVALID_VALUE;
    for (const void* p : {(const void*)initial_state, (const void*)d_o, (const void*)d_final, (const void*)dq,
                          (const void*)dk_out, (const void*)dv_out, (const void*)dg, (const void*)dbeta,
                          (const void*)d_initial, (const void*)cu_seqlens, (const void*)A_log,
                          (const void*)dt_bias, (const void*)d_A_log, (const void*)d_dt_bias,
                          (const void*)state_indices})
        if (p && !aligned(p, 4)) return GDN_ERROR_INVALID_VALUE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDN_ERROR_NOT_SUPPORTED;
    if (A_log && Hv > gdn::kBwdExMaxHv) return GDN_ERROR_NOT_SUPPORTED;
    const bool ex = A_log || state_indices || flags;
    const size_t need = ex ? gdn_chunk_bwd_ex_workspace_size(B, T, Hk, Hv, dk, dv, N, qkv_dtype, A_log != nullptr,
                                                             state_indices != nullptr, flags)
                           : gdn_chunk_bwd_workspace_size(B, T, Hk, Hv, dk, dv, N);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return GDN_ERROR_WORKSPACE;
    const gdn::BwdArgs a{q, k, v, g, beta, initial_state, cu_seqlens, d_o, d_final, B, T, Hk, Hv, dk, dv, N,
                         qkv_dtype, gate_dtype, dq, dk_out, dv_out, dg, dbeta, d_initial, workspace,
                         workspace_bytes, stream};
    hipError_t e;
    if (ex) {
        const gdn::BwdExArgs x{a, A_log, dt_bias, state_indices, num_slots,
                               (flags & GDN_FLAG_QK_L2NORM) ? 1 : 0, d_A_log, d_dt_bias};
        e = gdn::launch_chunk_bwd_ex(x);
    } else {
        e = gdn::launch_chunk_bwd(a);
    }
    return e == hipSuccess ? GDN_SUCCESS : GDN_ERROR_LAUNCH_FAILURE;
}

}  // namespace

extern "C" {

size_t gdn_chunk_bwd_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N) {
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1 || N < 1 || Hv % Hk != 0) return 0;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return 0;
    if (!sizes_fit(B, T, Hv, dv > dk ? dv : dk) || !sizes_fit(N, 1, Hv, (long long)dk * dv)) return 0;
    return gdn::chunk_bwd_workspace_size(B, T, Hv, dk, dv, N);
}

gdn_status gdn_chunk_bwd(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                         const float* d_o, const float* d_final, int B, int T, int Hk, int Hv,
                         int dk, int dv, int N, gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                         float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                         float* d_initial, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    return bwd_call(q, k, v, g, beta, nullptr, nullptr, initial_state, nullptr, 0, cu_seqlens, d_o, d_final,
                    B, T, Hk, Hv, dk, dv, N, qkv_dtype, gate_dtype, 0u, dq, dk_out, dv_out, dg, dbeta,
                    nullptr, nullptr, d_initial, workspace, workspace_bytes, stream);
}

size_t gdn_chunk_bwd_ex_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                       gdn_dtype qkv_dtype, int raw_gates, int pool, unsigned flags) {
    if (!gdn_chunk_bwd_workspace_size(B, T, Hk, Hv, dk, dv, N) || !dtype_ok(qkv_dtype)) return 0;
    return gdn::chunk_bwd_ex_workspace_size(B, T, Hk, Hv, dk, dv, N, raw_gates != 0, pool != 0,
                                            (flags & GDN_FLAG_QK_L2NORM) != 0, qkv_dtype);
}

gdn_status gdn_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* A_log, const float* dt_bias,
                            const float* initial_state, const int32_t* state_indices, int num_slots,
                            const int32_t* cu_seqlens, const float* d_o, const float* d_final, int B,
                            int T, int Hk, int Hv, int dk, int dv, int N, gdn_dtype qkv_dtype,
                            gdn_dtype gate_dtype, unsigned flags, float* dq, float* dk_out,
                            float* dv_out, float* dg, float* dbeta, float* d_A_log, float* d_dt_bias,
                            float* d_initial, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    return bwd_call(q, k, v, g, beta, A_log, dt_bias, initial_state, state_indices, num_slots, cu_seqlens,
                    d_o, d_final, B, T, Hk, Hv, dk, dv, N, qkv_dtype, gate_dtype, flags, dq, dk_out, dv_out,
                    dg, dbeta, d_A_log, d_dt_bias, d_initial, workspace, workspace_bytes, stream);
}

}  // extern "C"
