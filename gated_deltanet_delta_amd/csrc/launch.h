// launch.h -- host-side launchers behind the C ABI (one per kernel family).
#pragma once

#include <hip/hip_runtime_api.h>

#include "gdn.h"

namespace gdn {

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;                 // g, or the raw projection a when A_log is set
    const void* beta;              // beta, or the raw projection b when A_log is set
    const float* A_log;            // [Hv] or null: gates formed in the kernels from a, b
    const float* dt_bias;          // [Hv], with A_log
    const float* initial_state;
    const int32_t* cu_seqlens;
    const int32_t* state_indices;  // [N] or null: states live in a pool, sequence n in slot [n]
    int num_slots;                 // pool size with state_indices
    int B, T, Hk, Hv, dk, dv, N;
    gdn_dtype qkv_dtype, gate_dtype;
    float* o;
    float* final_state;
    void* workspace;
    size_t workspace_bytes;
    hipStream_t stream;
    int qk_l2norm;                 // q, k normalised to unit length inside the kernels
    // the gated output norm fused onto o (z set): y = o / sqrt(mean(o^2) + eps) * norm_weight *
    // silu(z) per (token, v-head) row takes o's place (o is then unused)
    const void* z = nullptr;       // [B, T, Hv, dv] z_dtype
    const float* norm_weight = nullptr;   // [dv]
    float eps = 0.f;
    gdn_dtype z_dtype = GDN_BF16, y_dtype = GDN_BF16;
    void* y = nullptr;             // [B, T, Hv, dv] y_dtype
};

struct RecurrentArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;                 // as in ChunkArgs
    const void* beta;
    const float* A_log;
    const float* dt_bias;
    float* state;
    const int32_t* state_indices;  // [B] or null: as in ChunkArgs
    int num_slots;
    int B, T, Hk, Hv, dk, dv;
    gdn_dtype qkv_dtype, gate_dtype;
    float* o;
    hipStream_t stream;
    int qk_l2norm;                 // as in ChunkArgs
};

struct NormArgs {
    const float* x;                // [rows, d] fp32
    const void* z;                 // [rows, d] z_dtype
    const float* weight;           // [d] fp32
    float eps;
    long long rows;
    int d;
    gdn_dtype z_dtype, out_dtype;
    void* out;                     // [rows, d] out_dtype
    hipStream_t stream;
};

struct ConvArgs {
    const void* x;                 // [B, T, C] x_dtype (packed: B == 1, sequences by cu_seqlens)
    const float* weight;           // [C, W]
    const float* bias;             // [C] or null
    void* conv_state;              // [N or num_slots, W - 1, C] x_dtype, or null
    const int32_t* state_indices;  // [N] or null
    int num_slots;
    const int32_t* cu_seqlens;     // [N + 1] or null
    int B, T, C, W, N;
    gdn_dtype x_dtype;
    int silu;
    void* y;                       // [B, T, C] x_dtype
    hipStream_t stream;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* initial_state;    // [N, Hv, dk, dv] or null
    const int32_t* cu_seqlens;
    const float* d_o;              // [B, T, Hv, dv]
    const float* d_final;          // [N, Hv, dk, dv] or null
    int B, T, Hk, Hv, dk, dv, N;
    gdn_dtype qkv_dtype, gate_dtype;
    float* dq;                     // [B, T, Hk, dk]
    float* dk_out;                 // [B, T, Hk, dk]
    float* dv_out;                 // [B, T, Hv, dv]
    float* dg;                     // [B, T, Hv]
    float* dbeta;                  // [B, T, Hv]
    float* d_initial;              // [N, Hv, dk, dv] or null
    void* workspace;
    size_t workspace_bytes;
    hipStream_t stream;
};

// Backward pass of the chunked rule (fp32 arithmetic).
size_t chunk_bwd_workspace_size(int B, int T, int Hv, int dk, int dv, int N);
hipError_t launch_chunk_bwd(const BwdArgs& a);

// The same with the forward's input options: raw gates, q/k normalisation, a state pool.
struct BwdExArgs {
    BwdArgs base;                  // g, beta hold a, b with A_log; initial_state is the pool with state_indices
    const float* A_log;            // [Hv] or null
    const float* dt_bias;          // [Hv], with A_log
    const int32_t* state_indices;  // [N] or null
    int num_slots;
    int qk_l2norm;
    float* dA_log;                 // [Hv], with A_log
    float* ddt_bias;               // [Hv], with A_log
};
constexpr int kBwdExMaxHv = 2048;  // v-heads the raw-gate gradients support (one block's tile)
size_t chunk_bwd_ex_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N, bool raw_gates,
                                   bool pool, bool l2, gdn_dtype qkv_dtype);
hipError_t launch_chunk_bwd_ex(const BwdExArgs& a);

// Depthwise causal convolution with its carried input cache.
hipError_t launch_causal_conv1d(const ConvArgs& a);

// The gated output norm (one row per head vector).
hipError_t launch_gated_rmsnorm(const NormArgs& a);

// Token-serial kernel: the state stays in registers for all T tokens of a call.
hipError_t launch_recurrent(const RecurrentArgs& a);

// Chunked kernel with fp32 arithmetic throughout (used for fp32 inputs; no workspace).
hipError_t launch_chunk_f32(const ChunkArgs& a);

// Chunked kernels on bf16 matrix cores (bf16 inputs).
bool chunk_mfma_supported(int dk, int dv, gdn_dtype qkv_dtype);
size_t chunk_mfma_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N, bool norm = false);
// Stages of a chunked call: prepare (every chunk in parallel: log-decay sums and the per-chunk
// triangular solve, into the workspace) and scan (the chunks in order).  A full call runs both.
constexpr unsigned kStagePrepare = 1u, kStageScan = 2u;
hipError_t launch_chunk_mfma(const ChunkArgs& a, unsigned stages);

}  // namespace gdn
