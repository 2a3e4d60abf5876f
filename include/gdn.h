/*
 * gdn.h -- C ABI of libgdn, the gated delta rule on AMD Instinct MI355X (gfx950).
 *
 * The operation.  Per (sequence, v-head) the library keeps a dk x dv fp32 state S and, for each
 * token t of the sequence in order, applies
 *
 *     S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,      o_t = S_t^T q_t
 *
 * i.e. decay the state, then correct it along the current key towards the current value with
 * strength beta, then read it out with the query (no query scale; the read-out includes token t).
 * This is the "delta rule state update and retrieval" of the Qwen3.5 Gated DeltaNet write-up
 * (wanger-sjtu.github.io, flowchart and section "Core mechanism: Gated DeltaNet": the state is
 * corrected along the current key instead of being accumulated), with the gates of the same
 * flowchart and of the Qwen3-Next architecture write-up (intelliparadigm.com, section 2.2):
 * beta = sigmoid(b) in (0,1) is the write strength and g = -exp(A_log) softplus(a + dt_bias) <= 0
 * is the log-decay.  Callers compute g and beta; the library takes them as inputs.
 *
 * The two entry points are the two modes of the Qwen3-Next Gated DeltaNet article (jsqmd.com,
 * section 2.2 "chunked parallel computation"): chunk_gated_delta_rule processes whole segments in
 * parallel chunks and returns the state to carry into the next segment; recurrent_gated_delta_rule
 * advances a cached state by one token at decode time.  The Qwen3.5 flowchart's "cache valid and
 * L = 1" switch picks between them; here the caller picks.
 *
 * Conventions shared by every call:
 *   - All tensor arguments are DEVICE pointers to contiguous row-major memory (innermost index
 *     last).  States, outputs and (for gdn_chunk_fwd) q, k, v must be 16-byte aligned; every other
 *     pointer needs only the alignment of its element type.  The caller owns every buffer; the
 *     library never allocates, frees or retains a pointer after the call returns.
 *   - q/k head sharing (grouped heads): v-head h reads q/k head h / (Hv / Hk) (v-heads 0..G-1 share
 *     q/k head 0, and so on, G = Hv / Hk).
 *   - Work is enqueued on `stream` and runs asynchronously; nothing synchronises.  A device fault
 *     surfaces at the caller's next synchronisation.  Calls on different streams are independent.
 *   - Arguments are checked on the host before anything is enqueued.  On any error the call
 *     returns a non-zero status and writes nothing.  Device memory is never read for validation:
 *     a cu_seqlens array that is not non-decreasing from 0 to T is a caller error with undefined
 *     results (but every kernel still stays inside the buffers the shapes describe).
 *   - NaN and Inf in inputs propagate to the outputs; they never stop a kernel.
 *   - Inputs are expected to satisfy g <= 0 and 0 <= beta <= 1 (the gates' ranges); q and k are
 *     used exactly as given (callers normalise them if their model does).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_SUCCESS = 0,
    GDN_ERROR_INVALID_VALUE = 1,    /* a null required pointer, a bad size or a bad combination */
    GDN_ERROR_NOT_SUPPORTED = 2,    /* valid, but a head size or dtype this build has no kernel for */
    GDN_ERROR_WORKSPACE = 3,        /* workspace pointer null or smaller than the size query says */
    GDN_ERROR_LAUNCH_FAILURE = 4,   /* the HIP runtime refused a launch (hipGetLastError) */
    GDN_STATUS_MAX_ENUM = 0x7fffffff  /* not a status: gives the type the range of a 32-bit int, so
                                         any int a caller passes is a valid value of it */
} gdn_status;

typedef enum {
    GDN_F32 = 0,                    /* IEEE binary32 */
    GDN_BF16 = 1,                   /* bfloat16 (upper half of binary32) */
    GDN_DTYPE_MAX_ENUM = 0x7fffffff /* not a dtype: as GDN_STATUS_MAX_ENUM (rejected by every call) */
} gdn_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* gdn_status_string(gdn_status status);

/* Library version as an integer: major * 10000 + minor * 100 + patch. */
int gdn_version(void);

/*
 * Bytes of device workspace gdn_chunk_fwd needs for these sizes (0 if none).  Pure host
 * arithmetic; never fails (returns 0 for sizes gdn_chunk_fwd would reject).
 */
size_t gdn_chunk_fwd_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                    gdn_dtype qkv_dtype);

/*
 * gdn_chunk_fwd -- chunk-parallel prefill (chunk_gated_delta_rule).
 *
 * Runs the rule above over every sequence and v-head and returns every token's output and every
 * sequence's final state.  Internally each sequence is cut into 64-token chunks (the last one may
 * be shorter); the result does not depend on the cut (up to rounding order).
 *
 * Inputs (device):
 *   q, k           [B, T, Hk, dk]  dtype qkv_dtype
 *   v              [B, T, Hv, dv]  dtype qkv_dtype
 *   g, beta        [B, T, Hv]      dtype gate_dtype
 *   initial_state  [N, Hv, dk, dv] fp32, or NULL for a zero initial state
 *   cu_seqlens     NULL: N == B and sequence n is batch row n (T tokens each).
 *                  Otherwise int32 [N+1] with B == 1: sequence n is tokens
 *                  [cu_seqlens[n], cu_seqlens[n+1]) of the packed T axis; cu_seqlens[0] == 0,
 *                  non-decreasing, cu_seqlens[N] == T.  Zero-length sequences are allowed (their
 *                  final state equals their initial state).  No chunk spans two sequences.
 *   (With T == 0 there are no tokens: q, k, v, g, beta and o may then be NULL.)
 * Outputs (device):
 *   o              [B, T, Hv, dv]  fp32; must not overlap any input
 *   final_state    [N, Hv, dk, dv] fp32; may be the same pointer as initial_state (the state is
 *                  then advanced in place), must not partially overlap it
 * Workspace (device): at least gdn_chunk_fwd_workspace_size(...) bytes, 256-byte aligned; may be
 *   NULL when that size is 0.  Its contents on entry do not matter; on return they are garbage.
 *   Two calls in flight at once need two workspaces.
 * Sizes: B >= 1, T >= 0, Hk >= 1, Hv >= 1 with Hv % Hk == 0, N >= 1; dk and dv each 64 or 128
 *   (other sizes: GDN_ERROR_NOT_SUPPORTED).  qkv_dtype and gate_dtype are GDN_BF16 or GDN_F32.
 * Precision: states and outputs are fp32 throughout.  bf16 inputs take the bf16 matrix-core path
 *   (fp32 accumulation, products that feed the output split into two bf16 terms); fp32 inputs take
 *   an fp32 path.
 */
gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v,
                         const void* g, const void* beta,
                         const float* initial_state, const int32_t* cu_seqlens,
                         int B, int T, int Hk, int Hv, int dk, int dv, int N,
                         gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                         float* o, float* final_state,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * gdn_chunk_fwd_noalloc -- gdn_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops, harnesses that forbid
 * hipMalloc).
 *
 * Arguments, checks and results are those of gdn_chunk_fwd on the same stream; the scratch between the
 * call's two phases comes from a static device array of GDN_NOALLOC_SCRATCH_BYTES (64 MiB) inside the
 * library instead of a caller's workspace.  Each GPU the library runs on holds its own copy of that
 * array until the process ends; nothing is allocated or freed by the call.  The array's address on a
 * device is looked up on the first call there (the stream must belong to the calling thread's current
 * device, else GDN_ERROR_INVALID_VALUE).
 *   - GDN_ERROR_WORKSPACE when gdn_chunk_fwd_workspace_size(...) for these sizes exceeds
 *     GDN_NOALLOC_SCRATCH_BYTES (e.g. more than about 11,600 tokens at 16 q/k and 32 v heads of 128).
 *   - Every call on one GPU shares that GPU's array, so two calls that overlap in time on one GPU
 *     (on different streams, or from different threads) race and give undefined results; calls
 *     ordered on one stream are safe.  The array keeps the last call's contents; no call depends on
 *     them.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
size_t gdn_chunk_fwd_noalloc_max_bytes(void);    /* GDN_NOALLOC_SCRATCH_BYTES, as built */
gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const void* g, const void* beta,
                                 const float* initial_state, const int32_t* cu_seqlens,
                                 int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                 gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                                 float* o, float* final_state,
                                 hipStream_t stream);

/*
 * gdn_chunk_fwd_prepare, gdn_chunk_fwd_scan -- the two halves of gdn_chunk_fwd.
 *
 * gdn_chunk_fwd(args) is exactly gdn_chunk_fwd_prepare(args) followed by gdn_chunk_fwd_scan(args)
 * on the same stream, with the same arguments and the same workspace.  prepare does the work that
 * is independent across chunks, every chunk at once (per-chunk log-decay sums and the chunk's
 * triangular solve, the UT/WY step of the jsqmd.com article's section 2.2 chunk form), and leaves
 * it in the workspace; scan walks each sequence's chunks in order and writes o and final_state.
 * The split exists so that a caller can time or schedule the two phases separately; between the
 * two calls the workspace must not be touched, and scan must not run before prepare has finished
 * on its stream.  Arguments, checks and status codes are those of gdn_chunk_fwd (both halves check
 * all of them).  For fp32 inputs prepare enqueues nothing and scan does the whole call.
 */
gdn_status gdn_chunk_fwd_prepare(const void* q, const void* k, const void* v,
                                 const void* g, const void* beta,
                                 const float* initial_state, const int32_t* cu_seqlens,
                                 int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                 gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                                 float* o, float* final_state,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);
gdn_status gdn_chunk_fwd_scan(const void* q, const void* k, const void* v,
                              const void* g, const void* beta,
                              const float* initial_state, const int32_t* cu_seqlens,
                              int B, int T, int Hk, int Hv, int dk, int dv, int N,
                              gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                              float* o, float* final_state,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * gdn_recurrent_step -- decode against a cached state (recurrent_gated_delta_rule).
 *
 * Advances B independent cached states by T tokens each (T == 1 is the usual decode step),
 * token by token, and writes each token's output.  The state is read once and written once per
 * call, in place.
 *
 * Inputs (device):
 *   q, k           [B, T, Hk, dk]  dtype qkv_dtype
 *   v              [B, T, Hv, dv]  dtype qkv_dtype
 *   g, beta        [B, T, Hv]      dtype gate_dtype
 * In/out (device):
 *   state          [B, Hv, dk, dv] fp32, updated in place
 * Output (device):
 *   o              [B, T, Hv, dv]  fp32; must not overlap any input or the state
 * Sizes: B >= 1, T >= 1, Hk >= 1, Hv >= 1 with Hv % Hk == 0; dk and dv each 64 or 128.
 */
gdn_status gdn_recurrent_step(const void* q, const void* k, const void* v,
                              const void* g, const void* beta,
                              float* state,
                              int B, int T, int Hk, int Hv, int dk, int dv,
                              gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                              float* o, hipStream_t stream);

/*
 * gdn_chunk_fwd_gating, gdn_recurrent_step_gating -- the same two calls with the gates formed inside
 * the kernels from the layer's raw per-token projections.
 *
 * The gate formulas are those of the Qwen3.5 flowchart (wanger-sjtu.github.io, "Core mechanism:
 * Gated DeltaNet") and of the Qwen3-Next write-up (intelliparadigm.com, section 2.2):
 *     beta = sigmoid(b),    g = -exp(A_log[h]) * softplus(a + dt_bias[h]),
 * evaluated in fp32 per (token, v-head) by the kernel that reads the gates, so the caller skips a
 * pass over [B, T, Hv] and never materialises g and beta.
 *
 * Arguments are those of gdn_chunk_fwd / gdn_recurrent_step with g, beta replaced by:
 *   a, b           [B, T, Hv]  dtype gate_dtype (device), the raw projections
 *   A_log, dt_bias [Hv]        fp32 (device), per v-head
 * Checks and status codes are those of the plain calls, plus GDN_ERROR_INVALID_VALUE for a null or
 * misaligned A_log / dt_bias.  Results equal the plain call's on g, beta computed by these formulas
 * in fp32.
 */
gdn_status gdn_chunk_fwd_gating(const void* q, const void* k, const void* v,
                                const void* a, const void* b,
                                const float* A_log, const float* dt_bias,
                                const float* initial_state, const int32_t* cu_seqlens,
                                int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                                float* o, float* final_state,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);
gdn_status gdn_recurrent_step_gating(const void* q, const void* k, const void* v,
                                     const void* a, const void* b,
                                     const float* A_log, const float* dt_bias,
                                     float* state,
                                     int B, int T, int Hk, int Hv, int dk, int dv,
                                     gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                                     float* o, hipStream_t stream);

/*
 * gdn_chunk_fwd_indexed, gdn_recurrent_step_indexed -- the two calls against a pool of cached
 * states, for continuous batching.
 *
 * The pages' decode loop (jsqmd.com, section 2.2) carries each request's state from one call to the
 * next, and the Qwen3.5 write-up ("Cache and state switching") keeps those states in a cache that the
 * serving side switches between requests.  Here the cache is one pool and each sequence (prefill)
 * or batch row (decode) names its slot:
 *   state_pool     [num_slots, Hv, dk, dv] fp32 (device), read and written in place
 *   state_indices  [N] int32 (device; N = number of sequences, B for decode): slot of each one
 * Sequence n starts from state_pool[state_indices[n]] and its final state is written back to the
 * same slot.  An index outside [0, num_slots) marks a padding row: prefill runs it from a zero state
 * and writes no state; decode leaves every state alone and writes zeros to the row's outputs.  The
 * valid indices of one call must be distinct (two rows on one slot race).  Slots not named are not
 * touched.  A prefill of a new request expects a zeroed slot.
 *
 * Other arguments, checks and status codes are those of gdn_chunk_fwd / gdn_recurrent_step
 * (gdn_chunk_fwd_indexed has no initial_state / final_state: the pool is both); in addition
 * num_slots >= 1 and a null or misaligned state_indices give GDN_ERROR_INVALID_VALUE.  The indices
 * themselves are read on the device only.
 */
gdn_status gdn_chunk_fwd_indexed(const void* q, const void* k, const void* v,
                                 const void* g, const void* beta,
                                 float* state_pool, const int32_t* state_indices, int num_slots,
                                 const int32_t* cu_seqlens,
                                 int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                 gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                                 float* o,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);
gdn_status gdn_recurrent_step_indexed(const void* q, const void* k, const void* v,
                                      const void* g, const void* beta,
                                      float* state_pool, const int32_t* state_indices, int num_slots,
                                      int B, int T, int Hk, int Hv, int dk, int dv,
                                      gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                                      float* o, hipStream_t stream);

/*
 * gdn_chunk_fwd_ex, gdn_recurrent_step_ex -- the two calls with every option at once: raw gates,
 * a state pool, and flags.
 *
 *   A_log, dt_bias   NULL: g and beta are the gates (gdn_chunk_fwd); both set: g and beta are the raw
 *                    projections a and b and the gates are formed as in gdn_chunk_fwd_gating
 *   state_indices    NULL: initial_state / final_state (chunk) or state (decode) are per sequence as
 *                    in the plain calls; set: they are one pool [num_slots, Hv, dk, dv] addressed as in
 *                    gdn_chunk_fwd_indexed (for the chunk call initial_state must equal final_state)
 *   flags            0 or GDN_FLAG_QK_L2NORM: q and k are normalised to unit length per (token,
 *                    q/k head) inside the kernels before the rule, q / sqrt(|q|^2 + 1e-6) and likewise
 *                    for k, in fp32 (the pages feed q and k to the rule without stating their scale;
 *                    the state correction along k is an exact partial overwrite only for unit keys)
 * Everything else, and every check and status code, is that of the plain calls; an unknown flag bit,
 * dt_bias without A_log, or a pool chunk call whose initial_state differs from final_state gives
 * GDN_ERROR_INVALID_VALUE.  With flags == 0 the results equal those of the matching plain, gating or
 * indexed call.
 */
#define GDN_FLAG_QK_L2NORM 1u
gdn_status gdn_chunk_fwd_ex(const void* q, const void* k, const void* v,
                            const void* g, const void* beta,
                            const float* A_log, const float* dt_bias,
                            const float* initial_state, float* final_state,
                            const int32_t* state_indices, int num_slots,
                            const int32_t* cu_seqlens,
                            int B, int T, int Hk, int Hv, int dk, int dv, int N,
                            gdn_dtype qkv_dtype, gdn_dtype gate_dtype, unsigned flags,
                            float* o,
                            void* workspace, size_t workspace_bytes,
                            hipStream_t stream);
gdn_status gdn_recurrent_step_ex(const void* q, const void* k, const void* v,
                                 const void* g, const void* beta,
                                 const float* A_log, const float* dt_bias,
                                 float* state, const int32_t* state_indices, int num_slots,
                                 int B, int T, int Hk, int Hv, int dk, int dv,
                                 gdn_dtype qkv_dtype, gdn_dtype gate_dtype, unsigned flags,
                                 float* o, hipStream_t stream);

/*
 * gdn_chunk_fwd_gated_norm -- the chunked prefill with the layer's gated output norm fused onto o.
 *
 * The Qwen3.5 Gated DeltaNet page (wanger-sjtu.github.io, flowchart nodes "AttnOut -> Norm",
 * "Z -> Norm" and section "Output and gated RMSNorm") feeds the rule's output straight into the
 * gated RMSNorm.  This call computes o as gdn_chunk_fwd_ex does (same options and flags) and, per
 * (token, v-head) row of dv channels, writes
 *     y = o / sqrt(mean(o^2) + eps) * weight * silu(z),     silu(z) = z / (1 + exp(-z)),
 * (gdn_gated_rmsnorm's formula, fp32 arithmetic) in place of o: o itself never reaches memory.
 *
 *   z       [B, T, Hv, dv] z_dtype (device), 16-byte aligned
 *   weight  [dv] fp32 (device), 16-byte aligned
 *   eps     >= 0 and finite
 *   y       [B, T, Hv, dv] y_dtype (device), 16-byte aligned; must not overlap any input
 * Everything else -- q, k, v, the gates (g, beta or the raw a, b with A_log and dt_bias), states,
 * state_indices, cu_seqlens, flags -- as in gdn_chunk_fwd_ex.
 * Workspace: gdn_chunk_fwd_gated_norm_workspace_size bytes, 256-byte aligned (0 only for rejected
 * sizes).  With bf16 q, k, v it holds gdn_chunk_fwd's scratch plus each row's sums of squares per
 * 16-channel slice; with fp32 inputs it holds o between the prefill and a separate norm pass.
 * Scheduling (bf16 inputs): the dv / 16 workgroups of one (sequence, v-head) trade their slices'
 * sums of squares while they run, so they must be able to run at the same time; the GPU dispatches
 * them close together, and on an otherwise busy GPU a workgroup that waits about a second for a
 * partner's sums gives up and writes NaN rows rather than hang.
 * Errors: those of gdn_chunk_fwd_ex, and GDN_ERROR_INVALID_VALUE for a null z, weight or y (T > 0),
 * a bad eps, dtype or alignment.
 */
size_t gdn_chunk_fwd_gated_norm_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                               gdn_dtype qkv_dtype);
gdn_status gdn_chunk_fwd_gated_norm(const void* q, const void* k, const void* v,
                                    const void* g, const void* beta,
                                    const float* A_log, const float* dt_bias,
                                    const float* initial_state, float* final_state,
                                    const int32_t* state_indices, int num_slots,
                                    const int32_t* cu_seqlens,
                                    const void* z, const float* weight, float eps,
                                    int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                    gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                                    gdn_dtype z_dtype, gdn_dtype y_dtype, unsigned flags,
                                    void* y,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * gdn_chunk_bwd -- the backward pass of gdn_chunk_fwd, for training: the gradients of a scalar loss
 * with respect to q, k, v, g, beta and the initial state, given its gradients d_o with respect to
 * o and d_final with respect to the final state.
 *
 * The Qwen3-Next article (jsqmd.com, section 2.2) names the chunked call as the training form of the
 * rule; this is its reverse: the chunk's products taken in reverse order (the UT/WY form of the
 * forward, differentiated), with the states at the chunk starts recomputed by a forward sweep.
 * fp32 arithmetic throughout.
 *
 * Inputs (device): q, k, v, g, beta, initial_state, cu_seqlens as in gdn_chunk_fwd (the gates as g
 * and beta; no pool); d_o [B, T, Hv, dv] fp32; d_final [N, Hv, dk, dv] fp32 or NULL (zero).
 * Outputs (device, fp32, every element written): d_q, d_k [B, T, Hk, dk] (summed over the v-heads
 * that share a q/k head); d_v [B, T, Hv, dv]; d_g, d_beta [B, T, Hv]; d_initial_state
 * [N, Hv, dk, dv] or NULL (not computed).
 * Workspace: gdn_chunk_bwd_workspace_size bytes, 256-byte aligned (per chunk: the state at its start,
 * the state gradient at its end, U and dY, and each 16-column slice's partial sums of dg and dbeta).
 * Sizes and dtypes as in gdn_chunk_fwd; dk and dv 64 or 128 (others: GDN_ERROR_NOT_SUPPORTED).
 * Alignment: q and k 16 bytes, every other pointer its element size.
 * Errors: GDN_ERROR_INVALID_VALUE for null or misaligned pointers, bad sizes or dtypes;
 * GDN_ERROR_WORKSPACE for a missing, short or misaligned workspace.
 */
size_t gdn_chunk_bwd_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N);
gdn_status gdn_chunk_bwd(const void* q, const void* k, const void* v,
                         const void* g, const void* beta,
                         const float* initial_state, const int32_t* cu_seqlens,
                         const float* d_o, const float* d_final,
                         int B, int T, int Hk, int Hv, int dk, int dv, int N,
                         gdn_dtype qkv_dtype, gdn_dtype gate_dtype,
                         float* d_q, float* d_k, float* d_v, float* d_g, float* d_beta,
                         float* d_initial_state,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * gdn_chunk_bwd_ex -- the backward pass of gdn_chunk_fwd_ex: the same gradients through the forward's
 * input options, so a layer that lets the library form its gates and normalise q and k trains
 * through the same call.
 *
 * The gate formulas are those of the Qwen3.5 flowchart (wanger-sjtu.github.io, "Core mechanism:
 * Gated DeltaNet") and of the Qwen3-Next write-up (intelliparadigm.com, section 2.2), differentiated:
 *     beta = sigmoid(b)                     ->  d_b = d_beta beta (1 - beta)
 *     g = -exp(A_log) softplus(a + dt_bias)  ->  d_a = d_g (-exp(A_log) sigmoid(a + dt_bias)),
 *                                              d_A_log[h] = sum over tokens of d_g g,
 *                                              d_dt_bias[h] = sum over tokens of d_a
 * and the q/k normalisation x^ = x / sqrt(|x|^2 + 1e-6) (GDN_FLAG_QK_L2NORM, as in gdn_chunk_fwd_ex):
 *     d_x = r d_x^ - r^3 (x . d_x^) x,   r = 1 / sqrt(|x|^2 + 1e-6).
 * The rule's own gradients are those of gdn_chunk_bwd on the formed gates and normalised q, k.
 *
 * Arguments are those of gdn_chunk_bwd plus:
 *   A_log, dt_bias   NULL: g and beta are the gates; both set: g and beta are the raw projections a
 *                    and b [B, T, Hv] (gate_dtype) and d_g, d_beta receive d_a, d_b
 *   d_A_log, d_dt_bias  [Hv] fp32 (device), written (not accumulated) when A_log is set, else unused
 *   state_indices    NULL: initial_state is per sequence as in gdn_chunk_bwd; set: initial_state is
 *                    the pool [num_slots, Hv, dk, dv] of gdn_chunk_fwd_ex (16-byte aligned) and
 *                    sequence n started from slot state_indices[n] (a zero state for an index outside
 *                    [0, num_slots), a padding row).  d_initial_state stays per sequence
 *                    [N, Hv, dk, dv]: the gradient with respect to the state each sequence started from.
 *   flags            0 or GDN_FLAG_QK_L2NORM (q, k are the raw vectors; d_q, d_k are with respect to them)
 * Workspace: gdn_chunk_bwd_ex_workspace_size bytes for the same sizes and options (raw_gates: A_log
 * set; pool: state_indices set), 256-byte aligned.  It adds to gdn_chunk_bwd's the formed gates, the
 * normalised q and k (and v widened to fp32 when q, k, v are bf16) and the gathered start states.
 * With no option set the call is gdn_chunk_bwd.  Determinism: d_A_log and d_dt_bias are summed in a
 * fixed order (per-block fp64 partial sums), so repeated calls give identical bits.
 * Errors: those of gdn_chunk_bwd, plus GDN_ERROR_INVALID_VALUE for an unknown flag bit, dt_bias without
 * A_log, A_log without d_A_log / d_dt_bias, a pool without initial_state or with num_slots < 1;
 * GDN_ERROR_NOT_SUPPORTED for raw gates with more than 2048 v-heads.
 */
size_t gdn_chunk_bwd_ex_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N,
                                       gdn_dtype qkv_dtype, int raw_gates, int pool, unsigned flags);
gdn_status gdn_chunk_bwd_ex(const void* q, const void* k, const void* v,
                            const void* g, const void* beta,
                            const float* A_log, const float* dt_bias,
                            const float* initial_state, const int32_t* state_indices, int num_slots,
                            const int32_t* cu_seqlens,
                            const float* d_o, const float* d_final,
                            int B, int T, int Hk, int Hv, int dk, int dv, int N,
                            gdn_dtype qkv_dtype, gdn_dtype gate_dtype, unsigned flags,
                            float* d_q, float* d_k, float* d_v, float* d_g, float* d_beta,
                            float* d_A_log, float* d_dt_bias, float* d_initial_state,
                            void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * gdn_gated_rmsnorm -- the layer's gated output norm, applied to the gated delta rule's output.
 *
 * The Qwen3.5 Gated DeltaNet page (wanger-sjtu.github.io, section "Output and gated RMSNorm", and
 * its flowchart nodes "AttnOut -> Norm", "Z -> Norm") sends the core output and the z branch into
 * one norm that normalises and then gates in the manner of SwiGLU.  Per row (one head vector of
 * d channels):
 *     y = x / sqrt(mean(x^2) + eps) * weight * silu(z),     silu(z) = z / (1 + exp(-z)),
 * in fp32 (the RMS normalisation as the Qwen3-Next article's section 3.2 writes it).
 *
 *   x       [rows, d] fp32 (device): e.g. o of gdn_chunk_fwd viewed as [B*T*Hv, dv]
 *   z       [rows, d] z_dtype (device)
 *   weight  [d] fp32 (device), per channel
 *   out     [rows, d] out_dtype (device); must not overlap x or z
 * Sizes: rows >= 0 (0: nothing is enqueued), d 64 or 128 (others: GDN_ERROR_NOT_SUPPORTED),
 * eps >= 0 and finite.  x and weight 16-byte aligned, z and out aligned to 4 elements.
 * Errors: GDN_ERROR_INVALID_VALUE for null pointers (rows > 0), bad sizes, dtypes or alignment.
 */
gdn_status gdn_gated_rmsnorm(const float* x, const void* z, const float* weight, float eps,
                             int64_t rows, int d, gdn_dtype z_dtype, gdn_dtype out_dtype,
                             void* out, hipStream_t stream);

/*
 * gdn_causal_conv1d -- the depthwise causal convolution of the QKV mixture, with its cache.
 *
 * The Qwen3.5 Gated DeltaNet page (wanger-sjtu.github.io) sends the QKV mixture (2K + V channels)
 * through "conv1d, Depthwise Causal Conv" before splitting it into q, k, v; the decode path reads the
 * conv_states cache and the layer then updates it ("Update Conv Cache").  Per sequence n and channel
 * c, with xp = [cache_n; x_n] (the W - 1 inputs before the sequence, oldest first, then its own):
 *     y[t, c] = act(sum_j weight[c, j] * xp[t + j, c] + bias[c])
 * and the cache of n becomes the last W - 1 rows of xp.  A prefill is one call over whole sequences,
 * a decode step the same call with T == 1.  The kernel width differs across the pages (4, 8, 12-16
 * by context length on one, 5 on another), so W (1 .. 16) is an argument.  The pages name no
 * activation: silu = 0 gives none; silu != 0 applies act(u) = u / (1 + exp(-u)).  fp32 arithmetic.
 *
 *   x           [B, T, C] x_dtype (device); packed sequences with cu_seqlens use B == 1
 *   weight      [C, W] fp32 (device); weight[c, W - 1] multiplies the current input
 *   bias        [C] fp32 (device) or NULL
 *   conv_state  [N, W - 1, C] x_dtype (device) or NULL (zeros in, nothing written); with
 *               state_indices, a pool [num_slots, W - 1, C] whose slot state_indices[n] serves
 *               sequence n (an index outside [0, num_slots): zeros in, nothing written).  Updated in
 *               place for every sequence with at least one token; the valid indices must be distinct.
 *               With W == 1 there is no history: conv_state and state_indices are ignored.
 *   cu_seqlens  [N + 1] int32 (device) or NULL (then N == B, sequence b = batch row b)
 *   y           [B, T, C] x_dtype (device); must not overlap x or the cache
 * Sizes: C a multiple of 4, W 1 .. 16 (others: GDN_ERROR_NOT_SUPPORTED), T >= 0.  x, y and
 * conv_state aligned to 4 elements, bias to 16 bytes.
 */
gdn_status gdn_causal_conv1d(const void* x, const float* weight, const float* bias,
                             void* conv_state, const int32_t* state_indices, int num_slots,
                             const int32_t* cu_seqlens, int B, int T, int C, int W, int N,
                             gdn_dtype x_dtype, int silu, void* y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
