// chunk_bwd_ex.hip -- backward pass of the chunked call with its input options: gates formed from
// the raw projections, q/k normalised to unit length, initial states taken from a pool.
//
// The options are steps in front of the rule, so their backward is the chain rule around the
// rule's own backward (chunk_bwd.hip), run unchanged on the transformed inputs:
//   before  g, beta from a, b (the same fp32 formula the forward kernels evaluate); q^ = q r and
//           k^ = k r with r = 1 / sqrt(|x|^2 + eps) as fp32 (and v widened to fp32 beside them, since
//           the rule's backward takes one input type); each sequence's start state gathered from its
//           pool slot (zeros for a padding row)
//   after   beta = sigmoid(b):                    db = dbeta beta (1 - beta)
//           g = -exp(A_log) softplus(a + dt_bias): da = dg (-exp(A_log) sigmoid(a + dt_bias)),
//                                                  dA_log = sum over tokens of dg g, ddt_bias = sum da
//           x^ = x r:                              dx = r dx^ - r^3 (x . dx^) x
// The per-head sums are taken in a fixed order (per-block partial sums in fp64, then one pass over
// the blocks), so results are bitwise reproducible.

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kGateRows = kBwdExMaxHv;   // (rows x v-heads) elements per gate-gradient block, at most

size_t align256b(size_t x) { return (x + 255) & ~(size_t)255; }

// Tokens of batch row 0 outside every packed sequence carry no gradient (the packed layout has
// B == 1 and its sequences are contiguous, from cu_seqlens[0] to cu_seqlens[N]).
__device__ __forceinline__ bool outside(const int32_t* cu_seqlens, int N, long long row) {
    return cu_seqlens && (row < cu_seqlens[0] || row >= cu_seqlens[N]);
}

// g and beta of every (token, v-head) from the raw projections, as fp32.
template <typename TG>
__global__ __launch_bounds__(kThreads) void bwd_ex_gates_kernel(const TG* __restrict__ a,
                                                                const TG* __restrict__ b,
                                                                const float* __restrict__ A_log,
                                                                const float* __restrict__ dt_bias, long long n,
                                                                int Hv, float* __restrict__ g,
                                                                float* __restrict__ beta) {
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    float gi, bi;
    gate_values(to_f32(a[i]), to_f32(b[i]), A_log, dt_bias, (int)(i % Hv), gi, bi);
    g[i] = gi;
    beta[i] = bi;
}

// One wave per head vector of D elements (D = 64 or 128): x / sqrt(|x|^2 + eps) as fp32.
template <int D, typename TIn>
__global__ __launch_bounds__(kThreads) void bwd_ex_l2norm_kernel(const TIn* __restrict__ x, long long vecs,
                                                                 float* __restrict__ y) {
    constexpr int E = D / kWave;
    const long long vec = (long long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (vec >= vecs) return;
    const TIn* p = x + vec * D + lane * E;
    float v[E], ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        v[e] = to_f32(p[e]);
        ss += v[e] * v[e];
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) ss += __shfl_xor(ss, off);
    const float r = 1.f / sqrtf(ss + kL2Eps);
#pragma unroll
    for (int e = 0; e < E; ++e) y[vec * D + lane * E + e] = v[e] * r;
}

// The same vectors' gradients, in place: dx = r dx^ - r^3 (x . dx^) x.
template <int D, typename TIn>
__global__ __launch_bounds__(kThreads) void bwd_ex_l2norm_grad_kernel(const TIn* __restrict__ x, long long vecs,
                                                                      int H, const int32_t* __restrict__ cu_seqlens,
                                                                      int N, float* __restrict__ dx) {
    constexpr int E = D / kWave;
    const long long vec = (long long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (vec >= vecs) return;
    const TIn* p = x + vec * D + lane * E;
    float* d = dx + vec * D + lane * E;
    float v[E], dn[E], ss = 0.f, xd = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        v[e] = to_f32(p[e]);
        dn[e] = d[e];
        ss += v[e] * v[e];
        xd += v[e] * dn[e];
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        ss += __shfl_xor(ss, off);
        xd += __shfl_xor(xd, off);
    }
    const float r = 1.f / sqrtf(ss + kL2Eps), c = r * r * r * xd;
    const bool out = outside(cu_seqlens, N, vec / H);
#pragma unroll
    for (int e = 0; e < E; ++e) d[e] = out ? 0.f : r * dn[e] - c * v[e];
}

// Widening copy of v (bf16 -> fp32), 4 elements per thread (every tensor here holds a multiple of 4;
// v is only 2-byte aligned, so its elements are read one by one).
__global__ __launch_bounds__(kThreads) void bwd_ex_widen_kernel(const bf16_t* __restrict__ x, long long n4,
                                                                float* __restrict__ y) {
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n4) return;
    const bf16_t* p = x + 4 * i;
    reinterpret_cast<float4*>(y)[i] = make_float4(to_f32(p[0]), to_f32(p[1]), to_f32(p[2]), to_f32(p[3]));
}

// Start state of every (sequence, v-head) from its pool slot, zeros for a padding row.
__global__ __launch_bounds__(kThreads) void bwd_ex_gather_kernel(const float* __restrict__ pool,
                                                                 const int32_t* __restrict__ state_indices,
                                                                 int num_slots, int Hv, int per_state4,
                                                                 float* __restrict__ s0) {
    const int n = blockIdx.x / Hv, h = blockIdx.x % Hv;
    int slot;
    const bool ok = state_slot(state_indices, num_slots, n, slot);
    const float4* src = reinterpret_cast<const float4*>(pool) + ((size_t)slot * Hv + h) * per_state4;
    float4* dst = reinterpret_cast<float4*>(s0) + (size_t)blockIdx.x * per_state4;
    for (int i = threadIdx.x; i < per_state4; i += kThreads) dst[i] = ok ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

// Gradients of the raw projections, in place over dg and dbeta, and per-block fp64 partial sums of
// dg * g (towards dA_log) and da (towards ddt_bias) for each v-head.  Block j covers rows
// [j * rows_per_block, ...) of the [rows, Hv] layout.
template <typename TG>
__global__ __launch_bounds__(kThreads) void bwd_ex_gates_grad_kernel(
    const TG* __restrict__ a, const TG* __restrict__ b, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const int32_t* __restrict__ cu_seqlens, int N, long long rows, int Hv,
    int rows_per_block, float* __restrict__ dg, float* __restrict__ dbeta, double* __restrict__ partial) {
    __shared__ double s_lg[kGateRows], s_lt[kGateRows];
    const long long r0 = (long long)blockIdx.x * rows_per_block;
    const long long r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;
    const long long e0 = r0 * Hv, ne = (r1 - r0) * Hv;
    for (long long j = threadIdx.x; j < ne; j += kThreads) {
        const long long i = e0 + j;
        const int h = (int)(i % Hv);
        const float z = to_f32(a[i]) + dt_bias[h];
        const float ea = expf(A_log[h]);
        const float sp = fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
        const float g = -ea * sp;
        const float bt = 1.f / (1.f + expf(-to_f32(b[i])));
        const bool out = outside(cu_seqlens, N, i / Hv);
        const float dgi = out ? 0.f : dg[i];
        const float da = dgi * (-ea / (1.f + expf(-z)));
        const float db = out ? 0.f : dbeta[i] * bt * (1.f - bt);
        dg[i] = da;
        dbeta[i] = db;
        s_lg[j] = out ? 0.0 : (double)dgi * (double)g;
        s_lt[j] = (double)da;
    }
    __syncthreads();
    for (int h = threadIdx.x; h < Hv; h += kThreads) {
        double sg = 0.0, st = 0.0;
        for (long long r = 0; r < r1 - r0; ++r) {
            sg += s_lg[r * Hv + h];
            st += s_lt[r * Hv + h];
        }
        partial[((size_t)blockIdx.x * Hv + h) * 2] = sg;
        partial[((size_t)blockIdx.x * Hv + h) * 2 + 1] = st;
    }
}

// dA_log and ddt_bias: the blocks' partial sums in block order.
__global__ __launch_bounds__(kThreads) void bwd_ex_gates_reduce_kernel(const double* __restrict__ partial,
                                                                       int blocks, int Hv,
                                                                       float* __restrict__ dA_log,
                                                                       float* __restrict__ ddt_bias) {
    const int h = blockIdx.x * kThreads + threadIdx.x;
    if (h >= Hv) return;
    double sg = 0.0, st = 0.0;
    for (int j = 0; j < blocks; ++j) {
        sg += partial[((size_t)j * Hv + h) * 2];
        st += partial[((size_t)j * Hv + h) * 2 + 1];
    }
    dA_log[h] = (float)sg;
    ddt_bias[h] = (float)st;
}

struct ExLayout {
    size_t g, beta, q, k, v, s0, partial, total;
    int gate_rows_per_block, gate_blocks;
};

ExLayout ex_layout(int B, int T, int Hk, int Hv, int dk, int dv, int N, bool raw_gates, bool pool, bool l2,
                   gdn_dtype qkv_dtype) {
    ExLayout l{};
    const size_t rows = (size_t)B * T;
    size_t off = align256b(chunk_bwd_workspace_size(B, T, Hv, dk, dv, N));
    l.gate_rows_per_block = kGateRows / Hv > 0 ? kGateRows / Hv : 1;
    l.gate_blocks = (int)((rows + l.gate_rows_per_block - 1) / l.gate_rows_per_block);
    if (raw_gates) {
        l.g = off;       off = align256b(off + sizeof(float) * rows * Hv);
        l.beta = off;    off = align256b(off + sizeof(float) * rows * Hv);
        l.partial = off; off = align256b(off + sizeof(double) * 2 * (size_t)l.gate_blocks * Hv);
    }
    if (l2) {
        l.q = off; off = align256b(off + sizeof(float) * rows * Hk * dk);
        l.k = off; off = align256b(off + sizeof(float) * rows * Hk * dk);
        if (qkv_dtype == GDN_BF16) {
            l.v = off; off = align256b(off + sizeof(float) * rows * Hv * dv);
        }
    }
    if (pool) {
        l.s0 = off; off = align256b(off + sizeof(float) * (size_t)N * Hv * dk * dv);
    }
    l.total = off;
    return l;
}

unsigned blocks_for(long long n, int per_block) { return (unsigned)((n + per_block - 1) / per_block); }

template <int D>
hipError_t l2norm_launch(const void* x, gdn_dtype t, long long vecs, float* y, hipStream_t s) {
    const unsigned grid = blocks_for(vecs, kThreads / kWave);
    if (t == GDN_BF16)
        hipLaunchKernelGGL((bwd_ex_l2norm_kernel<D, bf16_t>), dim3(grid), dim3(kThreads), 0, s,
                           static_cast<const bf16_t*>(x), vecs, y);
    else
        hipLaunchKernelGGL((bwd_ex_l2norm_kernel<D, float>), dim3(grid), dim3(kThreads), 0, s,
                           static_cast<const float*>(x), vecs, y);
    return hipGetLastError();
}

template <int D>
hipError_t l2norm_grad_launch(const void* x, gdn_dtype t, long long vecs, int H, const int32_t* cu, int N,
                              float* dx, hipStream_t s) {
    const unsigned grid = blocks_for(vecs, kThreads / kWave);
    if (t == GDN_BF16)
        hipLaunchKernelGGL((bwd_ex_l2norm_grad_kernel<D, bf16_t>), dim3(grid), dim3(kThreads), 0, s,
                           static_cast<const bf16_t*>(x), vecs, H, cu, N, dx);
    else
        hipLaunchKernelGGL((bwd_ex_l2norm_grad_kernel<D, float>), dim3(grid), dim3(kThreads), 0, s,
                           static_cast<const float*>(x), vecs, H, cu, N, dx);
    return hipGetLastError();
}

}  // namespace

size_t chunk_bwd_ex_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N, bool raw_gates,
                                   bool pool, bool l2, gdn_dtype qkv_dtype) {
    return ex_layout(B, T, Hk, Hv, dk, dv, N, raw_gates, pool, l2, qkv_dtype).total;
}

hipError_t launch_chunk_bwd_ex(const BwdExArgs& x) {
    const BwdArgs& a = x.base;
    const bool raw = x.A_log != nullptr, pool = x.state_indices != nullptr, l2 = x.qk_l2norm != 0;
    const ExLayout lay = ex_layout(a.B, a.T, a.Hk, a.Hv, a.dk, a.dv, a.N, raw, pool, l2, a.qkv_dtype);
    char* ws = static_cast<char*>(a.workspace);
    const long long rows = (long long)a.B * a.T;
    BwdArgs r = a;
    hipError_t e;
    if (raw && rows > 0) {
        float* g = reinterpret_cast<float*>(ws + lay.g);
        float* beta = reinterpret_cast<float*>(ws + lay.beta);
        const long long n = rows * a.Hv;
        if (a.gate_dtype == GDN_BF16)
            hipLaunchKernelGGL((bwd_ex_gates_kernel<bf16_t>), dim3(blocks_for(n, kThreads)), dim3(kThreads), 0,
                               a.stream, static_cast<const bf16_t*>(a.g), static_cast<const bf16_t*>(a.beta),
                               x.A_log, x.dt_bias, n, a.Hv, g, beta);
        else
            hipLaunchKernelGGL((bwd_ex_gates_kernel<float>), dim3(blocks_for(n, kThreads)), dim3(kThreads), 0,
                               a.stream, static_cast<const float*>(a.g), static_cast<const float*>(a.beta),
                               x.A_log, x.dt_bias, n, a.Hv, g, beta);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        r.g = g;
        r.beta = beta;
        r.gate_dtype = GDN_F32;
    }
    if (l2 && rows > 0) {
        float* qn = reinterpret_cast<float*>(ws + lay.q);
        float* kn = reinterpret_cast<float*>(ws + lay.k);
        const long long vecs = rows * a.Hk;
        for (int i = 0; i < 2; ++i) {
            const void* src = i == 0 ? a.q : a.k;
            float* dst = i == 0 ? qn : kn;
            e = a.dk == 128 ? l2norm_launch<128>(src, a.qkv_dtype, vecs, dst, a.stream)
                            : l2norm_launch<64>(src, a.qkv_dtype, vecs, dst, a.stream);
            if (e != hipSuccess) return e;
        }
        r.q = qn;
        r.k = kn;
        if (a.qkv_dtype == GDN_BF16) {
            float* vf = reinterpret_cast<float*>(ws + lay.v);
            const long long n4 = rows * a.Hv * a.dv / 4;
            hipLaunchKernelGGL(bwd_ex_widen_kernel, dim3(blocks_for(n4, kThreads)), dim3(kThreads), 0, a.stream,
                               static_cast<const bf16_t*>(a.v), n4, vf);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            r.v = vf;
        }
        r.qkv_dtype = GDN_F32;
    }
    if (pool) {
        float* s0 = reinterpret_cast<float*>(ws + lay.s0);
        hipLaunchKernelGGL(bwd_ex_gather_kernel, dim3((unsigned)(a.N * a.Hv)), dim3(kThreads), 0, a.stream,
                           a.initial_state, x.state_indices, x.num_slots, a.Hv, a.dk * a.dv / 4, s0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        r.initial_state = s0;
    }
    if ((e = launch_chunk_bwd(r)) != hipSuccess) return e;
    if (l2 && rows > 0) {
        const long long vecs = rows * a.Hk;
        for (int i = 0; i < 2; ++i) {
            const void* src = i == 0 ? a.q : a.k;
            float* d = i == 0 ? a.dq : a.dk_out;
            e = a.dk == 128 ? l2norm_grad_launch<128>(src, a.qkv_dtype, vecs, a.Hk, a.cu_seqlens, a.N, d, a.stream)
                            : l2norm_grad_launch<64>(src, a.qkv_dtype, vecs, a.Hk, a.cu_seqlens, a.N, d, a.stream);
            if (e != hipSuccess) return e;
        }
    }
    if (raw) {
        double* partial = reinterpret_cast<double*>(ws + lay.partial);
        if (rows > 0) {
            if (a.gate_dtype == GDN_BF16)
                hipLaunchKernelGGL((bwd_ex_gates_grad_kernel<bf16_t>), dim3((unsigned)lay.gate_blocks), dim3(kThreads),
                                   0, a.stream, static_cast<const bf16_t*>(a.g), static_cast<const bf16_t*>(a.beta),
                                   x.A_log, x.dt_bias, a.cu_seqlens, a.N, rows, a.Hv, lay.gate_rows_per_block, a.dg,
                                   a.dbeta, partial);
            else
                hipLaunchKernelGGL((bwd_ex_gates_grad_kernel<float>), dim3((unsigned)lay.gate_blocks), dim3(kThreads),
                                   0, a.stream, static_cast<const float*>(a.g), static_cast<const float*>(a.beta),
                                   x.A_log, x.dt_bias, a.cu_seqlens, a.N, rows, a.Hv, lay.gate_rows_per_block, a.dg,
                                   a.dbeta, partial);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        hipLaunchKernelGGL(bwd_ex_gates_reduce_kernel, dim3(blocks_for(a.Hv, kThreads)), dim3(kThreads), 0, a.stream,
                           partial, rows > 0 ? lay.gate_blocks : 0, a.Hv, x.dA_log, x.ddt_bias);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gdn
