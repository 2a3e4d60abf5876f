// chunk_f32.hip -- chunked gated delta rule with fp32 arithmetic throughout (fp32 inputs).
//
// One workgroup owns one (sequence, v-head, 32-column slice of the state) and walks the
// sequence's 64-token chunks in order.  Columns of the state never interact, so the slices are
// independent.  For a chunk with start state S (rows = key dim, columns = the slice), G_t the
// running sum of g inside the chunk and every decay factor formed as exp of a non-positive number:
//
//   A_tj = beta_t (k_t . k_j) e^(G_t - G_j)   (j < t)      P_tj = (q_t . k_j) e^(G_t - G_j)  (j <= t)
//   T    = (I + A)^-1                          (forward substitution, one column per lane)
//   R    = diag(beta) (V - diag(e^G) K S)      U = T R      (the per-token deltas of the chunk)
//   O    = diag(e^G) Q S + P U                 S <- e^(G_C) S + K^T diag(e^(G_C - G)) U
//
// Unrolling the per-token rule over the chunk gives exactly these identities.  A short last chunk
// is zero-padded: padded tokens have beta = 0 and g = 0, which leave the state untouched.
//
// With qk_l2norm, each staged row of K and Q is scaled to unit length in LDS (fp32) first.
//
// All operands live in LDS (~125 KB at dk = 128).  This path favours plain, exact fp32 arithmetic
// over speed; bf16 inputs take the matrix-core kernels instead.

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;        // chunk length
constexpr int kWS = 32;       // state columns per workgroup
constexpr int kThreads = 256;

template <int DK>
constexpr size_t lds_floats() {
    return 2 * (size_t)kC * (DK + 1) + (size_t)DK * kWS + 2 * (size_t)kC * (kC + 1) +
           (size_t)kC * (kWS + 1) + 4 * kC;
}

template <int DK, typename TIn, typename TG>
__global__ __launch_bounds__(kThreads) void chunk_f32_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TG* __restrict__ g, const TG* __restrict__ beta, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const float* initial_state,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ state_indices,
    int num_slots, int T, int Hk, int Hv, int dv, int qk_l2norm,
    float* __restrict__ o, float* final_state) {
    constexpr int LDK = DK + 1, LC = kC + 1, LW = kWS + 1;
    extern __shared__ float smem[];
    float* sK = smem;             // kC x LDK
    float* sQ = sK + kC * LDK;    // kC x LDK
    float* sS = sQ + kC * LDK;    // DK x kWS (state slice)
    float* sT = sS + DK * kWS;    // kC x LC  (A, then T)
    float* sP = sT + kC * LC;     // kC x LC
    float* sU = sP + kC * LC;     // kC x LW  (V, then R, then U)
    float* sG = sU + kC * LW;     // kC running log-decay
    float* sB = sG + kC;          // kC beta
    float* sE = sB + kC;          // kC e^G
    float* sD = sE + kC;          // kC e^(G_C - G)

    const int slices = dv / kWS;
    int unit = blockIdx.x;
    const int sl = unit % slices;
    unit /= slices;
    const int h = unit % Hv, n = unit / Hv;
    const int kh = h / (Hv / Hk);
    int row, t0, t1;
    sequence_range(cu_seqlens, n, T, row, t0, t1);
    const int c0 = sl * kWS;
    const int tid = threadIdx.x;

    // the sequence's state: its own, or a pool slot (a padding row starts from zero, writes none)
    int sslot;
    const bool has_slot = state_slot(state_indices, num_slots, n, sslot);
    const float* s_in = has_slot ? initial_state : nullptr;
    float* s_out = has_slot ? final_state : nullptr;
    const size_t sbase = ((size_t)sslot * Hv + h) * DK * dv;
    for (int e = tid; e < DK * kWS; e += kThreads) {
        const int i = e / kWS, c = e % kWS;
        sS[e] = s_in ? s_in[sbase + (size_t)i * dv + c0 + c] : 0.f;
    }
    __syncthreads();

    for (int cs = t0; cs < t1; cs += kC) {
        const int L = min(kC, t1 - cs);
        const size_t tok0 = (size_t)row * T + cs;

        for (int e = tid; e < kC * DK; e += kThreads) {
            const int t = e / DK, i = e % DK;
            float kv = 0.f, qv = 0.f;
            if (t < L) {
                const size_t off = ((tok0 + t) * Hk + kh) * DK + i;
                kv = to_f32(k[off]);
                qv = to_f32(q[off]);
            }
            sK[t * LDK + i] = kv;
            sQ[t * LDK + i] = qv;
        }
        for (int e = tid; e < kC * kWS; e += kThreads) {
            const int t = e / kWS, c = e % kWS;
            sU[t * LW + c] = t < L ? to_f32(v[((tok0 + t) * Hv + h) * dv + c0 + c]) : 0.f;
        }
        if (tid < kC) {
            float gt = 0.f, bt = 0.f;
            if (tid < L)
                gate_values(to_f32(g[(tok0 + tid) * Hv + h]), to_f32(beta[(tok0 + tid) * Hv + h]), A_log,
                            dt_bias, h, gt, bt);
            sG[tid] = gt;
            sB[tid] = bt;
        }
        __syncthreads();
        if (qk_l2norm) {
            // 2 kC rows (K then Q), two threads per row, each over half of it
            const int r = tid >> 1, half = tid & 1;
            float* xr = (r < kC ? sK + r * LDK : sQ + (r - kC) * LDK) + half * (DK / 2);
            float ss = 0.f;
            for (int i = 0; i < DK / 2; ++i) ss += xr[i] * xr[i];
            ss += __shfl_xor(ss, 1);
            const float rn = 1.f / sqrtf(ss + kL2Eps);
            for (int i = 0; i < DK / 2; ++i) xr[i] *= rn;
            __syncthreads();
        }
        if (tid == 0) {
            float acc = 0.f;
            for (int t = 0; t < kC; ++t) {
                acc += sG[t];
                sG[t] = acc;
            }
        }
        __syncthreads();
        if (tid < kC) {
            sE[tid] = expf(sG[tid]);
            sD[tid] = expf(sG[kC - 1] - sG[tid]);
        }

        // A (strictly lower) and P (lower with diagonal).
        for (int e = tid; e < kC * kC; e += kThreads) {
            const int t = e / kC, j = e % kC;
            float a = 0.f, p = 0.f;
            if (j <= t) {
                float dkk = 0.f, dqk = 0.f;
                for (int i = 0; i < DK; ++i) {
                    const float kj = sK[j * LDK + i];
                    dkk += sK[t * LDK + i] * kj;
                    dqk += sQ[t * LDK + i] * kj;
                }
                const float dec = expf(sG[t] - sG[j]);
                p = dqk * dec;
                if (j < t) a = sB[t] * dkk * dec;
            }
            sT[t * LC + j] = a;
            sP[t * LC + j] = p;
        }
        __syncthreads();

        // T = (I + A)^-1: lane c of wave 0 computes column c by forward substitution.
        float x[kC];
        if (tid < kC) {
#pragma unroll
            for (int t = 0; t < kC; ++t) {
                float acc = (t == tid) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < t; ++j) acc -= sT[t * LC + j] * x[j];
                x[t] = acc;
            }
        }
        __syncthreads();
        if (tid < kC) {
#pragma unroll
            for (int t = 0; t < kC; ++t) sT[t * LC + tid] = x[t];
        }
        __syncthreads();

        // R = beta (V - e^G (K S)), in place over V.
        for (int e = tid; e < kC * kWS; e += kThreads) {
            const int t = e / kWS, c = e % kWS;
            float ks = 0.f;
            for (int i = 0; i < DK; ++i) ks += sK[t * LDK + i] * sS[i * kWS + c];
            sU[t * LW + c] = sB[t] * (sU[t * LW + c] - sE[t] * ks);
        }
        __syncthreads();

        // U = T R.
        constexpr int PER = kC * kWS / kThreads;
        float ur[PER];
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int e = tid + kThreads * r, t = e / kWS, c = e % kWS;
            float acc = 0.f;
            for (int j = 0; j <= t; ++j) acc += sT[t * LC + j] * sU[j * LW + c];
            ur[r] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int e = tid + kThreads * r, t = e / kWS, c = e % kWS;
            sU[t * LW + c] = ur[r];
        }
        __syncthreads();

        // O = e^G (Q S) + P U.
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int e = tid + kThreads * r, t = e / kWS, c = e % kWS;
            if (t < L) {
                float qs = 0.f, pu = 0.f;
                for (int i = 0; i < DK; ++i) qs += sQ[t * LDK + i] * sS[i * kWS + c];
                for (int j = 0; j <= t; ++j) pu += sP[t * LC + j] * sU[j * LW + c];
                o[((tok0 + t) * Hv + h) * dv + c0 + c] = sE[t] * qs + pu;
            }
        }
        __syncthreads();

        // S <- e^(G_C) S + K^T diag(e^(G_C - G)) U.
        const float eC = sE[kC - 1];
        for (int e = tid; e < DK * kWS; e += kThreads) {
            const int i = e / kWS, c = e % kWS;
            float acc = 0.f;
            for (int t = 0; t < kC; ++t) acc += sK[t * LDK + i] * sD[t] * sU[t * LW + c];
            sS[e] = eC * sS[e] + acc;
        }
        __syncthreads();
    }

    if (s_out) {
        for (int e = tid; e < DK * kWS; e += kThreads) {
            const int i = e / kWS, c = e % kWS;
            s_out[sbase + (size_t)i * dv + c0 + c] = sS[e];
        }
    }
}

template <int DK, typename TIn, typename TG>
hipError_t launch_typed(const ChunkArgs& a) {
    const auto kern = chunk_f32_kernel<DK, TIn, TG>;
    const size_t bytes = lds_floats<DK>() * sizeof(float);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(a.N * a.Hv * (a.dv / kWS))), block(kThreads);
    hipLaunchKernelGGL(kern, grid, block, bytes, a.stream, static_cast<const TIn*>(a.q),
                       static_cast<const TIn*>(a.k), static_cast<const TIn*>(a.v),
                       static_cast<const TG*>(a.g), static_cast<const TG*>(a.beta), a.A_log,
                       a.dt_bias, a.initial_state, a.cu_seqlens, a.state_indices, a.num_slots, a.T,
                       a.Hk, a.Hv, a.dv, a.qk_l2norm, a.o, a.final_state);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const ChunkArgs& a) {
    const bool in_bf16 = a.qkv_dtype == GDN_BF16, g_bf16 = a.gate_dtype == GDN_BF16;
    if (in_bf16 && g_bf16) return launch_typed<DK, bf16_t, bf16_t>(a);
    if (in_bf16) return launch_typed<DK, bf16_t, float>(a);
    if (g_bf16) return launch_typed<DK, float, bf16_t>(a);
    return launch_typed<DK, float, float>(a);
}

}  // namespace

hipError_t launch_chunk_f32(const ChunkArgs& a) {
    return a.dk == 128 ? launch_dk<128>(a) : launch_dk<64>(a);
}

}  // namespace gdn
