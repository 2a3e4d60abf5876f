// recurrent.hip -- token-serial gated delta rule with the state held in registers.
//
// Serves gdn_recurrent_step (decode: T == 1 per call, or a few tokens).  One workgroup of 512
// threads owns one (sequence, v-head) state of DK x DV fp32 values; each thread holds a 4-column
// float4 strip of RPT rows in registers, so the state is read from HBM once and written once per
// call.  Per token:
//
//     a = exp(g);  p = S^T k;  u = beta (v - a p);  o = a S^T q + u (k . q);  S = a S + k u^T
//
// which is the decay -> predict -> correct -> read order of the rule with the two column
// reductions (S^T k and S^T q) taken from the same register pass over the old state.  With
// qk_l2norm, the staged q and k are first scaled to unit length in LDS (fp32).
//
// Memory pattern: rows of S are DV floats; a wave covers whole rows with 16-byte loads, so every
// load/store instruction of a wave touches 64 x 16 B of contiguous memory.  The work is ~1 flop
// per byte moved: the kernel is bound by HBM bandwidth.  The state is read and written with
// non-temporal accesses: each (sequence, head) state is touched once per call, and streaming it
// past the caches measured faster for this read-then-write-back pattern.

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kRecThreads = 512;

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int DK, int DV, typename TIn, typename TG>
__global__ __launch_bounds__(kRecThreads) void recurrent_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TG* __restrict__ g, const TG* __restrict__ beta, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, float* __restrict__ state,
    const int32_t* __restrict__ state_indices, int num_slots, float* __restrict__ o, int T, int Hk,
    int Hv, int qk_l2norm) {
    constexpr int CG = DV / 4;               // float4 column groups per row
    constexpr int RG = kRecThreads / CG;     // row groups
    constexpr int RPT = DK / RG;             // rows held per thread
    constexpr int NW = kRecThreads / kWave;  // waves per workgroup
    static_assert(DK % RG == 0 && RPT >= 1, "row split");
    static_assert(CG <= kWave && kWave % CG == 0, "column groups must tile a wave");

    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int lane = tid % kWave, wave = tid / kWave;
    const int bh = blockIdx.x;  // b * Hv + h
    const int b = bh / Hv, h = bh % Hv;
    const int kh = h / (Hv / Hk);
    int slot;  // the row's state: its own, or a pool slot
    if (!state_slot(state_indices, num_slots, b, slot)) {
        // a padding row: no state to advance; its outputs are zero
        for (int t = 0; t < T; ++t)
            for (int e = tid; e < DV; e += kRecThreads) o[(((size_t)b * T + t) * Hv + h) * DV + e] = 0.f;
        return;
    }

    __shared__ float sq[DK], sk[DK], sv[DV];
    __shared__ float red[NW][2 * DV + 1];

    f32x4v* S4 = reinterpret_cast<f32x4v*>(state + ((size_t)slot * Hv + h) * DK * DV);
    f32x4v s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) s[m] = __builtin_nontemporal_load(S4 + (size_t)(rg + RG * m) * CG + cg);

    for (int t = 0; t < T; ++t) {
        const size_t tok = (size_t)b * T + t;
        if (tid < DK) {
            sq[tid] = to_f32(q[(tok * Hk + kh) * DK + tid]);
            sk[tid] = to_f32(k[(tok * Hk + kh) * DK + tid]);
        }
        if (tid < DV) sv[tid] = to_f32(v[(tok * Hv + h) * DV + tid]);
        float gt, bt;
        gate_values(to_f32(g[tok * Hv + h]), to_f32(beta[tok * Hv + h]), A_log, dt_bias, h, gt, bt);
        __syncthreads();
        if (qk_l2norm) {
            if (wave < 2) {                              // wave 0 scales k, wave 1 q
                float* x = wave == 0 ? sk : sq;
                float ss = 0.f;
                for (int i = lane; i < DK; i += kWave) ss += x[i] * x[i];
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) ss += __shfl_xor(ss, off);
                const float rn = 1.f / sqrtf(ss + kL2Eps);
                for (int i = lane; i < DK; i += kWave) x[i] *= rn;
            }
            __syncthreads();
        }

        // Partial column sums over this thread's rows.
        float pk0 = 0.f, pk1 = 0.f, pk2 = 0.f, pk3 = 0.f;
        float pq0 = 0.f, pq1 = 0.f, pq2 = 0.f, pq3 = 0.f, kq = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            const float ki = sk[i], qi = sq[i];
            pk0 += s[m].x * ki; pk1 += s[m].y * ki; pk2 += s[m].z * ki; pk3 += s[m].w * ki;
            pq0 += s[m].x * qi; pq1 += s[m].y * qi; pq2 += s[m].z * qi; pq3 += s[m].w * qi;
            kq += ki * qi;
        }
        // Sum over the row groups inside the wave (lanes that differ only in row-group bits).
#pragma unroll
        for (int off = CG; off < kWave; off <<= 1) {
            pk0 += __shfl_xor(pk0, off); pk1 += __shfl_xor(pk1, off);
            pk2 += __shfl_xor(pk2, off); pk3 += __shfl_xor(pk3, off);
            pq0 += __shfl_xor(pq0, off); pq1 += __shfl_xor(pq1, off);
            pq2 += __shfl_xor(pq2, off); pq3 += __shfl_xor(pq3, off);
            kq += __shfl_xor(kq, off);
        }
        if (lane < CG) {
            float* r = red[wave];
            r[cg * 4 + 0] = pk0; r[cg * 4 + 1] = pk1; r[cg * 4 + 2] = pk2; r[cg * 4 + 3] = pk3;
            r[DV + cg * 4 + 0] = pq0; r[DV + cg * 4 + 1] = pq1;
            r[DV + cg * 4 + 2] = pq2; r[DV + cg * 4 + 3] = pq3;
            if (lane == 0) r[2 * DV] = kq;
        }
        __syncthreads();

        float PK[4] = {0.f, 0.f, 0.f, 0.f}, PQ[4] = {0.f, 0.f, 0.f, 0.f}, KQ = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                PK[c] += red[w][cg * 4 + c];
                PQ[c] += red[w][DV + cg * 4 + c];
            }
            KQ += red[w][2 * DV];
        }
        const float a = expf(gt);
        float u[4], out[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            u[c] = bt * (sv[cg * 4 + c] - a * PK[c]);
            out[c] = a * PQ[c] + u[c] * KQ;
        }
        if (rg == 0) {
            float4* o4 = reinterpret_cast<float4*>(o + (tok * Hv + h) * DV);
            o4[cg] = make_float4(out[0], out[1], out[2], out[3]);
        }
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float ki = sk[rg + RG * m];
            s[m].x = a * s[m].x + ki * u[0];
            s[m].y = a * s[m].y + ki * u[1];
            s[m].z = a * s[m].z + ki * u[2];
            s[m].w = a * s[m].w + ki * u[3];
        }
        __syncthreads();  // the staging buffers are rewritten by the next token
    }

#pragma unroll
    for (int m = 0; m < RPT; ++m) __builtin_nontemporal_store(s[m], S4 + (size_t)(rg + RG * m) * CG + cg);
}

template <int DK, int DV, typename TIn, typename TG>
hipError_t launch_typed(const RecurrentArgs& a) {
    const dim3 grid((unsigned)(a.B * a.Hv)), block(kRecThreads);
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, TIn, TG>), grid, block, 0, a.stream,
                       static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.v), static_cast<const TG*>(a.g),
                       static_cast<const TG*>(a.beta), a.A_log, a.dt_bias, a.state, a.state_indices,
                       a.num_slots, a.o, a.T, a.Hk, a.Hv, a.qk_l2norm);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const RecurrentArgs& a) {
    const bool in_bf16 = a.qkv_dtype == GDN_BF16, g_bf16 = a.gate_dtype == GDN_BF16;
    if (in_bf16 && g_bf16) return launch_typed<DK, DV, bf16_t, bf16_t>(a);
    if (in_bf16) return launch_typed<DK, DV, bf16_t, float>(a);
    if (g_bf16) return launch_typed<DK, DV, float, bf16_t>(a);
    return launch_typed<DK, DV, float, float>(a);
}

}  // namespace

hipError_t launch_recurrent(const RecurrentArgs& a) {
    if (a.dk == 128 && a.dv == 128) return launch_dims<128, 128>(a);
    if (a.dk == 128 && a.dv == 64) return launch_dims<128, 64>(a);
    if (a.dk == 64 && a.dv == 128) return launch_dims<64, 128>(a);
    return launch_dims<64, 64>(a);
}

}  // namespace gdn
