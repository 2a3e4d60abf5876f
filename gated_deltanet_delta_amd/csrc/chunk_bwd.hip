// chunk_bwd.hip -- backward pass of the chunked gated delta rule (fp32 arithmetic).
//
// Per 64-token chunk with start state S, G the running sum of g inside the chunk, gamma = e^G,
// f = e^(G_C - G), Gam_tj = e^(G_t - G_j), the forward is
//     Bm = (K K^T) o Gam (j < t)     T = (I + diag(beta) Bm)^-1
//     X  = V - diag(gamma) K S       U = T diag(beta) X
//     P  = (Q K^T) o Gam (j <= t)    O = diag(gamma) Q S + P U
//     S' = gamma_C S + K^T diag(f) U
// and, given dO and D = dL/dS', the reverse of those products:
//     dU = P^T dO + diag(f) K D       dY = T^T dU        dX = diag(beta) dY = dV
//     dA = -(dY U^T) (j < t)           (the product T^T dT T^T with dT = dU Y^T, Y = diag(beta) X)
//     dBm = diag(beta) dA              dP = (dO U^T) (j <= t)
//     dQ = diag(gamma) dO S^T + (dP o Gam) K
//     dK = (dP o Gam)^T Q + diag(f) U D^T - diag(gamma) dX S^T + ((dBm o Gam) + (dBm o Gam)^T) K
//     dbeta_t = X_t . dY_t + sum_j dA_tj Bm_tj
//     dG_t = gamma_t (QS)_t . dO_t - gamma_t (KS)_t . dX_t - f_t (KD)_t . U_t + rows - columns of
//            (dP o P + dBm o Bm);   dG_(C-1) += gamma_C <S, D> + sum_t f_t (KD)_t . U_t
//     dg = the reverse running sum of dG;   dL/dS = gamma_C D + Q^T diag(gamma) dO - K^T diag(gamma) dX
// A short last chunk is zero-padded (beta = 0, g = 0, zero rows), which contributes nothing.
//
// Three kernels:
//   bwd_prep_kernel   one workgroup per (chunk, q/k head): K K^T and Q K^T once, then per v-head the
//                     decayed Bm and P and the triangular inverse T, to the workspace.
//   bwd_slice_kernel  one workgroup per (sequence, v-head, 16-column slice of the state): a forward
//                     sweep for the chunk-start states, then the chunks in reverse with everything
//                     that involves the slice's columns: dV, dL/dS, this slice's parts of dbeta and
//                     dG, of the dq/dk terms that go through S, U or D, and of the two C x C
//                     matrices dP o Gam and dBm o Gam.  Columns never interact, so these are exact
//                     partial sums over the slices.
//   bwd_combine_kernel  one workgroup per (chunk, q/k head): sums the slices' partials (and the
//                     v-heads sharing the q/k head) in a fixed order, forms the three C x C x dk
//                     products once, and writes dq, dk, dg and dbeta.
// All products run on the vector ALU out of LDS, with small register tiles.

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;        // chunk length
constexpr int kW = 16;        // state columns per slice workgroup
constexpr int kThreads = 256;
constexpr int kLC = kC + 1;   // pitch of C x C matrices in LDS
constexpr int kMat = kC * kC; // one C x C matrix in the workspace

__device__ __forceinline__ float sum16(float x) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off);
    return x;
}
__device__ __forceinline__ float sum64(float x) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

// Chunk slots: the chunks of sequence 0, then sequence 1, ...  (nct chunks per batch row without
// cu_seqlens).
__device__ int bwd_slot0(const int32_t* cu_seqlens, int n, int T) {
    if (!cu_seqlens) return n * ((T + kC - 1) / kC);
    int s = 0;
    for (int m = 0; m < n; ++m) {
        int row, a, b;
        sequence_range(cu_seqlens, m, T, row, a, b);
        s += (b - a + kC - 1) / kC;
    }
    return s;
}
// slot -> (sequence n, its chunk's tokens [cs, cs + L) of batch row `row`)
__device__ bool bwd_locate(int slot, const int32_t* cu_seqlens, int N, int T, int& n, int& row, int& cs,
                           int& L) {
    const int nct = (T + kC - 1) / kC;
    int ci = 0, t0, t1;
    if (!cu_seqlens) {
        n = slot / nct;
        ci = slot % nct;
        if (n >= N) return false;
    } else {
        int s = 0;
        n = -1;
        for (int m = 0; m < N && n < 0; ++m) {
            int r, a, b;
            sequence_range(cu_seqlens, m, T, r, a, b);
            const int c = (b - a + kC - 1) / kC;
            if (slot < s + c) {
                n = m;
                ci = slot - s;
            }
            s += c;
        }
        if (n < 0) return false;
    }
    sequence_range(cu_seqlens, n, T, row, t0, t1);
    cs = t0 + ci * kC;
    L = min(kC, t1 - cs);
    return L > 0;
}

// The chunk's running log-decay G (in place over the gates), gamma and f, by the first wave.
__device__ __forceinline__ void chunk_decays(float* G, float* gam, float* f, int tid) {
    if (tid < kWave) {
        float x = G[tid];
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float y = __shfl_up(x, off);
            if (tid >= off) x += y;
        }
        G[tid] = x;
        const float gc = __shfl(x, kWave - 1);
        gam[tid] = expf(x);
        f[tid] = expf(gc - x);
    }
}

// ------------------------------------------------------------------------------------------------
template <int DK, typename TIn, typename TG>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TG* __restrict__ g,
    const TG* __restrict__ beta, const int32_t* __restrict__ cu_seqlens, int N, int T, int Hk, int Hv,
    float* __restrict__ mats) {
    constexpr int LK = DK + 1;
    __shared__ float sK[kC * LK], sQ[kC * LK];
    __shared__ float sKK[kC * kLC], sQK[kC * kLC], sBm[kC * kLC];
    __shared__ float sG[kC], sgam[kC], sf[kC], sb[kC];
    const int slot = blockIdx.x, kh = blockIdx.y;
    int n, row, cs, L;
    if (!bwd_locate(slot, cu_seqlens, N, T, n, row, cs, L)) return;
    const int tid = threadIdx.x;
    const size_t tok0 = (size_t)row * T + cs;
    for (int e = tid; e < kC * DK; e += kThreads) {
        const int t = e / DK, i = e % DK;
        const bool in = t < L;
        const size_t off = ((tok0 + t) * Hk + kh) * DK + i;
        sK[t * LK + i] = in ? to_f32(k[off]) : 0.f;
        sQ[t * LK + i] = in ? to_f32(q[off]) : 0.f;
    }
    __syncthreads();
    // K K^T and Q K^T: thread (ty, tx) forms the 4 x 4 tiles rows 4 ty.., columns 4 tx..
    {
        const int ty = tid >> 4, tx = tid & 15;
        float kk[4][4] = {}, qk[4][4] = {};
        for (int i = 0; i < DK; ++i) {
            float a[4], aq[4], b[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                a[r] = sK[(4 * ty + r) * LK + i];
                aq[r] = sQ[(4 * ty + r) * LK + i];
                b[r] = sK[(4 * tx + r) * LK + i];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    kk[r][s] += a[r] * b[s];
                    qk[r][s] += aq[r] * b[s];
                }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                sKK[(4 * ty + r) * kLC + 4 * tx + s] = kk[r][s];
                sQK[(4 * ty + r) * kLC + 4 * tx + s] = qk[r][s];
            }
    }
    const int G = Hv / Hk;
    for (int qh = 0; qh < G; ++qh) {
        const int h = kh * G + qh;
        if (tid < kC) {
            const bool in = tid < L;
            sG[tid] = in ? to_f32(g[(tok0 + tid) * Hv + h]) : 0.f;
            sb[tid] = in ? to_f32(beta[(tok0 + tid) * Hv + h]) : 0.f;
        }
        __syncthreads();
        chunk_decays(sG, sgam, sf, tid);
        __syncthreads();
        float* mT = mats + ((size_t)slot * Hv + h) * 3 * kMat;
        float* mB = mT + kMat;
        float* mP = mB + kMat;
        for (int e = tid; e < kMat; e += kThreads) {
            const int t = e / kC, j = e % kC;
            const float dec = j <= t ? expf(sG[t] - sG[j]) : 0.f;
            const float bm = j < t ? sKK[t * kLC + j] * dec : 0.f;
            sBm[t * kLC + j] = bm;
            mB[e] = bm;
            mP[e] = sQK[t * kLC + j] * dec;
        }
        __syncthreads();
        if (tid < kC) {            // T = (I + diag(beta) Bm)^-1, lane c: column c
            float x[kC];
#pragma unroll
            for (int t = 0; t < kC; ++t) {
                float acc = (t == tid) ? 1.f : 0.f;
                const float bt = sb[t];
#pragma unroll
                for (int j = 0; j < t; ++j) acc -= bt * sBm[t * kLC + j] * x[j];
                x[t] = acc;
            }
#pragma unroll
            for (int t = 0; t < kC; ++t) mT[t * kC + tid] = x[t];
        }
        __syncthreads();                   // sG, sb and sBm are rewritten for the next v-head
    }
}

// ------------------------------------------------------------------------------------------------
// The slice kernel runs 512 threads (two waves per SIMD, to hide LDS latency; more leaves too few
// registers): each row of a C x 16 slice product gets 16 lanes, each row of a C x C product a wave.
constexpr int kST = 512;
constexpr int kSW = kST / kWave;                // waves

template <int DK>
struct SliceLds {
    static constexpr int LK = DK + 1, LW = kW + 1;
    float K[kC * LK];
    float Q[kC * LK];
    float S[DK * kW];        // chunk-start state, this slice
    float D[DK * kW];        // dL/dS at the chunk end, this slice
    float T[kC * kLC];       // T, then E = dP o P + dBm o Bm
    float B[kC * kLC];       // Bm
    float P[kC * kLC];       // P
    float VX[kC * LW];       // V, then X
    float KS[kC * LW];
    float U[kC * LW];
    float dO[kC * LW];
    float dU[kC * LW];       // dU, then dY
    float G[kC], gam[kC], f[kC], beta[kC];
    float r_qsdo[kC], r_ksdx[kC], r_kdu[kC], r_db[kC], r_e[kC], dG[kC];
    float red[kSW];
    int slot0;
};

template <int DK, typename TIn, typename TG>
__global__ __launch_bounds__(kST) void bwd_slice_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TG* __restrict__ g, const TG* __restrict__ beta, const float* __restrict__ initial_state,
    const int32_t* __restrict__ cu_seqlens, const float* __restrict__ d_o,
    const float* __restrict__ d_final, int T, int Hk, int Hv, int dv, const float* __restrict__ mats,
    float* __restrict__ ckpt, float* __restrict__ pmat, float* __restrict__ part_dq,
    float* __restrict__ part_dk, float* __restrict__ part_dg, float* __restrict__ part_db,
    float* __restrict__ dv_out, float* __restrict__ d_initial, long long rows, int max_slots) {
    using L = SliceLds<DK>;
    constexpr int LK = L::LK, LW = L::LW;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    L& sm = *reinterpret_cast<L*>(smem_raw);

    const int slices = dv / kW;
    int unit = blockIdx.x;
    const int sl = unit % slices;
    unit /= slices;
    const int h = unit % Hv, n = unit / Hv;
    const int kh = h / (Hv / Hk);
    const int c0 = sl * kW;
    int row, t0, t1;
    sequence_range(cu_seqlens, n, T, row, t0, t1);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cc = tid & 15, rg = tid >> 4;                  // (row, column) of slice work
    constexpr int RPT = kC * kW / kST;                        // rows per thread (1)
    if (tid == 0) sm.slot0 = bwd_slot0(cu_seqlens, n, T);
    __syncthreads();
    const int slot0 = sm.slot0;
    // (a malformed cu_seqlens can claim more chunks than the workspace holds: stop at its end)
    const int nchunks = min((t1 - t0 + kC - 1) / kC, max(0, max_slots - slot0));
    const size_t SSL = (size_t)DK * dv;                       // one full state
    auto ck_at = [&](int ci) { return ckpt + ((size_t)(slot0 + ci) * Hv + h) * SSL; };

    // the chunk's inputs: K (and Q), this slice of V (and dO), the gates, G, gamma, f; T (and Bm, P)
    auto load_chunk = [&](int ci, bool rev) {
        const int cs = t0 + ci * kC, Lc = min(kC, t1 - cs);
        const size_t tok0 = (size_t)row * T + cs;
        for (int e = tid; e < kC * DK; e += kST) {
            const int t = e / DK, i = e % DK;
            const bool in = t < Lc;
            const size_t off = ((tok0 + t) * Hk + kh) * DK + i;
            sm.K[t * LK + i] = in ? to_f32(k[off]) : 0.f;
            if (rev) sm.Q[t * LK + i] = in ? to_f32(q[off]) : 0.f;
        }
        for (int e = tid; e < kC * kW; e += kST) {
            const int t = e / kW, c = e % kW;
            const bool in = t < Lc;
            const size_t off = ((tok0 + t) * Hv + h) * dv + c0 + c;
            sm.VX[t * LW + c] = in ? to_f32(v[off]) : 0.f;
            if (rev) sm.dO[t * LW + c] = in ? d_o[off] : 0.f;
        }
        const float* mT = mats + ((size_t)(slot0 + ci) * Hv + h) * 3 * kMat;
        for (int e = tid; e < kMat; e += kST) {
            const int t = e / kC, j = e % kC;
            sm.T[t * kLC + j] = mT[e];
            if (rev) {
                sm.B[t * kLC + j] = mT[kMat + e];
                sm.P[t * kLC + j] = mT[2 * kMat + e];
            }
        }
        if (tid < kC) {
            const bool in = tid < Lc;
            sm.G[tid] = in ? to_f32(g[(tok0 + tid) * Hv + h]) : 0.f;
            sm.beta[tid] = in ? to_f32(beta[(tok0 + tid) * Hv + h]) : 0.f;
        }
        __syncthreads();
        chunk_decays(sm.G, sm.gam, sm.f, tid);
        __syncthreads();
        return Lc;
    };
    // KS, X = V - gamma KS (in place over V), U = T diag(beta) X; 16 lanes per row, 4 rows each
    auto ks_x_u = [&]() {
#pragma unroll
        for (int it = 0; it < RPT; ++it) {
            const int t = rg + (kST / kW) * it, c = cc;
            float ks = 0.f;
            for (int i = 0; i < DK; ++i) ks += sm.K[t * LK + i] * sm.S[i * kW + c];
            sm.KS[t * LW + c] = ks;
            sm.VX[t * LW + c] -= sm.gam[t] * ks;
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < RPT; ++it) {
            const int t = rg + (kST / kW) * it, c = cc;
            float u = 0.f;
            for (int j = 0; j <= t; ++j) u += sm.T[t * kLC + j] * sm.beta[j] * sm.VX[j * LW + c];
            sm.U[t * LW + c] = u;
        }
        __syncthreads();
    };

    // ---------------- forward sweep: the state at every chunk start ----------------------------
    const size_t sbase = ((size_t)n * Hv + h) * SSL;
    for (int e = tid; e < DK * kW; e += kST) {
        const int i = e / kW, c = e % kW;
        sm.S[e] = initial_state ? initial_state[sbase + (size_t)i * dv + c0 + c] : 0.f;
    }
    __syncthreads();
    for (int ci = 0; ci < nchunks; ++ci) {
        for (int e = tid; e < DK * kW; e += kST) {
            const int i = e / kW, c = e % kW;
            ck_at(ci)[(size_t)i * dv + c0 + c] = sm.S[e];
        }
        load_chunk(ci, false);
        ks_x_u();
        const float gC = sm.gam[kC - 1];
        for (int e = tid; e < DK * kW; e += kST) {
            const int i = e / kW, c = e % kW;
            float acc = 0.f;
            for (int t = 0; t < kC; ++t) acc += sm.K[t * LK + i] * sm.f[t] * sm.U[t * LW + c];
            sm.S[e] = gC * sm.S[e] + acc;
        }
        __syncthreads();
    }

    // ---------------- reverse sweep ------------------------------------------------------------
    for (int e = tid; e < DK * kW; e += kST) {
        const int i = e / kW, c = e % kW;
        sm.D[e] = d_final ? d_final[sbase + (size_t)i * dv + c0 + c] : 0.f;
    }
    for (int ci = nchunks - 1; ci >= 0; --ci) {
        const int cs = t0 + ci * kC;
        const size_t tok0 = (size_t)row * T + cs;
        const int slot = slot0 + ci;
        for (int e = tid; e < DK * kW; e += kST) {
            const int i = e / kW, c = e % kW;
            sm.S[e] = ck_at(ci)[(size_t)i * dv + c0 + c];
        }
        const int Lc = load_chunk(ci, true);
        ks_x_u();

        // dU = P^T dO + f (K D); row sums (QS).dO and (KD).U
#pragma unroll
        for (int it = 0; it < RPT; ++it) {
            const int t = rg + (kST / kW) * it, c = cc;
            float kd = 0.f, qs = 0.f;
            for (int i = 0; i < DK; ++i) {
                kd += sm.K[t * LK + i] * sm.D[i * kW + c];
                qs += sm.Q[t * LK + i] * sm.S[i * kW + c];
            }
            float pdo = 0.f;
            for (int tp = t; tp < kC; ++tp) pdo += sm.P[tp * kLC + t] * sm.dO[tp * LW + c];
            sm.dU[t * LW + c] = pdo + sm.f[t] * kd;
            const float a = sum16(qs * sm.dO[t * LW + c]);
            const float b = sum16(kd * sm.U[t * LW + c]);
            if (c == 0) {
                sm.r_qsdo[t] = a;
                sm.r_kdu[t] = b;
            }
        }
        __syncthreads();
        // dY = T^T dU (in place, through registers), dX = beta dY = dV; row sums X.dY and (KS).dX
        float dy[RPT];
#pragma unroll
        for (int it = 0; it < RPT; ++it) {
            const int t = rg + (kST / kW) * it, c = cc;
            float acc = 0.f;
            for (int tp = t; tp < kC; ++tp) acc += sm.T[tp * kLC + t] * sm.dU[tp * LW + c];
            dy[it] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < RPT; ++it) {
            const int t = rg + (kST / kW) * it, c = cc;
            sm.dU[t * LW + c] = dy[it];
            const float dx = sm.beta[t] * dy[it];
            if (t < Lc) dv_out[((tok0 + t) * Hv + h) * dv + c0 + c] = dx;
            const float a = sum16(sm.VX[t * LW + c] * dy[it]);
            const float b = sum16(sm.KS[t * LW + c] * dx);
            if (c == 0) {
                sm.r_db[t] = a;
                sm.r_ksdx[t] = b;
            }
        }
        __syncthreads();
        // the C x C gradients, one wave per row t, lane j: this slice's dP o Gam and dBm o Gam go to
        // the workspace, E = dP o P + dBm o Bm stays for dG
        float* pP = pmat + (((size_t)slot * Hv + h) * slices + sl) * 2 * kMat;
        float* pB = pP + kMat;
        for (int it = 0; it < kC / kSW; ++it) {
            const int t = wave + kSW * it, j = lane;
            float dyu = 0.f, dou = 0.f;
#pragma unroll
            for (int c = 0; c < kW; ++c) {
                const float uj = sm.U[j * LW + c];
                dyu += sm.dU[t * LW + c] * uj;
                dou += sm.dO[t * LW + c] * uj;
            }
            const float dA = j < t ? -dyu : 0.f;
            const float dP = j <= t ? dou : 0.f;
            const float bm = sm.B[t * kLC + j], p = sm.P[t * kLC + j];
            const float dec = j <= t ? expf(sm.G[t] - sm.G[j]) : 0.f;
            const float dbm = sm.beta[t] * dA;
            const float e_tj = dP * p + dbm * bm;
            sm.T[t * kLC + j] = e_tj;
            pP[t * kC + j] = dP * dec;
            pB[t * kC + j] = dbm * dec;
            const float db = sum64(dA * bm);
            const float er = sum64(e_tj);
            if (lane == 0) {
                sm.r_db[t] += db;
                sm.r_e[t] = er;
            }
        }
        // <S, D> over the slice, for dG at the chunk's last row
        float sd = 0.f;
        for (int e = tid; e < DK * kW; e += kST) sd += sm.S[e] * sm.D[e];
        sd = sum64(sd);
        if (lane == 0) sm.red[wave] = sd;
        __syncthreads();

        // this slice's dq, dk terms through S, U, D: gamma dO S^T, f U D^T - gamma beta dY S^T
        float* pq = part_dq + (size_t)sl * rows * Hv * DK;
        float* pk = part_dk + (size_t)sl * rows * Hv * DK;
        for (int e = tid; e < kC * DK; e += kST) {
            const int t = e / DK, i = e % DK;
            if (t >= Lc) continue;
            float dos = 0.f, fud = 0.f, dys = 0.f;
#pragma unroll
            for (int c = 0; c < kW; ++c) {
                const float sic = sm.S[i * kW + c];
                dos += sm.dO[t * LW + c] * sic;
                fud += sm.U[t * LW + c] * sm.D[i * kW + c];
                dys += sm.dU[t * LW + c] * sic;
            }
            const size_t o = ((tok0 + t) * Hv + h) * DK + i;
            pq[o] = sm.gam[t] * dos;
            pk[o] = sm.f[t] * fud - sm.gam[t] * sm.beta[t] * dys;
        }
        // dG (this slice's part) and its reverse running sum, by the first wave (lane = row t)
        if (tid < kC) {
            const int t = tid;
            float ce = 0.f;
            for (int r = 0; r < kC; ++r) ce += sm.T[r * kLC + t];
            const float fkdu = sum64(sm.f[t] * sm.r_kdu[t]);
            float sdt = 0.f;
            for (int w = 0; w < kSW; ++w) sdt += sm.red[w];
            float x = sm.gam[t] * sm.r_qsdo[t] - sm.gam[t] * sm.r_ksdx[t] - sm.f[t] * sm.r_kdu[t] + sm.r_e[t] - ce;
            if (t == kC - 1) x += sm.gam[kC - 1] * sdt + fkdu;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float y = __shfl_down(x, off);
                if (t + off < kWave) x += y;
            }
            sm.dG[t] = x;
        }
        __syncthreads();
        if (tid < Lc) {
            const size_t o = (size_t)sl * rows * Hv + (tok0 + tid) * Hv + h;
            part_dg[o] = sm.dG[tid];
            part_db[o] = sm.r_db[tid];
        }
        // dL/dS for the previous chunk: gamma_C D + Q^T diag(gamma) dO - K^T diag(gamma beta) dY
        const float gC = sm.gam[kC - 1];
        float nd[DK * kW / kST];
#pragma unroll
        for (int r = 0; r < DK * kW / kST; ++r) {
            const int e = tid + kST * r, i = e / kW, c = e % kW;
            float acc = 0.f;
            for (int t = 0; t < kC; ++t)
                acc += sm.gam[t] * (sm.Q[t * LK + i] * sm.dO[t * LW + c] -
                                    sm.K[t * LK + i] * sm.beta[t] * sm.dU[t * LW + c]);
            nd[r] = gC * sm.D[e] + acc;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < DK * kW / kST; ++r) sm.D[tid + kST * r] = nd[r];
        __syncthreads();
    }
    if (d_initial) {
        for (int e = tid; e < DK * kW; e += kST) {
            const int i = e / kW, c = e % kW;
            d_initial[sbase + (size_t)i * dv + c0 + c] = sm.D[e];
        }
    }
}

// ------------------------------------------------------------------------------------------------
// One workgroup per (chunk, q/k head): dq = the slices' terms + (dP o Gam) K, and
// dk = their terms + (dP o Gam)^T Q + ((dBm o Gam) + (dBm o Gam)^T) K, with the two C x C matrices
// summed over the slices and the v-heads of the q/k head; dg and dbeta summed over the slices.
template <int DK, typename TIn>
__global__ __launch_bounds__(kThreads) void bwd_combine_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const int32_t* __restrict__ cu_seqlens, int N,
    int T, int Hk, int Hv, int slices, long long rows, const float* __restrict__ pmat,
    const float* __restrict__ part_dq, const float* __restrict__ part_dk, const float* __restrict__ part_dg,
    const float* __restrict__ part_db, float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dg,
    float* __restrict__ db) {
    constexpr int LK = DK + 1;
    __shared__ float sK[kC * LK], sQ[kC * LK];
    __shared__ float sP[kC * kLC], sB[kC * kLC];
    const int slot = blockIdx.x, kh = blockIdx.y;
    int n, row, cs, L;
    if (!bwd_locate(slot, cu_seqlens, N, T, n, row, cs, L)) return;
    const int tid = threadIdx.x;
    const size_t tok0 = (size_t)row * T + cs;
    const int G = Hv / Hk;
    for (int e = tid; e < kC * DK; e += kThreads) {
        const int t = e / DK, i = e % DK;
        const bool in = t < L;
        const size_t off = ((tok0 + t) * Hk + kh) * DK + i;
        sK[t * LK + i] = in ? to_f32(k[off]) : 0.f;
        sQ[t * LK + i] = in ? to_f32(q[off]) : 0.f;
    }
    // the two C x C matrices, summed over v-heads and slices; B symmetrised
    for (int e = tid; e < kMat; e += kThreads) {
        const int t = e / kC, j = e % kC;
        float ap = 0.f, ab = 0.f;
        for (int x = 0; x < G; ++x)
            for (int s = 0; s < slices; ++s) {
                const float* pm = pmat + (((size_t)slot * Hv + kh * G + x) * slices + s) * 2 * kMat;
                ap += pm[e];
                ab += pm[kMat + e] + pm[kMat + j * kC + t];
            }
        sP[t * kLC + j] = ap;
        sB[t * kLC + j] = ab;
    }
    __syncthreads();
    // dq, dk: thread (ty, tx) owns rows 4 ty .. 4 ty + 3 and keys tx, tx + 16, ..
    {
        constexpr int NI = DK / 16;
        const int ty = tid >> 4, tx = tid & 15;
        float aq[4][NI] = {}, ak[4][NI] = {};
        for (int j = 0; j < kC; ++j) {
            float p[4], pt[4], b[4], kj[NI], qj[NI];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[r] = sP[(4 * ty + r) * kLC + j];
                pt[r] = sP[j * kLC + 4 * ty + r];
                b[r] = sB[(4 * ty + r) * kLC + j];
            }
#pragma unroll
            for (int m = 0; m < NI; ++m) {
                kj[m] = sK[j * LK + tx + 16 * m];
                qj[m] = sQ[j * LK + tx + 16 * m];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int m = 0; m < NI; ++m) {
                    aq[r][m] += p[r] * kj[m];
                    ak[r][m] += pt[r] * qj[m] + b[r] * kj[m];
                }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * ty + r;
            if (t >= L) continue;
#pragma unroll
            for (int m = 0; m < NI; ++m) {
                const int i = tx + 16 * m;
                float sq = aq[r][m], skk = ak[r][m];
                for (int x = 0; x < G; ++x)
                    for (int s = 0; s < slices; ++s) {
                        const size_t o = (((size_t)s * rows + tok0 + t) * Hv + kh * G + x) * DK + i;
                        sq += part_dq[o];
                        skk += part_dk[o];
                    }
                dq[((tok0 + t) * Hk + kh) * DK + i] = sq;
                dk[((tok0 + t) * Hk + kh) * DK + i] = skk;
            }
        }
    }
    for (int e = tid; e < L * G; e += kThreads) {
        const int t = e / G, h = kh * G + e % G;
        float ag = 0.f, ab = 0.f;
        for (int s = 0; s < slices; ++s) {
            const size_t o = ((size_t)s * rows + tok0 + t) * Hv + h;
            ag += part_dg[o];
            ab += part_db[o];
        }
        dg[(tok0 + t) * Hv + h] = ag;
        db[(tok0 + t) * Hv + h] = ab;
    }
}

// dq, dk, dg, dbeta of tokens outside every packed sequence: zero (launched before the combine).
__global__ __launch_bounds__(kThreads) void bwd_zero_kernel(float* __restrict__ a, long long na,
                                                            float* __restrict__ b, long long nb,
                                                            float* __restrict__ c, long long nc,
                                                            float* __restrict__ d, long long nd) {
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (i < na) a[i] = 0.f;
    if (i < nb) b[i] = 0.f;
    if (i < nc) c[i] = 0.f;
    if (i < nd) d[i] = 0.f;
}

struct BwdLayout {
    size_t ckpt, mats, pmat, pq, pk, pg, pb, total;
    int slots;
};

size_t align256b(size_t x) { return (x + 255) & ~(size_t)255; }

BwdLayout bwd_layout(int B, int T, int Hv, int dk, int dv, int N) {
    BwdLayout l;
    const long long rows = (long long)B * T;
    l.slots = (int)(rows / kC) + N;
    const int slices = dv / kW;
    size_t off = 0;
    l.ckpt = off; off = align256b(off + sizeof(float) * (size_t)l.slots * Hv * dk * dv);
    l.mats = off; off = align256b(off + sizeof(float) * (size_t)l.slots * Hv * 3 * kMat);
    l.pmat = off; off = align256b(off + sizeof(float) * (size_t)l.slots * Hv * slices * 2 * kMat);
    l.pq = off;   off = align256b(off + sizeof(float) * (size_t)slices * rows * Hv * dk);
    l.pk = off;   off = align256b(off + sizeof(float) * (size_t)slices * rows * Hv * dk);
    l.pg = off;   off = align256b(off + sizeof(float) * (size_t)slices * rows * Hv);
    l.pb = off;   off = align256b(off + sizeof(float) * (size_t)slices * rows * Hv);
    l.total = off;
    return l;
}

template <int DK, typename TIn, typename TG>
hipError_t launch_bwd_typed(const BwdArgs& a) {
    const BwdLayout lay = bwd_layout(a.B, a.T, a.Hv, a.dk, a.dv, a.N);
    char* ws = static_cast<char*>(a.workspace);
    const long long rows = (long long)a.B * a.T;
    const int slices = a.dv / kW;
    const bool packed = a.cu_seqlens != nullptr;
    const int slots = packed ? lay.slots : a.B * ((a.T + kC - 1) / kC);
    float* ckpt = reinterpret_cast<float*>(ws + lay.ckpt);
    float* mats = reinterpret_cast<float*>(ws + lay.mats);
    float* pmat = reinterpret_cast<float*>(ws + lay.pmat);
    float* pq = reinterpret_cast<float*>(ws + lay.pq);
    float* pk = reinterpret_cast<float*>(ws + lay.pk);
    float* pg = reinterpret_cast<float*>(ws + lay.pg);
    float* pb = reinterpret_cast<float*>(ws + lay.pb);
    hipError_t e;
    if (slots > 0) {
        hipLaunchKernelGGL((bwd_prep_kernel<DK, TIn, TG>), dim3((unsigned)slots, (unsigned)a.Hk), dim3(kThreads), 0,
                           a.stream, static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                           static_cast<const TG*>(a.g), static_cast<const TG*>(a.beta), a.cu_seqlens, a.N, a.T,
                           a.Hk, a.Hv, mats);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const auto kern = bwd_slice_kernel<DK, TIn, TG>;
    const size_t bytes = sizeof(SliceLds<DK>);
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes)) != hipSuccess)
        return e;
    // (with no tokens this still runs: every sequence is empty and passes d_final through)
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.N * a.Hv * slices)), dim3(kST), bytes, a.stream,
                       static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.v), static_cast<const TG*>(a.g),
                       static_cast<const TG*>(a.beta), a.initial_state, a.cu_seqlens, a.d_o, a.d_final,
                       a.T, a.Hk, a.Hv, a.dv, mats, ckpt, pmat, pq, pk, pg, pb, a.dv_out, a.d_initial, rows,
                       lay.slots);
    if ((e = hipGetLastError()) != hipSuccess || rows == 0) return e;
    if (packed) {
        const long long nq = rows * a.Hk * a.dk, ng = rows * a.Hv, nmax = nq > ng ? nq : ng;
        hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((nmax + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                           a.stream, a.dq, nq, a.dk_out, nq, a.dg, ng, a.dbeta, ng);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (slots > 0) {
        hipLaunchKernelGGL((bwd_combine_kernel<DK, TIn>), dim3((unsigned)slots, (unsigned)a.Hk), dim3(kThreads), 0,
                           a.stream, static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k), a.cu_seqlens,
                           a.N, a.T, a.Hk, a.Hv, slices, rows, pmat, pq, pk, pg, pb, a.dq, a.dk_out, a.dg,
                           a.dbeta);
    }
    return hipGetLastError();
}

template <int DK>
hipError_t launch_bwd_dk(const BwdArgs& a) {
    const bool in_bf16 = a.qkv_dtype == GDN_BF16, g_bf16 = a.gate_dtype == GDN_BF16;
    if (in_bf16 && g_bf16) return launch_bwd_typed<DK, bf16_t, bf16_t>(a);
    if (in_bf16) return launch_bwd_typed<DK, bf16_t, float>(a);
    if (g_bf16) return launch_bwd_typed<DK, float, bf16_t>(a);
    return launch_bwd_typed<DK, float, float>(a);
}

}  // namespace

size_t chunk_bwd_workspace_size(int B, int T, int Hv, int dk, int dv, int N) {
    return bwd_layout(B, T, Hv, dk, dv, N).total;
}

hipError_t launch_chunk_bwd(const BwdArgs& a) {
    return a.dk == 128 ? launch_bwd_dk<128>(a) : launch_bwd_dk<64>(a);
}

}  // namespace gdn
