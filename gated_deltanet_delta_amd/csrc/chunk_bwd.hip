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
//                     that involves only the slice's columns: dV, dL/dS, and this slice's parts of
//                     dbeta and dG through the state (columns never interact, so these are exact
//                     partial sums over the slices), and its columns of U, dY and of D at every
//                     chunk's end, for the combine kernel.
//   bwd_combine_kernel  one workgroup per (chunk, q/k head), on the fp32 matrix cores: per v-head the
//                     C x C gradients dP, dA (contracted over dv) and their dG and dbeta terms; the
//                     dq and dk terms through the state (dO S^T, U D^T, dY S^T) and the three
//                     C x C x dk products with the C x C matrices summed over the v-heads in a fixed
//                     order; then dq, dk, dg and dbeta.
// The slice kernel's products against K or Q run, for bf16 inputs, on the bf16 matrix cores with the
// other operand in three bf16 pieces; its T and P products, and all of them for fp32 inputs, on the
// fp32 matrix cores.  The prepare kernel forms K K^T and
// Q K^T on the vector ALU with small register tiles, and T by 16 x 16 blocks: the diagonal ones by
// forward substitution, the others on the fp32 matrix cores.

#include <type_traits>

#include "common.h"
#include "launch.h"
#include "mfma_frag.h"

namespace gdn {
namespace {

constexpr int kC = 64;        // chunk length
constexpr int kW = 16;        // state columns per slice workgroup
constexpr int kThreads = 256;
constexpr int kLC = kC + 1;   // pitch of C x C matrices in LDS
constexpr int kMat = kC * kC; // one C x C matrix in the workspace


// 8 consecutive input elements as fp32 (one 16-byte load for bf16, two for fp32)
struct F8 {
    float x[8];
};
__device__ __forceinline__ F8 load8(const bf16_t* p) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const unsigned w[4] = {u.x, u.y, u.z, u.w};
    F8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.x[2 * i] = __uint_as_float(w[i] << 16);
        r.x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    return r;
}
__device__ __forceinline__ F8 load8(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    return F8{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}

// Rows [0, kC) x DK of a [token][head][DK] input into LDS rows of pitch LK, every load issued before
// the first LDS write; rows past Lc read row Lc - 1 (in bounds) and store zeros.
template <int DK, int LK, int NT, typename TIn>
__device__ __forceinline__ void stage_rows(const TIn* __restrict__ src, size_t tok0, int Hh, int head, int Lc,
                                           float* dst, int tid) {
    constexpr int PER = kC * DK / 8 / NT;       // 8-element pieces per thread
    F8 v[PER];
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int e = tid + NT * it, t = e / (DK / 8), c8 = 8 * (e % (DK / 8));
        const int tr = t < Lc ? t : Lc - 1;
        v[it] = load8(src + ((tok0 + tr) * Hh + head) * DK + c8);
    }
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int e = tid + NT * it, t = e / (DK / 8), c8 = 8 * (e % (DK / 8));
        const float m = t < Lc ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[t * LK + c8 + j] = m * v[it].x[j];
    }
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
        const float x = wave_prefix_sum(G[tid]);
        G[tid] = x;
        const float gc = lane_value(x, kWave - 1);
        gam[tid] = expf(x);
        f[tid] = expf(gc - x);
    }
}

// ------------------------------------------------------------------------------------------------
// fp32 matrix-core product on 16 x 16 tiles: lane (g, c) = (lane / 16, lane % 16) feeds A[c][k + g]
// and B[k + g][c]; element r of the result is row 4 g + r, column c
typedef float f32x4b __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4b mfma4(float a, float b, f32x4b c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int DK, typename TIn, typename TG>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TG* __restrict__ g,
    const TG* __restrict__ beta, const int32_t* __restrict__ cu_seqlens, int N, int T, int Hk, int Hv,
    float* __restrict__ mats) {
    constexpr int LK = DK + 1;
    // the staged K, Q rows and the C x C products share one region (67 KB at DK = 128: two
    // workgroups fit a CU)
    __shared__ float smem[2 * kC * LK > 4 * kC * kLC ? 2 * kC * LK : 4 * kC * kLC];
    float* sK = smem;
    float* sQ = smem + kC * LK;
    float* sKK = smem;
    float* sQK = smem + kC * kLC;
    float* sBm = smem + 2 * kC * kLC;
    float* sTT = smem + 3 * kC * kLC;
    __shared__ float sG[kC], sgam[kC], sf[kC], sb[kC];
    const int slot = blockIdx.x, kh = blockIdx.y;
    int n, row, cs, L;
    if (!bwd_locate(slot, cu_seqlens, N, T, n, row, cs, L)) return;
    const int tid = threadIdx.x;
    const size_t tok0 = (size_t)row * T + cs;
    stage_rows<DK, LK, kThreads>(k, tok0, Hk, kh, L, sK, tid);
    stage_rows<DK, LK, kThreads>(q, tok0, Hk, kh, L, sQ, tid);
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
        __syncthreads();                   // K and Q are read; their region takes the products
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
        // T = (I + A)^-1, A = diag(beta) Bm, by blocked forward substitution on 16 x 16 blocks.  Block
        // row a of (I + A) T = I gives, for b < a,  (I + A_aa) T_ab = -sum_{m=b}^{a-1} A_am T_mb:
        // the right-hand sides on the fp32 matrix cores, then every solve with I + A_aa in wave 0,
        // lane (g, c) taking column c of the g-th block of a level (DPP row broadcasts of A_aa).
        const int lane = tid & 63, wave = tid >> 6, gq = lane >> 4, c = lane & 15;
        // wave 0: (I + A_aa) x = y for the blocks (a, b) = (g + d, g), g < 4 - d, y read from sTT
        // (the identity for d = 0) and x written over it
        auto solve_level = [&](int d) {
            const int a = gq + d, b = gq;
            if (a > 3) return;
            float av[16], x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int row = 16 * a + t;
                av[t] = -sb[row] * sBm[row * kLC + 16 * a + c];   // (zero for t <= c: Bm is strictly lower)
                x[t] = d == 0 ? (t == c ? 1.f : 0.f) : sTT[row * kLC + 16 * b + c];
            }
            invert_blocks16(x, av);
#pragma unroll
            for (int t = 0; t < 16; ++t) sTT[(16 * a + t) * kLC + 16 * b + c] = x[t];
        };
        if (wave == 0) {
            solve_level(0);
        } else {
            for (int e = tid - kWave; e < kMat; e += kThreads - kWave) {
                const int t = e / kC, j = e % kC;
                if ((j >> 4) > (t >> 4)) sTT[t * kLC + j] = 0.f;
            }
        }
        __syncthreads();
        for (int d = 1; d < 4; ++d) {
            if (wave < 4 - d) {      // right-hand side of block (w + d, w)
                const int b = wave, a = wave + d;
                f32x4b X = {0.f, 0.f, 0.f, 0.f};
                for (int m = b; m < a; ++m) {
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        const int k = 16 * m + 4 * s4 + gq;
                        X = mfma4(sb[16 * a + c] * sBm[(16 * a + c) * kLC + k], sTT[k * kLC + 16 * b + c], X);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) sTT[(16 * a + 4 * gq + r) * kLC + 16 * b + c] = -X[r];
            }
            __syncthreads();
            if (wave == 0) solve_level(d);
            __syncthreads();
        }
        for (int e = tid; e < kMat; e += kThreads) mT[e] = sTT[(e / kC) * kLC + e % kC];
        __syncthreads();                   // sG, sb, sBm and sTT are rewritten for the next v-head
    }
}

// ------------------------------------------------------------------------------------------------
// The slice kernel: 512 threads, eight waves, each owning whole 16 x 16 output tiles (the C x 16
// slice products one row tile per wave, the K^T / Q^T products one key tile).  The fp32 products are
// chains of v_mfma_f32_16x16x4f32 (lane (g, c) = (lane / 16, lane % 16) feeds A[c][k + g] and
// B[k + g][c]; element r of the result is row 4 g + r, column c) with operands straight from LDS.
// For bf16 inputs the products against K or Q use v_mfma_f32_16x16x32_bf16 on fragments instead
// (rows_bf, keys_bf below).
constexpr int kST = 512;
constexpr int kSW = kST / kWave;                // waves
constexpr int kPieces = 3;                      // bf16 pieces of an fp32 operand (put_frag)


// K and Q of the chunk: fp32 rows (fp32 inputs), or for bf16 inputs the exact bf16 rows in the
// swizzled layout of mfma_frag.h, with the products' other operands as three-piece B fragments of
// v_mfma_f32_16x16x32_bf16 (put_frag), each written by the phase that forms the values:
//   Sf, Df   S and D over the keys: [32-key step kb][piece][lane (g, c)], element e = row 32 kb + 8 g + e
//   Yf, Zf   token-weighted operands over the chunk: [32-token step kb][piece][lane (g, c)], element
//            e = token 32 kb + 4 g + e (e < 4) or 32 kb + 16 + 4 g + e - 4 (e >= 4), the token order of
//            kt_frag; Yf holds f U (forward sweep) or gamma dO (reverse), Zf gamma beta dY
template <int DK, bool BF>
struct SliceKQ {
    float K[kC * (DK + 1)];
    float Q[kC * (DK + 1)];
};
template <int DK>
struct SliceKQ<DK, true> {
    __bf16 Kb[kC * DK];
    __bf16 Qb[kC * DK];
    bf16x8 Sf[DK / 32][kPieces][kWave];
    bf16x8 Df[DK / 32][kPieces][kWave];
    bf16x8 Yf[kC / 32][kPieces][kWave];
    bf16x8 Zf[kC / 32][kPieces][kWave];
};

template <int DK, bool BF>
struct SliceLds : SliceKQ<DK, BF> {
    static constexpr int LK = DK + 1, LW = kW + 1;
    float S[DK * LW];        // chunk-start state, this slice
    float D[DK * LW];        // dL/dS at the chunk end, this slice
    float T[kC * kLC];       // T
    float P[kC * kLC];       // P
    float VX[kC * LW];       // V, then X
    float KS[kC * LW];
    float U[kC * LW];
    float dO[kC * LW];
    float dU[kC * LW];
    float KD[kC * LW];       // K D, then dY
    float G[kC], gam[kC], f[kC], beta[kC];
    float r_qsdo[kC], r_ksdx[kC], r_kdu[kC], r_db[kC], dG[kC];
    float red[kSW];
    int slot0;
};

// Three bf16 pieces of fp32 values, x = hi + mid + lo to within 2^-27 |x| (each residual is exact in
// fp32; each rounding to bf16 leaves at most 2^-9 of what it rounds), into a B fragment array
// F[kb][piece][lane]: N = 4 or 2 consecutive elements of lane `ln`'s 8, from element e0 (a multiple
// of N).  Against exact bf16 K and Q, three products then carry the fp32 operand in full.
template <int N>
__device__ __forceinline__ void put_frag(bf16x8 (*F)[kPieces][kWave], int kb, int ln, int e0, const float* x) {
    unsigned w[kPieces][N / 2];
#pragma unroll
    for (int p = 0; p < N / 2; ++p) {
        float r0 = x[2 * p], r1 = x[2 * p + 1];
#pragma unroll
        for (int k = 0; k < kPieces; ++k) {
            const unsigned h = pack_bf16x2(r0, r1);
            w[k][p] = h;
            r0 -= __uint_as_float(h << 16);
            r1 -= __uint_as_float(h & 0xffff0000u);
        }
    }
#pragma unroll
    for (int k = 0; k < kPieces; ++k) {
        char* f = reinterpret_cast<char*>(&F[kb][k][ln]) + 2 * e0;
        if constexpr (N == 4) *reinterpret_cast<uint2*>(f) = uint2{w[k][0], w[k][1]};
        else *reinterpret_cast<unsigned*>(f) = w[k][0];
    }
}
__device__ __forceinline__ void put_frag4(bf16x8 (*F)[kPieces][kWave], int kb, int ln, int e0, const f32x4b& v) {
    const float x[4] = {v[0], v[1], v[2], v[3]};
    put_frag<4>(F, kb, ln, e0, x);
}

template <int DK, typename TIn, typename TG>
__global__ __launch_bounds__(kST) void bwd_slice_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TG* __restrict__ g, const TG* __restrict__ beta, const float* __restrict__ initial_state,
    const int32_t* __restrict__ cu_seqlens, const float* __restrict__ d_o,
    const float* __restrict__ d_final, int T, int Hk, int Hv, int dv, const float* __restrict__ mats,
    float* __restrict__ ckpt, float* __restrict__ ws_d,
    float* __restrict__ ws_u, float* __restrict__ ws_y, float* __restrict__ part_dg, float* __restrict__ part_db,
    float* __restrict__ dv_out, float* __restrict__ d_initial, long long rows, int max_slots) {
    constexpr bool BF = std::is_same<TIn, bf16_t>::value;   // exact bf16 K and Q: bf16 matrix cores
    using L = SliceLds<DK, BF>;
    constexpr int LK = L::LK, LW = L::LW;
    constexpr int KT = DK / 16;                  // key tiles
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    L& sm = *reinterpret_cast<L*>(smem_raw);

    const int slices = dv / kW;
    // Workgroups go to the XCDs round robin by index (i on XCD i % 8).  Units are dealt so that each
    // XCD gets one contiguous run of them: the slices of one v-head, which all read that v-head's
    // T and P, then share an L2.
    const int nwg = gridDim.x, xcd = blockIdx.x % 8, per = nwg / 8, extra = nwg % 8;
    int unit = xcd * per + min(xcd, extra) + blockIdx.x / 8;
    const int sl = unit % slices;
    unit /= slices;
    const int h = unit % Hv, n = unit / Hv;
    const int kh = h / (Hv / Hk);
    const int c0 = sl * kW;
    int row, t0, t1;
    sequence_range(cu_seqlens, n, T, row, t0, t1);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int gl = lane >> 4, cl = lane & 15;                      // (g, c) of the tile layout
    // Every product's LDS addresses derive from (g, c); left alone, the compiler hoists all of them
    // out of the chunk loops and runs out of registers.  Passing (g, c) through an empty asm at the
    // top of each chunk makes them loop-variant, so they are formed where they are used.
    auto refresh_lane = [&]() { asm volatile("" : "+v"(gl), "+v"(cl)); };
    if (tid == 0) sm.slot0 = bwd_slot0(cu_seqlens, n, T);
    lds_barrier();
    const int slot0 = sm.slot0;
    // (a malformed cu_seqlens can claim more chunks than the workspace holds: stop at its end)
    const int nchunks = min((t1 - t0 + kC - 1) / kC, max(0, max_slots - slot0));
    const size_t SSL = (size_t)DK * dv;                       // one full state
    auto ck_at = [&](int ci) { return ckpt + ((size_t)(slot0 + ci) * Hv + h) * SSL; };
    const f32x4b z4 = {0.f, 0.f, 0.f, 0.f};

    // the chunk's inputs: K (and Q), this slice of V (and dO), the gates, G, gamma, f; T (and Bm, P)
    // One chunk's inputs, fetched into registers a chunk before their use and written to LDS then:
    // K (and Q), this slice of V (and dO), the gates, T (and P).  The registers hold the loads as
    // they arrive (bf16 is widened only when written to LDS), so that nothing waits for them
    // before the commit.
    constexpr int NMX = 2, PM = kMat / 4 / kST;            // C x C matrices: T, P
    constexpr int PV = kC * kW / kST;                      // V, dO elements per thread
    constexpr int PR = kC * DK / 8 / kST;                  // 8-element K, Q pieces per thread
    using Raw8 = typename std::conditional<std::is_same<TIn, float>::value, float4[2], uint4>::type;
    struct ChunkIn {
        float4 mv[NMX][PM];
        TIn vv[PV];
        float ov[PV];
        Raw8 kr[PR], qr[PR];
        TG gr, br;
    };
    auto raw_load = [&](Raw8& d, const TIn* src) {
        if constexpr (std::is_same<TIn, float>::value) {
            d[0] = *reinterpret_cast<const float4*>(src);
            d[1] = *reinterpret_cast<const float4*>(src + 4);
        } else {
            d = *reinterpret_cast<const uint4*>(src);
        }
    };
    auto raw_store = [&](const Raw8& r, float* dst, float m) {
        if constexpr (std::is_same<TIn, float>::value) {
            const float x[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[j] = m * x[j];
        } else {
            const unsigned w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dst[2 * i] = m * __uint_as_float(w[i] << 16);
                dst[2 * i + 1] = m * __uint_as_float(w[i] & 0xffff0000u);
            }
        }
    };
    auto fetch_chunk = [&](ChunkIn& in, int ci, auto rev_c) {
        constexpr bool rev = decltype(rev_c)::value;
        const int cs = t0 + ci * kC, Lc = min(kC, t1 - cs);
        const size_t tok0 = (size_t)row * T + cs;
        // (T, and in the reverse sweep P: matrices 0 and 2 of the prep kernel's T, Bm, P)
        const float* mT = mats + ((size_t)(slot0 + ci) * Hv + h) * 3 * kMat;
#pragma unroll
        for (int m = 0; m < (rev ? 2 : 1); ++m)
#pragma unroll
            for (int it = 0; it < PM; ++it)
                in.mv[m][it] = *reinterpret_cast<const float4*>(mT + 2 * m * kMat + 4 * (tid + kST * it));
        // rows past the chunk's end read its last row (in bounds) and are zeroed at the commit
#pragma unroll
        for (int it = 0; it < PV; ++it) {
            const int e = tid + kST * it, t = e / kW, c = e % kW;
            const size_t off = ((tok0 + min(t, Lc - 1)) * Hv + h) * dv + c0 + c;
            in.vv[it] = v[off];
            if (rev) in.ov[it] = d_o[off];
        }
#pragma unroll
        for (int it = 0; it < PR; ++it) {
            const int e = tid + kST * it, t = min(e / (DK / 8), Lc - 1), c8 = 8 * (e % (DK / 8));
            raw_load(in.kr[it], k + ((tok0 + t) * Hk + kh) * DK + c8);
            if (rev) raw_load(in.qr[it], q + ((tok0 + t) * Hk + kh) * DK + c8);
        }
        if (tid < kC) {
            const size_t gi = (tok0 + min(tid, Lc - 1)) * Hv + h;
            in.gr = g[gi];
            in.br = beta[gi];
        }
    };
    auto commit_chunk = [&](const ChunkIn& in, int ci, auto rev_c) {
        constexpr bool rev = decltype(rev_c)::value;
        const int cs = t0 + ci * kC, Lc = min(kC, t1 - cs);
#pragma unroll
        for (int it = 0; it < PV; ++it) {
            const int e = tid + kST * it, t = e / kW, c = e % kW;
            const float m = t < Lc ? 1.f : 0.f;
            sm.VX[t * LW + c] = m * to_f32(in.vv[it]);
            if (rev) sm.dO[t * LW + c] = m * in.ov[it];
        }
#pragma unroll
        for (int it = 0; it < PR; ++it) {
            const int e = tid + kST * it, t = e / (DK / 8), c8 = 8 * (e % (DK / 8));
            if constexpr (BF) {
                // 16-byte chunk c8 / 8 of row t at its swizzled place; rows past the chunk's end zero
                // (component by component: a select of whole vectors becomes one of their addresses,
                // which puts the register prefetch on the stack)
                const int off = t * DK + 8 * ((c8 / 8) ^ kswz<DK>(t));
                const bool in_chunk = t < Lc;
                auto keep = [&](const uint4& x) {
                    return uint4{in_chunk ? x.x : 0u, in_chunk ? x.y : 0u, in_chunk ? x.z : 0u, in_chunk ? x.w : 0u};
                };
                *reinterpret_cast<uint4*>(sm.Kb + off) = keep(in.kr[it]);
                if (rev) *reinterpret_cast<uint4*>(sm.Qb + off) = keep(in.qr[it]);
            } else {
                const float m = t < Lc ? 1.f : 0.f;
                raw_store(in.kr[it], sm.K + t * LK + c8, m);
                if (rev) raw_store(in.qr[it], sm.Q + t * LK + c8, m);
            }
        }
        float* mdst[2] = {sm.T, sm.P};
#pragma unroll
        for (int m = 0; m < (rev ? 2 : 1); ++m)
#pragma unroll
            for (int it = 0; it < PM; ++it) {
                const int e = 4 * (tid + kST * it), t = e / kC, j = e % kC;
                float* d = mdst[m] + t * kLC + j;
                d[0] = in.mv[m][it].x;
                d[1] = in.mv[m][it].y;
                d[2] = in.mv[m][it].z;
                d[3] = in.mv[m][it].w;
            }
        if (tid < kC) {
            const bool inside = tid < Lc;
            sm.G[tid] = inside ? to_f32(in.gr) : 0.f;
            sm.beta[tid] = inside ? to_f32(in.br) : 0.f;
        }
        // (the first wave reads back only the gates its own lanes wrote: no barrier before)
        chunk_decays(sm.G, sm.gam, sm.f, tid);
        lds_barrier();
        return Lc;
    };
    // row tile a of M S (M = K or Q, C x DK, S DK x 16): A = M[16 a + c][k + g], B = S[k + g][c]
    auto rows_times_state = [&](const float* M, const float* Sx, int a) {
        f32x4b acc = z4;
        // (16-deep blocks of four products, so that a block's LDS reads are in flight together)
        for (int k0 = 0; k0 < DK; k0 += 16)
#pragma unroll
            for (int kk = k0; kk < k0 + 16; kk += 4)
                acc = mfma4(M[(16 * a + cl) * LK + kk + gl], Sx[(kk + gl) * LW + cl], acc);
        return acc;
    };
    // bf16 inputs: row tile a of M X over the keys, M = K or Q (exact bf16 rows), X = S or D as
    // three-piece fragments; three products per 32-key step
    auto rows_bf = [&](const __bf16* Mb, bf16x8 (*Xf)[kPieces][kWave], int a) {
        f32x4b acc = z4;
        const __bf16* mrow = Mb + 16 * a * DK;
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            const bf16x8 am = *reinterpret_cast<const bf16x8*>(mrow + kf_lane<DK>(cl, gl, kb));
#pragma unroll
            for (int k = 0; k < kPieces; ++k) acc = mma(am, Xf[kb][k][lane], acc);
        }
        return acc;
    };
    // bf16 inputs: key tile kt of M^T Y over the chunk's tokens (Y a token-weighted operand as
    // three-piece fragments); element r of lane (g, c) is key rho(kt, 4 g + r), column c
    auto keys_bf = [&](const __bf16* Mb, bf16x8 (*Yw)[kPieces][kWave], int kt) {
        f32x4b acc = z4;
        lds_u8* base = lds_at(Mb + kt_lane<DK>(cl, gl, kt >> 1));
#pragma unroll
        for (int kb = 0; kb < kC / 32; ++kb) {
            const bf16x8 at = kt_frag<DK>(base, kt & 1, kb);
#pragma unroll
            for (int k = 0; k < kPieces; ++k) acc = mma(at, Yw[kb][k][lane], acc);
        }
        return acc;
    };
    // the key that element r of a key tile b's result stands for
    auto key_of = [&](int b, int r) { return BF ? rho(b, 4 * gl + r) : 16 * b + 4 * gl + r; };

    // K S and X = V - gamma K S (waves 0-3); with `qs`, also the row sums (QS).dO and, for bf16
    // inputs, gamma dO as fragments for the state gradient (waves 4-7)
    auto ks_x = [&](bool qs) {
        if (wave < 4) {
            const int a = wave;
            f32x4b acc;
            if constexpr (BF) acc = rows_bf(sm.Kb, sm.Sf, a);
            else acc = rows_times_state(sm.K, sm.S, a);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * a + 4 * gl + r;
                sm.KS[t * LW + cl] = acc[r];
                sm.VX[t * LW + cl] -= sm.gam[t] * acc[r];
            }
        } else if (qs) {
            const int a = wave - 4;
            f32x4b acc, gdo;
            if constexpr (BF) acc = rows_bf(sm.Qb, sm.Sf, a);
            else acc = rows_times_state(sm.Q, sm.S, a);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * a + 4 * gl + r;
                const float o = sm.dO[t * LW + cl];
                const float s = row_sum16(acc[r] * o);
                if (cl == 0) sm.r_qsdo[t] = s;
                gdo[r] = sm.gam[t] * o;
            }
            if constexpr (BF) put_frag4(sm.Yf, a >> 1, lane, 4 * (a & 1), gdo);
        }
        lds_barrier();
    };
    // U = T diag(beta) X (waves 0-3, T lower triangular); with `kd`, K D into KD (waves 4-7)
    auto u_kd = [&](bool kd) {
        if (wave < 4) {
            const int a = wave;
            f32x4b acc = z4;
            for (int k0 = 0; k0 < 16 * (a + 1); k0 += 16)
#pragma unroll
                for (int kk = k0; kk < k0 + 16; kk += 4)
                    acc = mfma4(sm.T[(16 * a + cl) * kLC + kk + gl], sm.beta[kk + gl] * sm.VX[(kk + gl) * LW + cl], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.U[(16 * a + 4 * gl + r) * LW + cl] = acc[r];
            if constexpr (BF) {
                if (!kd) {                     // forward sweep: f U as fragments for the state update
                    f32x4b fu;
#pragma unroll
                    for (int r = 0; r < 4; ++r) fu[r] = sm.f[16 * a + 4 * gl + r] * acc[r];
                    put_frag4(sm.Yf, a >> 1, lane, 4 * (a & 1), fu);
                }
            }
        } else if (kd) {
            const int a = wave - 4;
            f32x4b acc;
            if constexpr (BF) acc = rows_bf(sm.Kb, sm.Df, a);
            else acc = rows_times_state(sm.K, sm.D, a);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.KD[(16 * a + 4 * gl + r) * LW + cl] = acc[r];
        }
        lds_barrier();
    };
    // key tile b of M^T (w o Y) over the chunk (M = K or Q [C][DK], Y C x 16, w per token)
    auto keys_times = [&](const float* M, const float* Y, const float* w1, const float* w2, int b) {
        f32x4b acc = z4;
        for (int k0 = 0; k0 < kC; k0 += 16)
#pragma unroll
            for (int kk = k0; kk < k0 + 16; kk += 4) {
                const int t = kk + gl;
                float wt = w1[t];
                if (w2) wt *= w2[t];
                acc = mfma4(M[t * LK + 16 * b + cl], wt * Y[t * LW + cl], acc);
            }
        return acc;
    };

    // ---------------- forward sweep: the state at every chunk start ----------------------------
    const size_t sbase = ((size_t)n * Hv + h) * SSL;
    // Per-thread elements of a slice state: column tid % 16, the PS consecutive keys PS (tid / 16) + j
    // (4 or 2 consecutive elements of one lane of a key fragment)
    constexpr int PS = DK * kW / kST;
    const int st_c = tid % kW, st_i = PS * (tid / kW);
    // X (fp32, pitch LW) and, for bf16 inputs, its fragments Xf from the thread's elements x
    auto put_state = [&](float* X, bf16x8 (*Xf)[kPieces][kWave], const float* x) {
#pragma unroll
        for (int j = 0; j < PS; ++j) X[(st_i + j) * LW + st_c] = x[j];
        if constexpr (BF) {
            const int i = st_i % 32;
            put_frag<PS>(Xf, st_i / 32, 16 * (i / 8) + st_c, i % 8, x);
        }
    };
    {
        float x[PS];
#pragma unroll
        for (int j = 0; j < PS; ++j)
            x[j] = initial_state ? initial_state[sbase + (size_t)(st_i + j) * dv + c0 + st_c] : 0.f;
        if constexpr (BF) put_state(sm.S, sm.Sf, x);
        else put_state(sm.S, nullptr, x);
    }
    // the chunk-start state of this slice, prefetched a chunk ahead in the reverse sweep
    float sck[PS];
    auto fetch_ckpt = [&](int ci) {
#pragma unroll
        for (int j = 0; j < PS; ++j) sck[j] = ck_at(ci)[(size_t)(st_i + j) * dv + c0 + st_c];
    };
    ChunkIn cin;
    if (nchunks > 0) fetch_chunk(cin, 0, std::false_type{});
    lds_barrier();
    for (int ci = 0; ci < nchunks; ++ci) {
        refresh_lane();
        commit_chunk(cin, ci, std::false_type{});
        // (each thread stores the elements it reads back with fetch_ckpt: the last chunk's are read
        // right away, with no barrier between)
#pragma unroll
        for (int j = 0; j < PS; ++j)
            ck_at(ci)[(size_t)(st_i + j) * dv + c0 + st_c] = sm.S[(st_i + j) * LW + st_c];
        // the next chunk's inputs; after the last, the reverse sweep's first chunk (this one)
        if (ci + 1 < nchunks) {
            fetch_chunk(cin, ci + 1, std::false_type{});
        } else {
            fetch_chunk(cin, ci, std::true_type{});
            fetch_ckpt(ci);
        }
        ks_x(false);
        u_kd(false);
        // S <- gamma_C S + K^T diag(f) U, key tile b per wave
        const float gC = sm.gam[kC - 1];
        for (int b = wave; b < KT; b += kSW) {
            f32x4b acc, sn;
            if constexpr (BF) acc = keys_bf(sm.Kb, sm.Yf, b);
            else acc = keys_times(sm.K, sm.U, sm.f, nullptr, b);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float* sp = &sm.S[key_of(b, r) * LW + cl];
                *sp = gC * *sp + acc[r];
                sn[r] = *sp;
            }
            if constexpr (BF) put_frag4(sm.Sf, b >> 1, lane, 4 * (b & 1), sn);
        }
        lds_barrier();
    }

    // ---------------- reverse sweep ------------------------------------------------------------
    {
        float x[PS];
#pragma unroll
        for (int j = 0; j < PS; ++j)
            x[j] = d_final ? d_final[sbase + (size_t)(st_i + j) * dv + c0 + st_c] : 0.f;
        if constexpr (BF) put_state(sm.D, sm.Df, x);
        else put_state(sm.D, nullptr, x);
    }
    for (int ci = nchunks - 1; ci >= 0; --ci) {
        refresh_lane();
        const int cs = t0 + ci * kC;
        const size_t tok0 = (size_t)row * T + cs;
        const int slot = slot0 + ci;
        float* wd = ws_d + ((size_t)slot * Hv + h) * SSL;
        if constexpr (BF) put_state(sm.S, sm.Sf, sck);
        else put_state(sm.S, nullptr, sck);
#pragma unroll
        for (int j = 0; j < PS; ++j)                            // D at this chunk's end, for the combine
            wd[(size_t)(st_i + j) * dv + c0 + st_c] = sm.D[(st_i + j) * LW + st_c];
        const int Lc = commit_chunk(cin, ci, std::true_type{});
        if (ci > 0) {
            fetch_chunk(cin, ci - 1, std::true_type{});
            fetch_ckpt(ci - 1);
        }
        ks_x(true);
        u_kd(true);

        // dU = P^T dO + f (K D) (P lower triangular: rows t' >= t), and the row sums (KD).U, on
        // waves 0-3; beside them waves 4-7 form <S, D> over the slice, for dG at the chunk's last
        // row (D is still the gradient at this chunk's end)
        if (wave < 4) {
            const int a = wave;
            f32x4b acc = z4;
            for (int k0 = 16 * a; k0 < kC; k0 += 16)
#pragma unroll
                for (int kk = k0; kk < k0 + 16; kk += 4)
                    acc = mfma4(sm.P[(kk + gl) * kLC + 16 * a + cl], sm.dO[(kk + gl) * LW + cl], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * a + 4 * gl + r;
                const float kd = sm.KD[t * LW + cl];
                sm.dU[t * LW + cl] = acc[r] + sm.f[t] * kd;
                const float s = row_sum16(kd * sm.U[t * LW + cl]);
                if (cl == 0) sm.r_kdu[t] = s;
            }
        } else {
            float sd = 0.f;
            for (int e = tid - kST / 2; e < DK * kW; e += kST / 2) {
                const int i = e / kW, c = e % kW;
                sd += sm.S[i * LW + c] * sm.D[i * LW + c];
            }
            sd = wave_sum64(sd);
            if (lane == 0) sm.red[wave - 4] = sd;
        }
        lds_barrier();
        // dY = T^T dU (into KD), dX = beta dY = dV, and the row sums X.dY and (KS).dX, on waves 0-3;
        // beside them waves 4-7 start dL/dS for the previous chunk, gamma_C D + Q^T diag(gamma) dO
        // (the part that does not need dY), in place over D
        if (wave < 4) {
            const int a = wave;
            f32x4b acc = z4;
            for (int k0 = 16 * a; k0 < kC; k0 += 16)
#pragma unroll
                for (int kk = k0; kk < k0 + 16; kk += 4)
                    acc = mfma4(sm.T[(kk + gl) * kLC + 16 * a + cl], sm.dU[(kk + gl) * LW + cl], acc);
            float* wu = ws_u + ((size_t)slot * Hv + h) * kC * dv + c0 + cl;
            float* wy = ws_y + ((size_t)slot * Hv + h) * kC * dv + c0 + cl;
            f32x4b zd;                                  // gamma beta dY, for bf16 inputs as fragments
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * a + 4 * gl + r;
                const float dy = acc[r], dx = sm.beta[t] * dy;
                zd[r] = sm.gam[t] * dx;
                sm.KD[t * LW + cl] = dy;
                wu[(size_t)t * dv] = sm.U[t * LW + cl];     // U and dY (zero past the chunk's end),
                wy[(size_t)t * dv] = dy;                    // for the combine
                if (t < Lc) dv_out[((tok0 + t) * Hv + h) * dv + c0 + cl] = dx;
                const float s1 = row_sum16(sm.VX[t * LW + cl] * dy);
                const float s2 = row_sum16(sm.KS[t * LW + cl] * dx);
                if (cl == 0) {
                    sm.r_db[t] = s1;
                    sm.r_ksdx[t] = s2;
                }
            }
            if constexpr (BF) put_frag4(sm.Zf, a >> 1, lane, 4 * (a & 1), zd);
        } else {
            const float gC = sm.gam[kC - 1];
            for (int b = wave - 4; b < KT; b += 4) {
                f32x4b a1;
                if constexpr (BF) a1 = keys_bf(sm.Qb, sm.Yf, b);
                else a1 = keys_times(sm.Q, sm.dO, sm.gam, nullptr, b);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float* dp = &sm.D[key_of(b, r) * LW + cl];
                    *dp = gC * *dp + a1[r];
                }
            }
        }
        lds_barrier();
        // dG (this slice's part: the terms through the state; those of the C x C matrices are the
        // combine kernel's) and its reverse running sum, by the last wave (lane = row t), beside the
        // rest of dL/dS, - K^T diag(gamma beta) dY, one key tile per wave
        if (wave == kSW - 1) {
            const int t = lane;
            const float fkdu = wave_sum64(sm.f[t] * sm.r_kdu[t]);
            const float sdt = (sm.red[0] + sm.red[1]) + (sm.red[2] + sm.red[3]);
            float x = sm.gam[t] * sm.r_qsdo[t] - sm.gam[t] * sm.r_ksdx[t] - sm.f[t] * sm.r_kdu[t];
            if (t == kC - 1) x += sm.gam[kC - 1] * sdt + fkdu;
            x = wave_suffix_sum(x, t);
            if (t < Lc) {
                const size_t o = (size_t)sl * rows * Hv + (tok0 + t) * Hv + h;
                part_dg[o] = x;
                part_db[o] = sm.r_db[t];
            }
        }
        for (int b = wave; b < KT; b += kSW) {
            f32x4b a2, dn;
            if constexpr (BF) a2 = keys_bf(sm.Kb, sm.Zf, b);
            else a2 = keys_times(sm.K, sm.KD, sm.gam, sm.beta, b);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float* dp = &sm.D[key_of(b, r) * LW + cl];
                *dp -= a2[r];
                dn[r] = *dp;
            }
            if constexpr (BF) put_frag4(sm.Df, b >> 1, lane, 4 * (b & 1), dn);
        }
        lds_barrier();
    }
    if (d_initial) {   // (the thread's own elements of D: with no chunk there is no barrier since they were written)
#pragma unroll
        for (int j = 0; j < PS; ++j)
            d_initial[sbase + (size_t)(st_i + j) * dv + c0 + st_c] = sm.D[(st_i + j) * LW + st_c];
    }
}

// ------------------------------------------------------------------------------------------------
// One workgroup per (chunk, q/k head): everything that needs a v-head's whole dv.  Per v-head h of
// the q/k head, with S the chunk-start state (the forward sweep's checkpoint), D the state gradient
// at the chunk's end, and U, dY from the slice kernel:
//     dP = (dO U^T) (j <= t),   dA = -(dY U^T) (j < t),   dBm = diag(beta) dA
//     E = dP o P + dBm o Bm:    dG_t += (rows - columns of E)_t,   dbeta_t += (rows of dA o Bm)_t
// added, as reverse running sums for dg, to the slices' partials; then, summed over the v-heads,
//     dq = sum_h diag(gamma) dO S^T + (dP o Gam) K
//     dk = sum_h [diag(f) U D^T - diag(gamma beta) dY S^T] + (dP o Gam)^T Q + ((dBm o Gam) + (dBm o Gam)^T) K
// All products run on the fp32 matrix cores.  Wave w of eight owns the 16 x 16 output tiles
// p = w, w + 8, .. of dq and of dk (row tile p / KT, key tile p % KT) and the tiles
// ((w + 8 j) / 4, w % 4) of the C x C matrices.  The products over dv take it in 32-column tiles
// staged in LDS; each tile's (and each 16-token block's) sum is formed on its own and then added to
// the running total, which keeps the fp32 chains short.
constexpr int kTC = 32;          // dv columns per staged tile of the state products
constexpr int kLT = kTC + 4;     // pitch of those tiles: rows 16 a + c, columns k + g land in distinct banks
constexpr int kLCc = kC + 4;     // pitch of the C x C matrices in the combine kernel
constexpr int kCT = 512;         // combine kernel threads: 8 waves, each owning 1/8 of the output tiles
constexpr int kMaxSlices = 8;    // 16-column slices of a state, at most (dv <= 128)

template <int DK>
struct CombineLds {
    static constexpr int LK = DK + 16;   // K, Q rows: reads at rows k + g, columns 16 b + c are conflict-free
    struct StateTerms {
        float S[DK * kLT], D[DK * kLT];              // [key][column]
        float O[kC * kLT], U[kC * kLT], Y[kC * kLT]; // [token][column], scaled by gamma, f, -gamma beta
        float Ou[kC * kLT], Uu[kC * kLT], Yu[kC * kLT];  // the same unscaled, for dP and dA
    };
    struct CCTerms {                                 // (over S and D once a v-head's dv is done)
        float E[kC * kLCc], F[kC * kLCc];            // E and dA o Bm
    };
    struct ChunkTerms {
        float K[kC * LK], Q[kC * LK];
        float P[kC * kLCc], B[kC * kLCc];
    };
    struct StateAndRaw {
        StateTerms st;
        // the next tile's S, D [DK][32] and dO, U, dY [C][32] as they arrive from memory
        // (global_load_lds), while the current tile's products run
        float rS[DK * kTC], rD[DK * kTC], rO[kC * kTC], rU[kC * kTC], rY[kC * kTC];
    };
    union {
        StateAndRaw sr;
        CCTerms cc;                                  // (between v-heads: overlaps st only)
        ChunkTerms ct;                               // (after the v-head loop)
    };
    float G[kC], gam[kC], f[kC], beta[kC];
};

static_assert(sizeof(CombineLds<128>) <= 160 * 1024, "combine LDS exceeds a CU's 160 KiB");

typedef __attribute__((address_space(1))) void glb_void_b;
typedef __attribute__((address_space(3))) void lds_void_b;
// 16 (4) bytes per lane from global memory straight into LDS: lane l writes dst + 16 l (4 l); dst is
// the same for the whole wave
__device__ __forceinline__ void lds_copy16(const float* src, float* dst) {
    __builtin_amdgcn_global_load_lds((glb_void_b*)src, (lds_void_b*)dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_copy4(const float* src, float* dst) {
    __builtin_amdgcn_global_load_lds((glb_void_b*)src, (lds_void_b*)dst, 4, 0, 0);
}
// s_waitcnt vmcnt(0), the other counters left alone: the wave's copies into LDS have landed
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int DK, typename TIn, typename TG>
__global__ __launch_bounds__(kCT) void bwd_combine_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TG* __restrict__ g,
    const TG* __restrict__ beta, const float* __restrict__ d_o, const int32_t* __restrict__ cu_seqlens,
    int N, int T, int Hk, int Hv, int dv, int slices, long long rows, const float* __restrict__ mats,
    const float* __restrict__ ckpt, const float* __restrict__ ws_d, const float* __restrict__ ws_u,
    const float* __restrict__ ws_y, const float* __restrict__ part_dg, const float* __restrict__ part_db,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dg, float* __restrict__ db) {
    using Lds = CombineLds<DK>;
    constexpr int LK = Lds::LK;
    constexpr int KT = DK / 16;                  // key tiles
    constexpr int NT = KT / 2;                   // output tiles per wave (of dq, and of dk)
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    Lds& sm = *reinterpret_cast<Lds*>(smem_raw);
    const int slot = blockIdx.x, kh = blockIdx.y;
    int n, row, cs, L;
    if (!bwd_locate(slot, cu_seqlens, N, T, n, row, cs, L)) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gl = lane >> 4, cl = lane & 15;
    const size_t tok0 = (size_t)row * T + cs;
    const int G = Hv / Hk;
    const f32x4b z4 = {0.f, 0.f, 0.f, 0.f};
    f32x4b aq[NT], ak[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) aq[j] = ak[j] = z4;
    // C x C tiles of this wave: (a, b) = ((wave + 8 j) / 4, wave % 4), j = 0, 1
    const int cb = wave & 3, ca0 = wave >> 2;
    f32x4b sp[2], sb[2];                         // sum over v-heads of dP o Gam, dBm o Gam
#pragma unroll
    for (int j = 0; j < 2; ++j) sp[j] = sb[j] = z4;

    // The 32-column tile (x, c0) of v-head kh G + x, copied from memory straight into the raw area:
    // wave w issues the copies j = w, w + 8, ..; copy j of a [rows][32] block covers its 16-byte
    // pieces 64 j .. 64 j + 63 (lane l: row (64 j + l) / 8, columns 4 ((64 j + l) % 8) ..), those of
    // dO 4-byte pieces (its rows need only 4-byte alignment), rows past the chunk's end read its
    // last row (zeroed when restaged).
    auto prefetch_tile = [&](int x, int c0) {
        const int h = kh * G + x;
        const float* Sg = ckpt + ((size_t)slot * Hv + h) * DK * dv + c0;
        const float* Dg = ws_d + ((size_t)slot * Hv + h) * DK * dv + c0;
        const float* Ug = ws_u + ((size_t)slot * Hv + h) * kC * dv + c0;
        const float* Yg = ws_y + ((size_t)slot * Hv + h) * kC * dv + c0;
        constexpr int CS = DK * kTC / 4 / kWave, CT = kC * kTC / 4 / kWave, CO = kC * kTC / kWave;
        for (int j = wave; j < CS; j += kCT / kWave) {
            const int p = kWave * j + lane, i = p / (kTC / 4), c = 4 * (p % (kTC / 4));
            lds_copy16(Sg + (size_t)i * dv + c, sm.sr.rS + 4 * kWave * j);
            lds_copy16(Dg + (size_t)i * dv + c, sm.sr.rD + 4 * kWave * j);
        }
        for (int j = wave; j < CT; j += kCT / kWave) {
            const int p = kWave * j + lane, t = p / (kTC / 4), c = 4 * (p % (kTC / 4));
            lds_copy16(Ug + (size_t)t * dv + c, sm.sr.rU + 4 * kWave * j);
            lds_copy16(Yg + (size_t)t * dv + c, sm.sr.rY + 4 * kWave * j);
        }
        for (int j = wave; j < CO; j += kCT / kWave) {
            const int p = kWave * j + lane, t = p / kTC, c = p % kTC;
            lds_copy4(d_o + ((tok0 + min(t, L - 1)) * Hv + h) * dv + c0 + c, sm.sr.rO + kWave * j);
        }
    };
    for (int x = 0; x < G; ++x) {
        const int h = kh * G + x;
        if (tid < kC) {
            const bool in = tid < L;
            sm.G[tid] = in ? to_f32(g[(tok0 + tid) * Hv + h]) : 0.f;
            sm.beta[tid] = in ? to_f32(beta[(tok0 + tid) * Hv + h]) : 0.f;
        }
        lds_barrier();
        chunk_decays(sm.G, sm.gam, sm.f, tid);
        lds_barrier();
        f32x4b cp[2], ca[2];                     // dO U^T and dY U^T on the wave's C x C tiles
#pragma unroll
        for (int j = 0; j < 2; ++j) cp[j] = ca[j] = z4;
        // ---- the products over dv, 32 columns at a time ----
        for (int c0 = 0; c0 < dv; c0 += kTC) {
            // this tile's inputs have landed in the raw area (issued during the previous tile, or
            // just below for a v-head's first): restage them with the padded pitch, unscaled and
            // scaled by gamma, f and -gamma beta
            if (x == 0 && c0 == 0) prefetch_tile(0, 0);
            wait_vmcnt0();
            lds_barrier();
            {
                constexpr int PS = DK * kTC / 4 / kCT, PT = kC * kTC / 4 / kCT;
#pragma unroll
                for (int it = 0; it < PS; ++it) {
                    const int e = 4 * (tid + kCT * it), i = e / kTC, c = e % kTC;
                    *reinterpret_cast<float4*>(&sm.sr.st.S[i * kLT + c]) = *reinterpret_cast<const float4*>(&sm.sr.rS[e]);
                    *reinterpret_cast<float4*>(&sm.sr.st.D[i * kLT + c]) = *reinterpret_cast<const float4*>(&sm.sr.rD[e]);
                }
                auto scaled = [](float s_, float4 v) { return make_float4(s_ * v.x, s_ * v.y, s_ * v.z, s_ * v.w); };
#pragma unroll
                for (int it = 0; it < PT; ++it) {
                    const int e = 4 * (tid + kCT * it), t = e / kTC, c = e % kTC;
                    const float m = t < L ? 1.f : 0.f;
                    const float4 vo = scaled(m, *reinterpret_cast<const float4*>(&sm.sr.rO[e]));
                    const float4 vu = *reinterpret_cast<const float4*>(&sm.sr.rU[e]);
                    const float4 vy = *reinterpret_cast<const float4*>(&sm.sr.rY[e]);
                    *reinterpret_cast<float4*>(&sm.sr.st.Ou[t * kLT + c]) = vo;
                    *reinterpret_cast<float4*>(&sm.sr.st.Uu[t * kLT + c]) = vu;
                    *reinterpret_cast<float4*>(&sm.sr.st.Yu[t * kLT + c]) = vy;
                    *reinterpret_cast<float4*>(&sm.sr.st.O[t * kLT + c]) = scaled(sm.gam[t], vo);
                    *reinterpret_cast<float4*>(&sm.sr.st.U[t * kLT + c]) = scaled(sm.f[t], vu);
                    *reinterpret_cast<float4*>(&sm.sr.st.Y[t * kLT + c]) = scaled(-sm.gam[t] * sm.beta[t], vy);
                }
            }
            lds_barrier();
            // the next tile: this v-head's, or the next v-head's first
            if (c0 + kTC < dv) prefetch_tile(x, c0 + kTC);
            else if (x + 1 < G) prefetch_tile(x + 1, 0);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int p = wave + 8 * j, a = p / KT, b = p % KT;
                f32x4b tq = z4, tk = z4;
#pragma unroll
                for (int kk = 0; kk < kTC; kk += 4) {
                    const float sb_ = sm.sr.st.S[(16 * b + cl) * kLT + kk + gl];
                    tq = mfma4(sm.sr.st.O[(16 * a + cl) * kLT + kk + gl], sb_, tq);
                    tk = mfma4(sm.sr.st.Y[(16 * a + cl) * kLT + kk + gl], sb_, tk);
                    tk = mfma4(sm.sr.st.U[(16 * a + cl) * kLT + kk + gl], sm.sr.st.D[(16 * b + cl) * kLT + kk + gl], tk);
                }
                aq[j] += tq;
                ak[j] += tk;
                __builtin_amdgcn_sched_barrier(0);   // (a tile's operand reads are not hoisted into the
            }                                        // previous tile: registers stay within budget)
            // dO U^T and dY U^T on the wave's C x C tiles on or below the diagonal
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int ra = ca0 + 2 * j;
                if (ra < cb) continue;
                f32x4b tp = z4, ta = z4;
#pragma unroll
                for (int kk = 0; kk < kTC; kk += 4) {
                    const float ub = sm.sr.st.Uu[(16 * cb + cl) * kLT + kk + gl];
                    tp = mfma4(sm.sr.st.Ou[(16 * ra + cl) * kLT + kk + gl], ub, tp);
                    ta = mfma4(sm.sr.st.Yu[(16 * ra + cl) * kLT + kk + gl], ub, ta);
                }
                cp[j] += tp;
                ca[j] += ta;
                __builtin_amdgcn_sched_barrier(0);
            }
            lds_barrier();
        }
        // ---- the C x C gradients of v-head h: E and dA o Bm to LDS, the v-head sums in registers ----
        {
            const float* Bmh = mats + ((size_t)slot * Hv + h) * 3 * kMat + kMat;     // (T, Bm, P)
            const float* Ph = Bmh + kMat;
            // every element's Bm and P in flight together, and no branch around the decay (its
            // argument clamped to <= 0, which leaves the elements on or below the diagonal as they
            // are): loads inside a branch were each waited for before the next
            float bmv[2][4], pvv[2][4];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * (ca0 + 2 * j) + 4 * gl + r, i = 16 * cb + cl;
                    bmv[j][r] = Bmh[t * kC + i];
                    pvv[j][r] = Ph[t * kC + i];
                }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * (ca0 + 2 * j) + 4 * gl + r, i = 16 * cb + cl;   // element (t, i)
                    const float dP = i <= t ? cp[j][r] : 0.f;
                    const float dA = i < t ? -ca[j][r] : 0.f;
                    const float bm = bmv[j][r], pv = pvv[j][r];
                    const float ed = expf(fminf(sm.G[t] - sm.G[i], 0.f));
                    const float dec = i <= t ? ed : 0.f;
                    const float dbm = sm.beta[t] * dA;
                    sm.cc.E[t * kLCc + i] = dP * pv + dbm * bm;
                    sm.cc.F[t * kLCc + i] = dA * bm;
                    sp[j][r] += dP * dec;
                    sb[j][r] += dbm * dec;
                }
        }
        lds_barrier();
        // rows minus columns of E (dG, as a reverse running sum) and rows of dA o Bm (dbeta), added
        // to the slices' partials, by the first wave (lane = row t)
        if (tid < kC) {
            const int t = tid;
            // the slices' partials first, all in flight together while the row sums run (a loop that
            // adds each as it arrives waits out one memory round trip per load); summed in slice order
            float pg[kMaxSlices], pb[kMaxSlices];
            const int tl = min(t, L - 1);
#pragma unroll
            for (int s = 0; s < kMaxSlices; ++s) {
                const size_t o = ((size_t)min(s, slices - 1) * rows + tok0 + tl) * Hv + h;
                pg[s] = part_dg[o];
                pb[s] = part_db[o];
            }
            float re = 0.f, ce = 0.f, rb = 0.f;
#pragma unroll 8
            for (int i = 0; i < kC; ++i) {
                re += sm.cc.E[t * kLCc + i];
                ce += sm.cc.E[i * kLCc + t];
                rb += sm.cc.F[t * kLCc + i];
            }
            const float xg = wave_suffix_sum(re - ce, t);
            if (t < L) {
                float ag = 0.f, ab = 0.f;
#pragma unroll
                for (int s = 0; s < kMaxSlices; ++s) {
                    if (s < slices) {
                        ag += pg[s];
                        ab += pb[s];
                    }
                }
                dg[(tok0 + t) * Hv + h] = ag + xg;
                db[(tok0 + t) * Hv + h] = ab + rb;
            }
        }
        lds_barrier();                         // E, F and the gates are rewritten for the next v-head
    }

    // ---- the chunk terms: K, Q, and the C x C matrices summed over the v-heads ----
    stage_rows<DK, LK, kCT>(k, tok0, Hk, kh, L, sm.ct.K, tid);
    stage_rows<DK, LK, kCT>(q, tok0, Hk, kh, L, sm.ct.Q, tid);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * (ca0 + 2 * j) + 4 * gl + r, i = 16 * cb + cl;
            sm.ct.P[t * kLCc + i] = sp[j][r];
            sm.ct.B[t * kLCc + i] = sb[j][r];
        }
    __syncthreads();
    {   // B symmetrised in LDS
        constexpr int PE = kMat / kCT;
        float ab[PE];
#pragma unroll
        for (int it = 0; it < PE; ++it) {
            const int e = tid + kCT * it, t = e / kC, i = e % kC;
            ab[it] = sm.ct.B[t * kLCc + i] + sm.ct.B[i * kLCc + t];
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < PE; ++it) {
            const int e = tid + kCT * it, t = e / kC, i = e % kC;
            sm.ct.B[t * kLCc + i] = ab[it];
        }
    }
    __syncthreads();
    // dq += P' K, dk += P'^T Q + B' K over the chunk's tokens (16-deep blocks of four products)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int p = wave + 8 * j, a = p / KT, b = p % KT;
        for (int k0 = 0; k0 < kC; k0 += 16) {
            f32x4b tq = z4, tk = z4;
#pragma unroll
            for (int kk = k0; kk < k0 + 16; kk += 4) {
                const float kb_ = sm.ct.K[(kk + gl) * LK + 16 * b + cl];
                tq = mfma4(sm.ct.P[(16 * a + cl) * kLCc + kk + gl], kb_, tq);
                tk = mfma4(sm.ct.P[(kk + gl) * kLCc + 16 * a + cl], sm.ct.Q[(kk + gl) * LK + 16 * b + cl], tk);
                tk = mfma4(sm.ct.B[(16 * a + cl) * kLCc + kk + gl], kb_, tk);
            }
            aq[j] += tq;
            ak[j] += tk;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // lane (g, c) of tile (a, b), element r: row 16 a + 4 g + r, key 16 b + c
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int p = wave + 8 * j, a = p / KT, b = p % KT;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * a + 4 * gl + r;
            if (t < L) {
                const size_t o = ((tok0 + t) * Hk + kh) * DK + 16 * b + cl;
                dq[o] = aq[j][r];
                dk[o] = ak[j][r];
            }
        }
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
    size_t ckpt, mats, wd, wu, wy, pg, pb, total;
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
    l.wd = off;   off = align256b(off + sizeof(float) * (size_t)l.slots * Hv * dk * dv);
    l.wu = off;   off = align256b(off + sizeof(float) * (size_t)l.slots * Hv * kC * dv);
    l.wy = off;   off = align256b(off + sizeof(float) * (size_t)l.slots * Hv * kC * dv);
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
    float* wd = reinterpret_cast<float*>(ws + lay.wd);
    float* wu = reinterpret_cast<float*>(ws + lay.wu);
    float* wy = reinterpret_cast<float*>(ws + lay.wy);
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
    const size_t bytes = sizeof(SliceLds<DK, std::is_same<TIn, bf16_t>::value>);
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes)) != hipSuccess)
        return e;
    // (with no tokens this still runs: every sequence is empty and passes d_final through)
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.N * a.Hv * slices)), dim3(kST), bytes, a.stream,
                       static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.v), static_cast<const TG*>(a.g),
                       static_cast<const TG*>(a.beta), a.initial_state, a.cu_seqlens, a.d_o, a.d_final,
                       a.T, a.Hk, a.Hv, a.dv, mats, ckpt, wd, wu, wy, pg, pb, a.dv_out, a.d_initial, rows,
                       lay.slots);
    if ((e = hipGetLastError()) != hipSuccess || rows == 0) return e;
    if (packed) {
        const long long nq = rows * a.Hk * a.dk, ng = rows * a.Hv, nmax = nq > ng ? nq : ng;
        hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((nmax + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                           a.stream, a.dq, nq, a.dk_out, nq, a.dg, ng, a.dbeta, ng);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (slots > 0) {
        const auto ck = bwd_combine_kernel<DK, TIn, TG>;
        const size_t cbytes = sizeof(CombineLds<DK>);
        if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(ck),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)cbytes)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(ck, dim3((unsigned)slots, (unsigned)a.Hk), dim3(kCT), cbytes, a.stream,
                           static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k), static_cast<const TG*>(a.g),
                           static_cast<const TG*>(a.beta), a.d_o, a.cu_seqlens, a.N, a.T, a.Hk, a.Hv, a.dv, slices,
                           rows, mats, ckpt, wd, wu, wy, pg, pb, a.dq, a.dk_out, a.dg, a.dbeta);
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
