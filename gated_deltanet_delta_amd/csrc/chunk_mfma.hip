// chunk_mfma.hip -- chunked gated delta rule on gfx950 bf16 matrix cores (dk = 128).
//
// Notation (one chunk of C = 64 tokens of one sequence and v-head, start state S (dk x dv), G_t the
// running sum of g inside the chunk, Gam_tj = e^(G_t - G_j) for j <= t):
//
//   A  = diag(beta) (K K^T o Gam), strictly lower        T  = (I + A)^-1
//   W  = T diag(beta e^G) K                               Ut = T diag(beta) V
//   P  = (Q K^T) o Gam, lower with diagonal
//   U  = Ut - W S                                         (the chunk's per-token deltas)
//   O  = diag(e^G) Q S + P U
//   S <- e^(G_C) S + K^T diag(e^(G_C - G)) U
//
// which is the per-token rule S_t = e^(g_t)(I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
// o_t = S_t^T q_t unrolled over the chunk.  Every decay factor is exp of a non-positive number.
//
// Two kernels:
//   chunk_prep_kernel   one workgroup per (chunk, v-head), all chunks in parallel: cumsum, A on
//                       the matrix cores, T by a blocked forward substitution (16 x 16 diagonal
//                       blocks by substitution, off-diagonal blocks by fp32 matrix-core products),
//                       then -W (bf16) and Ut (fp32) into the workspace.
//   chunk_state_kernel  one workgroup per (sequence, v-head, slice of WS state columns), walking
//                       the chunks in order.  Columns of S never interact, so slices are
//                       independent.  The slice of S stays in matrix-core accumulators for the
//                       whole sequence; each of the 4 waves owns 32 of the 128 key rows.
//
// Precision: q, k, v enter the matrix cores as exact bf16 values.  Quantities that feed the output
// with full weight (S, U, P, T diag(beta)) enter as two bf16 terms hi + lo (hi = bf16(x),
// lo = bf16(x - hi)), so their products carry ~16 significant bits; W enters as one bf16 term.
// Accumulation is fp32 everywhere; decay factors are applied on the fp32 side.
//
// MFMA lane layouts used (wave64, v_mfma_f32_16x16x32_bf16): lane l = 16 g + c holds A[c][8g..8g+7]
// and B[8g..8g+7][c]; the 16 x 16 result D[4g + r][c], r = 0..3, sits in lane l, element r.  The
// reduction index of one instruction may be permuted freely as long as A and B agree; the kernels
// use that to feed an accumulator tile straight back in as an operand without a transpose.

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;      // chunk length
constexpr int kDK = 128;    // key dimension handled by this file
constexpr int kThreads = 256;

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ __bf16 hi_of(float x) { return (__bf16)x; }
__device__ __forceinline__ __bf16 lo_of(float x, __bf16 hi) { return (__bf16)(x - (float)hi); }

__device__ __forceinline__ bf16x8 lds8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 lds4(const __bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ bf16x8 cat44(const bf16x4& a, const bf16x4& b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ------------------------------------------------------------------------------------------------
// Sequence -> chunk-slot bookkeeping for packed inputs (one workgroup).
//   chunk_start[n] = number of chunks in sequences 0..n-1 (chunk_start[N] = total)
//   order[r]       = sequence with the r-th largest length (ties by index), so that the state
//                    kernel starts the longest sequences first; identity when N > kOrderMax.
constexpr int kOrderMax = 1024;

__global__ __launch_bounds__(kThreads) void plan_kernel(const int32_t* __restrict__ cu_seqlens,
                                                        int N, int T,
                                                        int32_t* __restrict__ chunk_start,
                                                        int32_t* __restrict__ order) {
    __shared__ int32_t part[kThreads];
    __shared__ int32_t lens[kOrderMax];
    const int tid = threadIdx.x;
    const int per = (N + kThreads - 1) / kThreads;
    const int n0 = tid * per, n1 = min(N, n0 + per);
    auto len_of = [&](int n) {
        int a = cu_seqlens[n], b = cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        return b - a;
    };
    int sum = 0;
    for (int n = n0; n < n1; ++n) sum += (len_of(n) + kC - 1) / kC;
    part[tid] = sum;
    lds_barrier();
    for (int off = 1; off < kThreads; off <<= 1) {
        const int add = tid >= off ? part[tid - off] : 0;
        lds_barrier();
        part[tid] += add;
        lds_barrier();
    }
    int run = part[tid] - sum;  // exclusive prefix of this thread's block
    for (int n = n0; n < n1; ++n) {
        chunk_start[n] = run;
        run += (len_of(n) + kC - 1) / kC;
    }
    if (tid == kThreads - 1) chunk_start[N] = part[kThreads - 1];

    if (N <= kOrderMax) {
        for (int n = tid; n < N; n += kThreads) lens[n] = len_of(n);
        lds_barrier();
        for (int n = tid; n < N; n += kThreads) {
            const int ln = lens[n];
            int rank = 0;
            for (int m = 0; m < N; ++m) rank += (lens[m] > ln) || (lens[m] == ln && m < n);
            order[rank] = n;
        }
    } else {
        for (int n = tid; n < N; n += kThreads) order[n] = n;
    }
}

// Locate chunk slot `slot`: sequence n, chunk index ci, packed row, first token and length.
struct ChunkLoc {
    int n, ci, row, t0, len;
};

__device__ __forceinline__ bool locate_chunk(int slot, const int32_t* cu_seqlens,
                                             const int32_t* chunk_start, int N, int T, int nct,
                                             ChunkLoc& loc) {
    if (cu_seqlens) {
        if (slot >= chunk_start[N]) return false;
        int lo = 0, hi = N;  // largest n with chunk_start[n] <= slot
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (chunk_start[mid] <= slot) lo = mid; else hi = mid;
        }
        // skip zero-length sequences that share the same start
        int n = lo;
        while (n + 1 < N && chunk_start[n + 1] <= slot) ++n;
        int a = cu_seqlens[n], b = cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        loc.n = n;
        loc.ci = slot - chunk_start[n];
        loc.row = 0;
        loc.t0 = a + loc.ci * kC;
        loc.len = min(kC, b - loc.t0);
        return loc.len > 0;
    }
    loc.n = slot / nct;
    loc.ci = slot % nct;
    loc.row = loc.n;
    loc.t0 = loc.ci * kC;
    loc.len = min(kC, T - loc.t0);
    return loc.len > 0;
}

// ------------------------------------------------------------------------------------------------
// Staging helpers.
constexpr int kKP = kDK + 8;   // row pitch (elements) of 128-wide bf16 rows in LDS
constexpr int kTP = kC + 8;    // row pitch of transposed (token-contiguous) bf16 tiles
constexpr int kFP = kC + 4;    // row pitch of 64 x 64 fp32 tiles
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Two rows of eight bf16 (rows t and t+1) -> eight 32-bit words, word e = (row t [e], row t+1 [e]).
__device__ __forceinline__ uint32_t pair_word(const uint4& x0, const uint4& x1, int e) {
    const uint32_t a = (&x0.x)[e >> 1], b = (&x1.x)[e >> 1];
    return (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

// Writes the 16 x 8 block held as (rows 2m, 2m+1) x (columns 8p..8p+7) transposed into a
// token-contiguous tile tr[col][token] (pitch kTP): for each column one 32-bit word holds the two
// tokens.  Lanes m = 0..31 of a half-wave cover 32 consecutive words of one row.
__device__ __forceinline__ void store_pair_transposed(__bf16* tr, int m, int p, const uint4& x0,
                                                      const uint4& x1) {
    uint32_t* tr32 = reinterpret_cast<uint32_t*>(tr);
#pragma unroll
    for (int e = 0; e < 8; ++e) tr32[((8 * p + e) * kTP) / 2 + m] = pair_word(x0, x1, e);
}

// ------------------------------------------------------------------------------------------------
// chunk_prep_kernel: one workgroup per (chunk slot, v-head).
//
// LDS: sK  [64][kKP] bf16 (K rows)             sA [64][kFP] fp32
//      sKt [128][kTP] bf16 (K^T), later V^T     sT [64][kFP] fp32
// The log-decay is kept in log2 units (G2 = G log2 e) so every decay factor is one exp2.
template <int DV, typename TG>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const TG* __restrict__ g, const TG* __restrict__ beta, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ chunk_start, int N, int T, int Hk, int Hv, int nct,
    __bf16* __restrict__ ws_Wn, float* __restrict__ ws_U, float* __restrict__ ws_G,
    __bf16* __restrict__ ws_Kt, __bf16* __restrict__ ws_P) {
    static_assert(DV == 64 || DV == 128, "dv");
    static_assert(kC * kKP * 2 == kC * kFP * 4, "Q rows and A share one buffer");
    __shared__ __attribute__((aligned(16))) __bf16 sK[kC * kKP];
    __shared__ __attribute__((aligned(16))) __bf16 sKt[kDK * kTP];
    __shared__ __attribute__((aligned(16))) float sA[kC * kFP];
    __shared__ __attribute__((aligned(16))) float sT[kC * kFP];
    __shared__ float sG[kC], sB[kC], sBE[kC];
    __bf16* sVt = sKt;                            // V^T [DV][kTP] once K^T is dead
    __bf16* sQ = reinterpret_cast<__bf16*>(sA);   // Q rows [64][kKP] until A is formed

    const int slot = blockIdx.x, h = blockIdx.y;
    ChunkLoc loc;
    if (!locate_chunk(slot, cu_seqlens, chunk_start, N, T, nct, loc)) return;
    const int G = Hv / Hk, kh = h / G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, gq = lane >> 4;
    const int m = tid & 31, pg = tid >> 5;  // token pair (2m, 2m+1), column group
    const size_t tok0 = (size_t)loc.row * T + loc.t0;
    const int L = loc.len;
    const uint4 zero = make_uint4(0, 0, 0, 0);

    // ---- stage K (rows and transposed); V stays in registers until K^T is dead -----------------
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int p = pg + 8 * it;
        uint4 x0 = zero, x1 = zero;
        if (2 * m < L) x0 = *reinterpret_cast<const uint4*>(k + ((tok0 + 2 * m) * Hk + kh) * kDK + 8 * p);
        if (2 * m + 1 < L) x1 = *reinterpret_cast<const uint4*>(k + ((tok0 + 2 * m + 1) * Hk + kh) * kDK + 8 * p);
        *reinterpret_cast<uint4*>(sK + (2 * m) * kKP + 8 * p) = x0;
        *reinterpret_cast<uint4*>(sK + (2 * m + 1) * kKP + 8 * p) = x1;
        store_pair_transposed(sKt, m, p, x0, x1);
        uint4 y0 = zero, y1 = zero;
        if (2 * m < L) y0 = *reinterpret_cast<const uint4*>(q + ((tok0 + 2 * m) * Hk + kh) * kDK + 8 * p);
        if (2 * m + 1 < L) y1 = *reinterpret_cast<const uint4*>(q + ((tok0 + 2 * m + 1) * Hk + kh) * kDK + 8 * p);
        *reinterpret_cast<uint4*>(sQ + (2 * m) * kKP + 8 * p) = y0;
        *reinterpret_cast<uint4*>(sQ + (2 * m + 1) * kKP + 8 * p) = y1;
    }
    constexpr int kVIt = DV / 64;
    uint4 v0[kVIt], v1[kVIt];
#pragma unroll
    for (int it = 0; it < kVIt; ++it) {
        const int p = pg + 8 * it;
        v0[it] = zero;
        v1[it] = zero;
        if (2 * m < L) v0[it] = *reinterpret_cast<const uint4*>(v + ((tok0 + 2 * m) * Hv + h) * DV + 8 * p);
        if (2 * m + 1 < L) v1[it] = *reinterpret_cast<const uint4*>(v + ((tok0 + 2 * m + 1) * Hv + h) * DV + 8 * p);
    }
    const size_t ws_row = ((size_t)slot * Hv + h) * kC;
    if (wave == 0) {
        const float gt = lane < L ? to_f32(g[(tok0 + lane) * Hv + h]) * kLog2e : 0.f;
        const float bt = lane < L ? to_f32(beta[(tok0 + lane) * Hv + h]) : 0.f;
        float G2 = gt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(G2, off);
            if (lane >= off) G2 += y;
        }
        sG[lane] = G2;
        sB[lane] = bt;
        sBE[lane] = bt * exp2_fast(G2);
        ws_G[ws_row + lane] = G2;
    }
    for (int e = tid; e < kC * kFP; e += kThreads) sT[e] = 0.f;
    // P's strictly-upper 16x16 tiles are zero
    __bf16* Ph = ws_P + ((size_t)slot * Hv + h) * 2 * kC * kC;
    __bf16* Pl = Ph + kC * kC;
    for (int e = tid; e < kC * kC; e += kThreads) {
        const int t = e >> 6, tp = e & 63;
        if ((tp >> 4) > (t >> 4)) {
            Ph[e] = hi_of(0.f);
            Pl[e] = hi_of(0.f);
        }
    }
    lds_barrier();

    // K^T for the state kernel: written once per q/k head (by the group's first v-head)
    if (h % G == 0) {
        __bf16* dst = ws_Kt + ((size_t)slot * Hk + kh) * kDK * kC;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int e = tid + kThreads * it;  // 128 rows x 8 pieces
            const int i = e >> 3, p = e & 7;
            *reinterpret_cast<uint4*>(dst + i * kC + 8 * p) = *reinterpret_cast<const uint4*>(sKt + i * kTP + 8 * p);
        }
    }

    // ---- A = diag(beta) (K K^T o Gam), strictly lower: 10 lower 16x16 tiles over 4 waves ----------
    // wave 0: (0,0) (3,3) (3,0); wave 1: (1,1) (3,1) (1,0); wave 2: (2,2) (3,2); wave 3: (2,0) (2,1)
    auto tile_a = [](int w, int s) {
        return s == 0 ? (w == 3 ? 2 : w) : s == 1 ? (w == 3 ? 2 : 3) : (w < 2 ? (w == 0 ? 3 : 1) : -1);
    };
    auto tile_b = [](int w, int s) {
        return s == 0 ? (w == 3 ? 0 : w) : s == 1 ? (w == 3 ? 1 : w == 0 ? 3 : w) : 0;
    };
    f32x4 accA[3], accP[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int ta = tile_a(wave, s), tb = tile_b(wave, s);
        accA[s] = zero4();
        accP[s] = zero4();
        if (ta < 0) continue;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 b = lds8(sK + (16 * tb + c) * kKP + 32 * kb + 8 * gq);
            accA[s] = mma(lds8(sK + (16 * ta + c) * kKP + 32 * kb + 8 * gq), b, accA[s]);
            accP[s] = mma(lds8(sQ + (16 * ta + c) * kKP + 32 * kb + 8 * gq), b, accP[s]);
        }
        // P = (Q K^T) o Gam (lower with diagonal) as hi + lo, row-major [t][t']
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * ta + 4 * gq + r, j = 16 * tb + c;
            const float pv = j <= t ? accP[s][r] * exp2_fast(sG[t] - sG[j]) : 0.f;
            const __bf16 ph = hi_of(pv);
            Ph[t * kC + j] = ph;
            Pl[t * kC + j] = lo_of(pv, ph);
        }
    }
    lds_barrier();  // Q rows dead: A overwrites them
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int ta = tile_a(wave, s), tb = tile_b(wave, s);
        if (ta < 0) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * ta + 4 * gq + r, j = 16 * tb + c;
            sA[t * kFP + j] = j < t ? sB[t] * accA[s][r] * exp2_fast(sG[t] - sG[j]) : 0.f;
        }
    }
    lds_barrier();

    // ---- T = (I + A)^-1 ---------------------------------------------------------------------------
    // diagonal blocks: wave w inverts block w, lane c < 16 computes column c by substitution
    if (c == lane) {
        const int base = 16 * wave;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = (t == c) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < t; ++j) acc -= sA[(base + t) * kFP + base + j] * x[j];
            x[t] = acc;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) sT[(base + t) * kFP + base + c] = x[t];
    }
    lds_barrier();
    // off-diagonal blocks, by distance d = a - b:  T_ab = -T_aa * sum_{m=b}^{a-1} A_am T_mb
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        if (wave < 4 - d) {
            const int b = wave, a = wave + d;
            f32x4 X = zero4();
            for (int mm = b; mm < a; ++mm) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float av = sA[(16 * a + c) * kFP + 16 * mm + 4 * s + gq];
                    const float bv = sT[(16 * mm + 4 * s + gq) * kFP + 16 * b + c];
                    X = mma_f32(av, bv, X);
                }
            }
            // -T_aa X with X fed back from the accumulator: step s takes reduction rows 4g + s
            f32x4 Y = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float av = sT[(16 * a + c) * kFP + 16 * a + 4 * gq + s];
                Y = mma_f32(av, X[s], Y);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[(16 * a + 4 * gq + r) * kFP + 16 * b + c] = -Y[r];
        }
        lds_barrier();
    }

    // ---- -W = -T diag(beta e^G) K  (bf16) ---------------------------------------------------------
    // wave w computes key-dim tiles 2w, 2w+1 for all four token tiles
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        f32x4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
        for (int kb = 0; kb <= a / 2; ++kb) {
            const int t = 16 * a + c, j0 = 32 * kb + 8 * gq;
            const float4 t0 = *reinterpret_cast<const float4*>(sT + t * kFP + j0);
            const float4 t1 = *reinterpret_cast<const float4*>(sT + t * kFP + j0 + 4);
            const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
            bf16x8 af;
#pragma unroll
            for (int e = 0; e < 8; ++e) af[e] = hi_of(tv[e] * sBE[j0 + e]);
            const bf16x8 b0 = lds8(sKt + (16 * (2 * wave) + c) * kTP + j0);
            const bf16x8 b1 = lds8(sKt + (16 * (2 * wave + 1) + c) * kTP + j0);
            acc0 = mma(af, b0, acc0);
            acc1 = mma(af, b1, acc1);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * a + 4 * gq + r;
            ws_Wn[(ws_row + t) * kDK + 16 * (2 * wave) + c] = hi_of(-acc0[r]);
            ws_Wn[(ws_row + t) * kDK + 16 * (2 * wave + 1) + c] = hi_of(-acc1[r]);
        }
    }
    lds_barrier();  // K^T dead: V^T overwrites it

    // ---- Ut = T diag(beta) V  (fp32) --------------------------------------------------------------
#pragma unroll
    for (int it = 0; it < kVIt; ++it) store_pair_transposed(sVt, m, pg + 8 * it, v0[it], v1[it]);
    lds_barrier();
    constexpr int kTilesPerWave = DV / 16 / 4;  // value-dim tiles per wave
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        f32x4 acc[kTilesPerWave];
#pragma unroll
        for (int q2 = 0; q2 < kTilesPerWave; ++q2) acc[q2] = zero4();
#pragma unroll
        for (int kb = 0; kb <= a / 2; ++kb) {
            const int t = 16 * a + c, j0 = 32 * kb + 8 * gq;
            const float4 t0 = *reinterpret_cast<const float4*>(sT + t * kFP + j0);
            const float4 t1 = *reinterpret_cast<const float4*>(sT + t * kFP + j0 + 4);
            const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
            bf16x8 ah, al;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = tv[e] * sB[j0 + e];
                ah[e] = hi_of(x);
                al[e] = lo_of(x, ah[e]);
            }
#pragma unroll
            for (int q2 = 0; q2 < kTilesPerWave; ++q2) {
                const int ct = wave * kTilesPerWave + q2;
                const bf16x8 bv = lds8(sVt + (16 * ct + c) * kTP + j0);
                acc[q2] = mma(ah, bv, acc[q2]);
                acc[q2] = mma(al, bv, acc[q2]);
            }
        }
#pragma unroll
        for (int q2 = 0; q2 < kTilesPerWave; ++q2) {
            const int ct = wave * kTilesPerWave + q2;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * a + 4 * gq + r;
                ws_U[(ws_row + t) * DV + 16 * ct + c] = acc[q2][r];
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// chunk_state_kernel: one workgroup per (sequence, v-head, 16-column slice of S), chunks in order.
//
// Eight waves in two roles, both walking the sequence's chunks:
//   chain waves 0..3   carry the recurrence.  Chain wave w owns key rows [32w, 32w+32) of the
//                      slice of S as two 16 x 16 accumulator tiles.  For chunk i:
//                        - S (hi+lo) -> LDS, for the output waves
//                        - partial U_w = (-W)[:, rows_w] S[rows_w, :] -> LDS
//                        - (barrier) token tile w: U = Ut + sum_w U_w; U (hi+lo) and
//                          e^(G_C - G) U (hi+lo) -> LDS, token-contiguous
//                        - (barrier) S <- e^(G_C) S + K^T (e^(G_C - G) U)
//   output waves 4..7  one chunk behind: for chunk i-1, output wave w' forms token tile w' of
//                      O = e^G Q S + P U from the S and U the chain waves left in LDS.
// Every wave loads its own matrix-core operand fragments straight from memory into registers, one
// chunk ahead; LDS only carries what the waves exchange.  Two barriers per chunk.
constexpr int kStateThreads = 512;
constexpr int kWS = 16;          // state columns per workgroup
constexpr int kRP = kC + 4;      // pitch of the column-major fp32 partial tiles [16][64]
constexpr int kSP = kDK + 8;     // pitch of the key-contiguous state copies [16][128]

struct StateLds {
    float red[4][kWS * kRP];                     // chain waves' partial U, [column][token]
    __bf16 Dh[kWS * kTP], Dl[kWS * kTP];         // e^(G_C - G) U, [column][token]
    __bf16 Uh[2][kWS * kTP], Ul[2][kWS * kTP];   // U of the last two chunks, [column][token]
    __bf16 Sh[2][kWS * kSP], Sl[2][kWS * kSP];   // chunk-start S of the last two chunks, [column][key]
};

struct ChainFrag {
    bf16x4 wn[4][2];  // -W rows 16a + c, key columns 32w + 4g .. +3 and 32w + 16 + 4g .. +3
    bf16x8 kt[2][2];  // K^T rows 32w + 16it + c, tokens 32kb + 8g .. +7
    float ut[4];      // Ut rows 16w + 4g + r, column c0 + c
    float g2[4];      // G2 rows 16w + 4g + r
    float g2c;        // G2 of the chunk's last row
};

struct OutFrag {
    bf16x8 q[4];         // Q rows 16w' + c, key columns 32kb + 8g .. +7 (zero past the sequence)
    bf16x8 ph[2], pl[2]; // P rows 16w' + c, tokens 32kb + 8g .. +7
    float g2[4];         // G2 rows 16w' + 4g + r
};

template <int DV>
__device__ __forceinline__ void fetch_chain(ChainFrag& f, const __bf16* ws_Wn, const float* ws_U,
                                           const float* ws_G, const __bf16* ws_Kt, size_t ws_row,
                                           size_t kt_base, int w, int c0, int c, int gq) {
    const __bf16* wn = ws_Wn + ws_row * kDK;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int off = (16 * a + c) * kDK + 32 * w + 4 * gq;
        f.wn[a][0] = *reinterpret_cast<const bf16x4*>(wn + off);
        f.wn[a][1] = *reinterpret_cast<const bf16x4*>(wn + off + 16);
    }
    const __bf16* kt = ws_Kt + kt_base;
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            f.kt[it][kb] = *reinterpret_cast<const bf16x8*>(kt + (32 * w + 16 * it + c) * kC + 32 * kb + 8 * gq);
    const float* ut = ws_U + ws_row * DV + c0 + c;
    const float* g2 = ws_G + ws_row;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        f.ut[r] = ut[(16 * w + 4 * gq + r) * DV];
        f.g2[r] = g2[16 * w + 4 * gq + r];
    }
    f.g2c = g2[kC - 1];
}

__device__ __forceinline__ void fetch_out_q(OutFrag& f, const __bf16* q, const float* ws_G,
                                            size_t tok0, int L, int Hk, int kh, size_t ws_row,
                                            int w, int c, int gq) {
    // rows past the sequence's end read its last row and are then zeroed (no branch)
    const int t = 16 * w + c;
    const bool live = t < L;
    const __bf16* qr = q + ((tok0 + (live ? t : L - 1)) * Hk + kh) * kDK + 8 * gq;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const uint4 x = *reinterpret_cast<const uint4*>(qr + 32 * kb);
        const uint4 y = live ? x : make_uint4(0, 0, 0, 0);
        f.q[kb] = *reinterpret_cast<const bf16x8*>(&y);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) f.g2[r] = ws_G[ws_row + 16 * w + 4 * gq + r];
}

__device__ __forceinline__ void fetch_out_p(OutFrag& f, const __bf16* ws_P, size_t p_base, int w,
                                            int c, int gq) {
    const __bf16* ph = ws_P + p_base + (16 * w + c) * kC + 8 * gq;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        f.ph[kb] = *reinterpret_cast<const bf16x8*>(ph + 32 * kb);
        f.pl[kb] = *reinterpret_cast<const bf16x8*>(ph + kC * kC + 32 * kb);
    }
}

template <int DV>
__global__ __launch_bounds__(kStateThreads) void chunk_state_kernel(
    const __bf16* __restrict__ q, const float* initial_state,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ chunk_start,
    const int32_t* __restrict__ order, int N, int T, int Hk, int Hv, int nct, int max_slots,
    const __bf16* __restrict__ ws_Wn, const float* __restrict__ ws_U,
    const float* __restrict__ ws_G, const __bf16* __restrict__ ws_Kt,
    const __bf16* __restrict__ ws_P, float* __restrict__ o, float* final_state) {
    constexpr int S_SL = DV / kWS;  // slices per head
    __shared__ __attribute__((aligned(16))) StateLds sm;

    // blockIdx -> (unit, slice); all slices of a unit share blockIdx % 8 (the same XCD / L2)
    const int bid = blockIdx.x;
    const int sl = (bid / 8) % S_SL;
    const int u = ((bid / 8) / S_SL) * 8 + bid % 8;
    if (u >= N * Hv) return;
    const int rank = u / Hv, h = u % Hv;
    const int n = order ? order[rank] : rank;
    const int kh = h / (Hv / Hk);
    int row, t0, t1;
    sequence_range(cu_seqlens, n, T, row, t0, t1);
    const int slot0 = cu_seqlens ? chunk_start[n] : n * nct;
    // (a malformed cu_seqlens can claim more chunks than the workspace holds: stop at its end)
    const int nchunks = min((t1 - t0 + kC - 1) / kC, max(0, max_slots - slot0));
    const int c0 = sl * kWS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, gq = lane >> 4;
    const bool chain = wave < 4;
    const int w = chain ? wave : wave - 4;  // chain: key-row block; output: token tile

    auto tok0_of = [&](int ci) { return (size_t)row * T + t0 + (size_t)ci * kC; };
    auto len_of = [&](int ci) { return min(kC, t1 - t0 - ci * kC); };
    auto ws_row_of = [&](int ci) { return ((size_t)(slot0 + ci) * Hv + h) * kC; };
    auto kt_base_of = [&](int ci) { return ((size_t)(slot0 + ci) * Hk + kh) * kDK * kC; };
    auto p_base_of = [&](int ci) { return ((size_t)(slot0 + ci) * Hv + h) * 2 * kC * kC; };

    // chain waves: S slice rows 32w + 16it + 4g + r, column c0 + c
    f32x4 S[2] = {zero4(), zero4()};
    const size_t sbase = ((size_t)n * Hv + h) * kDK * DV;
    if (chain && initial_state) {
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[it][r] = initial_state[sbase + (size_t)(32 * w + 16 * it + 4 * gq + r) * DV + c0 + c];
    }

    // The two roles run separate loops (wave-uniform branch) so that neither role's in-flight
    // prefetches are drained at control-flow joins with the other's code.  Both loops execute the
    // same barriers: two per chunk, plus one pair for the output waves' one-chunk lag.
    if (chain) {
        // Chunk i with operands `cur`, prefetching chunk i+1 into `nxt` (the two sets alternate, so
        // no register copy has to wait for the prefetch to land).
        auto chain_step = [&](int i, const ChainFrag& cur, ChainFrag& nxt) {
            const int nx = min(i + 1, nchunks - 1);  // (the last prefetch repeats the last chunk)
            fetch_chain<DV>(nxt, ws_Wn, ws_U, ws_G, ws_Kt, ws_row_of(nx), kt_base_of(nx), w, c0, c, gq);
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch here, a whole chunk ahead of its use
            // S (hi + lo): B operand here, and the output waves' copy
            bf16x8 sh, sl8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = S[e >> 2][e & 3];
                sh[e] = hi_of(x);
                sl8[e] = lo_of(x, sh[e]);
            }
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int off = c * kSP + 32 * w + 16 * it + 4 * gq;
                *reinterpret_cast<bf16x4*>(sm.Sh[i & 1] + off) =
                    bf16x4{sh[4 * it], sh[4 * it + 1], sh[4 * it + 2], sh[4 * it + 3]};
                *reinterpret_cast<bf16x4*>(sm.Sl[i & 1] + off) =
                    bf16x4{sl8[4 * it], sl8[4 * it + 1], sl8[4 * it + 2], sl8[4 * it + 3]};
            }
            // partial U over this wave's 32 key rows, all 64 tokens
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const bf16x8 aw = cat44(cur.wn[a][0], cur.wn[a][1]);
                const f32x4 uh = mma(aw, sh, zero4());
                const f32x4 ul = mma(aw, sl8, zero4());
                *reinterpret_cast<f32x4*>(&sm.red[w][c * kRP + 16 * a + 4 * gq]) = uh + ul;
            }
            lds_barrier();

            // token tile w: U = Ut + sum of the four partials
            f32x4 uu = {cur.ut[0], cur.ut[1], cur.ut[2], cur.ut[3]};
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2)
                uu += *reinterpret_cast<const f32x4*>(&sm.red[w2][c * kRP + 16 * w + 4 * gq]);
            bf16x4 uh4, ul4, dh4, dl4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uh4[r] = hi_of(uu[r]);
                ul4[r] = lo_of(uu[r], uh4[r]);
                const float dd = exp2_fast(cur.g2c - cur.g2[r]) * uu[r];
                dh4[r] = hi_of(dd);
                dl4[r] = lo_of(dd, dh4[r]);
            }
            const int off = c * kTP + 16 * w + 4 * gq;
            *reinterpret_cast<bf16x4*>(sm.Uh[i & 1] + off) = uh4;
            *reinterpret_cast<bf16x4*>(sm.Ul[i & 1] + off) = ul4;
            *reinterpret_cast<bf16x4*>(sm.Dh + off) = dh4;
            *reinterpret_cast<bf16x4*>(sm.Dl + off) = dl4;
            lds_barrier();

            // S <- e^(G_C) S + K^T (e^(G_C - G) U)
            const float eC = exp2_fast(cur.g2c);
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                f32x4 a0 = S[it] * eC, a1 = zero4();
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int o2 = c * kTP + 32 * kb + 8 * gq;
                    a0 = mma(cur.kt[it][kb], lds8(sm.Dh + o2), a0);
                    a1 = mma(cur.kt[it][kb], lds8(sm.Dl + o2), a1);
                }
                S[it] = a0 + a1;
            }
        };
        // Both steps of the unrolled loop are unconditional (an odd count peels the first chunk),
        // so the compiler has no conditional block to sink a prefetch into.
        ChainFrag fa, fb;
        int i0 = 0;
        if (nchunks & 1) {
            fetch_chain<DV>(fb, ws_Wn, ws_U, ws_G, ws_Kt, ws_row_of(0), kt_base_of(0), w, c0, c, gq);
            chain_step(0, fb, fa);
            i0 = 1;
        } else if (nchunks > 0) {
            fetch_chain<DV>(fa, ws_Wn, ws_U, ws_G, ws_Kt, ws_row_of(0), kt_base_of(0), w, c0, c, gq);
        }
        for (int i = i0; i < nchunks; i += 2) {
            chain_step(i, fa, fb);
            chain_step(i + 1, fb, fa);
        }
        if (nchunks > 0) {  // the output waves' last chunk
            lds_barrier();
            lds_barrier();
        }
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                final_state[sbase + (size_t)(32 * w + 16 * it + 4 * gq + r) * DV + c0 + c] = S[it][r];
    } else {
        // Chunk i-1 with operands `cur`, prefetching chunk i into `nxt`.
        auto out_step = [&](int i, const OutFrag& cur, OutFrag& nxt) {
            const int pb = (i - 1) & 1;
            const int nx = min(i, nchunks - 1);
            fetch_out_q(nxt, q, ws_G, tok0_of(nx), len_of(nx), Hk, kh, ws_row_of(nx), w, c, gq);
            fetch_out_p(nxt, ws_P, p_base_of(nx), w, c, gq);
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch here, a whole chunk ahead of its use
            // O = e^G Q S for token tile w of chunk i-1
            f32x4 qs = zero4(), qs2 = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int off = c * kSP + 32 * kb + 8 * gq;
                qs = mma(cur.q[kb], lds8(sm.Sh[pb] + off), qs);
                qs2 = mma(cur.q[kb], lds8(sm.Sl[pb] + off), qs2);
            }
            f32x4 Ox;
#pragma unroll
            for (int r = 0; r < 4; ++r) Ox[r] = exp2_fast(cur.g2[r]) * (qs[r] + qs2[r]);
            lds_barrier();

            // O += P U for token tile w of chunk i-1, then store
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (2 * kb > w) continue;
                const int off = c * kTP + 32 * kb + 8 * gq;
                const bf16x8 uh = lds8(sm.Uh[pb] + off), ul = lds8(sm.Ul[pb] + off);
                Ox = mma(cur.ph[kb], uh, Ox);
                Ox = mma(cur.ph[kb], ul, Ox);
                Ox = mma(cur.pl[kb], uh, Ox);
            }
            const size_t tok0 = tok0_of(i - 1);
            const int L = len_of(i - 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * gq + r;
                if (t < L) o[((tok0 + t) * Hv + h) * DV + c0 + c] = Ox[r];
            }
            lds_barrier();
        };
        OutFrag fa, fb;
        int i0 = 1;
        if (nchunks > 0) {
            OutFrag& first = (nchunks & 1) ? fb : fa;
            fetch_out_q(first, q, ws_G, tok0_of(0), len_of(0), Hk, kh, ws_row_of(0), w, c, gq);
            fetch_out_p(first, ws_P, p_base_of(0), w, c, gq);
            lds_barrier();  // the chain waves' first chunk
            lds_barrier();
            if (nchunks & 1) {
                out_step(1, fb, fa);
                i0 = 2;
            }
        }
        for (int i = i0; i <= nchunks; i += 2) {
            out_step(i, fa, fb);
            out_step(i + 1, fb, fa);
        }
    }
}

// ------------------------------------------------------------------------------------------------
// workspace layout (each region 256-byte aligned):
//   chunk_start [N+1] int32 | order [N] int32 | G2 [slots][Hv][64] f32
//   | -W [slots][Hv][64][128] bf16 | Ut [slots][Hv][64][dv] f32 | K^T [slots][Hk][128][64] bf16
//   | P [slots][Hv][hi, lo][64][64] bf16
struct Layout {
    size_t chunk_start, order, G, Wn, U, Kt, P, total;
    int slots;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(int B, int T, int Hk, int Hv, int dv, int N) {
    Layout l;
    l.slots = (int)(((long long)B * T) / kC) + N;  // bounds B*ceil(T/64) and T/64 + N (packed)
    size_t off = 0;
    l.chunk_start = off; off = align256(off + sizeof(int32_t) * (size_t)(N + 1));
    l.order = off;       off = align256(off + sizeof(int32_t) * (size_t)N);
    l.G = off;           off = align256(off + sizeof(float) * (size_t)l.slots * Hv * kC);
    l.Wn = off;          off = align256(off + 2 * (size_t)l.slots * Hv * kC * kDK);
    l.U = off;           off = align256(off + sizeof(float) * (size_t)l.slots * Hv * kC * dv);
    l.Kt = off;          off = align256(off + 2 * (size_t)l.slots * Hk * kDK * kC);
    l.P = off;           off = align256(off + 2 * (size_t)l.slots * Hv * 2 * kC * kC);
    l.total = off;
    return l;
}

template <int DV>
hipError_t launch_state(const ChunkArgs& a, const Layout& lay, char* ws, int nct) {
    const int units = a.N * a.Hv;
    const int groups = (units + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * (DV / kWS))), block(kStateThreads);
    const bool packed = a.cu_seqlens != nullptr;
    hipLaunchKernelGGL((chunk_state_kernel<DV>), grid, block, 0, a.stream,
                       static_cast<const __bf16*>(a.q), a.initial_state, a.cu_seqlens,
                       packed ? reinterpret_cast<const int32_t*>(ws + lay.chunk_start) : nullptr,
                       packed ? reinterpret_cast<const int32_t*>(ws + lay.order) : nullptr,
                       a.N, a.T, a.Hk, a.Hv, nct, packed ? lay.slots : a.B * nct,
                       reinterpret_cast<const __bf16*>(ws + lay.Wn),
                       reinterpret_cast<const float*>(ws + lay.U),
                       reinterpret_cast<const float*>(ws + lay.G),
                       reinterpret_cast<const __bf16*>(ws + lay.Kt),
                       reinterpret_cast<const __bf16*>(ws + lay.P), a.o, a.final_state);
    return hipGetLastError();
}

template <int DV, typename TG>
hipError_t launch_dv(const ChunkArgs& a) {
    const Layout lay = layout(a.B, a.T, a.Hk, a.Hv, DV, a.N);
    char* ws = static_cast<char*>(a.workspace);
    const bool packed = a.cu_seqlens != nullptr;
    const int nct = (a.T + kC - 1) / kC;
    const int slots = packed ? lay.slots : a.B * nct;
    if (packed) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, a.stream, a.cu_seqlens, a.N,
                           a.T, reinterpret_cast<int32_t*>(ws + lay.chunk_start),
                           reinterpret_cast<int32_t*>(ws + lay.order));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (slots > 0) {
        hipLaunchKernelGGL((chunk_prep_kernel<DV, TG>), dim3((unsigned)slots, (unsigned)a.Hv),
                           dim3(kThreads), 0, a.stream, static_cast<const __bf16*>(a.q),
                           static_cast<const __bf16*>(a.k),
                           static_cast<const __bf16*>(a.v), static_cast<const TG*>(a.g),
                           static_cast<const TG*>(a.beta), a.cu_seqlens,
                           packed ? reinterpret_cast<const int32_t*>(ws + lay.chunk_start) : nullptr,
                           a.N, a.T, a.Hk, a.Hv, nct,
                           reinterpret_cast<__bf16*>(ws + lay.Wn), reinterpret_cast<float*>(ws + lay.U),
                           reinterpret_cast<float*>(ws + lay.G), reinterpret_cast<__bf16*>(ws + lay.Kt),
                           reinterpret_cast<__bf16*>(ws + lay.P));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_state<DV>(a, lay, ws, nct);
}

}  // namespace

bool chunk_mfma_supported(int dk, int dv, gdn_dtype qkv_dtype) {
    return qkv_dtype == GDN_BF16 && dk == kDK && (dv == 64 || dv == 128);
}

size_t chunk_mfma_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N) {
    (void)dk;
    return layout(B, T, Hk, Hv, dv, N).total;
}

hipError_t launch_chunk_mfma(const ChunkArgs& a) {
    const bool g_bf16 = a.gate_dtype == GDN_BF16;
    if (a.dv == 128) return g_bf16 ? launch_dv<128, bf16_t>(a) : launch_dv<128, float>(a);
    return g_bf16 ? launch_dv<64, bf16_t>(a) : launch_dv<64, float>(a);
}

}  // namespace gdn
