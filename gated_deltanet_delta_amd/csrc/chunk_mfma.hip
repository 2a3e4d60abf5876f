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
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const int add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int run = part[tid] - sum;  // exclusive prefix of this thread's block
    for (int n = n0; n < n1; ++n) {
        chunk_start[n] = run;
        run += (len_of(n) + kC - 1) / kC;
    }
    if (tid == kThreads - 1) chunk_start[N] = part[kThreads - 1];

    if (N <= kOrderMax) {
        for (int n = tid; n < N; n += kThreads) lens[n] = len_of(n);
        __syncthreads();
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
// chunk_prep_kernel: one workgroup per (chunk slot, v-head).
//
// LDS (bytes): sKA  [64][136] bf16 (K rows)  -- later reused as A [64][68] fp32
//              sKV  [128][72] bf16 (K^T)     -- later reused as V^T [DV][72] bf16
//              sT   [64][68] fp32
constexpr int kKP = kDK + 8;   // row pitch (elements) of K rows in LDS
constexpr int kTP = kC + 8;    // row pitch of transposed (token-contiguous) bf16 tiles
constexpr int kFP = kC + 4;    // row pitch of 64 x 64 fp32 tiles

template <int DV, typename TG>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(
    const __bf16* __restrict__ k, const __bf16* __restrict__ v, const TG* __restrict__ g,
    const TG* __restrict__ beta, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ chunk_start, int N, int T, int Hk, int Hv, int nct, int slots,
    __bf16* __restrict__ ws_Wn, float* __restrict__ ws_U, float* __restrict__ ws_G) {
    static_assert(DV == 64 || DV == 128, "dv");
    constexpr size_t kBytesKA = (size_t)kC * kKP * 2 > (size_t)kC * kFP * 4 ? (size_t)kC * kKP * 2
                                                                           : (size_t)kC * kFP * 4;
    constexpr size_t kBytesKV = (size_t)kDK * kTP * 2;
    __shared__ __attribute__((aligned(16))) unsigned char smem_ka[kBytesKA];
    __shared__ __attribute__((aligned(16))) unsigned char smem_kv[kBytesKV];
    __shared__ __attribute__((aligned(16))) float sT[kC * kFP];
    __shared__ float sG[kC], sB[kC], sBE[kC];

    __bf16* sK = reinterpret_cast<__bf16*>(smem_ka);   // [64][kKP]
    float* sA = reinterpret_cast<float*>(smem_ka);     // [64][kFP], after K rows are dead
    __bf16* sKt = reinterpret_cast<__bf16*>(smem_kv);  // [128][kTP]
    __bf16* sVt = reinterpret_cast<__bf16*>(smem_kv);  // [DV][kTP], after K^T is dead

    const int slot = blockIdx.x, h = blockIdx.y;
    ChunkLoc loc;
    if (!locate_chunk(slot, cu_seqlens, chunk_start, N, T, nct, loc)) return;
    const int kh = h / (Hv / Hk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, gq = lane >> 4;
    const size_t tok0 = (size_t)loc.row * T + loc.t0;
    const int L = loc.len;

    // ---- stage K (rows and transposed), prefetch V ----------------------------------------------
    {
        const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int e = tid + kThreads * it;  // 1024 16-byte pieces: row t, columns 8p..8p+7
            const int t = e >> 4, p = e & 15;
            uint4 x = zero;
            if (t < L) x = *reinterpret_cast<const uint4*>(k + ((tok0 + t) * Hk + kh) * kDK + 8 * p);
            *reinterpret_cast<uint4*>(sK + t * kKP + 8 * p) = x;
            const __bf16* xs = reinterpret_cast<const __bf16*>(&x);
#pragma unroll
            for (int j = 0; j < 8; ++j) sKt[(8 * p + j) * kTP + t] = xs[j];
        }
    }
    constexpr int kVPieces = kC * DV / 8 / kThreads;  // 16-byte pieces of V per thread
    uint4 vreg[kVPieces];
#pragma unroll
    for (int it = 0; it < kVPieces; ++it) {
        const int e = tid + kThreads * it;
        const int t = e / (DV / 8), p = e % (DV / 8);
        vreg[it] = make_uint4(0, 0, 0, 0);
        if (t < L) vreg[it] = *reinterpret_cast<const uint4*>(v + ((tok0 + t) * Hv + h) * DV + 8 * p);
    }
    if (wave == 0) {
        const float gt = lane < L ? to_f32(g[(tok0 + lane) * Hv + h]) : 0.f;
        const float bt = lane < L ? to_f32(beta[(tok0 + lane) * Hv + h]) : 0.f;
        float G = gt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(G, off);
            if (lane >= off) G += y;
        }
        sG[lane] = G;
        sB[lane] = bt;
        sBE[lane] = bt * expf(G);
        ws_G[((size_t)slot * Hv + h) * kC + lane] = G;
    }
    for (int e = tid; e < kC * kFP; e += kThreads) sT[e] = 0.f;
    __syncthreads();

    // ---- A = diag(beta) (K K^T o Gam), strictly lower: 10 lower 16x16 tiles over 4 waves ----------
    // wave 0: (0,0) (3,3) (3,0); wave 1: (1,1) (3,1) (1,0); wave 2: (2,2) (3,2); wave 3: (2,0) (2,1)
    auto tile_a = [](int w, int s) {
        return s == 0 ? (w == 3 ? 2 : w) : s == 1 ? (w == 3 ? 2 : 3) : (w < 2 ? (w == 0 ? 3 : 1) : -1);
    };
    auto tile_b = [](int w, int s) {
        return s == 0 ? (w == 3 ? 0 : w) : s == 1 ? (w == 3 ? 1 : w == 0 ? 3 : w) : 0;
    };
    f32x4 accA[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        accA[s] = zero4();
        const int ta = tile_a(wave, s), tb = tile_b(wave, s);
        if (ta < 0) continue;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 a = lds8(sK + (16 * ta + c) * kKP + 32 * kb + 8 * gq);
            const bf16x8 b = lds8(sK + (16 * tb + c) * kKP + 32 * kb + 8 * gq);
            accA[s] = mma(a, b, accA[s]);
        }
    }
    __syncthreads();  // K rows dead: sA overwrites them
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int ta = tile_a(wave, s), tb = tile_b(wave, s);
        if (ta < 0) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * ta + 4 * gq + r, j = 16 * tb + c;
            const float val = j < t ? sB[t] * accA[s][r] * expf(sG[t] - sG[j]) : 0.f;
            sA[t * kFP + j] = val;
        }
    }
    __syncthreads();

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
    __syncthreads();
    // off-diagonal blocks, by distance d = a - b:  T_ab = -T_aa * sum_{m=b}^{a-1} A_am T_mb
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        if (wave < 4 - d) {
            const int b = wave, a = wave + d;
            f32x4 X = zero4();
            for (int m = b; m < a; ++m) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float av = sA[(16 * a + c) * kFP + 16 * m + 4 * s + gq];
                    const float bv = sT[(16 * m + 4 * s + gq) * kFP + 16 * b + c];
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
        __syncthreads();
    }

    // ---- -W = -T diag(beta e^G) K  (bf16) ---------------------------------------------------------
    // wave w computes key-dim tiles 2w, 2w+1 for all four token tiles
    const size_t ws_row = ((size_t)slot * Hv + h) * kC;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        f32x4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
        for (int kb = 0; kb <= a / 2; ++kb) {
            const int t = 16 * a + c, j0 = 32 * kb + 8 * gq;
            bf16x8 af;
#pragma unroll
            for (int e = 0; e < 8; ++e) af[e] = hi_of(sT[t * kFP + j0 + e] * sBE[j0 + e]);
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
    __syncthreads();  // K^T dead: V^T overwrites it

    // ---- Ut = T diag(beta) V  (fp32) --------------------------------------------------------------
#pragma unroll
    for (int it = 0; it < kVPieces; ++it) {
        const int e = tid + kThreads * it;
        const int t = e / (DV / 8), p = e % (DV / 8);
        const __bf16* xs = reinterpret_cast<const __bf16*>(&vreg[it]);
#pragma unroll
        for (int j = 0; j < 8; ++j) sVt[(8 * p + j) * kTP + t] = xs[j];
    }
    __syncthreads();
    constexpr int kTilesPerWave = DV / 16 / 4;  // value-dim tiles per wave
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        f32x4 acc[kTilesPerWave];
#pragma unroll
        for (int q2 = 0; q2 < kTilesPerWave; ++q2) acc[q2] = zero4();
#pragma unroll
        for (int kb = 0; kb <= a / 2; ++kb) {
            const int t = 16 * a + c, j0 = 32 * kb + 8 * gq;
            bf16x8 ah, al;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = sT[t * kFP + j0 + e] * sB[j0 + e];
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
// chunk_state_kernel: one workgroup per (sequence, v-head, WS-column slice), chunks in order.
//
// Wave w owns key rows [32w, 32w+32) of the slice of S as two 16-row accumulator tiles per 16
// columns.  Per chunk:
//   1  partial U_w = (-W)[:, rows_w] S[rows_w, :] and QS_w = Q[:, rows_w] S[rows_w, :] (S as hi+lo)
//   2  partials -> LDS; wave w sums token tile w:  U = Ut + sum_w U_w,  O = e^G sum_w QS_w
//   3  U (hi+lo) and e^(G_C - G) U (hi+lo) -> LDS, transposed (token-contiguous)
//   4  S <- e^(G_C) S + K^T (e^(G_C-G) U);  P^T tiles = K Q^T (masked, decayed); O += P U;  store O
template <int WS>
struct StateLds {
    static constexpr int kNT = WS / 16;
    __bf16 Wn[kC * kKP];
    __bf16 Q[kC * kKP];
    __bf16 K[kC * kKP];
    __bf16 Kt[kDK * kTP];
    float Ut[kC * WS];
    float G[kC], EG[kC], ED[kC];
    float redU[4][kC * WS];
    float redQ[4][kC * WS];
    __bf16 Uh[WS * kTP], Ul[WS * kTP], Dh[WS * kTP], Dl[WS * kTP];
};

template <int DV, int WS>
__global__ __launch_bounds__(kThreads) void chunk_state_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const float* initial_state,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ chunk_start,
    const int32_t* __restrict__ order, int N, int T, int Hk, int Hv, int nct, int max_slots,
    const __bf16* __restrict__ ws_Wn, const float* __restrict__ ws_U,
    const float* __restrict__ ws_G, float* __restrict__ o, float* final_state) {
    constexpr int NT = WS / 16;        // 16-column tiles per slice
    constexpr int S_SL = DV / WS;      // slices per head
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    StateLds<WS>& sm = *reinterpret_cast<StateLds<WS>*>(smem_raw);

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
    const int c0 = sl * WS;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, gq = lane >> 4;

    // S slice: rows 32*wave + 16*it + 4*gq + r, column c0 + 16*ct + c
    f32x4 S[2][NT];
    const size_t sbase = ((size_t)n * Hv + h) * kDK * DV;
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 32 * wave + 16 * it + 4 * gq + r;
                S[it][ct][r] = initial_state ? initial_state[sbase + (size_t)i * DV + c0 + 16 * ct + c] : 0.f;
            }

    for (int ci = 0; ci < nchunks; ++ci) {
        const int slot = slot0 + ci;
        const size_t tok0 = (size_t)row * T + t0 + (size_t)ci * kC;
        const int L = min(kC, t1 - t0 - ci * kC);
        const size_t ws_row = ((size_t)slot * Hv + h) * kC;

        // ---- stage this chunk -------------------------------------------------------------------
        __syncthreads();  // previous chunk done with every staged buffer
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int e = tid + kThreads * it;
            const int t = e >> 4, p = e & 15;
            const uint4 zero = make_uint4(0, 0, 0, 0);
            uint4 xq = zero, xk = zero;
            if (t < L) {
                const size_t off = ((tok0 + t) * Hk + kh) * kDK + 8 * p;
                xq = *reinterpret_cast<const uint4*>(q + off);
                xk = *reinterpret_cast<const uint4*>(k + off);
            }
            const uint4 xw = *reinterpret_cast<const uint4*>(ws_Wn + (ws_row + t) * kDK + 8 * p);
            *reinterpret_cast<uint4*>(sm.Q + t * kKP + 8 * p) = xq;
            *reinterpret_cast<uint4*>(sm.K + t * kKP + 8 * p) = xk;
            *reinterpret_cast<uint4*>(sm.Wn + t * kKP + 8 * p) = xw;
            const __bf16* xs = reinterpret_cast<const __bf16*>(&xk);
#pragma unroll
            for (int j = 0; j < 8; ++j) sm.Kt[(8 * p + j) * kTP + t] = xs[j];
        }
        for (int e = tid; e < kC * WS / 4; e += kThreads) {
            const int t = e / (WS / 4), p = e % (WS / 4);
            *reinterpret_cast<float4*>(sm.Ut + t * WS + 4 * p) =
                *reinterpret_cast<const float4*>(ws_U + (ws_row + t) * DV + c0 + 4 * p);
        }
        if (tid < kC) sm.G[tid] = ws_G[ws_row + tid];
        __syncthreads();
        const float GC = sm.G[kC - 1];
        if (tid < kC) {
            sm.EG[tid] = expf(sm.G[tid]);
            sm.ED[tid] = expf(GC - sm.G[tid]);
        }
        const float eC = expf(GC);

        // ---- 1: partial U and QS over this wave's 32 key rows ----------------------------------
        bf16x8 Sh[NT], Sl[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = S[e >> 2][ct][e & 3];
                Sh[ct][e] = hi_of(x);
                Sl[ct][e] = lo_of(x, Sh[ct][e]);
            }
        const int kr = 32 * wave + 4 * gq;  // key rows of slots 0..3; slots 4..7 are kr + 16
        f32x4 Up[4][NT], Qp[4][NT];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int t = 16 * a + c;
            const bf16x8 aw = cat44(lds4(sm.Wn + t * kKP + kr), lds4(sm.Wn + t * kKP + kr + 16));
            const bf16x8 aq = cat44(lds4(sm.Q + t * kKP + kr), lds4(sm.Q + t * kKP + kr + 16));
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                Up[a][ct] = mma(aw, Sh[ct], zero4());
                Up[a][ct] = mma(aw, Sl[ct], Up[a][ct]);
                Qp[a][ct] = mma(aq, Sh[ct], zero4());
                Qp[a][ct] = mma(aq, Sl[ct], Qp[a][ct]);
            }
        }
        // ---- 2: cross-wave sums for token tile `wave` -----------------------------------------
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * a + 4 * gq + r, j = 16 * ct + c;
                    sm.redU[wave][t * WS + j] = Up[a][ct][r];
                    sm.redQ[wave][t * WS + j] = Qp[a][ct][r];
                }
        __syncthreads();
        f32x4 Ox[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * wave + 4 * gq + r, j = 16 * ct + c;
                float uu = sm.Ut[t * WS + j], qs = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    uu += sm.redU[w2][t * WS + j];
                    qs += sm.redQ[w2][t * WS + j];
                }
                Ox[ct][r] = sm.EG[t] * qs;
                const __bf16 uh = hi_of(uu), ul = lo_of(uu, uh);
                const float dd = sm.ED[t] * uu;
                const __bf16 dh = hi_of(dd), dl = lo_of(dd, dh);
                sm.Uh[j * kTP + t] = uh;
                sm.Ul[j * kTP + t] = ul;
                sm.Dh[j * kTP + t] = dh;
                sm.Dl[j * kTP + t] = dl;
            }
        __syncthreads();

        // ---- 4a: S <- e^(G_C) S + K^T (e^(G_C - G) U) --------------------------------------------
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) S[it][ct] *= eC;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int j0 = 32 * kb + 8 * gq;
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const bf16x8 ak = lds8(sm.Kt + (32 * wave + 16 * it + c) * kTP + j0);
#pragma unroll
                for (int ct = 0; ct < NT; ++ct) {
                    const int jc = 16 * ct + c;
                    S[it][ct] = mma(ak, lds8(sm.Dh + jc * kTP + j0), S[it][ct]);
                    S[it][ct] = mma(ak, lds8(sm.Dl + jc * kTP + j0), S[it][ct]);
                }
            }
        }

        // ---- 4b: P^T tiles (a, wave) for a <= wave: rows t' = 16a + 4g + r, column t = 16 wave + c
        f32x4 PT[4];
        const int tq = 16 * wave + c;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            PT[a] = zero4();
            if (a > wave) continue;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const bf16x8 ak = lds8(sm.K + (16 * a + c) * kKP + 32 * kb + 8 * gq);
                const bf16x8 bq = lds8(sm.Q + tq * kKP + 32 * kb + 8 * gq);
                PT[a] = mma(ak, bq, PT[a]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tp = 16 * a + 4 * gq + r;
                PT[a][r] = tp <= tq ? PT[a][r] * expf(sm.G[tq] - sm.G[tp]) : 0.f;
            }
        }
        // ---- 4c: O += P U for token tile `wave` ---------------------------------------------------
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (2 * kb > wave) continue;
            bf16x8 ph, pl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = PT[2 * kb + (e >> 2)][e & 3];
                ph[e] = hi_of(x);
                pl[e] = lo_of(x, ph[e]);
            }
            const int j0 = 32 * kb + 4 * gq;  // token slots j0..j0+3 and j0+16..j0+19
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const int jc = 16 * ct + c;
                const bf16x8 uh = cat44(lds4(sm.Uh + jc * kTP + j0), lds4(sm.Uh + jc * kTP + j0 + 16));
                const bf16x8 ul = cat44(lds4(sm.Ul + jc * kTP + j0), lds4(sm.Ul + jc * kTP + j0 + 16));
                Ox[ct] = mma(ph, uh, Ox[ct]);
                Ox[ct] = mma(ph, ul, Ox[ct]);
                Ox[ct] = mma(pl, uh, Ox[ct]);
            }
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * wave + 4 * gq + r;
                if (t < L) o[((tok0 + t) * Hv + h) * DV + c0 + 16 * ct + c] = Ox[ct][r];
            }
    }

#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 32 * wave + 16 * it + 4 * gq + r;
                final_state[sbase + (size_t)i * DV + c0 + 16 * ct + c] = S[it][ct][r];
            }
}

// ------------------------------------------------------------------------------------------------
// workspace layout (each region 256-byte aligned):
//   chunk_start [N+1] int32 | order [N] int32 | G [slots][Hv][64] f32 | -W [slots][Hv][64][128] bf16
//   | Ut [slots][Hv][64][dv] f32
struct Layout {
    size_t chunk_start, order, G, Wn, U, total;
    int slots;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(int B, int T, int Hv, int dv, int N) {
    Layout l;
    l.slots = (int)(((long long)B * T) / kC) + N;  // bounds B*ceil(T/64) and T/64 + N (packed)
    size_t off = 0;
    l.chunk_start = off; off = align256(off + sizeof(int32_t) * (size_t)(N + 1));
    l.order = off;       off = align256(off + sizeof(int32_t) * (size_t)N);
    l.G = off;           off = align256(off + sizeof(float) * (size_t)l.slots * Hv * kC);
    l.Wn = off;          off = align256(off + 2 * (size_t)l.slots * Hv * kC * kDK);
    l.U = off;           off = align256(off + sizeof(float) * (size_t)l.slots * Hv * kC * dv);
    l.total = off;
    return l;
}

template <int DV, int WS>
hipError_t launch_state(const ChunkArgs& a, const Layout& lay, char* ws, int nct) {
    const auto kern = chunk_state_kernel<DV, WS>;
    const size_t bytes = sizeof(StateLds<WS>);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    const int units = a.N * a.Hv;
    const int groups = (units + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * (DV / WS))), block(kThreads);
    const bool packed = a.cu_seqlens != nullptr;
    hipLaunchKernelGGL(kern, grid, block, bytes, a.stream, static_cast<const __bf16*>(a.q),
                       static_cast<const __bf16*>(a.k), a.initial_state, a.cu_seqlens,
                       packed ? reinterpret_cast<const int32_t*>(ws + lay.chunk_start) : nullptr,
                       packed ? reinterpret_cast<const int32_t*>(ws + lay.order) : nullptr,
                       a.N, a.T, a.Hk, a.Hv, nct, packed ? lay.slots : a.B * nct,
                       reinterpret_cast<const __bf16*>(ws + lay.Wn),
                       reinterpret_cast<const float*>(ws + lay.U),
                       reinterpret_cast<const float*>(ws + lay.G), a.o, a.final_state);
    return hipGetLastError();
}

template <int DV, typename TG>
hipError_t launch_dv(const ChunkArgs& a) {
    const Layout lay = layout(a.B, a.T, a.Hv, DV, a.N);
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
                           dim3(kThreads), 0, a.stream, static_cast<const __bf16*>(a.k),
                           static_cast<const __bf16*>(a.v), static_cast<const TG*>(a.g),
                           static_cast<const TG*>(a.beta), a.cu_seqlens,
                           packed ? reinterpret_cast<const int32_t*>(ws + lay.chunk_start) : nullptr,
                           a.N, a.T, a.Hk, a.Hv, nct, slots,
                           reinterpret_cast<__bf16*>(ws + lay.Wn), reinterpret_cast<float*>(ws + lay.U),
                           reinterpret_cast<float*>(ws + lay.G));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // Narrow slices when there are few (sequence, head) units, wide ones otherwise.
    const long long units = (long long)a.N * a.Hv;
    if (units * (DV / 16) <= 2048) return launch_state<DV, 16>(a, lay, ws, nct);
    return launch_state<DV, 32>(a, lay, ws, nct);
}

}  // namespace

bool chunk_mfma_supported(int dk, int dv, gdn_dtype qkv_dtype) {
    return qkv_dtype == GDN_BF16 && dk == kDK && (dv == 64 || dv == 128);
}

size_t chunk_mfma_workspace_size(int B, int T, int Hv, int dk, int dv, int N) {
    (void)dk;
    return layout(B, T, Hv, dv, N).total;
}

hipError_t launch_chunk_mfma(const ChunkArgs& a) {
    const bool g_bf16 = a.gate_dtype == GDN_BF16;
    if (a.dv == 128) return g_bf16 ? launch_dv<128, bf16_t>(a) : launch_dv<128, float>(a);
    return g_bf16 ? launch_dv<64, bf16_t>(a) : launch_dv<64, float>(a);
}

}  // namespace gdn
