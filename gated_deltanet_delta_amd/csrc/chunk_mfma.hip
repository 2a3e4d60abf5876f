// chunk_mfma.hip -- chunked gated delta rule on gfx950 bf16 matrix cores (dk = 128).
//
// Notation (one chunk of C = 64 tokens of one sequence and v-head, start state S (dk x dv), G_t the
// running sum of g inside the chunk, Gam_tj = e^(G_t - G_j) for j <= t):
//
//   A  = diag(beta) (K K^T o Gam), strictly lower        T  = (I + A)^-1,   M = T diag(beta)
//   W  = M diag(e^G) K                                    Ut = M V
//   P  = (Q K^T) o Gam, lower with diagonal
//   U  = Ut - W S                                         (the chunk's per-token deltas)
//   O  = diag(e^G) Q S + P U
//   S <- e^(G_C) S + K^T diag(e^(G_C - G)) U
//
// which is the per-token rule S_t = e^(g_t)(I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
// o_t = S_t^T q_t unrolled over the chunk.  Every decay factor is exp of a non-positive number.
//
// Two kernels:
//   chunk_solve_kernel  one workgroup per (chunk, v-head), all chunks in parallel: the part with a
//                       serial dependence inside a chunk.  Cumsum, A on the matrix cores, T by a
//                       blocked forward substitution (16 x 16 diagonal blocks by substitution,
//                       off-diagonal blocks by fp32 matrix-core products), M = T diag(beta) as
//                       hi + lo bf16 into the workspace (16 KiB per chunk and v-head).
//   chunk_fused_kernel  one workgroup per (sequence, v-head, 16-column slice of S), walking the
//                       chunks in order with three wave roles (see there).  Everything else is
//                       formed on the fly from q, k, v, M and G; nothing else round-trips memory.
//
// Precision: q, k, v enter the matrix cores as exact bf16 values.  Quantities that feed the output
// with full weight (S, U, P, M) enter as two bf16 terms hi + lo (hi = bf16(x), lo = bf16(x - hi)),
// so their products carry ~16 significant bits; W enters as one bf16 term.  Accumulation is fp32
// everywhere; decay factors are applied on the fp32 side.
//
// Lane layouts used (wave64, checked on the device):
//   v_mfma_f32_16x16x32_bf16: lane l = 16 g + c holds A[c][8g..8g+7] and B[8g..8g+7][c]; the 16x16
//     result D[4g + r][c], r = 0..3, sits in lane l, element r.  The reduction index of one
//     instruction may be permuted freely as long as A and B agree; the kernels use that to feed
//     an accumulator tile straight back in as an operand.
//   ds_read_b64_tr_b16: within each 16-lane group, if lane j addresses four 16-bit values
//     X[j][0..3], lane i receives X[4m + i/4][i%4], m = 0..3.  Pointing lane c of group g at row
//     8g + c/4, columns c0 + 4(c%4) of a row-major tile therefore hands lane (g, c) the column
//     segment X[8g .. 8g+3][c0 + c]: a row-major tile serves directly as a transposed operand.

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
// Shared helpers.
constexpr int kKP = kDK + 8;   // row pitch (elements) of 128-wide bf16 rows in LDS
constexpr int kTP = kC + 8;    // row pitch of token-contiguous bf16 tiles [column][token]
constexpr int kFP = kC + 4;    // row pitch of 64 x 64 fp32 tiles
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// MFMA operand from a row-major bf16 tile X (pitch in elements) read transposed: lane (g, c)
// receives X[r0 + 8g + e][c0 + c], e = 0..7, i.e. rows are the reduction index.
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* X, int pitch, int r0, int c0, int g, int c) {
    const __bf16* p0 = X + (r0 + 8 * g + (c >> 2)) * pitch + c0 + 4 * (c & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 4 * pitch));
    return cat44(lo, hi);
}

// ------------------------------------------------------------------------------------------------
// chunk_solve_kernel: one workgroup per (chunk slot, v-head).
//
// Writes G2 = running sum of g log2(e) (64 floats) and M = T diag(beta) as hi and lo bf16 tiles
// [64][64] (row-major, zero above the diagonal and in rows/columns past the chunk's length).
template <typename TG>
__global__ __launch_bounds__(kThreads) void chunk_solve_kernel(
    const __bf16* __restrict__ k, const TG* __restrict__ g, const TG* __restrict__ beta,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ chunk_start, int N, int T,
    int Hk, int Hv, int nct, float* __restrict__ ws_G, __bf16* __restrict__ ws_M) {
    __shared__ __attribute__((aligned(16))) __bf16 sK[kC * kKP];
    __shared__ __attribute__((aligned(16))) float sA[kC * kFP];
    __shared__ __attribute__((aligned(16))) float sT[kC * kFP];
    __shared__ float sG[kC], sB[kC];

    const int slot = blockIdx.x, h = blockIdx.y;
    ChunkLoc loc;
    if (!locate_chunk(slot, cu_seqlens, chunk_start, N, T, nct, loc)) return;
    const int kh = h / (Hv / Hk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, gq = lane >> 4;
    const size_t tok0 = (size_t)loc.row * T + loc.t0;
    const int L = loc.len;

#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = tid + kThreads * it;  // 1024 pieces: row e/16, columns 8 (e%16) .. +7
        const int t = e >> 4, p = e & 15;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (t < L) x = *reinterpret_cast<const uint4*>(k + ((tok0 + t) * Hk + kh) * kDK + 8 * p);
        *reinterpret_cast<uint4*>(sK + t * kKP + 8 * p) = x;
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
        ws_G[ws_row + lane] = G2;
    }
    for (int e = tid; e < kC * kFP; e += kThreads) sT[e] = 0.f;
    lds_barrier();

    // A = diag(beta) (K K^T o Gam), strictly lower: 10 lower 16x16 tiles over 4 waves
    // wave 0: (0,0) (3,3) (3,0); wave 1: (1,1) (3,1) (1,0); wave 2: (2,2) (3,2); wave 3: (2,0) (2,1)
    auto tile_a = [](int w, int s) {
        return s == 0 ? (w == 3 ? 2 : w) : s == 1 ? (w == 3 ? 2 : 3) : (w < 2 ? (w == 0 ? 3 : 1) : -1);
    };
    auto tile_b = [](int w, int s) {
        return s == 0 ? (w == 3 ? 0 : w) : s == 1 ? (w == 3 ? 1 : w == 0 ? 3 : w) : 0;
    };
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int ta = tile_a(wave, s), tb = tile_b(wave, s);
        if (ta < 0) continue;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            acc = mma(lds8(sK + (16 * ta + c) * kKP + 32 * kb + 8 * gq),
                      lds8(sK + (16 * tb + c) * kKP + 32 * kb + 8 * gq), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * ta + 4 * gq + r, j = 16 * tb + c;
            sA[t * kFP + j] = j < t ? sB[t] * acc[r] * exp2_fast(sG[t] - sG[j]) : 0.f;
        }
    }
    lds_barrier();

    // T = (I + A)^-1: diagonal blocks, wave w inverts block w (lane c < 16 computes column c)
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

    // M = T diag(beta) as hi and lo rows: 64 rows x 8 pieces of 8 columns
    __bf16* Mh = ws_M + ((size_t)slot * Hv + h) * 2 * kC * kC;
    __bf16* Ml = Mh + kC * kC;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int e = tid + kThreads * it;
        const int t = e >> 3, p = e & 7;
        const float4 a0 = *reinterpret_cast<const float4*>(sT + t * kFP + 8 * p);
        const float4 a1 = *reinterpret_cast<const float4*>(sT + t * kFP + 8 * p + 4);
        const float tv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        bf16x8 hv, lv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = tv[j] * sB[8 * p + j];
            hv[j] = hi_of(x);
            lv[j] = lo_of(x, hv[j]);
        }
        *reinterpret_cast<bf16x8*>(Mh + t * kC + 8 * p) = hv;
        *reinterpret_cast<bf16x8*>(Ml + t * kC + 8 * p) = lv;
    }
}

// ------------------------------------------------------------------------------------------------
// chunk_fused_kernel: one workgroup per (sequence, v-head, 16-column slice of S).
//
// With M = T diag(beta) from chunk_solve_kernel, the chunk's deltas are
//     U = Ut - W S = M (V - diag(e^G) K S)
// so no W is formed: the chain needs K S (K exact bf16, S as hi + lo), one elementwise step and one
// 64 x 64 product with M.  Eight waves step through the chunks together, three barriers per chunk:
//
//   chain waves 0..3 (wave w owns key rows [32w, 32w+32) of S as two 16x16 accumulator tiles)
//     phase 1  S (hi + lo) -> LDS for the output waves; partial (K S)_w over its 32 key rows
//     phase 2  token tile w: X = V - e^G sum_w (K S)_w  -> LDS as hi + lo
//     phase 3  token tile w: U = M X; U (hi + lo) and e^(G_C - G) U (hi + lo) -> LDS
//     phase 4  S <- e^(G_C) S + K^T (e^(G_C - G) U), K^T read transposed from the K rows
//   output waves 4..7 (wave w' owns token tile w' of O)
//     phase 1  P^T tiles (a, w') = K Q^T for a < 2 (masked, decayed)
//     phase 2  O = e^G Q S from the chain's S copy
//     phase 3  P^T tiles for a >= 2
//     phase 4  O += P U from the chain's U copy; store
// Both roles stage the next chunk's K rows and log-decay into a three-chunk LDS ring at phase 1.
// All global operands (K, G for staging; M and V for the chain; q for the output waves) are
// fetched into registers one chunk ahead, alternating between two register sets.
constexpr int kFusedThreads = 512;
constexpr int kWS = 16;          // state columns per workgroup
constexpr int kRP = kC + 4;      // pitch of the column-major fp32 tiles [16][64]
constexpr int kSP = kDK + 8;     // pitch of the key-contiguous state copy [16][128]

struct FusedLds {
    __bf16 Kr[3][kC * kKP];        // K rows (ring of three chunks)
    float G2[3][kC];               // running log2-decay (ring of three chunks)
    float EG[3][kC];               // exp2(G2)
    __bf16 Sh[kWS * kSP], Sl[kWS * kSP];   // chunk-start S, [column][key]
    __bf16 Xh[kWS * kTP], Xl[kWS * kTP];   // V - e^G K S, [column][token]
    __bf16 Uh[kWS * kTP], Ul[kWS * kTP];   // U, [column][token]
    __bf16 Dh[kWS * kTP], Dl[kWS * kTP];   // e^(G_C - G) U, [column][token]
    float red[4][kWS * kRP];       // chain waves' partial K S, [column][token]
};

struct StageFrag {                 // one thread's share of the next chunk's K rows and G
    uint4 k[2];                    // K pieces e = tid + 512 it: row e/16, columns 8 (e%16) .. +7
    float g2;                      // G2 row tid (tid < 64)
};

struct ChainFrag {
    bf16x8 mh[2], ml[2];           // M rows 16w + c, columns 32 kb + 8 g .. +7
    __bf16 vv[4];                  // V rows 16w + 4g + r, column c0 + c (zero past the chunk)
};

struct OutFrag {
    bf16x8 q[4];                   // Q rows 16w' + c, key columns 32 kb + 8 g .. +7 (zero past L)
};

template <int DV>
__global__ __launch_bounds__(kFusedThreads) void chunk_fused_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* initial_state, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ order, int N, int T,
    int Hk, int Hv, int nct, int max_slots, const float* __restrict__ ws_G,
    const __bf16* __restrict__ ws_M, float* __restrict__ o, float* final_state) {
    constexpr int S_SL = DV / kWS;  // slices per head
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    FusedLds& sm = *reinterpret_cast<FusedLds*>(smem_raw);

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
    const size_t sbase = ((size_t)n * Hv + h) * kDK * DV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, gq = lane >> 4;
    const bool chain = wave < 4;
    const int w = wave & 3;

    auto tok0_of = [&](int ci) { return (size_t)row * T + t0 + (size_t)ci * kC; };
    auto len_of = [&](int ci) { return min(kC, t1 - t0 - ci * kC); };
    auto ws_row_of = [&](int ci) { return ((size_t)(slot0 + ci) * Hv + h) * kC; };

    if (nchunks == 0) {  // zero-length sequence: the state passes through
        if (chain) {
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const size_t idx = sbase + (size_t)(32 * w + 16 * it + 4 * gq + r) * DV + c0 + c;
                    final_state[idx] = initial_state ? initial_state[idx] : 0.f;
                }
        }
        return;
    }

    // ---- staging of K rows and G (both roles, one chunk ahead) -------------------------------
    auto fetch_stage = [&](StageFrag& f, int ci) {
        const size_t tok0 = tok0_of(ci);
        const int L = len_of(ci);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int e = tid + kFusedThreads * it, t = e >> 4, p = e & 15;
            const bool live = t < L;
            const uint4 x = *reinterpret_cast<const uint4*>(k + ((tok0 + (live ? t : L - 1)) * Hk + kh) * kDK + 8 * p);
            f.k[it] = live ? x : make_uint4(0, 0, 0, 0);
        }
        f.g2 = ws_G[ws_row_of(ci) + (tid & 63)];
    };
    auto store_stage = [&](const StageFrag& f, int ci) {
        __bf16* kr = sm.Kr[ci % 3];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int e = tid + kFusedThreads * it, t = e >> 4, p = e & 15;
            *reinterpret_cast<uint4*>(kr + t * kKP + 8 * p) = f.k[it];
        }
        if (tid < kC) {
            sm.G2[ci % 3][tid] = f.g2;
            sm.EG[ci % 3][tid] = exp2_fast(f.g2);
        }
    };
    StageFrag sa, sb;
    fetch_stage(sa, 0);
    store_stage(sa, 0);  // chunk 0 is staged before the loop; chunk i+1 at phase 1 of chunk i

    if (chain) {
        // ------------------------------------------------ chain waves -------------------------
        auto fetch_chain = [&](ChainFrag& f, int ci) {
            const __bf16* mb = ws_M + ((size_t)(slot0 + ci) * Hv + h) * 2 * kC * kC + (16 * w + c) * kC + 8 * gq;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f.mh[kb] = *reinterpret_cast<const bf16x8*>(mb + 32 * kb);
                f.ml[kb] = *reinterpret_cast<const bf16x8*>(mb + kC * kC + 32 * kb);
            }
            const size_t tok0 = tok0_of(ci);
            const int L = len_of(ci);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * gq + r;
                const bool live = t < L;
                const __bf16 x = v[((tok0 + (live ? t : L - 1)) * Hv + h) * DV + c0 + c];
                f.vv[r] = live ? x : (__bf16)0.f;
            }
        };
        f32x4 S[2] = {zero4(), zero4()};
        if (initial_state) {
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[it][r] = initial_state[sbase + (size_t)(32 * w + 16 * it + 4 * gq + r) * DV + c0 + c];
        }
        auto step = [&](int i, const ChainFrag& cur, ChainFrag& nxt, const StageFrag& st, StageFrag& stn) {
            store_stage(st, i + 1);  // (the last step stages a repeat of the last chunk: unread)
            fetch_stage(stn, min(i + 2, nchunks - 1));
            fetch_chain(nxt, min(i + 1, nchunks - 1));
            __builtin_amdgcn_sched_barrier(0);
            const __bf16* kr = sm.Kr[i % 3];
            // phase 1: S (hi + lo) -> LDS; partial K S over this wave's 32 key rows
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
                *reinterpret_cast<bf16x4*>(sm.Sh + off) = bf16x4{sh[4 * it], sh[4 * it + 1], sh[4 * it + 2], sh[4 * it + 3]};
                *reinterpret_cast<bf16x4*>(sm.Sl + off) = bf16x4{sl8[4 * it], sl8[4 * it + 1], sl8[4 * it + 2], sl8[4 * it + 3]};
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const __bf16* kk = kr + (16 * a + c) * kKP + 32 * w + 4 * gq;
                const bf16x8 ak = cat44(lds4(kk), lds4(kk + 16));
                const f32x4 ph = mma(ak, sh, zero4());
                const f32x4 pl = mma(ak, sl8, zero4());
                *reinterpret_cast<f32x4*>(&sm.red[w][c * kRP + 16 * a + 4 * gq]) = ph + pl;
            }
            lds_barrier();

            // phase 2: token tile w: X = V - e^G K S  (hi + lo)
            const int tr0 = 16 * w + 4 * gq;
            f32x4 ks = *reinterpret_cast<const f32x4*>(&sm.red[0][c * kRP + tr0]);
#pragma unroll
            for (int w2 = 1; w2 < 4; ++w2) ks += *reinterpret_cast<const f32x4*>(&sm.red[w2][c * kRP + tr0]);
            const f32x4 eg = *reinterpret_cast<const f32x4*>(&sm.EG[i % 3][tr0]);
            bf16x4 xh4, xl4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = (float)cur.vv[r] - eg[r] * ks[r];
                xh4[r] = hi_of(x);
                xl4[r] = lo_of(x, xh4[r]);
            }
            *reinterpret_cast<bf16x4*>(sm.Xh + c * kTP + tr0) = xh4;
            *reinterpret_cast<bf16x4*>(sm.Xl + c * kTP + tr0) = xl4;
            lds_barrier();

            // phase 3: token tile w: U = M X; U and e^(G_C - G) U (hi + lo) -> LDS
            f32x4 uu = zero4(), uu2 = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (2 * kb > w) continue;
                const int off = c * kTP + 32 * kb + 8 * gq;
                const bf16x8 xh = lds8(sm.Xh + off), xl = lds8(sm.Xl + off);
                uu = mma(cur.mh[kb], xh, uu);
                uu2 = mma(cur.mh[kb], xl, uu2);
                uu2 = mma(cur.ml[kb], xh, uu2);
            }
            uu += uu2;
            const f32x4 g2 = *reinterpret_cast<const f32x4*>(&sm.G2[i % 3][tr0]);
            const float g2c = sm.G2[i % 3][kC - 1];
            bf16x4 uh4, ul4, dh4, dl4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uh4[r] = hi_of(uu[r]);
                ul4[r] = lo_of(uu[r], uh4[r]);
                const float dd = exp2_fast(g2c - g2[r]) * uu[r];
                dh4[r] = hi_of(dd);
                dl4[r] = lo_of(dd, dh4[r]);
            }
            const int off = c * kTP + tr0;
            *reinterpret_cast<bf16x4*>(sm.Uh + off) = uh4;
            *reinterpret_cast<bf16x4*>(sm.Ul + off) = ul4;
            *reinterpret_cast<bf16x4*>(sm.Dh + off) = dh4;
            *reinterpret_cast<bf16x4*>(sm.Dl + off) = dl4;
            lds_barrier();

            // phase 4: S <- e^(G_C) S + K^T (e^(G_C - G) U)
            const float eC = sm.EG[i % 3][kC - 1];
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                f32x4 a0 = S[it] * eC, a1 = zero4();
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 kt = tr_frag(kr, kKP, 32 * kb, 32 * w + 16 * it, gq, c);
                    const int o2 = c * kTP + 32 * kb + 8 * gq;
                    a0 = mma(kt, lds8(sm.Dh + o2), a0);
                    a1 = mma(kt, lds8(sm.Dl + o2), a1);
                }
                S[it] = a0 + a1;
            }
        };
        ChainFrag ca, cb;
        fetch_chain(ca, 0);
        fetch_stage(sb, min(1, nchunks - 1));
        lds_barrier();  // chunk 0 staged
        int i = 0;
        for (; i + 1 < nchunks; i += 2) {
            step(i, ca, cb, sb, sa);
            step(i + 1, cb, ca, sa, sb);
        }
        if (i < nchunks) step(i, ca, cb, sb, sa);
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                final_state[sbase + (size_t)(32 * w + 16 * it + 4 * gq + r) * DV + c0 + c] = S[it][r];
    } else {
        // ------------------------------------------------ output waves ------------------------
        auto fetch_out = [&](OutFrag& f, int ci) {
            // rows past the sequence's end read its last row and are then zeroed (no branch)
            const int t = 16 * w + c, L = len_of(ci);
            const bool live = t < L;
            const __bf16* qr = q + ((tok0_of(ci) + (live ? t : L - 1)) * Hk + kh) * kDK + 8 * gq;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const uint4 x = *reinterpret_cast<const uint4*>(qr + 32 * kb);
                const uint4 y = live ? x : make_uint4(0, 0, 0, 0);
                f.q[kb] = *reinterpret_cast<const bf16x8*>(&y);
            }
        };
        const int tq = 16 * w + c;
        // P^T tile (a, w): rows t' = 16a + 4g + r, column t = tq; masked and decayed
        auto ptile = [&](const OutFrag& cur, const __bf16* kr, const float* g2, float gt, int a) {
            f32x4 pt = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                pt = mma(lds8(kr + (16 * a + c) * kKP + 32 * kb + 8 * gq), cur.q[kb], pt);
            const f32x4 gp = *reinterpret_cast<const f32x4*>(g2 + 16 * a + 4 * gq);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tp = 16 * a + 4 * gq + r;
                pt[r] = tp <= tq ? pt[r] * exp2_fast(gt - gp[r]) : 0.f;
            }
            return pt;
        };
        auto step = [&](int i, const OutFrag& cur, OutFrag& nxt, const StageFrag& st, StageFrag& stn) {
            store_stage(st, i + 1);
            fetch_stage(stn, min(i + 2, nchunks - 1));
            fetch_out(nxt, min(i + 1, nchunks - 1));
            __builtin_amdgcn_sched_barrier(0);
            const __bf16* kr = sm.Kr[i % 3];
            const float* g2 = sm.G2[i % 3];
            const float gt = g2[tq];
            // phase 1: P^T tiles a = 0, 1
            f32x4 PT[4] = {zero4(), zero4(), zero4(), zero4()};
            PT[0] = ptile(cur, kr, g2, gt, 0);
            if (w >= 1) PT[1] = ptile(cur, kr, g2, gt, 1);
            lds_barrier();
            // phase 2: O = e^G Q S
            f32x4 qs = zero4(), qs2 = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int off = c * kSP + 32 * kb + 8 * gq;
                qs = mma(cur.q[kb], lds8(sm.Sh + off), qs);
                qs2 = mma(cur.q[kb], lds8(sm.Sl + off), qs2);
            }
            const f32x4 eg = *reinterpret_cast<const f32x4*>(&sm.EG[i % 3][16 * w + 4 * gq]);
            f32x4 Ox = eg * (qs + qs2);
            lds_barrier();
            // phase 3: P^T tiles a = 2, 3
            if (w >= 2) PT[2] = ptile(cur, kr, g2, gt, 2);
            if (w >= 3) PT[3] = ptile(cur, kr, g2, gt, 3);
            lds_barrier();
            // phase 4: O += P U, then store
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (2 * kb > w) continue;
                bf16x8 ph, pl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = PT[2 * kb + (e >> 2)][e & 3];
                    ph[e] = hi_of(x);
                    pl[e] = lo_of(x, ph[e]);
                }
                const int j0 = c * kTP + 32 * kb + 4 * gq;  // token slots j..j+3 and j+16..j+19
                const bf16x8 uh = cat44(lds4(sm.Uh + j0), lds4(sm.Uh + j0 + 16));
                const bf16x8 ul = cat44(lds4(sm.Ul + j0), lds4(sm.Ul + j0 + 16));
                Ox = mma(ph, uh, Ox);
                Ox = mma(ph, ul, Ox);
                Ox = mma(pl, uh, Ox);
            }
            const size_t tok0 = tok0_of(i);
            const int L = len_of(i);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * gq + r;
                if (t < L) o[((tok0 + t) * Hv + h) * DV + c0 + c] = Ox[r];
            }
        };
        OutFrag fa, fb;
        fetch_out(fa, 0);
        fetch_stage(sb, min(1, nchunks - 1));
        lds_barrier();  // chunk 0 staged
        int i = 0;
        for (; i + 1 < nchunks; i += 2) {
            step(i, fa, fb, sb, sa);
            step(i + 1, fb, fa, sa, sb);
        }
        if (i < nchunks) step(i, fa, fb, sb, sa);
    }
}

// ------------------------------------------------------------------------------------------------
// workspace layout (each region 256-byte aligned):
//   chunk_start [N+1] int32 | order [N] int32 | G2 [slots][Hv][64] f32
//   | M [slots][Hv][hi, lo][64][64] bf16
struct Layout {
    size_t chunk_start, order, G, M, total;
    int slots;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(int B, int T, int Hv, int N) {
    Layout l;
    l.slots = (int)(((long long)B * T) / kC) + N;  // bounds B*ceil(T/64) and T/64 + N (packed)
    size_t off = 0;
    l.chunk_start = off; off = align256(off + sizeof(int32_t) * (size_t)(N + 1));
    l.order = off;       off = align256(off + sizeof(int32_t) * (size_t)N);
    l.G = off;           off = align256(off + sizeof(float) * (size_t)l.slots * Hv * kC);
    l.M = off;           off = align256(off + 2 * (size_t)l.slots * Hv * 2 * kC * kC);
    l.total = off;
    return l;
}

template <int DV, typename TG>
hipError_t launch_dv(const ChunkArgs& a, unsigned stages) {
    const Layout lay = layout(a.B, a.T, a.Hv, a.N);
    char* ws = static_cast<char*>(a.workspace);
    const bool packed = a.cu_seqlens != nullptr;
    const int nct = (a.T + kC - 1) / kC;
    const int slots = packed ? lay.slots : a.B * nct;
    const int32_t* chunk_start = packed ? reinterpret_cast<const int32_t*>(ws + lay.chunk_start) : nullptr;
    const int32_t* order = packed ? reinterpret_cast<const int32_t*>(ws + lay.order) : nullptr;
    float* ws_G = reinterpret_cast<float*>(ws + lay.G);
    __bf16* ws_M = reinterpret_cast<__bf16*>(ws + lay.M);
    hipError_t e;
    if ((stages & kStagePrepare) && packed) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, a.stream, a.cu_seqlens, a.N,
                           a.T, reinterpret_cast<int32_t*>(ws + lay.chunk_start),
                           reinterpret_cast<int32_t*>(ws + lay.order));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((stages & kStagePrepare) && slots > 0) {
        hipLaunchKernelGGL((chunk_solve_kernel<TG>), dim3((unsigned)slots, (unsigned)a.Hv),
                           dim3(kThreads), 0, a.stream, static_cast<const __bf16*>(a.k),
                           static_cast<const TG*>(a.g), static_cast<const TG*>(a.beta),
                           a.cu_seqlens, chunk_start, a.N, a.T, a.Hk, a.Hv, nct, ws_G, ws_M);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (!(stages & kStageScan)) return hipSuccess;
    const auto kern = chunk_fused_kernel<DV>;
    const size_t bytes = sizeof(FusedLds);
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes)) != hipSuccess)
        return e;
    const int units = a.N * a.Hv;
    const int groups = (units + 7) / 8;
    hipLaunchKernelGGL(kern, dim3((unsigned)(groups * 8 * (DV / kWS))), dim3(kFusedThreads), bytes,
                       a.stream, static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                       static_cast<const __bf16*>(a.v), a.initial_state, a.cu_seqlens, chunk_start,
                       order, a.N, a.T, a.Hk, a.Hv, nct, packed ? lay.slots : a.B * nct, ws_G, ws_M,
                       a.o, a.final_state);
    return hipGetLastError();
}

}  // namespace

bool chunk_mfma_supported(int dk, int dv, gdn_dtype qkv_dtype) {
    return qkv_dtype == GDN_BF16 && dk == kDK && (dv == 64 || dv == 128);
}

size_t chunk_mfma_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N) {
    (void)Hk;
    (void)dk;
    (void)dv;
    return layout(B, T, Hv, N).total;
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, unsigned stages) {
    const bool g_bf16 = a.gate_dtype == GDN_BF16;
    if (a.dv == 128) return g_bf16 ? launch_dv<128, bf16_t>(a, stages) : launch_dv<128, float>(a, stages);
    return g_bf16 ? launch_dv<64, bf16_t>(a, stages) : launch_dv<64, float>(a, stages);
}

}  // namespace gdn
