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
//                       hi + lo bf16 into the workspace (16 KiB per chunk and v-head), and the
//                       chunk's decay factors.
//   chunk_scan_kernel   one workgroup per (sequence, v-head, 32 columns of S), walking the chunks
//                       in order with chain and output waves (see there).  With M, the chunk's
//                       deltas are U = Ut - W S = M (V - diag(e^G) K S), so W and Ut are never
//                       formed; everything else comes from q, k, v on the fly.
//
// Precision: q, k, v enter the matrix cores as exact bf16 values.  Quantities that feed the output
// with full weight (S, U, P, M) enter as two bf16 terms hi + lo (hi = bf16(x), lo = bf16(x - hi)),
// so their products carry ~16 significant bits.  Accumulation is fp32 everywhere; decay factors
// are applied on the fp32 side.
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

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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
constexpr int kFP = kC + 4;    // row pitch of 64 x 64 fp32 tiles
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Shared-memory address for the hot loops, hidden from the optimizer (an empty asm): accesses at
// constant byte offsets from it then use the instructions' offset field, instead of one
// precomputed address register per access.
__device__ __forceinline__ lds_u8* lds_at(const void* p) {
    lds_u8* q = (lds_u8*)p;
    asm volatile("" : "+v"(q));
    return q;
}
template <typename T>
__device__ __forceinline__ T ld(lds_u8* b, int off) {
    return *(__attribute__((address_space(3))) const T*)(b + off);
}
template <typename T>
__device__ __forceinline__ void st(lds_u8* b, int off, const T& x) {
    *(__attribute__((address_space(3))) T*)(b + off) = x;
}
__device__ __forceinline__ bf16x4 read_tr(lds_u8* b, int off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(b + off));
}

// ------------------------------------------------------------------------------------------------
// chunk_solve_kernel: one workgroup per (chunk slot, v-head).
//
// Writes the chunk's gate block [3][64] floats: G2 = running sum of g log2(e), 2^G2 and
// 2^(G2_C - G2) (G2_C = G2 at the chunk's last row; padding rows past the chunk's length have
// g = 0), and M = T diag(beta) as hi and lo bf16 tiles [64][64] (row-major with the column order
// described at the store, zero above the diagonal and in rows/columns past the chunk's length).
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
    const size_t ws_row = ((size_t)slot * Hv + h) * 3 * kC;
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
        const float G2c = __shfl(G2, 63);
        ws_G[ws_row + lane] = G2;
        ws_G[ws_row + kC + lane] = exp2_fast(G2);
        ws_G[ws_row + 2 * kC + lane] = exp2_fast(G2c - G2);
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

    // M = T diag(beta) as hi and lo rows: 64 rows x 8 pieces of 8 columns.  Within each block of 32
    // columns the stored order is the scan kernel's B-fragment order: stored columns 8 g + e are
    // columns 4 g + e (e < 4) and 16 + 4 g + e - 4 (e >= 4).
    __bf16* Mh = ws_M + ((size_t)slot * Hv + h) * 2 * kC * kC;
    __bf16* Ml = Mh + kC * kC;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int e = tid + kThreads * it;
        const int t = e >> 3, p = e & 7;
        const int j0 = 32 * (p >> 2) + 4 * (p & 3);
        const float4 a0 = *reinterpret_cast<const float4*>(sT + t * kFP + j0);
        const float4 a1 = *reinterpret_cast<const float4*>(sT + t * kFP + j0 + 16);
        const float tv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        bf16x8 hv, lv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = tv[j] * sB[j0 + (j & 3) + 16 * (j >> 2)];
            hv[j] = hi_of(x);
            lv[j] = lo_of(x, hv[j]);
        }
        *reinterpret_cast<bf16x8*>(Mh + t * kC + 8 * p) = hv;
        *reinterpret_cast<bf16x8*>(Ml + t * kC + 8 * p) = lv;
    }
}

// ------------------------------------------------------------------------------------------------
// chunk_scan_kernel: one workgroup of four waves per (sequence, v-head, 32 columns of S).
//
// Waves 0 and 1 are chain waves.  Each owns one 16-column slice of S whole (128 keys x 16 columns,
// eight 16 x 16 fp32 accumulator tiles), so the chunk step
//     KS = K S,   X = V - diag(e^G) KS,   U = M X,   D = diag(e^(G_C - G)) U,
//     S <- e^(G_C) S + K^T D
// runs inside one wave with no reduction across waves: every product's result stays in registers
// and is fed straight back as the next product's B operand.  For that the accumulator rows are
// given a fixed permutation of keys and tokens: row m (m = 4g + r) of tile a stands for index
//     rho(a, m) = 32 (a / 2) + 8 (m / 4) + 4 (a % 2) + m % 4,
// so that tiles 2j and 2j + 1 together hand lane (g, c) the eight consecutive indices
// 32 j + 8 g .. + 7: exactly the B-operand fragment of a 32-deep product.  The A operands are then
// plain 16-byte rows (K rows from LDS, M rows from memory), and K^T for the state update comes from
// the same K rows through ds_read_b64_tr_b16.
//
// Waves 2 and 3 are output waves, running one chunk behind the chain.  Output wave w' owns token
// tiles {0, 3} (w' = 0) or {1, 2} (w' = 1) of O^T = S^T Q^T diag(e^G) + U^T P^T for both slices
// (tokens in natural order here): P^T tiles = K Q^T (masked, decayed) in registers, S^T and U^T
// from the copies the chain waves leave in LDS.  They also stage the next chunk's K rows, V columns
// and gate block into a three-chunk LDS ring.
//
// One LDS barrier per chunk step.  At step s: chain waves do chunk s (read ring slot s % 3, write
// S/U copies to buffer s % 2); output waves finish chunk s - 1 (ring slot (s - 1) % 3, buffer
// (s - 1) % 2) and store chunk s + 1 into ring slot (s + 1) % 3.
constexpr int kScanThreads = 256;
constexpr int kWS = 16;          // state columns per chain wave
constexpr int kSlices = 2;       // chain waves (16-column slices) per workgroup
constexpr int kSP = kDK + 8;     // row pitch of the S^T copies [column][key]
constexpr int kUP = kC + 8;      // row pitch of the U^T copies [column][token]
constexpr int kVP = 48;          // row pitch of the staged V columns [token][32 columns]
// K ring rows: pitch kKR elements (320 bytes, 20 sixteen-byte chunks), and the 16-byte chunk q of
// row t stored at chunk q ^ ((t >> 2) & 3).  With 64 four-byte banks, both ways the rows are read
// then touch 16 different chunk positions per 16 lanes: a row fragment (16 rows, one chunk each,
// rows t..t+15) and a transposed fragment (4 consecutive rows x 4 consecutive chunks).
constexpr int kKR = 160;
__host__ __device__ constexpr int kswz(int t) { return (t >> 2) & 3; }

struct ScanLds {
    __bf16 Kr[3][kC * kKR];                    // K rows [token][key], ring of three chunks
    float Gt[3][3 * kC];                       // gate block: G2, 2^G2, 2^(G2_C - G2)
    __bf16 Vr[3][kC * kVP];                    // V [token][this workgroup's 32 columns]
    __bf16 Ut[kSlices][2][2][kWS * kUP];       // U^T [slice][buffer][hi, lo]
    __bf16 St[kSlices][2][2][kWS * kSP];       // S^T at chunk start [slice][buffer][hi, lo]
};

// index (token or key) that accumulator row m of tile a stands for
__device__ __forceinline__ int rho(int a, int m) {
    return 32 * (a >> 1) + 8 * (m >> 2) + 4 * (a & 1) + (m & 3);
}

// K^T fragment for the state update: lane (g, c) receives K[32 kb + 8 g + e][rho(kt, c)], e = 0..7
// (keys in the state tiles' row order, tokens consecutive as in the D fragments).  Each half is a
// transposed read of rows 32 kb + 8 g + 4 h + c / 4 at logical chunk 4 (kt / 2) + c % 4, half
// kt % 2 of the chunk; `k0`, `k1` hold the ring slot plus the lane's part of the two halves'
// addresses (the chunk swizzle of those rows depends on g and h only).
__device__ __forceinline__ bf16x8 kt_frag(lds_u8* k0, lds_u8* k1, int kt, int kb) {
    const int off = 2 * (32 * kb * kKR + 32 * (kt >> 1) + 4 * (kt & 1));
    return cat44(read_tr(k0, off), read_tr(k1, off));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats -> two RNE bf16 values packed in one register (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ unsigned pack_bf16x2(float x0, float x1) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
}

// x = hi + lo for the eight values {a, b}: hi = bf16(x), lo = bf16(x - hi), as B fragments
__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, bf16x8& h, bf16x8& l) {
    u32x4 hp, lp;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float x0 = p < 2 ? a[2 * p] : b[2 * p - 4];
        const float x1 = p < 2 ? a[2 * p + 1] : b[2 * p - 3];
        const unsigned hh = pack_bf16x2(x0, x1);
        hp[p] = hh;
        lp[p] = pack_bf16x2(x0 - __uint_as_float(hh << 16), x1 - __uint_as_float(hh & 0xffff0000u));
    }
    h = __builtin_bit_cast(bf16x8, hp);
    l = __builtin_bit_cast(bf16x8, lp);
}

struct ChainIn {                   // one chunk's M fragments for a chain wave
    bf16x8 mh[6], ml[6];           // M rows rho(a', c), columns 32 kb + 8 g ..: (a', kb) =
                                   // (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
};

struct OutIn {                     // one chunk's Q fragments for an output wave (registers)
    bf16x8 q[2][4];                // Q rows 16 a + c of its two tiles, columns 32 kb + 8 g ..
};

struct StageIn {                   // an output wave's half of one chunk's staged inputs
    u32x4 k[8];                    // K piece e = lane + 64 (2 it + w'): row e / 16, columns 8 (e % 16)
    u32x4 v[2];                    // V piece e = lane + 64 (2 it + w'): row e / 4, columns 8 (e % 4)
    f32x4 gt;                      // gate piece lane (lanes < 24), 4 floats each per output wave
};

template <int DV>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chunk_scan_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* initial_state, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ order, int N, int T,
    int Hk, int Hv, int nct, int max_slots, const float* __restrict__ ws_G,
    const __bf16* __restrict__ ws_M, float* __restrict__ o, float* final_state) {
    constexpr int NP = DV / (kWS * kSlices);  // column pairs per v-head
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    ScanLds& sm = *reinterpret_cast<ScanLds*>(smem_raw);

    // blockIdx -> (group, member): a group is one (sequence, q/k head); its members are the
    // (v-head, column pair) workgroups that read the same q and k.  All members of a group share
    // blockIdx % 8, hence one XCD and its L2.
    const int Gq = Hv / Hk, MB = Gq * NP;
    const int bid = blockIdx.x;
    const int xr = bid >> 3;
    const int member = xr % MB;
    const int grp = (xr / MB) * 8 + (bid & 7);
    if (grp >= N * Hk) return;
    const int rank = grp / Hk, kh = grp % Hk;
    const int h = kh * Gq + member / NP;
    const int pair = member % NP;
    const int n = order ? order[rank] : rank;
    int row, t0, t1;
    sequence_range(cu_seqlens, n, T, row, t0, t1);
    const int slot0 = cu_seqlens ? chunk_start[n] : n * nct;
    // (a malformed cu_seqlens can claim more chunks than the workspace holds: stop at its end)
    const int nchunks = min((t1 - t0 + kC - 1) / kC, max(0, max_slots - slot0));
    const size_t sbase = ((size_t)n * Hv + h) * kDK * DV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;

    auto tok0_of = [&](int ci) { return (size_t)row * T + t0 + (size_t)ci * kC; };
    auto len_of = [&](int ci) { return min(kC, t1 - t0 - ci * kC); };

    if (wave < kSlices) {
        // ------------------------------------------------ chain waves -------------------------
        const int c0 = (pair * kSlices + wave) * kWS;
        auto state_idx = [&](int kt, int r) {
            return sbase + (size_t)rho(kt, 4 * g + r) * DV + c0 + c;
        };
        if (nchunks == 0) {  // zero-length sequence: the state passes through
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    final_state[state_idx(kt, r)] = initial_state ? initial_state[state_idx(kt, r)] : 0.f;
            return;
        }
        constexpr int ta[6] = {0, 1, 2, 2, 3, 3}, tb[6] = {0, 0, 0, 1, 0, 1};
        auto fetch = [&](ChainIn& f, int ci) {
            const __bf16* mb = ws_M + ((size_t)(slot0 + ci) * Hv + h) * 2 * kC * kC;
#pragma unroll
            for (int p = 0; p < 6; ++p) {
                const __bf16* mp = mb + rho(ta[p], c) * kC + 32 * tb[p] + 8 * g;
                f.mh[p] = *reinterpret_cast<const bf16x8*>(mp);
                f.ml[p] = *reinterpret_cast<const bf16x8*>(mp + kC * kC);
            }
        };

        f32x4 S[8];
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[kt][r] = initial_state ? initial_state[state_idx(kt, r)] : 0.f;
        // lane parts of the LDS addresses (the rest are compile-time offsets)
        const int l_kf = c * kKR + 8 * (g ^ kswz(c));                     // K row c, logical chunk g
        const int l_kt0 = (8 * g + (c >> 2)) * kKR + 8 * ((c & 3) ^ kswz(8 * g));
        const int l_kt1 = (8 * g + 4 + (c >> 2)) * kKR + 8 * ((c & 3) ^ kswz(8 * g + 4));
        const int l_v = (4 * g + (c >> 2)) * kVP + kWS * wave + 4 * (c & 3);
        const int l_st = c * kSP + 8 * g, l_ut = c * kUP + 8 * g;

        // one set of M registers: chunk i's fragments are consumed by U = M X, then the same
        // registers are refilled with chunk i + 1's, a whole step ahead of their use
        ChainIn mc;
        auto step = [&](int i) {
            const __bf16* kr = sm.Kr[i % 3];
            const __bf16* vr = sm.Vr[i % 3];
            const float* gt = sm.Gt[i % 3];
            // K rows for K S, all issued before the first product
            bf16x8 kf[4][4];                             // K rows 16 a + c, keys 32 j + 8 g ..
            lds_u8* kfl = lds_at(kr + l_kf);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int a = 0; a < 4; ++a) kf[j][a] = ld<bf16x8>(kfl, 2 * (16 * a * kKR + 32 * j));
            __builtin_amdgcn_sched_barrier(0);
            // S as hi + lo B fragments (keys 32 j + 8 g + e)
            bf16x8 sh[4], sl[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split8(S[2 * j], S[2 * j + 1], sh[j], sl[j]);
            // KS: token tile a, rows 16 a + m
            f32x4 ks[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    ks[a] = mma(kf[j][a], sh[j], ks[a]);
                    ks[a] = mma(kf[j][a], sl[j], ks[a]);
                }
            __builtin_amdgcn_sched_barrier(0);
            // V[16 a + 4 g + r][c0 + c], r = 0..3 (one transposed read of four consecutive rows),
            // the decay factors, the first half of the K^T fragments; the S copy for the output
            lds_u8* vl = lds_at(vr + l_v);
            lds_u8* kt0 = lds_at(kr + l_kt0);
            lds_u8* kt1 = lds_at(kr + l_kt1);
            lds_u8* gl = lds_at(gt + 4 * g);
            lds_u8* gd = lds_at(gt + 8 * g);
            bf16x4 vv[4];
            f32x4 eg[4], dg[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                vv[a] = read_tr(vl, 2 * 16 * a * kVP);
                eg[a] = ld<f32x4>(gl, 4 * (kC + 16 * a));                   // 2^G2 at 16 a + 4 g + r
                dg[a] = ld<f32x4>(gd, 4 * (2 * kC + 32 * (a >> 1) + 4 * (a & 1)));  // at rho(a, 4 g + r)
            }
            const float ec = gt[2 * kC - 1];
            bf16x8 kt[8][2];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) kt[t][kb] = kt_frag(kt0, kt1, t, kb);
            lds_u8* stb = lds_at(sm.St[wave][i & 1][0] + l_st);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                st(stb, 2 * 32 * j, sh[j]);
                st(stb, 2 * (kWS * kSP + 32 * j), sl[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
            // X = V - e^G KS as hi + lo B fragments (tokens 32 kb + 4 g + e for e < 4 and
            // 32 kb + 16 + 4 g + e - 4 for e >= 4: the stored column order of M)
            f32x4 xs[4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int r = 0; r < 4; ++r) xs[a][r] = (float)vv[a][r] - eg[a][r] * ks[a][r];
            bf16x8 xh[2], xl[2];
            split8(xs[0], xs[1], xh[0], xl[0]);
            split8(xs[2], xs[3], xh[1], xl[1]);
            // U = M X (M lower triangular: token tiles 0, 1 need kb = 0 only)
            f32x4 u[4], u2[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) { u[a] = zero4(); u2[a] = zero4(); }
#pragma unroll
            for (int p = 0; p < 6; ++p) {
                u[ta[p]] = mma(mc.mh[p], xh[tb[p]], u[ta[p]]);
                u2[ta[p]] = mma(mc.mh[p], xl[tb[p]], u2[ta[p]]);
                u2[ta[p]] = mma(mc.ml[p], xh[tb[p]], u2[ta[p]]);
            }
            __builtin_amdgcn_sched_barrier(0);
            fetch(mc, min(i + 1, nchunks - 1));
            // second half of the K^T fragments
#pragma unroll
            for (int t = 4; t < 8; ++t)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) kt[t][kb] = kt_frag(kt0, kt1, t, kb);
            f32x4 ds[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                u[a] += u2[a];
                ds[a] = u[a] * dg[a];
            }
            bf16x8 dh[2], dl[2];
            split8(ds[0], ds[1], dh[0], dl[0]);
            split8(ds[2], ds[3], dh[1], dl[1]);
            // S <- e^(G_C) S + K^T D
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                f32x4 acc = S[t] * ec;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    acc = mma(kt[t][kb], dh[kb], acc);
                    acc = mma(kt[t][kb], dl[kb], acc);
                }
                S[t] = acc;
            }
            // U (hi + lo) for the output waves
            bf16x8 uh[2], ul[2];
            split8(u[0], u[1], uh[0], ul[0]);
            split8(u[2], u[3], uh[1], ul[1]);
            lds_u8* utb = lds_at(sm.Ut[wave][i & 1][0] + l_ut);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                st(utb, 2 * 32 * kb, uh[kb]);
                st(utb, 2 * (kWS * kUP + 32 * kb), ul[kb]);
            }
            lds_barrier();
        };
        fetch(mc, 0);
        lds_barrier();  // chunk 0 staged
        for (int i = 0; i < nchunks; ++i) step(i);
        lds_barrier();  // the output waves' last step
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) final_state[state_idx(kt, r)] = S[kt][r];
    } else {
        // ------------------------------------------------ output waves ------------------------
        if (nchunks == 0) return;
        auto run = [&](auto w2c) {
            constexpr int w2 = decltype(w2c)::value;     // 0: tiles {0, 3}; 1: tiles {1, 2}
            constexpr int tiles[2] = {w2, 3 - w2};
            const int l_kf = c * kKR + 8 * (g ^ kswz(c));                 // K row c, logical chunk g
            const int l_st = c * kSP + 8 * g, l_ut = c * kUP + 4 * g;
            const int l_sk = (lane >> 4) * kKR + 8 * (lane & 15);          // staged K piece (physical)
            const int l_sv = (lane >> 2) * kVP + 8 * (lane & 3);           // staged V piece
            // staging: K rows (8 pieces per lane), this workgroup's 32 V columns (2 pieces), the
            // gate block (48 pieces of 4 floats: lanes 0..23 of each output wave).  Rows past a
            // partial chunk's end repeat its last row (so every load is in bounds and unmasked):
            // they meet zero rows and columns of M (beta = 0 there), so they contribute nothing,
            // and outputs of those rows are never stored.
            auto fetch_stage = [&](StageIn& f, int ci) {
                const size_t tok0 = tok0_of(ci);
                const int L = len_of(ci);
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    // row 4 (2 it + w') + lane / 16, physical chunk lane % 16: logical chunk
                    // (lane % 16) ^ kswz(row)
                    const int e = lane + 64 * (2 * it + w2), t = e >> 4;
                    const int p = (e & 15) ^ kswz(t);
                    f.k[it] = *reinterpret_cast<const u32x4*>(k + ((tok0 + min(t, L - 1)) * Hk + kh) * kDK + 8 * p);
                }
#pragma unroll
                for (int it = 0; it < 2; ++it) {
                    const int e = lane + 64 * (2 * it + w2), t = min(e >> 2, L - 1), p = e & 3;
                    f.v[it] = *reinterpret_cast<const u32x4*>(
                        v + ((tok0 + t) * Hv + h) * DV + pair * kSlices * kWS + 8 * p);
                }
                const float* gb = ws_G + ((size_t)(slot0 + ci) * Hv + h) * 3 * kC;
                f.gt = *reinterpret_cast<const f32x4*>(gb + 4 * min(lane + 24 * w2, 47));
            };
            auto store_stage = [&](const StageIn& f, int ci) {
                lds_u8* kl = lds_at(sm.Kr[ci % 3] + l_sk);
#pragma unroll
                for (int it = 0; it < 8; ++it)                           // rows 4 (2 it + w') + lane / 16
                    st(kl, 2 * 4 * (2 * it + w2) * kKR, f.k[it]);
                lds_u8* vl = lds_at(sm.Vr[ci % 3] + l_sv);
#pragma unroll
                for (int it = 0; it < 2; ++it)                           // rows 16 (2 it + w') + lane / 4
                    st(vl, 2 * 16 * (2 * it + w2) * kVP, f.v[it]);
                if (lane < 24) *reinterpret_cast<f32x4*>(sm.Gt[ci % 3] + 4 * (lane + 24 * w2)) = f.gt;
            };
            auto fetch_out = [&](OutIn& f, int ci) {
                const size_t tok0 = tok0_of(ci);
                const int L = len_of(ci);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int t = min(16 * tiles[x] + c, L - 1);
                    const __bf16* qr = q + ((tok0 + t) * Hk + kh) * kDK + 8 * g;
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) f.q[x][kb] = *reinterpret_cast<const bf16x8*>(qr + 32 * kb);
                }
            };
            // one set of staging registers and one of Q registers, each refilled right after its
            // last use in a step, a whole step ahead of the next use
            StageIn st;
            OutIn cur;
            auto step = [&](int s) {
                // stage chunk s + 1 (fetched one step ago), then fetch chunk s + 2 into the same
                // registers (repeats of the last chunk near the end: never read)
                store_stage(st, s + 1);
                fetch_stage(st, min(s + 2, nchunks - 1));
                const int ci = s - 1;                    // the chunk finished in this step
                const __bf16* kr = sm.Kr[ci % 3];
                const float* gt = sm.Gt[ci % 3];
                const int buf = ci & 1;
                // LDS operands, all issued up front: K rows of the P^T tiles (b <= 3 - w'), the
                // gate values, S^T (hi, lo) and U^T (hi, lo) of both slices
                constexpr int NB = 4 - w2;
                bf16x8 kf[NB][4];
                lds_u8* kfl = lds_at(kr + l_kf);
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) kf[b][kb] = ld<bf16x8>(kfl, 2 * (16 * b * kKR + 32 * kb));
                f32x4 gp[NB];
                lds_u8* gl = lds_at(gt + 4 * g);
#pragma unroll
                for (int b = 0; b < NB; ++b) gp[b] = ld<f32x4>(gl, 4 * 16 * b);
                float gq[2], eq[2];
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    gq[x] = gt[16 * tiles[x] + c];
                    eq[x] = gt[kC + 16 * tiles[x] + c];
                }
                bf16x8 sf[kSlices][2][4], uf[kSlices][2][2];
#pragma unroll
                for (int j = 0; j < kSlices; ++j)
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl) {
                        lds_u8* sp = lds_at(sm.St[j][buf][hl] + l_st);
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) sf[j][hl][kb] = ld<bf16x8>(sp, 2 * 32 * kb);
                        lds_u8* up = lds_at(sm.Ut[j][buf][hl] + l_ut);
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
                            uf[j][hl][kb] = cat44(ld<bf16x4>(up, 2 * 32 * kb), ld<bf16x4>(up, 2 * (32 * kb + 16)));
                    }
                __builtin_amdgcn_sched_barrier(0);
                f32x4 ot[2][kSlices];
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int a = tiles[x];
                    const int t = 16 * a + c;
                    // P^T tiles (b, a) = K Q^T for b <= a: rows t' = 16 b + m, masked to t' <= t
                    f32x4 pt[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        pt[b] = zero4();
                        if (b > a) continue;
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) pt[b] = mma(kf[b][kb], cur.q[x][kb], pt[b]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int tp = 16 * b + 4 * g + r;
                            pt[b][r] = tp <= t ? pt[b][r] * exp2_fast(gq[x] - gp[b][r]) : 0.f;
                        }
                    }
                    // B fragments for P U: reduction rows 32 kb + 4 g + e (e < 4), + 16 (e >= 4)
                    bf16x8 ph[2], pl[2];
                    split8(pt[0], pt[1], ph[0], pl[0]);
                    split8(pt[2], pt[3], ph[1], pl[1]);
#pragma unroll
                    for (int j = 0; j < kSlices; ++j) {
                        f32x4 qs = zero4(), qs2 = zero4();
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) {
                            qs = mma(sf[j][0][kb], cur.q[x][kb], qs);
                            qs2 = mma(sf[j][1][kb], cur.q[x][kb], qs2);
                        }
                        f32x4 acc = (qs + qs2) * eq[x];
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            if (2 * kb > a) continue;
                            acc = mma(uf[j][0][kb], ph[kb], acc);
                            acc = mma(uf[j][0][kb], pl[kb], acc);
                            acc = mma(uf[j][1][kb], ph[kb], acc);
                        }
                        ot[x][j] = acc;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                fetch_out(cur, min(s, nchunks - 1));             // chunk s's Q rows, for the next step
                const size_t tok0 = tok0_of(ci);
                const int L = len_of(ci);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int t = 16 * tiles[x] + c;
                    if (t < L) {
#pragma unroll
                        for (int j = 0; j < kSlices; ++j) {
                            const int c0 = (pair * kSlices + j) * kWS;
                            *reinterpret_cast<f32x4*>(o + ((tok0 + t) * Hv + h) * DV + c0 + 4 * g) = ot[x][j];
                        }
                    }
                }
                lds_barrier();
            };
            fetch_stage(st, 0);
            store_stage(st, 0);
            fetch_stage(st, min(1, nchunks - 1));
            lds_barrier();  // chunk 0 staged
            // step 0: stage chunk 1, fetch chunk 2 and chunk 0's Q rows
            store_stage(st, 1);
            fetch_stage(st, min(2, nchunks - 1));
            fetch_out(cur, 0);
            lds_barrier();
            for (int s = 1; s <= nchunks; ++s) step(s);
        };
        if (wave == kSlices) run(std::integral_constant<int, 0>{});
        else run(std::integral_constant<int, 1>{});
    }
}

// ------------------------------------------------------------------------------------------------
// workspace layout (each region 256-byte aligned):
//   chunk_start [N+1] int32 | order [N] int32 | gates [slots][Hv][G2, 2^G2, 2^(G2_C - G2)][64] f32
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
    l.G = off;           off = align256(off + sizeof(float) * (size_t)l.slots * Hv * 3 * kC);
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
    const auto kern = chunk_scan_kernel<DV>;
    const size_t bytes = sizeof(ScanLds);
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes)) != hipSuccess)
        return e;
    const int groups = a.N * a.Hk;                        // (sequence, q/k head)
    const int members = (a.Hv / a.Hk) * (DV / (kWS * kSlices));
    const unsigned grid = (unsigned)(((groups + 7) / 8) * 8 * members);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kScanThreads), bytes,
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
