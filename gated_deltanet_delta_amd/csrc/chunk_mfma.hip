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
//   chunk_solve_kernel  one workgroup per (chunk, q/k head), all chunks in parallel: the part with
//                       a serial dependence inside a chunk.  Cumsum, A on the matrix cores, T by a
//                       blocked forward substitution (16 x 16 diagonal blocks by substitution,
//                       off-diagonal blocks by fp32 matrix-core products), M = T diag(beta) as
//                       hi + lo bf16 into the workspace (12 KiB per chunk and v-head), the chunk's
//                       decay factors, and N = K K_prev^T (16 KiB per chunk and q/k head).
//   chunk_scan_kernel   one workgroup per (sequence, v-head, 16 columns of S), walking the chunks
//                       in order with chain, state and output waves (see there).  With M, the
//                       chunk's deltas are U = Ut - W S = M (V - diag(e^G) K S), so W and Ut are
//                       never formed; everything else comes from q, k, v on the fly.
//
// Precision: q, k, v enter the matrix cores as exact bf16 values.  Quantities that feed the output
// with full weight (S, X, U, D, P, M, N) enter as two bf16 terms hi + lo (hi = bf16(x),
// lo = bf16(x - hi)), so their products carry ~16 significant bits.  Accumulation is fp32
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
constexpr int kGRows = 5;   // rows of a chunk's gate block (of kC floats each)
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
// Fragment layouts shared by the solve kernel (writer) and the scan kernel (reader).
//
// A "fragment" is the A operand of one v_mfma_f32_16x16x32_bf16 as the 64 lanes hold it: lane
// (g, c) has eight bf16 values, 16 bytes; a fragment is stored as 64 x 16 = 1 KiB with lane l at
// byte 16 l, so that one wave loads it with one fully coalesced instruction.
//
// The B operands these fragments meet in the scan kernel are accumulator tiles fed straight back:
// tiles 2j and 2j + 1 with natural token rows hand lane (g, c) the tokens 32 j + 4 g + e (e < 4)
// and 32 j + 16 + 4 g + e - 4 (e >= 4).  Element e of an A fragment's lane (g, c) therefore holds
// column 32 j + colperm(g, e) of its row, colperm(g, e) = 4 g + (e & 3) + 16 (e >> 2).
//
//   M (per chunk and v-head): the nonzero pairs (row tile a, k-step j) of the lower-triangular
//     M = T diag(beta), in the order (0,0) (1,0) (2,0) (2,1) (3,0) (3,1), each as hi then lo:
//     12 fragments.  Lane (g, c) of pair (a, j) holds row 16 a + c.
//   N (per chunk and q/k head, chunks with a predecessor in the same sequence only): N = K K_p^T,
//     rows the chunk's tokens, columns the previous chunk's, all pairs (a, j) in the order
//     (0,0) (0,1) (1,0) ... (3,1), each as hi then lo: 16 fragments.
constexpr int kFragElems = 512;  // bf16 per fragment
constexpr int kMFrags = 12;
constexpr int kNFrags = 16;
__host__ __device__ constexpr int m_pair_row(int p) { return p < 2 ? p : (p < 4 ? 2 : 3); }
__host__ __device__ constexpr int m_pair_step(int p) { return (p == 3 || p == 5) ? 1 : 0; }
__device__ __forceinline__ int colperm(int g, int e) { return 4 * g + (e & 3) + 16 * (e >> 2); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats -> two RNE bf16 values packed in one register (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ unsigned pack_bf16x2(float x0, float x1) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
}

// x = hi + lo for the eight values {a, b}: hi = bf16(x), lo = bf16(x - hi), as fragments
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

// ------------------------------------------------------------------------------------------------
// chunk_solve_kernel: one workgroup per (chunk slot, q/k head), for each of the head's v-heads.
//
// Writes, per (chunk, v-head), the chunk's gate block [5][64] floats: G2 = running sum of
// g log2(e), 2^G2, 2^(G2_C - G2) (G2_C = G2 at the chunk's last row; padding rows past the
// chunk's length have g = 0) and, with L2, the key and query scales r_t = 1 / |k_t| and
// rq_t = 1 / |q_t| (rows 3 and 4); and M = T diag(beta) as the 12 fragments described above (zero
// above the diagonal and in rows/columns past the chunk's length).  Per (chunk, q/k head) it writes
// N = K K_p^T for the scan kernel's K S recurrence.
//
// L2 (q and k normalised to unit length): the normalised keys are diag(r) K, so the chunk's
// K K^T becomes diag(r) K K^T diag(r) (applied to the product tiles in fp32), and every later use of
// a normalised key or query is a per-token factor on the scan kernel's fp32 side; K and Q
// themselves stay the exact bf16 inputs.
//
// K enters the matrix cores straight from memory (its rows are both operands of K K^T), and
// K K^T is formed once for all v-heads of the q/k head.  A and T live in shared memory as their
// lower 16 x 16 blocks only (22 KB in all).
constexpr int kBP = 17;          // row pitch (floats) of the 16 x 16 blocks of A and T
__device__ __forceinline__ int blk(int a, int b) { return a * (a + 1) / 2 + b; }   // a >= b

// (at most 128 registers per lane: four waves per SIMD, so a whole 4096-token prefill's chunk
// workgroups are resident at once)
template <typename TG, bool L2>
__global__ __launch_bounds__(kThreads, 4) void chunk_solve_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const TG* __restrict__ g,
    const TG* __restrict__ beta, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ chunk_start, int N, int T,
    int Hk, int Hv, int nct, float* __restrict__ ws_G, __bf16* __restrict__ ws_M,
    __bf16* __restrict__ ws_N) {
    __shared__ float sA[10][16 * kBP];     // blocks (a, b), a > b, of A
    __shared__ float sT[10][16 * kBP];     // blocks (a, b), a >= b, of T = (I + A)^-1
    __shared__ float sB[kC];

    const int slot = blockIdx.x, kh = blockIdx.y;
    ChunkLoc loc;
    if (!locate_chunk(slot, cu_seqlens, chunk_start, N, T, nct, loc)) return;
    const int Gq = Hv / Hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, gq = lane >> 4;
    const size_t tok0 = (size_t)loc.row * T + loc.t0;
    const int L = loc.len;
    const bool has_prev = loc.ci > 0;   // the previous chunk (always a full one) is in this sequence

    // K K^T as 16x16 tiles; wave w owns diagonal tile (w, w) and some below it: wave 0 (0,0) (1,0);
    // wave 1 (1,1) (2,1) (2,0); wave 2 (2,2) (3,2); wave 3 (3,3) (3,0) (3,1).  The K rows of the (at
    // most three) token tiles a wave needs are all loaded before the first product.  K rows past
    // the chunk's end repeat its last row: they only meet rows with beta = 0.
    auto kfrag = [&](int t, int kb) {
        const int r = min(16 * t + c, L - 1);
        return *reinterpret_cast<const bf16x8*>(k + ((tok0 + r) * Hk + kh) * kDK + 32 * kb + 8 * gq);
    };
    // token tiles of the K rows: wave 0 {0, 1}, wave 1 {1, 2, 0}, wave 2 {2, 3}, wave 3 {3, 0, 1}
    const int tt0 = wave, tt1 = (wave + 1) & 3, tt2 = wave == 1 ? 0 : 1;
    bf16x8 k0[4], k1[4], k2[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        k0[kb] = kfrag(tt0, kb);
        k1[kb] = kfrag(tt1, kb);
    }
    if (wave & 1) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) k2[kb] = kfrag(tt2, kb);
    }
    // the previous chunk's K rows 16 b + c, b = 0..3, for N
    bf16x8 kp[4][4];
    if (has_prev) {
        const __bf16* pb = k + ((tok0 - kC + c) * Hk + kh) * kDK + 8 * gq;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                kp[b][kb] = *reinterpret_cast<const bf16x8*>(pb + (size_t)16 * b * Hk * kDK + 32 * kb);
    }
    auto kkt = [&](const bf16x8* ka, const bf16x8* kb_) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = mma(ka[kb], kb_[kb], acc);
        return acc;
    };
    // lane (g, c) element r of tile (ta, tb) holds (K K^T)[16 ta + 4 g + r][16 tb + c]
    f32x4 kd = kkt(k0, k0);                                        // (w, w)
    f32x4 kx = wave == 3 ? kkt(k0, k1) : kkt(k1, k0);              // (1,0) (2,1) (3,2) / (3,0)
    f32x4 ky = zero4();                                            // (2,0) / (3,1)
    if (wave == 1) ky = kkt(k1, k2);
    if (wave == 3) ky = kkt(k0, k2);
    const int xa = wave == 3 ? 3 : wave + 1, xb = wave == 3 ? 0 : wave;
    const int ya = wave == 1 ? 2 : 3, yb = wave == 1 ? 0 : 1;

    // N: wave w forms the tiles (b, w) of N^T = K_p K^T, whose lane (g, c) element r is
    // N[16 w + c][16 b + 4 g + r]; tiles 2j and 2j + 1 together are exactly fragment (w, j)
    if (has_prev) {
        f32x4 nt[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) nt[b] = kkt(kp[b], k0);
        __bf16* nb = ws_N + ((size_t)slot * Hk + kh) * kNFrags * kFragElems + 8 * lane;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            bf16x8 hv, lv;
            split8(nt[2 * j], nt[2 * j + 1], hv, lv);
            *reinterpret_cast<bf16x8*>(nb + (2 * (2 * wave + j)) * kFragElems) = hv;
            *reinterpret_cast<bf16x8*>(nb + (2 * (2 * wave + j) + 1) * kFragElems) = lv;
        }
    }


    if constexpr (L2) {
        // r_t = 1 / sqrt(|k_t|^2 + eps) for the rows of the wave's K tiles (lane (g, c) holds 32 of
        // row 16 tt + c's keys; the sum over g leaves every lane with its column's r), then
        // K K^T -> diag(r) K K^T diag(r) tile by tile: a tile's column factor is the lane's own, its
        // row factors come from lanes 4 g + r.  Each wave writes r of its own tile `wave` to the gate
        // blocks of every v-head.
        auto rnorm = [&](const bf16x8* kf) {
            float ss = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = (float)kf[kb][e];
                    ss += x * x;
                }
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            return 1.f / sqrtf(ss + kL2Eps);
        };
        const float r0 = rnorm(k0), r1 = rnorm(k1), r2 = (wave & 1) ? rnorm(k2) : 1.f;
        auto scale_tile = [&](f32x4& acc, float rrow, float rcol) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= __shfl(rrow, 4 * gq + r) * rcol;
        };
        scale_tile(kd, r0, r0);
        if (wave == 3) scale_tile(kx, r0, r1);       // (3, 0): rows k0, columns k1
        else scale_tile(kx, r1, r0);                 // (w + 1, w)
        if (wave == 1) scale_tile(ky, r1, r2);       // (2, 0)
        if (wave == 3) scale_tile(ky, r0, r2);       // (3, 1)
        if (gq == 0)
            for (int qh = 0; qh < Gq; ++qh)
                ws_G[((size_t)slot * Hv + kh * Gq + qh) * kGRows * kC + 3 * kC + 16 * wave + c] = r0;
    }
    // the gates of the first kPre v-heads are loaded together with K (one memory round trip)
    constexpr int kPre = 4;
    float gpre[kPre], bpre[kPre];
    const size_t grow = (tok0 + min(lane, L - 1)) * Hv + (size_t)kh * Gq;
#pragma unroll
    for (int qh = 0; qh < kPre; ++qh) {
        const int qq = min(qh, Gq - 1);
        gpre[qh] = to_f32(g[grow + qq]);
        bpre[qh] = to_f32(beta[grow + qq]);
    }

    for (int qh = 0; qh < Gq; ++qh) {
        const int h = kh * Gq + qh;
        // the chunk's gates and the running log2-decay G2 (a wave prefix sum, in every wave)
        float graw, braw;
        if (qh < kPre) {
            graw = gpre[0]; braw = bpre[0];
#pragma unroll
            for (int j = 1; j < kPre; ++j)
                if (qh == j) { graw = gpre[j]; braw = bpre[j]; }
        } else {
            graw = to_f32(g[grow + qh]);
            braw = to_f32(beta[grow + qh]);
        }
        float gv, bv;
        gate_values(graw, braw, A_log, dt_bias, h, gv, bv);
        const float gt = lane < L ? gv * kLog2e : 0.f;
        const float bt = lane < L ? bv : 0.f;
        float G2 = gt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(G2, off);
            if (lane >= off) G2 += y;
        }
        if (wave == 0) {
            const size_t ws_row = ((size_t)slot * Hv + h) * kGRows * kC;
            const float G2c = __shfl(G2, 63);
            ws_G[ws_row + lane] = G2;
            ws_G[ws_row + kC + lane] = exp2_fast(G2);
            ws_G[ws_row + 2 * kC + lane] = exp2_fast(G2c - G2);
            sB[lane] = bt;
        }
        // A = diag(beta) (K K^T o Gam), strictly lower, tile by tile
        auto atile = [&](int ta, int tb, f32x4 acc) {
            const float Gj = __shfl(G2, 16 * tb + c);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * ta + 4 * gq + r, j = 16 * tb + c;
                const float Gt = __shfl(G2, t), Bt = __shfl(bt, t);
                acc[r] = j < t ? Bt * acc[r] * exp2_fast(Gt - Gj) : 0.f;
            }
            return acc;
        };
        auto store_a = [&](int ta, int tb, const f32x4& x) {
            float* dst = sA[blk(ta, tb)];
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(4 * gq + r) * kBP + c] = x[r];
        };
        store_a(xa, xb, atile(xa, xb, kx));
        if (wave & 1) store_a(ya, yb, atile(ya, yb, ky));
        // T_ww = (I + A_ww)^-1 by forward substitution, lane c computing column c, column-sweep
        // order (x_j final, then subtracted from every later row: 15 dependent steps); the entries
        // of A_ww come out of the accumulator tile one by one, broadcast with readlane
        {
            const f32x4 ad = atile(wave, wave, kd);
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) x[t] = (t == c) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < 15; ++j)
#pragma unroll
                for (int t = j + 1; t < 16; ++t)
                    x[t] -= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ad[t & 3]), 16 * (t >> 2) + j)) * x[j];
            if (lane < 16) {
                float* Td = sT[blk(wave, wave)];
#pragma unroll
                for (int t = 0; t < 16; ++t) Td[t * kBP + c] = x[t];
            }
        }
        lds_barrier();
        // off-diagonal blocks, by distance d = a - b:  T_ab = -T_aa * sum_{m=b}^{a-1} A_am T_mb
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            if (wave < 4 - d) {
                const int b = wave, a = wave + d;
                f32x4 X = zero4();
                for (int mm = b; mm < a; ++mm) {
                    const float* Am = sA[blk(a, mm)];
                    const float* Tm = sT[blk(mm, b)];
#pragma unroll
                    for (int s = 0; s < 4; ++s) X = mma_f32(Am[c * kBP + 4 * s + gq], Tm[(4 * s + gq) * kBP + c], X);
                }
                // -T_aa X with X fed back from the accumulator: step s takes reduction rows 4g + s
                const float* Ta = sT[blk(a, a)];
                f32x4 Y = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) Y = mma_f32(Ta[c * kBP + 4 * gq + s], X[s], Y);
                float* Tab = sT[blk(a, b)];
#pragma unroll
                for (int r = 0; r < 4; ++r) Tab[(4 * gq + r) * kBP + c] = -Y[r];
            }
            lds_barrier();
        }

        // M = T diag(beta) as its 12 fragments: item e = (pair p, lane ln) writes the hi and lo
        // fragment rows of that lane, one 1 KiB fragment per wave and pass
        __bf16* Mb = ws_M + ((size_t)slot * Hv + h) * kMFrags * kFragElems;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int e = tid + kThreads * it;
            if (e >= 6 * 64) break;
            const int p = e >> 6, ln = e & 63, lg = ln >> 4;
            const int t = 16 * m_pair_row(p) + (ln & 15), j0 = 32 * m_pair_step(p);
            bf16x8 hv, lv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = j0 + colperm(lg, j);
                const int ba = t >> 4, bb = col >> 4;
                const float tv = bb <= ba ? sT[blk(ba, bb)][(t & 15) * kBP + (col & 15)] : 0.f;
                const float x = tv * sB[col];
                hv[j] = hi_of(x);
                lv[j] = lo_of(x, hv[j]);
            }
            *reinterpret_cast<bf16x8*>(Mb + (2 * p) * kFragElems + 8 * ln) = hv;
            *reinterpret_cast<bf16x8*>(Mb + (2 * p + 1) * kFragElems + 8 * ln) = lv;
        }
        lds_barrier();                 // sT and sB are rewritten for the next v-head
    }
    if constexpr (L2) {
        // rq_t = 1 / sqrt(|q_t|^2 + eps) for token tile `wave` (lane (g, c): 32 of row 16 wave + c's
        // keys), into every v-head's gate block; read last, when the solve's registers are free
        const int qrow = min(16 * wave + c, L - 1);
        const __bf16* qr = q + ((tok0 + qrow) * Hk + kh) * kDK + 8 * gq;
        bf16x8 qf[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) qf[kb] = *reinterpret_cast<const bf16x8*>(qr + 32 * kb);
        float ss = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = (float)qf[kb][e];
                ss += x * x;
            }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        if (gq == 0) {
            const float rq = 1.f / sqrtf(ss + kL2Eps);
            for (int qh = 0; qh < Gq; ++qh)
                ws_G[((size_t)slot * Hv + kh * Gq + qh) * kGRows * kC + 4 * kC + 16 * wave + c] = rq;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// chunk_scan_kernel: one workgroup of six waves per (sequence, v-head, 16-column slice of S).
//
// Per chunk s of the sequence (start state S_{s-1}, U_s = M_s X_s its deltas):
//     X_s = V_s - diag(e^G) K_s S_{s-1}
//     U_s = M_s X_s,   D_s = diag(e^(G_C - G)) U_s
//     S_s = e^(G_C) S_{s-1} + K_s^T D_s
//     O_s = diag(e^G) Q_s S_{s-1} + P_s U_s
// Only X -> U -> D -> X is a true chain from chunk to chunk once the state is eliminated from it:
//     K_s S_{s-1} = e^(G_C,s-1) K_s S_{s-2} + N_s D_{s-1},     N_s = K_s K_{s-1}^T
// where K_s S_{s-2} is known a whole chunk earlier.  The roles:
//
//   chain wave (0)   per chunk: N_s D_{s-1}, X_s = Y_s - diag(e^G) N_s D_{s-1}, U_s = M_s X_s and
//                    D_s, with Y_s = V_s - diag(e^G) e^(G_C,s-1) K_s S_{s-2} from the state waves.
//                    64 x 16 quantities, four 16 x 16 fp32 accumulator tiles each; N and M from
//                    the solve kernel, loaded into registers a chunk ahead.
//   state waves (1, 4)  one per half of the keys (64 keys x 16 columns, four tiles): one chunk
//                    behind the chain, S <- e^(G_C) S + K^T D from the chain's U; then the half's
//                    part of Y for the next chunk (half 0 adds V), and S^T (hi + lo) in LDS for
//                    the output waves.
//   output waves (2, 3)  one chunk behind the chain: wave w' owns token tiles {w', 3 - w'} of
//                    O^T = S^T Q^T diag(e^G) + U^T P^T, P^T tiles = K Q^T masked and decayed in
//                    registers, Q from memory a chunk ahead.
//   staging wave (5) copies each chunk's K rows, V columns and gate block straight from memory into
//                    a five-chunk LDS ring (global_load_lds), three chunks ahead of the chain.
//
// L2 (q and k normalised to unit length, r = 1 / |k|, rq = 1 / |q| per token, from the solve's gate
// block): the kernel keeps the exact bf16 K and Q and applies the scales on the fp32 side.  The
// chain hands out diag(r) U in place of U, which is what the normalised keys' K^T D, N_s D_{s-1} and
// P U need; the e^G factors of Y and X take r_s; the output rows take rq.
//
// Waves w and w + 4 share a SIMD: the chain with state half 1, state half 0 with the staging
// wave; the output waves have one each.  The state waves run at a higher priority than the chain:
// on the shared SIMD the chain has the slack (measured), and the state half is the one the next
// chunk waits for.
//
// Every product's result stays in registers and feeds the next product as its B operand.  The
// chain's tiles (and the K S tiles of the state waves) use natural token rows: tiles 2j and 2j + 1
// then hand lane (g, c) tokens 32 j + 4 g + e (e < 4) and 32 j + 16 + 4 g + e - 4 (e >= 4), the
// column order of the N and M fragments.  The state tiles stand for keys in the order
//     rho(a, m) = 32 (a / 2) + 8 (m / 4) + 4 (a % 2) + m % 4      (row m = 4g + r of tile a),
// so that tiles 2j and 2j + 1 hand lane (g, c) the consecutive keys 32 j + 8 g .. + 7, matching
// K rows read as plain A fragments; K^T for the state update is read from the same K rows with
// ds_read_b64_tr_b16.
//
// One LDS barrier per chunk step.  Step s: the chain does chunk s, the state waves apply D_{s-1}
// and form chunk s + 1's Y, the output waves finish chunk s - 1, the staging wave starts chunk
// s + 3's copy and waits for chunk s + 2's.
constexpr int kScanThreads = 384;
constexpr int kWS = 16;          // state columns per workgroup
constexpr int kSP = kDK + 8;     // row pitch of the S^T copies [column][key]
constexpr int kRing = 5;         // chunks in the staging ring
// K ring rows: pitch kKR elements (320 bytes, 20 sixteen-byte chunks, the last 4 unused), and the
// 16-byte chunk q of row t stored at chunk q ^ ((t >> 2) & 3).  With 64 four-byte banks, both ways
// the rows are read then touch 16 different chunk positions per 16 lanes: a row fragment (16
// rows, one chunk each) and a transposed fragment (4 consecutive rows x 4 consecutive chunks).
constexpr int kKR = 160;
constexpr int kKDma = kC * kKR * 2 / 1024;   // 1 KiB copy instructions per K slot (20)
// copy instructions per chunk: K, V (2 KiB), gate block (768 bytes; with L2 1 KiB + 256 bytes)
constexpr int kDmaOps = kKDma + 2 + 1;
// L2 prefetch: kPfAhead chunks ahead of the step that issues it, every line a workgroup group
// reads for a chunk (Q and K rows, the N block; per v-head the M block, V rows and gate block) is
// touched once, so that the chain's M and N loads and the output waves' Q loads (issued one step
// before use) and the staging copies (two steps) meet L2 rather than HBM.
constexpr int kPfAhead = 4;
constexpr int kLinesQ = kC * kDK * 2 / 128;                  // also K's
constexpr int kLinesN = kNFrags * kFragElems * 2 / 128;
constexpr int kLinesM = kMFrags * kFragElems * 2 / 128;
constexpr int kLinesG = kGRows * kC * 4 / 128;
__host__ __device__ constexpr int kswz(int t) { return (t >> 2) & 3; }

struct ScanLds {
    __bf16 Kr[kRing][kC * kKR];                // K rows [token][key]
    __bf16 Vr[kRing][kC * kWS];                // V [token][this slice's 16 columns]
    float Gt[kRing][kGRows * kC];              // gate block: G2, 2^G2, 2^(G2_C - G2), (r, rq)
    __bf16 St[2][2][kWS * kSP];                // S^T at chunk start [buffer][hi, lo]
    f32x4 Ut[2][4][64];                        // U [buffer][token tile][lane], the chain's tiles
    f32x4 Yt[2][2][4][64];                     // Y in two parts [buffer][key half][tile][lane]
    uint32_t sink[64];                         // landing row of the L2 prefetches (never read)
};
static_assert(sizeof(ScanLds) <= 160 * 1024, "scan LDS exceeds a CU's 160 KiB");

// index (token or key) that accumulator row m of tile a stands for
__device__ __forceinline__ int rho(int a, int m) {
    return 32 * (a >> 1) + 8 * (m >> 2) + 4 * (a & 1) + (m & 3);
}

// K^T fragment for the state update: lane (g, c) receives K[32 kb + 4 g + e][rho(kt, c)] (e < 4)
// and K[32 kb + 16 + 4 g + e - 4][rho(kt, c)] (e >= 4): keys in the state tiles' row order, tokens
// as in the chain's D fragments.  Each half is a transposed read of row 32 kb + 4 g (+ 16) + c / 4
// at logical chunk 4 (kt / 2) + c % 4, half kt % 2 of the chunk; `k0` holds the ring slot plus the
// lane's part of the address (the chunk swizzle of those rows is g).
__device__ __forceinline__ bf16x8 kt_frag(lds_u8* k0, int kt, int kb) {
    const int off = 2 * (32 * kb * kKR + 32 * (kt >> 1) + 4 * (kt & 1));
    return cat44(read_tr(k0, off), read_tr(k0, off + 2 * 16 * kKR));
}

typedef __attribute__((address_space(1))) void glb_void;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16 bytes per lane from global memory straight into LDS: lane l writes dst + 16 l
__device__ __forceinline__ void copy_to_lds(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)dst, 16, 0, 0);
}

struct OutIn {                     // one chunk's Q fragments for an output wave (registers)
    bf16x8 q[2][4];                // Q rows 16 a + c of its two tiles, columns 32 kb + 8 g ..
};

template <int DV, bool L2>
__global__ __launch_bounds__(kScanThreads) void chunk_scan_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* initial_state, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ state_indices, int num_slots,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ order, int N, int T,
    int Hk, int Hv, int nct, int max_slots, const float* __restrict__ ws_G,
    const __bf16* __restrict__ ws_M, const __bf16* __restrict__ ws_N, float* __restrict__ o,
    float* final_state) {
    constexpr int NS = DV / kWS;  // slices per v-head
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    ScanLds& sm = *reinterpret_cast<ScanLds*>(smem_raw);

    // blockIdx -> (group, member): a group is one (sequence, q/k head); its members are the
    // (v-head, slice) workgroups that read the same q and k.  All members of a group share
    // blockIdx % 8, hence one XCD and its L2.
    const int Gq = Hv / Hk, MB = Gq * NS;
    const int bid = blockIdx.x;
    const int xr = bid >> 3;
    const int member = xr % MB;
    const int grp = (xr / MB) * 8 + (bid & 7);
    if (grp >= N * Hk) return;
    const int rank = grp / Hk, kh = grp % Hk;
    const int h = kh * Gq + member / NS;
    const int c0 = (member % NS) * kWS;
    const int n = order ? order[rank] : rank;
    int row, t0, t1;
    sequence_range(cu_seqlens, n, T, row, t0, t1);
    const int slot0 = cu_seqlens ? chunk_start[n] : n * nct;
    // (a malformed cu_seqlens can claim more chunks than the workspace holds: stop at its end)
    const int nchunks = min((t1 - t0 + kC - 1) / kC, max(0, max_slots - slot0));
    // the sequence's state: its own, or a pool slot (a padding row starts from zero, writes none)
    int sslot;
    const bool has_slot = state_slot(state_indices, num_slots, n, sslot);
    const float* s_in = has_slot ? initial_state : nullptr;
    float* s_out = has_slot ? final_state : nullptr;
    const size_t sbase = ((size_t)sslot * Hv + h) * kDK * DV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;

    auto tok0_of = [&](int ci) { return (size_t)row * T + t0 + (size_t)ci * kC; };
    auto len_of = [&](int ci) { return min(kC, t1 - t0 - ci * kC); };

    if (wave == 0) {
        // ------------------------------------------------ chain wave --------------------------
        if (nchunks == 0) return;
        __builtin_amdgcn_s_setprio(1);
        bf16x8 mf[kMFrags];              // M_s fragments, refilled with M_{s+1}'s once used
        bf16x8 nf[kNFrags];              // N_s fragments, likewise
        auto fetch_m = [&](int ci) {
            const __bf16* b = ws_M + ((size_t)(slot0 + ci) * Hv + h) * kMFrags * kFragElems + 8 * lane;
#pragma unroll
            for (int f = 0; f < kMFrags; ++f) mf[f] = *reinterpret_cast<const bf16x8*>(b + f * kFragElems);
        };
        auto fetch_n = [&](int ci) {
            const __bf16* b = ws_N + ((size_t)(slot0 + ci) * Hk + kh) * kNFrags * kFragElems + 8 * lane;
#pragma unroll
            for (int f = 0; f < kNFrags; ++f) nf[f] = *reinterpret_cast<const bf16x8*>(b + f * kFragElems);
        };
        f32x4 u[4];                      // U of the previous chunk
        fetch_m(0);
        if (nchunks > 1) fetch_n(1);
        lds_barrier();  // P: chunks 0 and 1 staged
        lds_barrier();  // B0: Y_0 ready
        auto step = [&](int s, auto first) {
            constexpr bool kFirst = decltype(first)::value;
            const float* gt = sm.Gt[s % kRing];
            lds_u8* yl = lds_at(&sm.Yt[s & 1][0][0][lane]);
            lds_u8* gl = lds_at(gt + kC + 4 * g);                    // 2^G2 at rows 16 a + 4 g + r
            f32x4 y[4], eg[4], rk[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                y[a] = ld<f32x4>(yl, 16 * 64 * a) + ld<f32x4>(yl, 16 * 64 * (4 + a));
                eg[a] = ld<f32x4>(gl, 4 * 16 * a);
                if constexpr (L2) {
                    rk[a] = ld<f32x4>(gl, 4 * 16 * a + 4 * 2 * kC);                     // r_s
                    eg[a] *= rk[a];
                }
            }
            f32x4 x[4];
            if constexpr (kFirst) {
#pragma unroll
                for (int a = 0; a < 4; ++a) x[a] = y[a];
            } else {
                // D_{s-1} = diag(e^(G_C - G)) U_{s-1} as hi + lo B fragments
                lds_u8* dl_ = lds_at(sm.Gt[(s - 1) % kRing] + 2 * kC + 4 * g);
                f32x4 ds[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) ds[a] = u[a] * ld<f32x4>(dl_, 4 * 16 * a);
                bf16x8 dh[2], dlo[2];
                split8(ds[0], ds[1], dh[0], dlo[0]);
                split8(ds[2], ds[3], dh[1], dlo[1]);
                // N_s D_{s-1}
                f32x4 nd[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    nd[a] = zero4();
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        nd[a] = mma(nf[2 * (2 * a + j)], dh[j], nd[a]);
                        nd[a] = mma(nf[2 * (2 * a + j)], dlo[j], nd[a]);
                        nd[a] = mma(nf[2 * (2 * a + j) + 1], dh[j], nd[a]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                fetch_n(min(s + 1, nchunks - 1));   // unconditional: see fetch_m
#pragma unroll
                for (int a = 0; a < 4; ++a) x[a] = y[a] - eg[a] * nd[a];
            }
            bf16x8 xh[2], xl[2];
            split8(x[0], x[1], xh[0], xl[0]);
            split8(x[2], x[3], xh[1], xl[1]);
            // U = M X (M lower triangular: pairs (a, j) with 2 j <= a)
#pragma unroll
            for (int a = 0; a < 4; ++a) u[a] = zero4();
#pragma unroll
            for (int p = 0; p < 6; ++p) {
                const int a = m_pair_row(p), j = m_pair_step(p);
                u[a] = mma(mf[2 * p], xh[j], u[a]);
                u[a] = mma(mf[2 * p], xl[j], u[a]);
                u[a] = mma(mf[2 * p + 1], xh[j], u[a]);
            }
            if constexpr (L2) {
#pragma unroll
                for (int a = 0; a < 4; ++a) u[a] *= rk[a];         // diag(r) U
            }
            __builtin_amdgcn_sched_barrier(0);
            // unconditional (the last chunk refetches itself): a conditional fetch makes the
            // compiler's wait before the next use also wait for every load issued after it
            fetch_m(min(s + 1, nchunks - 1));
            lds_u8* ul = lds_at(&sm.Ut[s & 1][0][lane]);
#pragma unroll
            for (int a = 0; a < 4; ++a) st(ul, 16 * 64 * a, u[a]);
            lds_barrier();
        };
        step(0, std::true_type{});
        for (int s = 1; s < nchunks; ++s) step(s, std::false_type{});
        lds_barrier();  // the other roles' last step
    } else if (wave == 1 || wave == 4) {
        // ------------------------------------------------ state waves -------------------------
        auto state_role = [&](auto hc) {
            constexpr int hh = decltype(hc)::value;   // key half: state tiles 4 hh .. 4 hh + 3
            auto state_idx = [&](int t, int r) {
                return sbase + (size_t)rho(4 * hh + t, 4 * g + r) * DV + c0 + c;
            };
            if (nchunks == 0) {  // zero-length sequence: the state passes through
                if (s_out) {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            s_out[state_idx(t, r)] = s_in ? s_in[state_idx(t, r)] : 0.f;
                }
                return;
            }
            __builtin_amdgcn_s_setprio(2);
            f32x4 S[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[t][r] = s_in ? s_in[state_idx(t, r)] : 0.f;
            // lane parts of the LDS addresses (the rest are compile-time offsets)
            const int l_kf = c * kKR + 8 * (g ^ kswz(c));                 // K row c, logical chunk g
            const int l_kt = (4 * g + (c >> 2)) * kKR + 8 * ((c & 3) ^ g);
            const int l_v = (4 * g + (c >> 2)) * kWS + 4 * (c & 3);
            const int l_st = c * kSP + 8 * g;
            bf16x8 sh[2], sl[2];             // this half of S as hi + lo B fragments
                                             // (keys 32 (2 hh + u) + 8 g + e)
            auto split_s = [&]() {
#pragma unroll
                for (int u = 0; u < 2; ++u) split8(S[2 * u], S[2 * u + 1], sh[u], sl[u]);
            };
            // this half's part of Y for chunk ci: -diag(e^G) e^(G_C, ci - 1) K S over its keys,
            // plus V in half 0 (ec = that decay factor)
            auto make_y = [&](int ci, float ec) {
                const int slot = ci % kRing;
                lds_u8* kfl = lds_at(sm.Kr[slot] + l_kf);
                lds_u8* gl = lds_at(sm.Gt[slot] + kC + 4 * g);
                f32x4 ks[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    bf16x8 kf[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) kf[u] = ld<bf16x8>(kfl, 2 * (16 * a * kKR + 32 * (2 * hh + u)));
                    ks[a] = zero4();
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        ks[a] = mma(kf[u], sh[u], ks[a]);
                        ks[a] = mma(kf[u], sl[u], ks[a]);
                    }
                }
                lds_u8* yl = lds_at(&sm.Yt[ci & 1][hh][0][lane]);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f32x4 eg = ld<f32x4>(gl, 4 * 16 * a) * ec;
                    if constexpr (L2) eg *= ld<f32x4>(gl, 4 * 16 * a + 4 * 2 * kC);      // r_s
                    f32x4 y;
                    if constexpr (hh == 0) {
                        lds_u8* vl = lds_at(sm.Vr[slot] + l_v);
                        const bf16x4 vv = read_tr(vl, 2 * 16 * a * kWS);        // V[16 a + 4 g + r][c]
#pragma unroll
                        for (int r = 0; r < 4; ++r) y[r] = (float)vv[r] - eg[r] * ks[a][r];
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) y[r] = -eg[r] * ks[a][r];
                    }
                    st(yl, 16 * 64 * a, y);
                }
            };
            lds_barrier();  // P: chunks 0 and 1 staged
            split_s();
            make_y(0, 1.f);
            lds_barrier();  // B0
            for (int s = 0; s <= nchunks; ++s) {
                if (s >= 1) {
                    // S <- e^(G_C) S + K^T D with chunk s - 1's D, from the chain's U
                    const int ps = (s - 1) % kRing;
                    const float* gp = sm.Gt[ps];
                    const float ec = gp[2 * kC - 1];
                    lds_u8* ul = lds_at(&sm.Ut[(s - 1) & 1][0][lane]);
                    lds_u8* dl_ = lds_at(gp + 2 * kC + 4 * g);
                    f32x4 ds[4];
#pragma unroll
                    for (int a = 0; a < 4; ++a) ds[a] = ld<f32x4>(ul, 16 * 64 * a) * ld<f32x4>(dl_, 4 * 16 * a);
                    bf16x8 dh[2], dlo[2];
                    split8(ds[0], ds[1], dh[0], dlo[0]);
                    split8(ds[2], ds[3], dh[1], dlo[1]);
                    lds_u8* ktl = lds_at(sm.Kr[ps] + l_kt);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        bf16x8 kt[2];
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) kt[kb] = kt_frag(ktl, 4 * hh + t, kb);
                        f32x4 acc = S[t] * ec;
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            acc = mma(kt[kb], dh[kb], acc);
                            acc = mma(kt[kb], dlo[kb], acc);
                        }
                        S[t] = acc;
                    }
                }
                if (s < nchunks) {
                    // S_{s-1} (chunk s's start state) for the output waves, and chunk s + 1's Y
                    split_s();
                    lds_u8* stb = lds_at(sm.St[s & 1][0] + l_st);
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        st(stb, 2 * 32 * (2 * hh + u), sh[u]);
                        st(stb, 2 * (kWS * kSP + 32 * (2 * hh + u)), sl[u]);
                    }
                    if (s + 1 < nchunks) make_y(s + 1, sm.Gt[s % kRing][2 * kC - 1]);
                }
                lds_barrier();
            }
            if (s_out) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) s_out[state_idx(t, r)] = S[t][r];
            }
        };
        if (wave == 1) state_role(std::integral_constant<int, 0>{});
        else state_role(std::integral_constant<int, 1>{});
    } else if (wave < 4) {
        // ------------------------------------------------ output waves ------------------------
        if (nchunks == 0) return;
        auto run = [&](auto oc) {
            constexpr int ow = decltype(oc)::value;      // 0: tiles {0, 3}; 1: tiles {1, 2}
            constexpr int tiles[2] = {ow, 3 - ow};
            const int l_kf = c * kKR + 8 * (g ^ kswz(c));                 // K row c, logical chunk g
            const int l_st = c * kSP + 8 * g;
            auto fetch_out = [&](OutIn& f, int ci) {
                const size_t tok0 = tok0_of(ci);
                const int L = len_of(ci);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    // rows past a partial chunk's end repeat its last row: their outputs are never
                    // stored, and they enter no other row's output
                    const int t = min(16 * tiles[x] + c, L - 1);
                    const __bf16* qr = q + ((tok0 + t) * Hk + kh) * kDK + 8 * g;
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) f.q[x][kb] = *reinterpret_cast<const bf16x8*>(qr + 32 * kb);
                }
            };
            auto step = [&](int s, const OutIn& cur, OutIn& nxt) {
                fetch_out(nxt, min(s, nchunks - 1));             // chunk s's Q rows, for the next step
                const int ci = s - 1;                            // the chunk finished in this step
                const int slot = ci % kRing;
                const __bf16* kr = sm.Kr[slot];
                const float* gt = sm.Gt[slot];
                const int buf = ci & 1;
                // S^T (hi, lo), U^T (hi, lo) and the gate values of this wave's rows
                lds_u8* kfl = lds_at(kr + l_kf);
                lds_u8* gl = lds_at(gt + 4 * g);
                float gq[2], eq[2], rq[2];
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    gq[x] = gt[16 * tiles[x] + c];
                    eq[x] = gt[kC + 16 * tiles[x] + c];
                    if constexpr (L2) rq[x] = gt[4 * kC + 16 * tiles[x] + c];
                }
                bf16x8 sf[2][4], uf[2][2];
#pragma unroll
                for (int hl = 0; hl < 2; ++hl) {
                    lds_u8* sp = lds_at(sm.St[buf][hl] + l_st);
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) sf[hl][kb] = ld<bf16x8>(sp, 2 * 32 * kb);
                }
                // U^T fragments: lane (g, c) of the chain's tiles 2 kb, 2 kb + 1 holds U at
                // tokens 32 kb + 4 g + r and 32 kb + 16 + 4 g + r, column c: the P^T row order
                lds_u8* ul = lds_at(&sm.Ut[buf][0][lane]);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    split8(ld<f32x4>(ul, 16 * 64 * (2 * kb)), ld<f32x4>(ul, 16 * 64 * (2 * kb + 1)), uf[0][kb],
                           uf[1][kb]);
                f32x4 ot[2];
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int a = tiles[x];
                    const int t = 16 * a + c;
                    // P^T tiles (b, a) = K Q^T for b <= a: rows t' = 16 b + m, masked to t' <= t
                    bf16x8 kf[4][4];
#pragma unroll
                    for (int b = 0; b <= a; ++b)
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) kf[b][kb] = ld<bf16x8>(kfl, 2 * (16 * b * kKR + 32 * kb));
                    f32x4 pt[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        pt[b] = zero4();
                        if (b > a) continue;
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) pt[b] = mma(kf[b][kb], cur.q[x][kb], pt[b]);
                        const f32x4 gp = ld<f32x4>(gl, 4 * 16 * b);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int tp = 16 * b + 4 * g + r;
                            pt[b][r] = tp <= t ? pt[b][r] * exp2_fast(gq[x] - gp[r]) : 0.f;
                        }
                    }
                    // B fragments for P U: reduction rows 32 kb + 4 g + e (e < 4), + 16 (e >= 4)
                    bf16x8 ph[2], pl[2];
                    split8(pt[0], pt[1], ph[0], pl[0]);
                    split8(pt[2], pt[3], ph[1], pl[1]);
                    f32x4 qs = zero4(), qs2 = zero4();
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        qs = mma(sf[0][kb], cur.q[x][kb], qs);
                        qs2 = mma(sf[1][kb], cur.q[x][kb], qs2);
                    }
                    f32x4 acc = (qs + qs2) * eq[x];
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        if (2 * kb > a) continue;
                        acc = mma(uf[0][kb], ph[kb], acc);
                        acc = mma(uf[0][kb], pl[kb], acc);
                        acc = mma(uf[1][kb], ph[kb], acc);
                    }
                    if constexpr (L2) acc *= rq[x];
                    ot[x] = acc;
                }
                const size_t tok0 = tok0_of(ci);
                const int L = len_of(ci);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int t = 16 * tiles[x] + c;
                    if (t < L) *reinterpret_cast<f32x4*>(o + ((tok0 + t) * Hv + h) * DV + c0 + 4 * g) = ot[x];
                }
                lds_barrier();
            };
            OutIn fa, fb;
            fetch_out(fa, 0);
            lds_barrier();  // P
            lds_barrier();  // B0
            lds_barrier();  // step 0: nothing finishes yet
            int s = 1;
            for (; s + 1 <= nchunks; s += 2) {
                step(s, fa, fb);
                step(s + 1, fb, fa);
            }
            if (s <= nchunks) step(s, fa, fb);
        };
        if (wave == 2) run(std::integral_constant<int, 0>{});
        else run(std::integral_constant<int, 1>{});
    } else {
        // ------------------------------------------------ staging wave ------------------------
        if (nchunks == 0) return;
        // K piece of copy instruction ii: byte 1024 ii + 16 lane of the slot, i.e. row t, physical
        // chunk pc (pc >= 16 is row padding: any in-bounds source will do)
        int krow[kKDma], kcol[kKDma];
#pragma unroll
        for (int ii = 0; ii < kKDma; ++ii) {
            const int ob = 1024 * ii + 16 * lane;
            const int t = ob / (2 * kKR), pc = (ob % (2 * kKR)) / 16;
            krow[ii] = t;
            kcol[ii] = 8 * (pc < 16 ? (pc ^ kswz(t)) : 0);
        }
        auto dma = [&](int ci) {
            const int slot = ci % kRing;
            const size_t tok0 = tok0_of(ci);
            const int L = len_of(ci);
            const __bf16* kb = k + (tok0 * Hk + kh) * kDK;
#pragma unroll
            for (int ii = 0; ii < kKDma; ++ii)
                copy_to_lds(kb + (size_t)min(krow[ii], L - 1) * Hk * kDK + kcol[ii], sm.Kr[slot] + 512 * ii);
            const __bf16* vb = v + (tok0 * Hv + h) * DV + c0;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)          // rows 32 jj + lane / 2, columns 8 (lane % 2)
                copy_to_lds(vb + (size_t)min(32 * jj + (lane >> 1), L - 1) * Hv * DV + 8 * (lane & 1),
                            sm.Vr[slot] + 512 * jj);
            const float* gb = ws_G + ((size_t)(slot0 + ci) * Hv + h) * kGRows * kC;
            if constexpr (L2) {
                copy_to_lds(gb + 4 * lane, sm.Gt[slot]);                  // rows 0-3
                if (lane < 16) copy_to_lds(gb + 4 * kC + 4 * lane, sm.Gt[slot] + 4 * kC);   // row 4
            } else {
                copy_to_lds(gb + 4 * min(lane, 47), sm.Gt[slot]);         // rows 0-2
            }
        };
        // The group's lines of chunk cp, dealt out over its MB = Gq DV / 16 members: lane l of
        // member m touches lines m + MB (l + 64 i), i < kPf.  Line order: Q rows, K rows, N, then
        // per v-head of the group its M block, V rows and gate block.  Addresses are clamped into
        // the chunk (a repeated line costs an L2 hit), so every instruction is issued with all
        // lanes and the copy counts below stay exact.  Each instruction lands 64 dwords in sm.sink.
        constexpr int kRowLines = DV / 64;                     // 128-byte lines per V row
        constexpr int kLinesV = kC * kRowLines;
        constexpr int kPerHead = kLinesM + kLinesV + kLinesG;
        constexpr int kPf = DV == 64 ? 3 : 2;                  // covers Gq = 1, the widest share
        auto prefetch = [&](int cp) {
            const size_t tok0 = tok0_of(cp);
            const int L = len_of(cp);
            const int total = 2 * kLinesQ + kLinesN + Gq * kPerHead;
#pragma unroll
            for (int i = 0; i < kPf; ++i) {
                const int line = min(member + MB * (lane + 64 * i), total - 1);
                const void* src;
                if (line < 2 * kLinesQ) {
                    const __bf16* base = line < kLinesQ ? q : k;
                    const int ln = line % kLinesQ;
                    src = base + ((tok0 + min(ln >> 1, L - 1)) * Hk + kh) * kDK + 64 * (ln & 1);
                } else if (line < 2 * kLinesQ + kLinesN) {
                    src = ws_N + ((size_t)(slot0 + cp) * Hk + kh) * kNFrags * kFragElems +
                          64 * (line - 2 * kLinesQ);
                } else {
                    const int j = line - 2 * kLinesQ - kLinesN;
                    const int hv = kh * Gq + j / kPerHead, r = j % kPerHead;
                    if (r < kLinesM) {
                        src = ws_M + ((size_t)(slot0 + cp) * Hv + hv) * kMFrags * kFragElems + 64 * r;
                    } else if (r < kLinesM + kLinesV) {
                        const int rv = r - kLinesM;
                        src = v + ((tok0 + min(rv / kRowLines, L - 1)) * Hv + hv) * DV + 64 * (rv % kRowLines);
                    } else {
                        src = ws_G + ((size_t)(slot0 + cp) * Hv + hv) * kGRows * kC + 32 * (r - kLinesM - kLinesV);
                    }
                }
                __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)sm.sink, 4, 0, 0);
            }
        };
        dma(0);
        if (nchunks > 1) dma(1);
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();       // P: chunks 0 and 1 staged
        if (nchunks > 2) {
            dma(2);
            prefetch(min(kPfAhead - 1, nchunks - 1));
        }
        __builtin_amdgcn_s_barrier();       // B0
        for (int s = 0; s <= nchunks; ++s) {
            // chunk s + 3 goes into the slot chunk s - 2 left; chunk s + 2 must have landed before
            // the step ends.  Every chunk copy from chunk 2 on is followed by one prefetch, so the
            // copies of chunk s + 2 are older than the newest kDmaOps (+1) + 2 kPf instructions.
            if (s + 3 < nchunks) {
                dma(s + 3);
                prefetch(min(s + kPfAhead, nchunks - 1));
                wait_vmcnt<kDmaOps + (L2 ? 1 : 0) + 2 * kPf>();
            } else {
                wait_vmcnt<0>();
            }
            __builtin_amdgcn_s_barrier();
        }
    }
}

// ------------------------------------------------------------------------------------------------
// workspace layout (each region 256-byte aligned):
//   chunk_start [N+1] int32 | order [N] int32 | gates [slots][Hv][G2, 2^G2, 2^(G2_C - G2), r][64] f32
//   | M [slots][Hv][12 fragments] bf16 | N [slots][Hk][16 fragments] bf16
struct Layout {
    size_t chunk_start, order, G, M, Nm, total;
    int slots;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(int B, int T, int Hk, int Hv, int N) {
    Layout l;
    l.slots = (int)(((long long)B * T) / kC) + N;  // bounds B*ceil(T/64) and T/64 + N (packed)
    size_t off = 0;
    l.chunk_start = off; off = align256(off + sizeof(int32_t) * (size_t)(N + 1));
    l.order = off;       off = align256(off + sizeof(int32_t) * (size_t)N);
    l.G = off;           off = align256(off + sizeof(float) * (size_t)l.slots * Hv * kGRows * kC);
    l.M = off;           off = align256(off + 2 * (size_t)l.slots * Hv * kMFrags * kFragElems);
    l.Nm = off;          off = align256(off + 2 * (size_t)l.slots * Hk * kNFrags * kFragElems);
    l.total = off;
    return l;
}

template <int DV, typename TG, bool L2>
hipError_t launch_dv(const ChunkArgs& a, unsigned stages) {
    const Layout lay = layout(a.B, a.T, a.Hk, a.Hv, a.N);
    char* ws = static_cast<char*>(a.workspace);
    const bool packed = a.cu_seqlens != nullptr;
    const int nct = (a.T + kC - 1) / kC;
    const int slots = packed ? lay.slots : a.B * nct;
    const int32_t* chunk_start = packed ? reinterpret_cast<const int32_t*>(ws + lay.chunk_start) : nullptr;
    const int32_t* order = packed ? reinterpret_cast<const int32_t*>(ws + lay.order) : nullptr;
    float* ws_G = reinterpret_cast<float*>(ws + lay.G);
    __bf16* ws_M = reinterpret_cast<__bf16*>(ws + lay.M);
    __bf16* ws_N = reinterpret_cast<__bf16*>(ws + lay.Nm);
    hipError_t e;
    if ((stages & kStagePrepare) && packed) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, a.stream, a.cu_seqlens, a.N,
                           a.T, reinterpret_cast<int32_t*>(ws + lay.chunk_start),
                           reinterpret_cast<int32_t*>(ws + lay.order));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((stages & kStagePrepare) && slots > 0) {
        hipLaunchKernelGGL((chunk_solve_kernel<TG, L2>), dim3((unsigned)slots, (unsigned)a.Hk),
                           dim3(kThreads), 0, a.stream, static_cast<const __bf16*>(a.q),
                           static_cast<const __bf16*>(a.k),
                           static_cast<const TG*>(a.g), static_cast<const TG*>(a.beta), a.A_log,
                           a.dt_bias, a.cu_seqlens, chunk_start, a.N, a.T, a.Hk, a.Hv, nct, ws_G, ws_M,
                           ws_N);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (!(stages & kStageScan)) return hipSuccess;
    const auto kern = chunk_scan_kernel<DV, L2>;
    const size_t bytes = sizeof(ScanLds);
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes)) != hipSuccess)
        return e;
    const int groups = a.N * a.Hk;                        // (sequence, q/k head)
    const int members = (a.Hv / a.Hk) * (DV / kWS);
    const unsigned grid = (unsigned)(((groups + 7) / 8) * 8 * members);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kScanThreads), bytes,
                       a.stream, static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                       static_cast<const __bf16*>(a.v), a.initial_state, a.cu_seqlens,
                       a.state_indices, a.num_slots, chunk_start,
                       order, a.N, a.T, a.Hk, a.Hv, nct, packed ? lay.slots : a.B * nct, ws_G, ws_M,
                       ws_N, a.o, a.final_state);
    return hipGetLastError();
}

}  // namespace

bool chunk_mfma_supported(int dk, int dv, gdn_dtype qkv_dtype) {
    return qkv_dtype == GDN_BF16 && dk == kDK && (dv == 64 || dv == 128);
}

size_t chunk_mfma_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N) {
    (void)dk;
    (void)dv;
    return layout(B, T, Hk, Hv, N).total;
}

template <bool L2>
hipError_t launch_l2(const ChunkArgs& a, unsigned stages) {
    const bool g_bf16 = a.gate_dtype == GDN_BF16;
    if (a.dv == 128) return g_bf16 ? launch_dv<128, bf16_t, L2>(a, stages) : launch_dv<128, float, L2>(a, stages);
    return g_bf16 ? launch_dv<64, bf16_t, L2>(a, stages) : launch_dv<64, float, L2>(a, stages);
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, unsigned stages) {
    return a.qk_l2norm ? launch_l2<true>(a, stages) : launch_l2<false>(a, stages);
}

}  // namespace gdn
