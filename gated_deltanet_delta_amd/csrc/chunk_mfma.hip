// chunk_mfma.hip -- chunked gated delta rule on gfx950 matrix cores (bf16 inputs, dk = 64 or 128).
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
//                       fp16 into the workspace (6 KiB per chunk and v-head), the chunk's decay
//                       factors, and N = K K_prev^T (8 KiB per chunk and q/k head).
//   chunk_scan_kernel   one workgroup per (sequence, v-head, 16 columns of S), walking the chunks
//                       in order with chain, state and output waves (see there).  With M, the
//                       chunk's deltas are U = Ut - W S = M (V - diag(e^G) K S), so W and Ut are
//                       never formed; everything else comes from q, k, v on the fly.
//
// Precision: q, k, v enter the matrix cores as exact bf16 values.  S, U, P and the state update's D
// enter as two bf16 terms hi + lo (hi = bf16(x), lo = bf16(x - hi)), so their products carry ~16
// significant bits.  The chunk-to-chunk chain (N D and M X, see the scan kernel) runs on fp16
// operands (11 significant bits, 8x finer than one bf16 term): a single product per tile instead of
// three.  Their entries are bounded by the inputs' scale: |M| and |N| by the keys' norms (the
// normalised keys' N is stored for the L2 option), |X| and |D| by |v| and |S|; fp16 holds them
// while those stay below ~6e4 and keeps full relative precision above ~6e-5 (smaller entries keep
// an absolute precision of 6e-8).  Accumulation is fp32 everywhere; decay factors are applied on
// the fp32 side.
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
#include "mfma_frag.h"

namespace gdn {
namespace {

constexpr int kC = kChunk; // chunk length
constexpr int kGRows = 5;   // rows of a chunk's gate block (of kC floats each)
// Key dimension DK (64 or 128) is a template parameter of both kernels; KB = DK / 32 is the number of
// 32-key steps of one matrix-core product over the keys.
constexpr int kThreads = 256;
constexpr int kXcds = 8;     // XCDs of an MI355X; workgroup i runs on XCD i % 8

__device__ __forceinline__ f32x4 mma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }


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
        int row, a, b;
        sequence_range(cu_seqlens, n, T, row, a, b);
        return b - a;
    };
    int sum = 0;
    for (int n = n0; n < n1; ++n) sum += sequence_chunks(cu_seqlens, n, T);
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
        run += sequence_chunks(cu_seqlens, n, T);
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

// ------------------------------------------------------------------------------------------------
// Shared helpers.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------------------------------------
// Fragment layouts shared by the solve kernel (writer) and the scan kernel (reader).
//
// A "fragment" is the A operand of one v_mfma_f32_16x16x32 (bf16 or fp16) as the 64 lanes hold it: lane
// (g, c) has eight 16-bit values, 16 bytes; a fragment is stored as 64 x 16 = 1 KiB with lane l at
// byte 16 l, so that one wave loads it with one fully coalesced instruction.
//
// The B operands these fragments meet in the scan kernel are accumulator tiles fed straight back:
// tiles 2j and 2j + 1 with natural token rows hand lane (g, c) the tokens 32 j + 4 g + e (e < 4)
// and 32 j + 16 + 4 g + e - 4 (e >= 4).  Element e of an A fragment's lane (g, c) therefore holds
// column 32 j + colperm(g, e) of its row, colperm(g, e) = 4 g + (e & 3) + 16 (e >> 2).
//
//   M (per chunk and v-head): the nonzero pairs (row tile a, k-step j) of the lower-triangular
//     M = T diag(beta), in the order (0,0) (1,0) (2,0) (2,1) (3,0) (3,1), fp16: 6 fragments.  Lane
//     (g, c) of pair (a, j) holds row 16 a + c.
//   N (per chunk and q/k head, chunks with a predecessor in the same sequence only): N = K K_p^T,
//     rows the chunk's tokens, columns the previous chunk's, all pairs (a, j) in the order
//     (0,0) (0,1) (1,0) ... (3,1), fp16: 8 fragments.
constexpr int kFragElems = 512;  // 16-bit values per fragment
constexpr int kMFrags = 6;
constexpr int kNFrags = 8;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8 pack_f16(const f32x4& a, const f32x4& b) {
    return __builtin_convertvector((f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}, f16x8);
}
__device__ __forceinline__ f32x4 mma16(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__host__ __device__ constexpr int m_pair_row(int p) { return p < 2 ? p : (p < 4 ? 2 : 3); }
__host__ __device__ constexpr int m_pair_step(int p) { return (p == 3 || p == 5) ? 1 : 0; }
__device__ __forceinline__ int colperm(int g, int e) { return 4 * g + (e & 3) + 16 * (e >> 2); }

// ------------------------------------------------------------------------------------------------
// chunk_solve_kernel: one workgroup per (chunk slot, q/k head), for each of the head's v-heads.
//
// Writes, per (chunk, v-head), the chunk's gate block [5][64] floats: G2 = running sum of
// g log2(e), 2^G2, 2^(G2_C - G2) (G2_C = G2 at the chunk's last row; padding rows past the
// chunk's length have g = 0) and, with L2, the key and query scales r_t = 1 / |k_t| and
// rq_t = 1 / |q_t| (rows 3 and 4); and M = T diag(beta) as the 6 fp16 fragments described above (zero
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

// Stores that write through to memory (sc0 sc1) for the solve's outputs, which only the next kernel
// reads: they leave no dirty L2 lines for the write-back at the end of the kernel (measured: the
// prepare kernel 25.2 -> 23.5 us).
__device__ __forceinline__ void store_through(f16x8* p, const f16x8& v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_through(float* p, float v) {
    asm volatile("global_store_dword %0, %1, off sc0 sc1" : : "v"(p), "v"(v) : "memory");
}

// Orders one wave's shared-memory writes before its later reads of what other lanes wrote.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// (at most 128 registers per lane: four waves per SIMD, so a whole 4096-token prefill's chunk
// workgroups are resident at once)
template <int DK, typename TG, bool L2>
__global__ __launch_bounds__(kThreads, 4) void chunk_solve_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const TG* __restrict__ g,
    const TG* __restrict__ beta, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ chunk_start, int N, int T,
    int Hk, int Hv, int nct, float* __restrict__ ws_G, __bf16* __restrict__ ws_M,
    __bf16* __restrict__ ws_N, float* __restrict__ ws_X, int x_per_head) {
    // The chunk's K rows and the previous chunk's, staged once in the swizzled row layout of
    // mfma_frag.h (whole-row copies straight into shared memory) and read from there as matrix-core
    // fragments by all four waves; the blocks of A and T reuse the same space afterwards.
    // (head size 64 keeps its fragment loads from memory: a staged build failed its parity tests there
    // with non-finite final states, for a cause not found)
    constexpr bool kStageK = DK == 128;
    constexpr int kKBytes = kC * DK * 2;
    constexpr int kATBytes = 2 * 10 * 16 * kBP * 4;
    constexpr int kRawBytes = 2 * kKBytes > kATBytes ? 2 * kKBytes : kATBytes;
    __shared__ __attribute__((aligned(16))) unsigned char s_raw[kRawBytes];
    float (*sA)[16 * kBP] = reinterpret_cast<float (*)[16 * kBP]>(s_raw);                 // blocks (a, b), a > b, of A
    float (*sT)[16 * kBP] = reinterpret_cast<float (*)[16 * kBP]>(s_raw + kATBytes / 2);  // (a, b), a >= b, of T = (I + A)^-1
    __bf16* const sKc = reinterpret_cast<__bf16*>(s_raw);              // this chunk's K rows
    __bf16* const sKp = reinterpret_cast<__bf16*>(s_raw + kKBytes);    // the previous chunk's
    __shared__ float sB[kC];
    // per wave: the current v-head's G2 and beta, read by address in the tile loops (instead of by
    // cross-lane broadcasts)
    __shared__ __attribute__((aligned(16))) float sW[4][2][kC];

    constexpr int KB = DK / 32;
    // Workgroups go to the XCDs round robin by linear index.  The (chunk slot, q/k head) items are
    // dealt so that each XCD gets one contiguous run of them: a chunk and the next one, which reads
    // its keys again as its previous chunk's, then share an L2.
    const int nwg = gridDim.x * gridDim.y, lin = blockIdx.x + gridDim.x * blockIdx.y;
    const int xcd = lin % kXcds, per = nwg / kXcds, extra = nwg % kXcds;
    const int item = xcd * per + min(xcd, extra) + lin / kXcds;
    const int slot = item % gridDim.x, kh = item / gridDim.x;
    ChunkLoc loc;
    if (!locate_chunk(slot, cu_seqlens, chunk_start, N, T, nct, loc)) return;
    const int Gq = Hv / Hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, gq = lane >> 4;
    const size_t tok0 = (size_t)loc.row * T + loc.t0;
    const int L = loc.len;
    const bool has_prev = loc.ci > 0;   // the previous chunk (always a full one) is in this sequence

    // fused output norm: this chunk's exchange rows of the head's v-heads start out as -1, a value
    // no sum of squares takes, so that the scan can tell a published sum from a missing one
    if (ws_X) {
        float* xb = ws_X + ((size_t)slot * Hv + (size_t)kh * Gq) * x_per_head;
        for (int i = 4 * tid; i < Gq * x_per_head; i += 4 * kThreads)
            *reinterpret_cast<f32x4*>(xb + i) = f32x4{-1.f, -1.f, -1.f, -1.f};
    }

    // Stage K: each 1 KiB copy instruction writes four rows; lane l lands at byte 16 l of the copy,
    // row t, physical chunk p, and so fetches logical chunk p ^ kswz(t) of row t.  Rows past the
    // chunk's end repeat its last row: they only meet rows with beta = 0.
    {
        constexpr int kCopies = kKBytes / 1024;          // per chunk of K rows
        auto stage = [&](__bf16* dst, size_t row0, int rows, int j) {
            const int byte = j * 1024 + 16 * lane;
            const int t = byte / (2 * DK), pch = (byte % (2 * DK)) / 16;
            const __bf16* src = k + ((row0 + min(t, rows - 1)) * Hk + kh) * DK + 8 * (pch ^ kswz<DK>(t));
            __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(reinterpret_cast<unsigned char*>(dst) + j * 1024),
                                             16, 0, 0);
        };
        if constexpr (kStageK) {
            for (int j = wave; j < kCopies; j += 4) stage(sKc, tok0, L, j);
            if (has_prev)
                for (int j = wave; j < kCopies; j += 4) stage(sKp, tok0 - kC, kC, j);
            __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): this wave's copies have landed
            __syncthreads();                             // and every other wave's
        }
    }
    // K K^T as 16x16 tiles; wave w owns diagonal tile (w, w) and some below it: wave 0 (0,0) (1,0);
    // wave 1 (1,1) (2,1) (2,0); wave 2 (2,2) (3,2); wave 3 (3,3) (3,0) (3,1).  The K rows of the (at
    // most three) token tiles a wave needs are all read before the first product.
    auto kfrag = [&](int t, int kb) {
        if constexpr (kStageK) return *reinterpret_cast<const bf16x8*>(sKc + 16 * t * DK + kf_lane<DK>(c, gq, kb));
        const int r = min(16 * t + c, L - 1);
        return *reinterpret_cast<const bf16x8*>(k + ((tok0 + r) * Hk + kh) * DK + 32 * kb + 8 * gq);
    };
    // token tiles of the K rows: wave 0 {0, 1}, wave 1 {1, 2, 0}, wave 2 {2, 3}, wave 3 {3, 0, 1}
    const int tt0 = wave, tt1 = (wave + 1) & 3, tt2 = wave == 1 ? 0 : 1;
    bf16x8 k0[KB], k1[KB], k2[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        k0[kb] = kfrag(tt0, kb);
        k1[kb] = kfrag(tt1, kb);
    }
    if (wave & 1) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) k2[kb] = kfrag(tt2, kb);
    }
    // the previous chunk's K rows 16 b + c, b = 0..3, for N
    bf16x8 kp[4][KB];
    if (has_prev) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                kp[b][kb] = kStageK ? *reinterpret_cast<const bf16x8*>(sKp + 16 * b * DK + kf_lane<DK>(c, gq, kb))
                                    : *reinterpret_cast<const bf16x8*>(k + ((tok0 - kC + 16 * b + c) * Hk + kh) * DK
                                                                       + 32 * kb + 8 * gq);
    }
    // every wave holds its fragments before any writes the blocks of A and T over the staged rows
    if constexpr (kStageK) __syncthreads();
    auto kkt = [&](const bf16x8* ka, const bf16x8* kb_) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = mma(ka[kb], kb_[kb], acc);
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

    // L2: r_t = 1 / sqrt(|k_t|^2 + eps) for K rows held as matrix-core fragments (lane (g, c) holds 32
    // of row 16 t + c's keys; the sum over g leaves every lane with its row's r)
    auto rnorm = [&](const bf16x8* kf) {
        float ss = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = (float)kf[kb][e];
                ss += x * x;
            }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        return 1.f / sqrtf(ss + kL2Eps);
    };
    float r0 = 1.f;
    if constexpr (L2) {
        // K K^T -> diag(r) K K^T diag(r) tile by tile: a tile's column factor is the lane's own, its
        // row factors come from lanes 4 g + r.  Each wave writes r of its own tile `wave` to the gate
        // blocks of every v-head.
        r0 = rnorm(k0);
        const float r1 = rnorm(k1), r2 = (wave & 1) ? rnorm(k2) : 1.f;
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

    // N: wave w forms the tiles (b, w) of N^T = K_p K^T, whose lane (g, c) element r is
    // N[16 w + c][16 b + 4 g + r]; tiles 2j and 2j + 1 together are exactly fragment (w, j), stored as
    // single fp16 values.  With L2 it is the normalised keys' N: each entry times r of its row (the
    // lane's own r0) and r_p of its column (previous chunk's row 16 b + 4 g + r), so that its entries
    // stay within |N| <= 1 whatever the raw keys' scale.
    if (has_prev) {
        f32x4 nt[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            nt[b] = kkt(kp[b], k0);
            if constexpr (L2) {
                const float rp = rnorm(kp[b]);
#pragma unroll
                for (int r = 0; r < 4; ++r) nt[b][r] *= r0 * __shfl(rp, 4 * gq + r);
            }
        }
        __bf16* nb = ws_N + ((size_t)slot * Hk + kh) * kNFrags * kFragElems + 8 * lane;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            store_through(reinterpret_cast<f16x8*>(nb + (2 * wave + j) * kFragElems), pack_f16(nt[2 * j], nt[2 * j + 1]));
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
        const float G2 = wave_prefix_sum(gt);
        if (wave == 0) {
            const size_t ws_row = ((size_t)slot * Hv + h) * kGRows * kC;
            const float G2c = __shfl(G2, 63);
            store_through(ws_G + ws_row + lane, G2);
            store_through(ws_G + ws_row + kC + lane, exp2_fast(G2));
            store_through(ws_G + ws_row + 2 * kC + lane, exp2_fast(G2c - G2));
            sB[lane] = bt;
        }
        float* wG = sW[wave][0];
        float* wB = sW[wave][1];
        wG[lane] = G2;
        wB[lane] = bt;
        wave_lds_sync();
        // A = diag(beta) (K K^T o Gam), strictly lower, tile by tile
        auto atile = [&](int ta, int tb, f32x4 acc) {
            const f32x4 Gt = *reinterpret_cast<const f32x4*>(wG + 16 * ta + 4 * gq);
            const f32x4 Bt = *reinterpret_cast<const f32x4*>(wB + 16 * ta + 4 * gq);
            const float Gj = wG[16 * tb + c];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * ta + 4 * gq + r, j = 16 * tb + c;
                acc[r] = j < t ? Bt[r] * acc[r] * exp2_fast(Gt[r] - Gj) : 0.f;
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
        // the diagonal blocks A_ww (zero on and above the diagonal) go where T_ww will be
        {
            const f32x4 ad = atile(wave, wave, kd);
            float* Ad = sT[blk(wave, wave)];
#pragma unroll
            for (int r = 0; r < 4; ++r) Ad[(4 * gq + r) * kBP + c] = ad[r];
        }
        lds_barrier();
        // T_gg = (I + A_gg)^-1 for all four diagonal blocks in wave 0: lane (g, c) computes column c
        // of block g, in place
        if (wave == 0) {
            float* Tg = sT[blk(gq, gq)];
            float a[16], x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                a[t] = -Tg[t * kBP + c];
                x[t] = (t == c) ? 1.f : 0.f;
            }
            invert_blocks16(x, a);
#pragma unroll
            for (int t = 0; t < 16; ++t) Tg[t * kBP + c] = x[t];
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

        // M = T diag(beta) as its 6 fp16 fragments: item e = (pair p, lane ln) writes that lane's
        // eight values of the pair's fragment, one 1 KiB fragment per wave and pass
        __bf16* Mb = ws_M + ((size_t)slot * Hv + h) * kMFrags * kFragElems;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int e = tid + kThreads * it;
            if (e >= 6 * 64) break;
            const int p = e >> 6, ln = e & 63, lg = ln >> 4;
            const int t = 16 * m_pair_row(p) + (ln & 15), j0 = 32 * m_pair_step(p);
            f16x8 hv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = j0 + colperm(lg, j);
                const int ba = t >> 4, bb = col >> 4;
                const float tv = bb <= ba ? sT[blk(ba, bb)][(t & 15) * kBP + (col & 15)] : 0.f;
                hv[j] = (_Float16)(tv * sB[col]);
            }
            store_through(reinterpret_cast<f16x8*>(Mb + p * kFragElems + 8 * ln), hv);
        }
        lds_barrier();                 // sT and sB are rewritten for the next v-head
    }
    if constexpr (L2) {
        // rq_t = 1 / sqrt(|q_t|^2 + eps) for token tile `wave` (lane (g, c): 32 of row 16 wave + c's
        // keys), into every v-head's gate block; read last, when the solve's registers are free
        const int qrow = min(16 * wave + c, L - 1);
        const __bf16* qr = q + ((tok0 + qrow) * Hk + kh) * DK + 8 * gq;
        bf16x8 qf[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qf[kb] = *reinterpret_cast<const bf16x8*>(qr + 32 * kb);
        float ss = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
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
//                    64 x 16 quantities, four 16 x 16 fp32 accumulator tiles each, fed to fp16
//                    products; N and M (fp16) from the solve kernel, loaded into registers two
//                    chunks ahead (two buffers).
//   state waves (1, 4)  one per half of the keys (64 keys x 16 columns, four tiles): one chunk
//                    behind the chain, S <- e^(G_C) S + K^T D from the chain's U; then the half's
//                    part of Y for the next chunk (half 0 adds V), and S^T (hi + lo) in LDS for
//                    the output waves.
//   output waves (2, 3)  one chunk behind the chain: wave w' owns token tiles {w', 3 - w'} of
//                    O^T = S^T Q^T diag(e^G) + U^T P^T, P^T tiles = K Q^T masked and decayed in
//                    registers, Q from memory a chunk ahead.
//   staging wave (5) copies each chunk's K rows, V columns and gate block straight from memory into
//                    LDS rings (global_load_lds; five chunks of K and gates, three of V, whose
//                    rows are read a step before their chunk's), three chunks ahead of the chain;
//                    for a full chunk every lane's source is a fixed offset from one uniform base.
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
constexpr int kRing = 5;         // chunks in the staging ring (K rows, gate blocks)
constexpr int kVRing = 3;        // chunks of V in LDS (each is read in the step after it lands)
// Geometry that depends on the key dimension DK.
template <int DK>
struct Geom {
    static constexpr int KB = DK / 32;                  // 32-key steps of a product over the keys
    static constexpr int KR = DK;                       // K ring row pitch (elements)
    static constexpr int SP = DK + 8;                   // row pitch of the S^T copies [column][key]
    static constexpr int KDma = kC * KR * 2 / 1024;     // 1 KiB copy instructions per K slot (16, 8)
    static constexpr int DmaOps = KDma + 2 + 1;         // per chunk: K, V (2 KiB), gate block
    static constexpr int TPH = DK / 32;                 // 16-key state tiles per key half
    static constexpr int UPH = DK / 64;                 // 32-key blocks per key half
    static constexpr int LinesQ = kC * DK * 2 / 128;    // 128-byte lines of a chunk's Q (also K) rows
    static constexpr int RowLines = DK / 64;            // 128-byte lines per Q or K row
    static_assert(DK == 64 || DK == 128, "key dimension");
    static_assert(kC * KR * 2 % 1024 == 0, "K slot is a whole number of copy instructions");
};
// L2 prefetch: kPfAhead chunks ahead of the step that issues it, every line a workgroup group
// reads for a chunk (Q and K rows, the N block; per v-head the M block, V rows and gate block) is
// touched once, so that the chain's M and N loads and the output waves' Q loads (issued one step
// before use) and the staging copies (two steps) meet L2 rather than HBM.
constexpr int kPfAhead = 4;
constexpr int kLinesN = kNFrags * kFragElems * 2 / 128;
constexpr int kLinesM = kMFrags * kFragElems * 2 / 128;
constexpr int kLinesG = kGRows * kC * 4 / 128;
template <int DK>
struct ScanLds {
    __bf16 Kr[kRing][kC * Geom<DK>::KR];       // K rows [token][key]
    __bf16 Vr[kVRing][kC * kWS];               // V [token][this slice's 16 columns]
    float Gt[kRing][kGRows * kC];              // gate block: G2, 2^G2, 2^(G2_C - G2), (r, rq)
    __bf16 St[2][2][kWS * Geom<DK>::SP];       // S^T at chunk start [buffer][hi, lo]
    bf16x8 Us[2][2][2][64];                    // U as B fragments [buffer][32-token step][hi, lo][lane]
    bf16x8 Ds[2][2][2][64];                    // D = diag(e^(G_C - G)) U, likewise
    f32x4 Yt[2][2][4][64];                     // Y in two parts [buffer][key half][tile][lane]
    uint32_t sink[64];                         // landing row of the L2 prefetches (never read)
};
static_assert(sizeof(ScanLds<128>) <= 160 * 1024, "scan LDS exceeds a CU's 160 KiB");

// The gated output norm fused onto o, y = o / sqrt(mean(o^2) + eps) * weight * silu(z) per (token,
// v-head) row of DV channels.  A row's channels come from the NS = DV / 16 slice workgroups of its
// v-head.  The output waves hand each chunk's o tile to the two norm waves through a two-chunk LDS
// ring; a norm wave (32 rows, two lanes of 8 channels per row) keeps its rows in registers, publishes
// the row's 16 channels' sum of
// squares of every row into the exchange block of that chunk and v-head (device-scope stores over
// the solve kernel's -1 fill), and kNormLag steps later normalises, gates and stores its channels
// of y, with the other slices' sums and z loaded kNormAhead steps before.  A sum still at -1 when it
// is needed is waited for; every slice publishes each chunk kNormLag - kNormAhead steps before any
// slice loads it, so that only happens when one slice runs behind.
constexpr int kScanThreadsNorm = kScanThreads + 128;  // plus the norm waves (6, 7)
constexpr int kORing = 2;                             // chunks of o in LDS
constexpr int kNormLag = 4;                           // steps from publishing to normalising
constexpr int kNormAhead = 2;                         // steps from loading to normalising
constexpr int kNormSpin = 1 << 20;                    // polls of a missing sum before giving up
struct ScanNorm {
    const void* z;               // [rows of o] x DV, bf16 or fp32
    const float* weight;         // [DV]
    float eps;
    int z_bf16, y_bf16;
    float* xs;                   // [slots][Hv][NS][64] each slice's sum of squares of each row
    void* y;                     // [B, T, Hv, DV], bf16 or fp32
};
template <int DK>
constexpr size_t scan_lds_bytes(bool norm) {
    return sizeof(ScanLds<DK>) + (norm ? sizeof(float) * kORing * kC * kWS : 0);
}
static_assert(scan_lds_bytes<128>(true) <= 160 * 1024, "fused-norm scan LDS exceeds a CU's 160 KiB");


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

template <int KB>
struct OutIn {                     // one chunk's Q fragments for an output wave (registers)
    bf16x8 q[2][KB];               // Q rows 16 a + c of its two tiles, columns 32 kb + 8 g ..
};

template <int DK, int DV, bool L2, bool NORM>
__global__ __launch_bounds__(NORM ? kScanThreadsNorm : kScanThreads) void chunk_scan_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* initial_state, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ state_indices, int num_slots,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ order, int N, int T,
    int Hk, int Hv, int nct, int max_slots, const float* __restrict__ ws_G,
    const __bf16* __restrict__ ws_M, const __bf16* __restrict__ ws_N, float* __restrict__ o,
    float* final_state, ScanNorm nrm) {
    constexpr int NS = DV / kWS;  // slices per v-head
    using GM = Geom<DK>;
    constexpr int KB = GM::KB, KR = GM::KR, SP = GM::SP, TPH = GM::TPH, UPH = GM::UPH;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    ScanLds<DK>& sm = *reinterpret_cast<ScanLds<DK>*>(smem_raw);
    float* const o_ring = reinterpret_cast<float*>(smem_raw + sizeof(ScanLds<DK>));   // NORM: [kORing][kC][kWS]

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
    const size_t sbase = ((size_t)sslot * Hv + h) * DK * DV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;

    auto tok0_of = [&](int ci) { return (size_t)row * T + t0 + (size_t)ci * kC; };
    auto len_of = [&](int ci) { return min(kC, t1 - t0 - ci * kC); };

    if (wave == 0) {
        // ------------------------------------------------ chain wave --------------------------
        if (nchunks == 0) return;
        __builtin_amdgcn_s_setprio(1);
        // M and N fragments of two chunks in flight: buffer ci % 2 holds chunk ci's, refilled with
        // chunk ci + 2's as soon as the last product using them has issued
        f16x8 mf[2][kMFrags];
        f16x8 nf[2][kNFrags];
        auto fetch_m = [&](int ci, auto pc) {
            constexpr int par = decltype(pc)::value;
            const __bf16* b = ws_M + ((size_t)(slot0 + ci) * Hv + h) * kMFrags * kFragElems + 8 * lane;
#pragma unroll
            for (int f = 0; f < kMFrags; ++f) mf[par][f] = *reinterpret_cast<const f16x8*>(b + f * kFragElems);
        };
        auto fetch_n = [&](int ci, auto pc) {
            constexpr int par = decltype(pc)::value;
            const __bf16* b = ws_N + ((size_t)(slot0 + ci) * Hk + kh) * kNFrags * kFragElems + 8 * lane;
#pragma unroll
            for (int f = 0; f < kNFrags; ++f) nf[par][f] = *reinterpret_cast<const f16x8*>(b + f * kFragElems);
        };
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        f32x4 dprev[4];                  // D of the previous chunk, fp32
        fetch_m(0, P0{});
        fetch_m(min(1, nchunks - 1), P1{});
        fetch_n(min(1, nchunks - 1), P1{});
        fetch_n(min(2, nchunks - 1), P0{});
        lds_barrier();  // P: chunks 0 and 1 staged
        lds_barrier();  // B0: Y_0 ready
        auto step = [&](int s, auto first, auto pc) {
            constexpr bool kFirst = decltype(first)::value;
            constexpr int par = decltype(pc)::value;
            const float* gt = sm.Gt[s % kRing];
            lds_u8* yl = lds_at(&sm.Yt[s & 1][0][0][lane]);
            lds_u8* gl = lds_at(gt + kC + 4 * g);                    // 2^G2 at rows 16 a + 4 g + r
            f32x4 y[4], eg[4], rk[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                y[a] = ld<f32x4>(yl, 16 * 64 * a) + ld<f32x4>(yl, 16 * 64 * (4 + a));
                eg[a] = ld<f32x4>(gl, 4 * 16 * a);
                if constexpr (L2) rk[a] = ld<f32x4>(gl, 4 * 16 * a + 4 * 2 * kC);          // r_s
            }
            f32x4 x[4];
            if constexpr (kFirst) {
#pragma unroll
                for (int a = 0; a < 4; ++a) x[a] = y[a];
            } else {
                // D_{s-1} = diag(e^(G_C - G)) U_{s-1} (kept from the previous step) as fp16 B fragments
                const f16x8 d16[2] = {pack_f16(dprev[0], dprev[1]), pack_f16(dprev[2], dprev[3])};
                // N_s D_{s-1}
                f32x4 nd[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    nd[a] = zero4();
#pragma unroll
                    for (int j = 0; j < 2; ++j) nd[a] = mma16(nf[par][2 * a + j], d16[j], nd[a]);
                }
                __builtin_amdgcn_sched_barrier(0);
                fetch_n(min(s + 2, nchunks - 1), pc);   // unconditional: see fetch_m
#pragma unroll
                for (int a = 0; a < 4; ++a) x[a] = y[a] - eg[a] * nd[a];
            }
            const f16x8 x16[2] = {pack_f16(x[0], x[1]), pack_f16(x[2], x[3])};
            // U = M X (M lower triangular: pairs (a, j) with 2 j <= a)
            f32x4 u[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) u[a] = zero4();
#pragma unroll
            for (int p = 0; p < 6; ++p) {
                const int a = m_pair_row(p), j = m_pair_step(p);
                u[a] = mma16(mf[par][p], x16[j], u[a]);
            }

            // D_s for the next chunk's N D, and U_s, D_s as hi + lo B fragments for the state and
            // output waves (with L2 as diag(r) U and diag(r) D: the raw keys then act as normalised ones)
            lds_u8* dcl = lds_at(gt + 2 * kC + 4 * g);               // 2^(G2_C - G2) at rows 16 a + 4 g + r
#pragma unroll
            for (int a = 0; a < 4; ++a) dprev[a] = u[a] * ld<f32x4>(dcl, 4 * 16 * a);
            f32x4 ur[4], dr[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                ur[a] = u[a];
                dr[a] = dprev[a];
                if constexpr (L2) {
                    ur[a] *= rk[a];
                    dr[a] *= rk[a];
                }
            }
            lds_u8* dsl = lds_at(&sm.Ds[s & 1][0][0][lane]);
            lds_u8* usl = lds_at(&sm.Us[s & 1][0][0][lane]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                bf16x8 hi, lo;
                split8(dr[2 * j], dr[2 * j + 1], hi, lo);
                st(dsl, 16 * 64 * (2 * j), hi);
                st(dsl, 16 * 64 * (2 * j + 1), lo);
                split8(ur[2 * j], ur[2 * j + 1], hi, lo);
                st(usl, 16 * 64 * (2 * j), hi);
                st(usl, 16 * 64 * (2 * j + 1), lo);
            }
            __builtin_amdgcn_sched_barrier(0);
            // unconditional (the last chunk refetches itself): a conditional fetch makes the
            // compiler's wait before the next use also wait for every load issued after it
            fetch_m(min(s + 2, nchunks - 1), pc);
            lds_barrier();
        };
        step(0, std::true_type{}, P0{});
        int s = 1;
        for (; s + 1 < nchunks; s += 2) {
            step(s, std::false_type{}, P1{});
            step(s + 1, std::false_type{}, P0{});
        }
        if (s < nchunks) step(s, std::false_type{}, P1{});
        lds_barrier();  // the other roles' last step
    } else if (wave == 1 || wave == 4) {
        // ------------------------------------------------ state waves -------------------------
        auto state_role = [&](auto hc) {
            constexpr int hh = decltype(hc)::value;   // key half: state tiles TPH hh .. TPH hh + TPH - 1
            auto state_idx = [&](int t, int r) {
                return sbase + (size_t)rho(TPH * hh + t, 4 * g + r) * DV + c0 + c;
            };
            if (nchunks == 0) {  // zero-length sequence: the state passes through
                if (s_out) {
#pragma unroll
                    for (int t = 0; t < TPH; ++t)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            s_out[state_idx(t, r)] = s_in ? s_in[state_idx(t, r)] : 0.f;
                }
                return;
            }
            __builtin_amdgcn_s_setprio(2);
            f32x4 S[TPH];
#pragma unroll
            for (int t = 0; t < TPH; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[t][r] = s_in ? s_in[state_idx(t, r)] : 0.f;
            // lane parts of the LDS addresses (the rest are compile-time offsets)
            int l_kf[UPH], l_kt[UPH];        // this half's 32-key blocks (row fragments, K^T quads)
#pragma unroll
            for (int u = 0; u < UPH; ++u) {
                l_kf[u] = kf_lane<DK>(c, g, UPH * hh + u);
                l_kt[u] = kt_lane<DK>(c, g, UPH * hh + u);
            }
            const int l_v = (4 * g + (c >> 2)) * kWS + 4 * (c & 3);
            const int l_st = c * SP + 8 * g;
            bf16x8 sh[UPH], sl[UPH];         // this half of S as hi + lo B fragments
                                             // (keys 32 (UPH hh + u) + 8 g + e)
            auto split_s = [&]() {
#pragma unroll
                for (int u = 0; u < UPH; ++u) split8(S[2 * u], S[2 * u + 1], sh[u], sl[u]);
            };
            // this half's part of Y for chunk ci: -diag(e^G) e^(G_C, ci - 1) K S over its keys,
            // plus V in half 0 (ec = that decay factor)
            auto make_y = [&](int ci, float ec) {
                const int slot = ci % kRing, vslot = ci % kVRing;
                lds_u8* kfl[UPH];
#pragma unroll
                for (int u = 0; u < UPH; ++u) kfl[u] = lds_at(sm.Kr[slot] + l_kf[u]);
                lds_u8* gl = lds_at(sm.Gt[slot] + kC + 4 * g);
                f32x4 ks[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    bf16x8 kf[UPH];
#pragma unroll
                    for (int u = 0; u < UPH; ++u) kf[u] = ld<bf16x8>(kfl[u], 2 * 16 * a * KR);
                    ks[a] = zero4();
#pragma unroll
                    for (int u = 0; u < UPH; ++u) {
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
                        lds_u8* vl = lds_at(sm.Vr[vslot] + l_v);
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
                    lds_u8* dsl = lds_at(&sm.Ds[(s - 1) & 1][0][0][lane]);   // the chain's D, hi + lo
                    bf16x8 dh[2], dlo[2];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        dh[j] = ld<bf16x8>(dsl, 16 * 64 * (2 * j));
                        dlo[j] = ld<bf16x8>(dsl, 16 * 64 * (2 * j + 1));
                    }
                    lds_u8* ktl[UPH];
#pragma unroll
                    for (int u = 0; u < UPH; ++u) ktl[u] = lds_at(sm.Kr[ps] + l_kt[u]);
#pragma unroll
                    for (int t = 0; t < TPH; ++t) {
                        bf16x8 kt[2];
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) kt[kb] = kt_frag<KR>(ktl[t >> 1], t & 1, kb);
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
                    for (int u = 0; u < UPH; ++u) {
                        st(stb, 2 * 32 * (UPH * hh + u), sh[u]);
                        st(stb, 2 * (kWS * SP + 32 * (UPH * hh + u)), sl[u]);
                    }
                    if (s + 1 < nchunks) make_y(s + 1, sm.Gt[s % kRing][2 * kC - 1]);
                }
                lds_barrier();
            }
            if (s_out) {
#pragma unroll
                for (int t = 0; t < TPH; ++t)
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
            int l_kf[KB];                                  // K row c, logical chunk 4 kb + g
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) l_kf[kb] = kf_lane<DK>(c, g, kb);
            const int l_st = c * SP + 8 * g;
            auto fetch_out = [&](OutIn<KB>& f, int ci) {
                const size_t tok0 = tok0_of(ci);
                const int L = len_of(ci);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    // rows past a partial chunk's end repeat its last row: their outputs are never
                    // stored, and they enter no other row's output
                    const int t = min(16 * tiles[x] + c, L - 1);
                    const __bf16* qr = q + ((tok0 + t) * Hk + kh) * DK + 8 * g;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) f.q[x][kb] = *reinterpret_cast<const bf16x8*>(qr + 32 * kb);
                }
            };
            auto step = [&](int s, const OutIn<KB>& cur, OutIn<KB>& nxt) {
                fetch_out(nxt, min(s, nchunks - 1));             // chunk s's Q rows, for the next step
                const int ci = s - 1;                            // the chunk finished in this step
                const int slot = ci % kRing;
                const __bf16* kr = sm.Kr[slot];
                const float* gt = sm.Gt[slot];
                const int buf = ci & 1;
                // S^T (hi, lo), U^T (hi, lo) and the gate values of this wave's rows
                lds_u8* kfl[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) kfl[kb] = lds_at(kr + l_kf[kb]);
                lds_u8* gl = lds_at(gt + 4 * g);
                float gq[2], eq[2], rq[2];
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    gq[x] = gt[16 * tiles[x] + c];
                    eq[x] = gt[kC + 16 * tiles[x] + c];
                    if constexpr (L2) rq[x] = gt[4 * kC + 16 * tiles[x] + c];
                }
                bf16x8 sf[2][KB], uf[2][2];
#pragma unroll
                for (int hl = 0; hl < 2; ++hl) {
                    lds_u8* sp = lds_at(sm.St[buf][hl] + l_st);
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) sf[hl][kb] = ld<bf16x8>(sp, 2 * 32 * kb);
                }
                // U^T fragments (hi, lo, split by the chain): lane (g, c) of the chain's tiles 2 kb,
                // 2 kb + 1 holds U at tokens 32 kb + 4 g + r and 32 kb + 16 + 4 g + r, column c: the
                // P^T row order
                lds_u8* usl = lds_at(&sm.Us[buf][0][0][lane]);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    uf[0][kb] = ld<bf16x8>(usl, 16 * 64 * (2 * kb));
                    uf[1][kb] = ld<bf16x8>(usl, 16 * 64 * (2 * kb + 1));
                }
                f32x4 ot[2];
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int a = tiles[x];
                    const int t = 16 * a + c;
                    // P^T tiles (b, a) = K Q^T for b <= a: rows t' = 16 b + m, masked to t' <= t
                    bf16x8 kf[4][KB];
#pragma unroll
                    for (int b = 0; b <= a; ++b)
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) kf[b][kb] = ld<bf16x8>(kfl[kb], 2 * 16 * b * KR);
                    f32x4 pt[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        pt[b] = zero4();
                        if (b > a) continue;
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) pt[b] = mma(kf[b][kb], cur.q[x][kb], pt[b]);
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
                    for (int kb = 0; kb < KB; ++kb) {
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
                if constexpr (NORM) {      // to the norm wave's ring: row t, channels 4 g ..
                    lds_u8* orl = lds_at(o_ring + (ci % kORing) * kC * kWS + c * kWS + 4 * g);
#pragma unroll
                    for (int x = 0; x < 2; ++x) st(orl, 4 * 16 * tiles[x] * kWS, ot[x]);
                } else {
                    const size_t tok0 = tok0_of(ci);
                    const int L = len_of(ci);
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        const int t = 16 * tiles[x] + c;
                        if (t < L) *reinterpret_cast<f32x4*>(o + ((tok0 + t) * Hv + h) * DV + c0 + 4 * g) = ot[x];
                    }
                }
                lds_barrier();
            };
            OutIn<KB> fa, fb;
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
    } else if (wave >= 6) {
        // ------------------------------------------------ norm waves (fused output norm) ------
        if constexpr (NORM) {
            if (nchunks == 0) return;
            constexpr int kCh = kWS / 2;               // channels per lane
            const int slice = c0 / kWS;
            const int t = 32 * (wave - 6) + (lane >> 1);   // this lane's row: token t of the chunk
            const int ch = kCh * (lane & 1);               // and its channels ch .. ch + 7 of the slice
            float wv[kCh];
#pragma unroll
            for (int j = 0; j < kCh; ++j) wv[j] = nrm.weight[c0 + ch + j];
            // chunk ci's exchange block: [slice][row] (each slice's 64 sums one contiguous run)
            auto xblk = [&](int ci) { return nrm.xs + ((size_t)(slot0 + ci) * Hv + h) * NS * kC; };
            struct NIn {                               // one chunk's inputs, loaded kNormAhead steps ahead
                float sum[NS];                         // every slice's sum of squares of row t
                u32x4 z[2];                            // z at row t, the lane's channels (bf16: z[0])
            };
            auto load_sums = [&](NIn& f, int d) {
                float* xb = xblk(d) + t;
#pragma unroll
                for (int e = 0; e < NS; ++e)
                    f.sum[e] = __hip_atomic_load(xb + e * kC, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            };
            // the same instructions whatever the chunk and z's dtype (bf16 z loads its 16 bytes twice):
            // every load the compiler waits for then has the same number of later ones behind it
            auto fetch = [&](NIn& f, int d) {
                load_sums(f, d);
                const size_t row = ((tok0_of(d) + min(t, len_of(d) - 1)) * Hv + h) * DV + c0 + ch;
                const u32x4* zp = nrm.z_bf16
                                      ? reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(nrm.z) + row)
                                      : reinterpret_cast<const u32x4*>(static_cast<const float*>(nrm.z) + row);
                const int zhi = nrm.z_bf16 ? 0 : 1;
                f.z[0] = zp[0];
                f.z[1] = zp[zhi];
            };
            auto normalize = [&](NIn& f, const float* orow, int d) {
                if (t >= len_of(d)) return;            // rows past a partial chunk's end
                auto ready = [&]() {
                    bool r = true;
#pragma unroll
                    for (int e = 0; e < NS; ++e) r = r && !(f.sum[e] < 0.f);
                    return r;
                };
                bool ok = ready();
                for (int it = 0; !ok && it < kNormSpin; ++it) {    // a slice running behind
                    __builtin_amdgcn_s_sleep(2);
                    load_sums(f, d);
                    ok = ready();
                }
                float tot = 0.f;
#pragma unroll
                for (int e = 0; e < NS; ++e) tot += f.sum[e];
                // (a sum that never arrived leaves the row NaN rather than wrong)
                const float inv = ok ? 1.f / sqrtf(tot / DV + nrm.eps) : __builtin_nanf("");
                float yv[kCh];
#pragma unroll
                for (int j = 0; j < kCh; ++j) {
                    const unsigned zw = nrm.z_bf16 ? f.z[0][j >> 1] : f.z[j >> 2][j & 3];
                    const float zf = nrm.z_bf16 ? __uint_as_float((j & 1) ? (zw & 0xffff0000u) : (zw << 16))
                                                : __uint_as_float(zw);
                    yv[j] = orow[j] * inv * wv[j] * silu(zf);
                }
                const size_t row = ((tok0_of(d) + t) * Hv + h) * DV + c0 + ch;
                if (nrm.y_bf16) {
                    *reinterpret_cast<u32x4*>(static_cast<__bf16*>(nrm.y) + row) =
                        u32x4{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]), pack_bf16x2(yv[4], yv[5]),
                              pack_bf16x2(yv[6], yv[7])};
                } else {
                    f32x4* yp = reinterpret_cast<f32x4*>(static_cast<float*>(nrm.y) + row);
                    yp[0] = f32x4{yv[0], yv[1], yv[2], yv[3]};
                    yp[1] = f32x4{yv[4], yv[5], yv[6], yv[7]};
                }
            };
            // this lane's part of its row in the last kNormLag chunks (chunk p in orow[p % kNormLag])
            // and the loaded inputs of the next kNormAhead chunks to normalise (chunk d in
            // nin[d % kNormAhead])
            float orow[kNormLag][kCh];
            NIn nin[kNormAhead];
            // step s (the other roles' step s while they run): normalise chunk d = s - 2 - kNormLag,
            // take chunk s - 2's rows (they landed in step s - 1) into the slot d leaves and publish
            // their sums, load the inputs of chunk d + kNormAhead into the slot d leaves
            auto nstep = [&](int s, auto ic) {
                constexpr int i = decltype(ic)::value;              // s % kPeriod
                constexpr int os = ((i - 2) % kNormLag + kNormLag) % kNormLag;
                constexpr int ns = ((i - 2 - kNormLag) % kNormAhead + kNormAhead) % kNormAhead;
                const int d = s - 2 - kNormLag, p = s - 2;
                if (d >= 0 && d < nchunks) normalize(nin[ns], orow[os], d);
                if (p >= 0 && p < nchunks) {
                    lds_u8* orl = lds_at(o_ring + (p % kORing) * kC * kWS + t * kWS + ch);
                    float ss = 0.f;
#pragma unroll
                    for (int j4 = 0; j4 < 2; ++j4) {
                        const f32x4 x = ld<f32x4>(orl, 16 * j4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            orow[os][4 * j4 + e] = x[e];
                            ss += x[e] * x[e];
                        }
                    }
                    ss += __shfl_xor(ss, 1);                // the row's other 8 channels
                    // (both lanes of the row store the same value)
                    __hip_atomic_store(xblk(p) + slice * kC + t, ss, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                fetch(nin[ns], min(max(d + kNormAhead, 0), nchunks - 1));   // unconditional: see fetch
                if (s <= nchunks) lds_barrier();
            };
            lds_barrier();  // P
            lds_barrier();  // B0
            constexpr int kPeriod = 4;                // slot patterns repeat every kPeriod steps
            static_assert(kPeriod % kNormLag == 0 && kPeriod % kNormAhead == 0, "slot period");
            const int last = nchunks + 1 + kNormLag;  // the step that normalises the last chunk
            // (whole periods, up to kPeriod - 1 idle steps past `last`: every step of an iteration
            // then runs, so the loads the compiler waits for always have the same ones behind them)
            for (int s = 0; s <= last; s += kPeriod) {
                using std::integral_constant;
                nstep(s, integral_constant<int, 0>{});
                nstep(s + 1, integral_constant<int, 1>{});
                nstep(s + 2, integral_constant<int, 2>{});
                nstep(s + 3, integral_constant<int, 3>{});
            }
        }
    } else {
        // ------------------------------------------------ staging wave ------------------------
        if (nchunks == 0) return;
        // K piece of copy instruction ii: byte 1024 ii + 16 lane of the slot, i.e. row t, physical
        // chunk pc, which holds the row's logical chunk pc ^ kswz(t)
        constexpr int KDma = GM::KDma;
        int krow[KDma], kcol[KDma];
#pragma unroll
        for (int ii = 0; ii < KDma; ++ii) {
            const int ob = 1024 * ii + 16 * lane;
            const int t = ob / (2 * KR), pc = (ob % (2 * KR)) / 16;
            krow[ii] = t;
            kcol[ii] = 8 * (pc ^ kswz<DK>(t));
        }
        // byte offsets of each lane's pieces inside a full chunk (the same for every chunk)
        uint32_t koff[KDma], voff[2];
#pragma unroll
        for (int ii = 0; ii < KDma; ++ii) koff[ii] = 2u * ((uint32_t)krow[ii] * Hk * DK + kcol[ii]);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) voff[jj] = 2u * ((uint32_t)(32 * jj + (lane >> 1)) * Hv * DV + 8 * (lane & 1));
        auto dma = [&](int ci) {
            const int slot = ci % kRing, vslot = ci % kVRing;
            const size_t tok0 = tok0_of(ci);
            const int L = len_of(ci);
            const __bf16* kb = k + (tok0 * Hk + kh) * DK;
            const __bf16* vb = v + (tok0 * Hv + h) * DV + c0;
            if (L == kC) {      // full chunk: uniform base plus the lane's fixed offset
                const char* kbc = reinterpret_cast<const char*>(kb);
                const char* vbc = reinterpret_cast<const char*>(vb);
#pragma unroll
                for (int ii = 0; ii < KDma; ++ii) copy_to_lds(kbc + koff[ii], sm.Kr[slot] + 512 * ii);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) copy_to_lds(vbc + voff[jj], sm.Vr[vslot] + 512 * jj);
            } else {
#pragma unroll
                for (int ii = 0; ii < KDma; ++ii)
                    copy_to_lds(kb + (size_t)min(krow[ii], L - 1) * Hk * DK + kcol[ii], sm.Kr[slot] + 512 * ii);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)          // rows 32 jj + lane / 2, columns 8 (lane % 2)
                    copy_to_lds(vb + (size_t)min(32 * jj + (lane >> 1), L - 1) * Hv * DV + 8 * (lane & 1),
                                sm.Vr[vslot] + 512 * jj);
            }
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
        constexpr int kLinesQ = GM::LinesQ, kQRow = GM::RowLines;
        // per lane and prefetch instruction: the line's address in chunk 0 and its stride per chunk
        const char* pf0[kPf];
        uint32_t pfstride[kPf];
        {
            const int total = 2 * kLinesQ + kLinesN + Gq * kPerHead;
            const size_t tok0 = tok0_of(0);
#pragma unroll
            for (int i = 0; i < kPf; ++i) {
                const int line = min(member + MB * (lane + 64 * i), total - 1);
                const void* src;
                uint32_t stride;
                if (line < 2 * kLinesQ) {
                    const __bf16* base = line < kLinesQ ? q : k;
                    const int ln = line % kLinesQ;
                    src = base + ((tok0 + ln / kQRow) * Hk + kh) * DK + 64 * (ln % kQRow);
                    stride = 2u * kC * Hk * DK;
                } else if (line < 2 * kLinesQ + kLinesN) {
                    src = ws_N + ((size_t)slot0 * Hk + kh) * kNFrags * kFragElems + 64 * (line - 2 * kLinesQ);
                    stride = 2u * Hk * kNFrags * kFragElems;
                } else {
                    const int j = line - 2 * kLinesQ - kLinesN;
                    const int hv = kh * Gq + j / kPerHead, r = j % kPerHead;
                    if (r < kLinesM) {
                        src = ws_M + ((size_t)slot0 * Hv + hv) * kMFrags * kFragElems + 64 * r;
                        stride = 2u * Hv * kMFrags * kFragElems;
                    } else if (r < kLinesM + kLinesV) {
                        const int rv = r - kLinesM;
                        src = v + ((tok0 + rv / kRowLines) * Hv + hv) * DV + 64 * (rv % kRowLines);
                        stride = 2u * kC * Hv * DV;
                    } else {
                        src = ws_G + ((size_t)slot0 * Hv + hv) * kGRows * kC + 32 * (r - kLinesM - kLinesV);
                        stride = 4u * Hv * kGRows * kC;
                    }
                }
                pf0[i] = static_cast<const char*>(src);
                pfstride[i] = stride;
            }
        }
        auto prefetch = [&](int cp) {
            const size_t tok0 = tok0_of(cp);
            const int L = len_of(cp);
            const int total = 2 * kLinesQ + kLinesN + Gq * kPerHead;
            if (L == kC) {     // full chunk: no clamping of rows
#pragma unroll
                for (int i = 0; i < kPf; ++i)
                    __builtin_amdgcn_global_load_lds((glb_void*)(pf0[i] + (size_t)cp * pfstride[i]), (lds_void*)sm.sink,
                                                     4, 0, 0);
                return;
            }
#pragma unroll
            for (int i = 0; i < kPf; ++i) {
                const int line = min(member + MB * (lane + 64 * i), total - 1);
                const void* src;
                if (line < 2 * kLinesQ) {
                    const __bf16* base = line < kLinesQ ? q : k;
                    const int ln = line % kLinesQ;
                    src = base + ((tok0 + min(ln / kQRow, L - 1)) * Hk + kh) * DK + 64 * (ln % kQRow);
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
            // copies of chunk s + 2 are older than the newest DmaOps (+1) + 2 kPf instructions.
            if (s + 3 < nchunks) {
                dma(s + 3);
                prefetch(min(s + kPfAhead, nchunks - 1));
                wait_vmcnt<GM::DmaOps + (L2 ? 1 : 0) + 2 * kPf>();
            } else {
                wait_vmcnt<0>();
            }
            __builtin_amdgcn_s_barrier();
        }
    }
}

// ------------------------------------------------------------------------------------------------
// workspace layout (each region 256-byte aligned):
//   chunk_start [N+1] int32 | order [N] int32 | gates [slots][Hv][kGRows][64] f32
//   | M [slots][Hv][6 fragments] fp16 | N [slots][Hk][8 fragments] fp16
//   | with the fused norm: sums of squares [slots][Hv][dv / 16][64] f32
struct Layout {
    size_t chunk_start, order, G, M, Nm, X, total;
    int slots;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(int B, int T, int Hk, int Hv, int N, int dv = 0, bool norm = false) {
    Layout l;
    l.slots = (int)(((long long)B * T) / kC) + N;  // bounds B*ceil(T/64) and T/64 + N (packed)
    size_t off = 0;
    l.chunk_start = off; off = align256(off + sizeof(int32_t) * (size_t)(N + 1));
    l.order = off;       off = align256(off + sizeof(int32_t) * (size_t)N);
    l.G = off;           off = align256(off + sizeof(float) * (size_t)l.slots * Hv * kGRows * kC);
    l.M = off;           off = align256(off + 2 * (size_t)l.slots * Hv * kMFrags * kFragElems);
    l.Nm = off;          off = align256(off + 2 * (size_t)l.slots * Hk * kNFrags * kFragElems);
    l.X = off;           off = norm ? align256(off + sizeof(float) * (size_t)l.slots * Hv * kC * (dv / kWS)) : off;
    l.total = off;
    return l;
}

template <int DK, int DV, typename TG, bool L2>
hipError_t launch_dv(const ChunkArgs& a, unsigned stages) {
    const bool norm = a.z != nullptr;
    const Layout lay = layout(a.B, a.T, a.Hk, a.Hv, a.N, DV, norm);
    char* ws = static_cast<char*>(a.workspace);
    const bool packed = a.cu_seqlens != nullptr;
    const int nct = (a.T + kC - 1) / kC;
    const int slots = packed ? lay.slots : a.B * nct;
    const int32_t* chunk_start = packed ? reinterpret_cast<const int32_t*>(ws + lay.chunk_start) : nullptr;
    const int32_t* order = packed ? reinterpret_cast<const int32_t*>(ws + lay.order) : nullptr;
    float* ws_G = reinterpret_cast<float*>(ws + lay.G);
    __bf16* ws_M = reinterpret_cast<__bf16*>(ws + lay.M);
    __bf16* ws_N = reinterpret_cast<__bf16*>(ws + lay.Nm);
    float* ws_X = norm ? reinterpret_cast<float*>(ws + lay.X) : nullptr;
    hipError_t e;
    if ((stages & kStagePrepare) && packed) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, a.stream, a.cu_seqlens, a.N,
                           a.T, reinterpret_cast<int32_t*>(ws + lay.chunk_start),
                           reinterpret_cast<int32_t*>(ws + lay.order));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((stages & kStagePrepare) && slots > 0) {
        hipLaunchKernelGGL((chunk_solve_kernel<DK, TG, L2>), dim3((unsigned)slots, (unsigned)a.Hk),
                           dim3(kThreads), 0, a.stream, static_cast<const __bf16*>(a.q),
                           static_cast<const __bf16*>(a.k),
                           static_cast<const TG*>(a.g), static_cast<const TG*>(a.beta), a.A_log,
                           a.dt_bias, a.cu_seqlens, chunk_start, a.N, a.T, a.Hk, a.Hv, nct, ws_G, ws_M,
                           ws_N, ws_X, kC * (DV / kWS));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (!(stages & kStageScan)) return hipSuccess;
    const auto kern = norm ? chunk_scan_kernel<DK, DV, L2, true> : chunk_scan_kernel<DK, DV, L2, false>;
    const size_t bytes = scan_lds_bytes<DK>(norm);
    const ScanNorm nrm{a.z, a.norm_weight, a.eps, a.z_dtype == GDN_BF16, a.y_dtype == GDN_BF16, ws_X, a.y};
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes)) != hipSuccess)
        return e;
    const int groups = a.N * a.Hk;                        // (sequence, q/k head)
    const int members = (a.Hv / a.Hk) * (DV / kWS);
    const unsigned grid = (unsigned)(((groups + 7) / 8) * 8 * members);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(norm ? kScanThreadsNorm : kScanThreads), bytes,
                       a.stream, static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                       static_cast<const __bf16*>(a.v), a.initial_state, a.cu_seqlens,
                       a.state_indices, a.num_slots, chunk_start,
                       order, a.N, a.T, a.Hk, a.Hv, nct, packed ? lay.slots : a.B * nct, ws_G, ws_M,
                       ws_N, a.o, a.final_state, nrm);
    return hipGetLastError();
}

}  // namespace

bool chunk_mfma_supported(int dk, int dv, gdn_dtype qkv_dtype) {
    return qkv_dtype == GDN_BF16 && (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

size_t chunk_mfma_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int N, bool norm) {
    (void)dk;
    return layout(B, T, Hk, Hv, N, dv, norm).total;
}

template <int DK, bool L2>
hipError_t launch_dk(const ChunkArgs& a, unsigned stages) {
    const bool g_bf16 = a.gate_dtype == GDN_BF16;
    if (a.dv == 128)
        return g_bf16 ? launch_dv<DK, 128, bf16_t, L2>(a, stages) : launch_dv<DK, 128, float, L2>(a, stages);
    return g_bf16 ? launch_dv<DK, 64, bf16_t, L2>(a, stages) : launch_dv<DK, 64, float, L2>(a, stages);
}

template <bool L2>
hipError_t launch_l2(const ChunkArgs& a, unsigned stages) {
    return a.dk == 128 ? launch_dk<128, L2>(a, stages) : launch_dk<64, L2>(a, stages);
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, unsigned stages) {
    return a.qk_l2norm ? launch_l2<true>(a, stages) : launch_l2<false>(a, stages);
}

}  // namespace gdn
