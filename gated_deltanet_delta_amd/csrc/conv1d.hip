// conv1d.hip -- depthwise causal convolution over time with a carried input cache (the conv that
// the QKV mixture passes through before the gated delta rule, and its conv_states on decode).
//
// Per sequence n and channel c, with xp = [cache_n; x_n] (the W - 1 inputs before the sequence,
// oldest first, then the sequence's own):
//     y[t, c] = act(sum_j w[c, j] xp[t + j, c] + bias[c])
// and the cache becomes the last W - 1 rows of xp.
//
// Memory-bound.  A thread owns 4 consecutive channels and a block of kConvTok tokens of the
// (packed) token stream; it keeps the last W inputs of its channels in registers, so every input
// is read once (plus W - 1 rows of halo per block), and every load and store of a wave covers 256
// consecutive channels.  Sequences may start and end inside a block: the window restarts from the
// sequence's cache at each start.
//
// The caches are rewritten by a second launch, one thread per (sequence, 4 channels): a sequence
// longer than a block is read near its start by one block and ends in another, so a rewrite from
// the first launch could overtake the read.

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvTok = 64;       // tokens per thread

typedef float f32x4c __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4c __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4c cload(const float* p) { return *reinterpret_cast<const f32x4c*>(p); }
__device__ __forceinline__ f32x4c cload(const bf16_t* p) {
    const u16x4c b = *reinterpret_cast<const u16x4c*>(p);
    return f32x4c{__uint_as_float(unsigned(b[0]) << 16), __uint_as_float(unsigned(b[1]) << 16),
                  __uint_as_float(unsigned(b[2]) << 16), __uint_as_float(unsigned(b[3]) << 16)};
}
__device__ __forceinline__ unsigned short to_bf16c(float f) {
    const unsigned u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40);
    return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ void cstore(float* p, const f32x4c& y) { *reinterpret_cast<f32x4c*>(p) = y; }
__device__ __forceinline__ void cstore(bf16_t* p, const f32x4c& y) {
    *reinterpret_cast<u16x4c*>(p) = u16x4c{to_bf16c(y[0]), to_bf16c(y[1]), to_bf16c(y[2]), to_bf16c(y[3])};
}

template <int W, typename TX>
__global__ __launch_bounds__(kConvThreads) void causal_conv1d_kernel(
    const TX* __restrict__ x, const float* __restrict__ weight, const float* __restrict__ bias,
    TX* conv_state, const int32_t* __restrict__ state_indices, int num_slots,
    const int32_t* __restrict__ cu_seqlens, int N, int T, long long total, int C, int silu,
    TX* __restrict__ y) {
    const int c0 = 4 * (blockIdx.x * kConvThreads + threadIdx.x);
    if (c0 >= C) return;
    const long long tb0 = (long long)blockIdx.y * kConvTok;
    const long long tb1 = tb0 + kConvTok < total ? tb0 + kConvTok : total;

    // the taps (w[c][j] multiplies the input j - W + 1 steps back) and the bias of these channels
    f32x4c wr[W];
#pragma unroll
    for (int j = 0; j < W; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[j][i] = weight[(size_t)(c0 + i) * W + j];
    f32x4c bv = bias ? cload(bias + c0) : f32x4c{0.f, 0.f, 0.f, 0.f};

    // sequence n holding token t: its range [s0, s1) of the token stream
    int n;
    long long s0, s1;
    auto find_seq = [&](long long t) {
        if (cu_seqlens) {
            int lo = 0, hi = N;                           // largest n with cu[n] <= t
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (cu_seqlens[mid] <= t) lo = mid; else hi = mid;
            }
            n = lo;
            int row, a, b;
            sequence_range(cu_seqlens, n, (int)total, row, a, b);
            while (b <= t && n + 1 < N) {                 // (skip empty sequences at the same start)
                ++n;
                sequence_range(cu_seqlens, n, (int)total, row, a, b);
            }
            s0 = a;
            s1 = b;
        } else {
            n = (int)(t / T);
            s0 = (long long)n * T;
            s1 = s0 + T;
        }
    };
    // the cache rows of sequence n (null: no cache, zeros in and nothing written)
    auto cache_of = [&](int seq) -> TX* {
        if (!conv_state) return nullptr;
        int slot;
        if (!state_slot(state_indices, num_slots, seq, slot)) return nullptr;
        return conv_state + (size_t)slot * (W - 1) * C;
    };

    f32x4c win[W];                                       // win[j]: input W - 1 - j steps back
    auto input_at = [&](long long row, const TX* cache) -> f32x4c {
        if (row >= s0) return cload(x + (size_t)row * C + c0);
        const long long k = row - s0 + (W - 1);          // row of the cache, 0 = oldest
        // (k < 0 only for a malformed, decreasing cu_seqlens: read nothing outside the cache)
        return cache && k >= 0 ? cload(cache + (size_t)k * C + c0) : f32x4c{0.f, 0.f, 0.f, 0.f};
    };
    find_seq(tb0);
    TX* cache = cache_of(n);
#pragma unroll
    for (int j = 0; j < W - 1; ++j) win[j] = input_at(tb0 - (W - 1) + j, cache);

    for (long long t = tb0; t < tb1; ++t) {
        if (t >= s1) {                                   // a new sequence starts here
            find_seq(t);
            cache = cache_of(n);
#pragma unroll
            for (int j = 0; j < W - 1; ++j) win[j] = input_at(t - (W - 1) + j, cache);
        }
        win[W - 1] = cload(x + (size_t)t * C + c0);
        f32x4c acc = bv;
#pragma unroll
        for (int j = 0; j < W; ++j) acc += wr[j] * win[j];
        if (silu) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = acc[i] / (1.f + expf(-acc[i]));
        }
        cstore(y + (size_t)t * C + c0, acc);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) win[j] = win[j + 1];
    }
}

// The new cache of sequence n: the last W - 1 rows of [cache_n; x_n], all read before any is written.
template <int W, typename TX>
__global__ __launch_bounds__(kConvThreads) void conv_cache_kernel(
    const TX* __restrict__ x, TX* conv_state, const int32_t* __restrict__ state_indices,
    int num_slots, const int32_t* __restrict__ cu_seqlens, int T, long long total, int C) {
    const int c0 = 4 * (blockIdx.x * kConvThreads + threadIdx.x);
    const int n = blockIdx.y;
    if (c0 >= C) return;
    long long s0, s1;
    if (cu_seqlens) {
        int row, a, b;
        sequence_range(cu_seqlens, n, (int)total, row, a, b);
        s0 = a;
        s1 = b;
    } else {
        s0 = (long long)n * T;
        s1 = s0 + T;
    }
    const long long len = s1 - s0;
    int slot;
    if (len == 0 || !state_slot(state_indices, num_slots, n, slot)) return;
    TX* cache = conv_state + (size_t)slot * (W - 1) * C;
    f32x4c v[W > 1 ? W - 1 : 1];                         // (never launched for W == 1)
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const long long r = len + j;                     // row of [cache; x], 0 = oldest cache row
        v[j] = r < W - 1 ? cload(cache + (size_t)r * C + c0)
                         : cload(x + (size_t)(s0 + r - (W - 1)) * C + c0);
    }
#pragma unroll
    for (int j = 0; j < W - 1; ++j) cstore(cache + (size_t)j * C + c0, v[j]);
}

template <int W, typename TX>
hipError_t launch_conv_typed(const ConvArgs& a) {
    const long long total = a.cu_seqlens ? (long long)a.T : (long long)a.B * a.T;
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((a.C / 4 + kConvThreads - 1) / kConvThreads),
                    (unsigned)((total + kConvTok - 1) / kConvTok));
    hipLaunchKernelGGL((causal_conv1d_kernel<W, TX>), grid, dim3(kConvThreads), 0, a.stream,
                       static_cast<const TX*>(a.x), a.weight, a.bias, static_cast<TX*>(a.conv_state),
                       a.state_indices, a.num_slots, a.cu_seqlens, a.N, a.T, total, a.C, a.silu,
                       static_cast<TX*>(a.y));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || W == 1 || !a.conv_state) return e;
    const dim3 grid2((unsigned)((a.C / 4 + kConvThreads - 1) / kConvThreads), (unsigned)a.N);
    hipLaunchKernelGGL((conv_cache_kernel<W, TX>), grid2, dim3(kConvThreads), 0, a.stream,
                       static_cast<const TX*>(a.x), static_cast<TX*>(a.conv_state), a.state_indices,
                       a.num_slots, a.cu_seqlens, a.T, total, a.C);
    return hipGetLastError();
}

template <int W>
hipError_t launch_conv_w(const ConvArgs& a) {
    return a.x_dtype == GDN_BF16 ? launch_conv_typed<W, bf16_t>(a) : launch_conv_typed<W, float>(a);
}

}  // namespace

hipError_t launch_causal_conv1d(const ConvArgs& a) {
    switch (a.W) {
        case 1: return launch_conv_w<1>(a);
        case 2: return launch_conv_w<2>(a);
        case 3: return launch_conv_w<3>(a);
        case 4: return launch_conv_w<4>(a);
        case 5: return launch_conv_w<5>(a);
        case 6: return launch_conv_w<6>(a);
        case 7: return launch_conv_w<7>(a);
        case 8: return launch_conv_w<8>(a);
        case 9: return launch_conv_w<9>(a);
        case 10: return launch_conv_w<10>(a);
        case 11: return launch_conv_w<11>(a);
        case 12: return launch_conv_w<12>(a);
        case 13: return launch_conv_w<13>(a);
        case 14: return launch_conv_w<14>(a);
        case 15: return launch_conv_w<15>(a);
        default: return launch_conv_w<16>(a);
    }
}

}  // namespace gdn
