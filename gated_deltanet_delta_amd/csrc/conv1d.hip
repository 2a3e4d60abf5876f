// conv1d.hip -- depthwise causal convolution over time with a carried input cache (the conv that
// the QKV mixture passes through before the gated delta rule, and its conv_states on decode).
//
// Per sequence n and channel c, with xp = [cache_n; x_n] (the W - 1 inputs before the sequence,
// oldest first, then the sequence's own):
//     y[t, c] = act(sum_j w[c, j] xp[t + j, c] + bias[c])
// and the cache becomes the last W - 1 rows of xp.
//
// Memory-bound.  A thread owns 4 consecutive channels and a tile of TOK tokens of the (packed)
// token stream, so every input is read once (plus W - 1 rows of halo per tile), and every load and
// store of a wave covers 256 consecutive channels.  TOK is 8 for prefills (short tiles give the
// launch several rounds of waves, which overlap one another's loads, arithmetic and stores), 1 for
// decode-like calls (sequences of a token or a few).  A tile whose tokens and halo all lie inside one
// sequence (nearly every tile of a prefill) issues all its loads at once into registers and then
// computes; a tile that meets a sequence start walks its tokens one by one, keeping the last W
// inputs in registers and restarting the window from the sequence's cache at each start.
//
// Only a sequence's first W - 1 tokens read its old cache.  When they all lie in the tile that holds
// the sequence's start (nearly always), the thread that reads the old cache there also writes the
// new one: from its window registers at the last token if the whole sequence lies in the tile,
// otherwise right after the read, by copying the sequence's last W - 1 inputs.  When those tokens
// span two tiles, a rewrite by either could overtake the other's read: a second launch rewrites such
// caches, and is skipped when the host can see that no sequence needs it (equal-length sequences
// without cu_seqlens).

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kConvThreads = 256;
constexpr int kPrefillTok = 8;     // tokens per thread when sequences are long

typedef float f32x4c __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4c __attribute__((ext_vector_type(4)));

// 4-channel loads: raw (bf16 kept packed until used) and widened to fp32
__device__ __forceinline__ f32x4c rload(const float* p) { return *reinterpret_cast<const f32x4c*>(p); }
__device__ __forceinline__ u16x4c rload(const bf16_t* p) { return *reinterpret_cast<const u16x4c*>(p); }
__device__ __forceinline__ f32x4c widen(const f32x4c& v) { return v; }
__device__ __forceinline__ f32x4c widen(const u16x4c& b) {
    return f32x4c{__uint_as_float(unsigned(b[0]) << 16), __uint_as_float(unsigned(b[1]) << 16),
                  __uint_as_float(unsigned(b[2]) << 16), __uint_as_float(unsigned(b[3]) << 16)};
}
template <typename TX>
__device__ __forceinline__ f32x4c cload(const TX* p) { return widen(rload(p)); }

__device__ __forceinline__ unsigned short to_bf16c(float f) {
    const unsigned u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40);
    return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ void cstore(float* p, const f32x4c& y) { *reinterpret_cast<f32x4c*>(p) = y; }
__device__ __forceinline__ void cstore(bf16_t* p, const f32x4c& y) {
    *reinterpret_cast<u16x4c*>(p) = u16x4c{to_bf16c(y[0]), to_bf16c(y[1]), to_bf16c(y[2]), to_bf16c(y[3])};
}
// a cache row holds an input unchanged (same type, exact)
__device__ __forceinline__ void rstore(float* p, const f32x4c& v) { *reinterpret_cast<f32x4c*>(p) = v; }
__device__ __forceinline__ void rstore(bf16_t* p, const u16x4c& v) { *reinterpret_cast<u16x4c*>(p) = v; }

__device__ __forceinline__ f32x4c act(f32x4c a, int silu_on) {
    if (silu_on) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = silu(a[i]);
    }
    return a;
}

// Sequence n's token range [s0, s1) in the packed stream (clamped like sequence_range).
__device__ __forceinline__ void seq_bounds(const int32_t* cu_seqlens, int n, int T, long long total,
                                           long long& s0, long long& s1) {
    if (cu_seqlens) {
        int row, a, b;
        sequence_range(cu_seqlens, n, (int)total, row, a, b);
        s0 = a;
        s1 = b;
    } else {
        s0 = (long long)n * T;
        s1 = s0 + T;
    }
}

// Every token of sequence [s0, s1) that reads its cache (the first W - 1) lies in the tile of TOK
// tokens holding s0: one thread reads the old cache and may write the new one.
template <int TOK, int W>
__host__ __device__ __forceinline__ bool cache_in_one_tile(long long s0, long long s1) {
    const long long e = s1 < s0 + (W - 1) ? s1 : s0 + (W - 1);
    return s1 > s0 && s0 / TOK == (e - 1) / TOK;
}

// The new cache of sequence [s0, s1): the last W - 1 rows of [cache; x], all read before any is
// written (the oldest rows come from the cache itself when the sequence is shorter than W - 1).
template <int W, typename TX>
__device__ __forceinline__ void rewrite_cache(const TX* __restrict__ x, TX* cache, long long s0,
                                              long long s1, int C, int c0) {
    if constexpr (W > 1) {
        const long long len = s1 - s0;
        decltype(rload(x)) v[W - 1];
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const long long r = len + j;                 // row of [cache; x], 0 = oldest cache row
            v[j] = r < W - 1 ? rload(cache + (size_t)r * C + c0) : rload(x + (size_t)(s0 + r - (W - 1)) * C + c0);
        }
#pragma unroll
        for (int j = 0; j < W - 1; ++j) rstore(cache + (size_t)j * C + c0, v[j]);
    }
}

template <int W, int TOK, typename TX>
__global__ __launch_bounds__(kConvThreads) void causal_conv1d_kernel(
    const TX* __restrict__ x, const float* __restrict__ weight, const float* __restrict__ bias,
    TX* conv_state, const int32_t* __restrict__ state_indices, int num_slots,
    const int32_t* __restrict__ cu_seqlens, int N, int T, long long total, int C, int silu_on,
    TX* __restrict__ y) {
    using Raw = decltype(rload(x));
    const int c0 = 4 * (blockIdx.x * kConvThreads + threadIdx.x);
    if (c0 >= C) return;
    const long long tb0 = (long long)blockIdx.y * TOK;
    const long long tb1 = tb0 + TOK < total ? tb0 + TOK : total;

    // the taps (w[c][j] multiplies the input j - W + 1 steps back) and the bias of these channels
    f32x4c wr[W];
#pragma unroll
    for (int j = 0; j < W; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[j][i] = weight[(size_t)(c0 + i) * W + j];
    const f32x4c bv = bias ? cload(bias + c0) : f32x4c{0.f, 0.f, 0.f, 0.f};

    // sequence n holding token t, and its range [s0, s1)
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
            seq_bounds(cu_seqlens, n, T, total, s0, s1);
            while (s1 <= t && n + 1 < N) {                // (skip empty sequences at the same start)
                ++n;
                seq_bounds(cu_seqlens, n, T, total, s0, s1);
            }
        } else {
            n = (int)(t / T);
            seq_bounds(nullptr, n, T, total, s0, s1);
        }
    };
    find_seq(tb0);

    if (s0 <= tb0 - (W - 1) && tb0 + TOK <= s1) {
        // the whole window lies in this sequence's own rows: every load first, then the sums
        constexpr int R = TOK + W - 1;
        Raw r[R];
        const TX* xb = x + (size_t)(tb0 - (W - 1)) * C + c0;
#pragma unroll
        for (int j = 0; j < R; ++j) r[j] = rload(xb + (size_t)j * C);
        TX* yb = y + (size_t)tb0 * C + c0;
#pragma unroll
        for (int i = 0; i < TOK; ++i) {
            f32x4c acc = bv;
#pragma unroll
            for (int j = 0; j < W; ++j) acc += wr[j] * widen(r[i + j]);
            cstore(yb + (size_t)i * C, act(acc, silu_on));
        }
        return;
    }

    // the cache rows of sequence n (null: no cache, zeros in and nothing written)
    auto cache_of = [&](int seq) -> TX* {
        if (!conv_state) return nullptr;
        int slot;
        if (!state_slot(state_indices, num_slots, seq, slot)) return nullptr;
        return conv_state + (size_t)slot * (W - 1) * C;
    };
    Raw win[W];                                          // win[j]: input W - 1 - j steps back
    auto input_at = [&](long long row, const TX* cache) -> Raw {
        if (row >= s0) return rload(x + (size_t)row * C + c0);
        const long long k = row - s0 + (W - 1);          // row of the cache, 0 = oldest
        // (k < 0 only for a malformed, decreasing cu_seqlens: read nothing outside the cache)
        return cache && k >= 0 ? rload(cache + (size_t)k * C + c0) : Raw{0, 0, 0, 0};
    };
    TX* cache = cache_of(n);
#pragma unroll
    for (int j = 0; j < W - 1; ++j) win[j] = input_at(tb0 - (W - 1) + j, cache);
    // a sequence that starts here and runs past the tile: its cache is its last W - 1 inputs
    auto copy_tail = [&]() {
        if (cache && s0 / TOK != (s1 - 1) / TOK && cache_in_one_tile<TOK, W>(s0, s1)) {
            Raw v[W];
#pragma unroll
            for (int j = 0; j < W - 1; ++j) v[j] = rload(x + (size_t)(s1 - (W - 1) + j) * C + c0);
#pragma unroll
            for (int j = 0; j < W - 1; ++j) rstore(cache + (size_t)j * C + c0, v[j]);
        }
    };
    if (s0 == tb0) copy_tail();

    for (long long t = tb0; t < tb1; ++t) {
        if (t >= s1) {                                   // a new sequence starts here
            find_seq(t);
            cache = cache_of(n);
#pragma unroll
            for (int j = 0; j < W - 1; ++j) win[j] = input_at(t - (W - 1) + j, cache);
            if (s0 == t) copy_tail();
        }
        win[W - 1] = rload(x + (size_t)t * C + c0);
        f32x4c acc = bv;
#pragma unroll
        for (int j = 0; j < W; ++j) acc += wr[j] * widen(win[j]);
        cstore(y + (size_t)t * C + c0, act(acc, silu_on));
        if (t == s1 - 1 && cache && s0 / TOK == t / TOK) {
            // a sequence inside this tile ends: the window's last W - 1 rows are its new cache
#pragma unroll
            for (int j = 0; j < W - 1; ++j) rstore(cache + (size_t)j * C + c0, win[j + 1]);
        }
#pragma unroll
        for (int j = 0; j < W - 1; ++j) win[j] = win[j + 1];
    }
}

// The new cache of every sequence whose cache-reading tokens span two tiles.
template <int W, int TOK, typename TX>
__global__ __launch_bounds__(kConvThreads) void conv_cache_kernel(
    const TX* __restrict__ x, TX* conv_state, const int32_t* __restrict__ state_indices,
    int num_slots, const int32_t* __restrict__ cu_seqlens, int T, long long total, int C) {
    const int c0 = 4 * (blockIdx.x * kConvThreads + threadIdx.x);
    const int n = blockIdx.y;
    if (c0 >= C) return;
    long long s0, s1;
    seq_bounds(cu_seqlens, n, T, total, s0, s1);
    int slot;
    if (s1 == s0 || cache_in_one_tile<TOK, W>(s0, s1) || !state_slot(state_indices, num_slots, n, slot)) return;
    rewrite_cache<W>(x, conv_state + (size_t)slot * (W - 1) * C, s0, s1, C, c0);
}

template <int W, int TOK, typename TX>
hipError_t launch_conv_tok(const ConvArgs& a, long long total) {
    const unsigned cblocks = (unsigned)((a.C / 4 + kConvThreads - 1) / kConvThreads);
    const dim3 grid(cblocks, (unsigned)((total + TOK - 1) / TOK));
    hipLaunchKernelGGL((causal_conv1d_kernel<W, TOK, TX>), grid, dim3(kConvThreads), 0, a.stream,
                       static_cast<const TX*>(a.x), a.weight, a.bias, static_cast<TX*>(a.conv_state),
                       a.state_indices, a.num_slots, a.cu_seqlens, a.N, a.T, total, a.C, a.silu,
                       static_cast<TX*>(a.y));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || W == 1 || !a.conv_state) return e;
    if (!a.cu_seqlens) {                                 // equal lengths: the host can tell
        bool all_done = true;
        for (long long b = 0; b < a.B && all_done; ++b)
            all_done = cache_in_one_tile<TOK, W>(b * a.T, (b + 1) * a.T);
        if (all_done) return hipSuccess;
    }
    hipLaunchKernelGGL((conv_cache_kernel<W, TOK, TX>), dim3(cblocks, (unsigned)a.N), dim3(kConvThreads), 0,
                       a.stream, static_cast<const TX*>(a.x), static_cast<TX*>(a.conv_state),
                       a.state_indices, a.num_slots, a.cu_seqlens, a.T, total, a.C);
    return hipGetLastError();
}

template <int W, typename TX>
hipError_t launch_conv_typed(const ConvArgs& a) {
    const long long total = a.cu_seqlens ? (long long)a.T : (long long)a.B * a.T;
    if (total == 0) return hipSuccess;
    // sequences of a few tokens (decode steps, short packed requests): one token per thread, so the
    // sequences' loads proceed in parallel rather than one after another
    if (total < 8LL * a.N) return launch_conv_tok<W, 1, TX>(a, total);
    return launch_conv_tok<W, kPrefillTok, TX>(a, total);
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
