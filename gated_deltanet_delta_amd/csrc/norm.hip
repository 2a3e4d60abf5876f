// norm.hip -- the layer's gated output norm: y = x / sqrt(mean(x^2) + eps) * weight * silu(z) per
// row of D channels (one head vector of the gated delta rule's output, gated by the z branch).
//
// Memory-bound: per row it reads x (fp32) and z, writes y, and does a handful of flops per value.
// Each lane owns 4 consecutive channels (one 16-byte fp32 load of x, one load of z, one store of
// y), so D / 4 lanes cover a row and a wave covers 256 / D rows; the mean square is reduced with
// shuffles inside those lanes.

#include "common.h"
#include "launch.h"

namespace gdn {
namespace {

constexpr int kNormThreads = 256;

typedef float f32x4n __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4n load4(const float* p) { return *reinterpret_cast<const f32x4n*>(p); }
__device__ __forceinline__ f32x4n load4(const bf16_t* p) {
    const u16x4 b = *reinterpret_cast<const u16x4*>(p);
    return f32x4n{__uint_as_float(unsigned(b[0]) << 16), __uint_as_float(unsigned(b[1]) << 16),
                  __uint_as_float(unsigned(b[2]) << 16), __uint_as_float(unsigned(b[3]) << 16)};
}

// fp32 -> bf16, round to nearest even (NaN kept a quiet NaN)
__device__ __forceinline__ unsigned short to_bf16(float f) {
    const unsigned u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40);
    return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ void store4(float* p, const f32x4n& y) { *reinterpret_cast<f32x4n*>(p) = y; }
__device__ __forceinline__ void store4(bf16_t* p, const f32x4n& y) {
    *reinterpret_cast<u16x4*>(p) = u16x4{to_bf16(y[0]), to_bf16(y[1]), to_bf16(y[2]), to_bf16(y[3])};
}

template <int D, typename TZ, typename TO>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(
    const float* __restrict__ x, const TZ* __restrict__ z, const float* __restrict__ weight,
    float eps, long long rows, TO* __restrict__ out) {
    constexpr int LPR = D / 4;                      // lanes per row
    constexpr int RPB = kNormThreads / LPR;         // rows per workgroup
    const int tid = threadIdx.x;
    const int lr = tid % LPR, rr = tid / LPR;
    const long long row = (long long)blockIdx.x * RPB + rr;
    if (row >= rows) return;                        // (whole row groups leave together)
    const size_t base = (size_t)row * D + 4 * lr;
    const f32x4n xv = load4(x + base);
    const f32x4n zv = load4(z + base);
    const f32x4n wv = load4(weight + 4 * lr);
    float ss = xv[0] * xv[0] + xv[1] * xv[1] + xv[2] * xv[2] + xv[3] * xv[3];
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off);
    const float inv_rms = 1.f / sqrtf(ss / D + eps);
    f32x4n y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        y[i] = xv[i] * inv_rms * wv[i] * silu(zv[i]);
    }
    store4(out + base, y);
}

template <int D, typename TZ, typename TO>
hipError_t launch_norm_typed(const NormArgs& a) {
    constexpr int RPB = kNormThreads / (D / 4);
    const long long blocks = (a.rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((gated_rmsnorm_kernel<D, TZ, TO>), dim3((unsigned)blocks), dim3(kNormThreads), 0,
                       a.stream, a.x, static_cast<const TZ*>(a.z), a.weight, a.eps, a.rows,
                       static_cast<TO*>(a.out));
    return hipGetLastError();
}

template <int D>
hipError_t launch_norm_dims(const NormArgs& a) {
    const bool zb = a.z_dtype == GDN_BF16, ob = a.out_dtype == GDN_BF16;
    if (zb && ob) return launch_norm_typed<D, bf16_t, bf16_t>(a);
    if (zb) return launch_norm_typed<D, bf16_t, float>(a);
    if (ob) return launch_norm_typed<D, float, bf16_t>(a);
    return launch_norm_typed<D, float, float>(a);
}

}  // namespace

hipError_t launch_gated_rmsnorm(const NormArgs& a) {
    if (a.rows == 0) return hipSuccess;
    return a.d == 128 ? launch_norm_dims<128>(a) : launch_norm_dims<64>(a);
}

}  // namespace gdn
