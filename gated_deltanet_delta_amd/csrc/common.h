// common.h -- small device helpers shared by the libgdn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <utility>

#include "seqmath.h"

namespace gdn {

constexpr int kWave = 64;

// bf16 values travel as raw 16-bit patterns; widening to fp32 is exact (shift into the top half).
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x.bits) << 16); }

// Row/offset helpers with 64-bit arithmetic (packed sequences reach ~1e9 elements).
__device__ __forceinline__ size_t idx3(size_t a, size_t b, size_t B_, size_t c, size_t C_) {
    return (a * B_ + b) * C_ + c;
}

// Unit lower-triangular inverses of four 16 x 16 blocks at once, one block per row of 16 lanes:
// lane (g, c) holds in a[t] = -A_g[t][c] (zero for t <= c) and returns in x[t] = T_g[t][c],
// T_g = (I + A_g)^-1.  Column sweep: once x[j] is final it is subtracted from every later row, the
// row's A_g[t][j] broadcast from lane j of the row (DPP row_newbcast:j), 15 dependent steps.
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + J, 0xf, 0xf, true));
}
template <int J>
__device__ __forceinline__ void subst_step(float (&x)[16], const float (&a)[16]) {
#pragma unroll
    for (int t = J + 1; t < 16; ++t) x[t] = fmaf(row_bcast<J>(a[t]), x[J], x[t]);
}
template <int... J>
__device__ __forceinline__ void subst_blocks(float (&x)[16], const float (&a)[16], std::integer_sequence<int, J...>) {
    (subst_step<J>(x, a), ...);
}
__device__ __forceinline__ void invert_blocks16(float (&x)[16], const float (&a)[16]) {
    subst_blocks(x, a, std::make_integer_sequence<int, 15>{});
}

// Cross-lane sums on the vector ALU (DPP), with no LDS round trip.  dpp<CTRL, ROWS> returns the value
// of the lane that CTRL names, in the rows of 16 lanes that ROWS selects; lanes whose source falls
// outside their row, and rows not selected, take 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float lane_value(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Sum over each row of 16 lanes, left in every lane of the row.  A butterfly: quad_perm [1 0 3 2],
// quad_perm [2 3 0 1], row_half_mirror, row_mirror.  After each step every lane of a group holds the
// same partial sum, so the result is the xor butterfly's bit for bit.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0xb1>(x);
    x += dpp<0x4e>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    return x;
}

// Sum over the wave, the same in every lane: (R0 + R1) + (R2 + R3) of the four row sums.
__device__ __forceinline__ float wave_sum64(float x) {
    x = row_sum16(x);
    return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8 lanes inside each row of
// 16 lanes (row_shr), then lane 15's total added to rows 1 and 3 and lane 31's to rows 2 and 3 (DPP
// row broadcasts).
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp<0x111>(x);
    x += dpp<0x112>(x);
    x += dpp<0x114>(x);
    x += dpp<0x118>(x);
    x += dpp<0x142, 0xa>(x);
    x += dpp<0x143, 0xc>(x);
    return x;
}

// Inclusive suffix sum over the 64 lanes of a wave (lane t gets the sum of lanes t .. 63): shifts
// by 1, 2, 4, 8 lanes toward lower lanes inside each row (row_shl), then every row adds the totals
// of the rows above it, which lanes 16, 32 and 48 hold.
__device__ __forceinline__ float wave_suffix_sum(float x, int lane) {
    x += dpp<0x101>(x);
    x += dpp<0x102>(x);
    x += dpp<0x104>(x);
    x += dpp<0x108>(x);
    const float s3 = lane_value(x, 48), s2 = lane_value(x, 32) + s3, s1 = lane_value(x, 16) + s2;
    const int row = lane >> 4;
    return x + (row == 0 ? s1 : row == 1 ? s2 : row == 2 ? s3 : 0.f);
}

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global memory at
// workgroup scope, which on gfx950 waits for every outstanding global load and store of the wave
// (vmcnt(0)); that would stall register prefetches of the next chunk at every barrier.  The kernels
// here never exchange data through global memory within a launch, so an LDS-scoped fence suffices.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Gates of one (token, v-head): with `A_log` null, `x` and `y` are g and beta themselves; otherwise
// they are the raw projections a and b, and beta = sigmoid(b), g = -exp(A_log[h]) softplus(a +
// dt_bias[h]) (softplus in the form max(z, 0) + log(1 + exp(-|z|)), which neither overflows nor
// loses the small tail).  g <= 0 then holds by construction.
__device__ __forceinline__ void gate_values(float x, float y, const float* A_log, const float* dt_bias,
                                            int h, float& g, float& beta) {
    if (A_log) {
        const float z = x + dt_bias[h];
        const float sp = fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
        g = -expf(A_log[h]) * sp;
        beta = 1.f / (1.f + expf(-y));
    } else {
        g = x;
        beta = y;
    }
}

// eps of the optional q/k L2 normalisation x / sqrt(|x|^2 + eps) (the eps of the model's RMS norms)
constexpr float kL2Eps = 1e-6f;

// SiLU, u * sigmoid(u), from the hardware exp2 and reciprocal (each within about an ulp).  The
// correctly rounded library exp and an IEEE division cost some 25 instructions per element, which a
// streaming kernel cannot hide behind its memory traffic.
__device__ __forceinline__ float silu(float u) { return u * __builtin_amdgcn_rcpf(1.f + __expf(-u)); }

}  // namespace gdn
