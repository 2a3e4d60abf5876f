// common.h -- small device helpers shared by the libgdn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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

// State slot of sequence (or batch row) n: n itself, or state_indices[n] in a pool of num_slots
// states.  An index outside [0, num_slots) marks a padding row, which has no state: false is
// returned and slot is set to 0 (any in-bounds value; nothing is read or written through it).
__device__ __forceinline__ bool state_slot(const int32_t* state_indices, int num_slots, int n, int& slot) {
    if (!state_indices) {
        slot = n;
        return true;
    }
    const int s = state_indices[n];
    const bool ok = s >= 0 && s < num_slots;
    slot = ok ? s : 0;
    return ok;
}

// Sequence n's token range [t0, t1) inside batch row `row`, clamped to [0, T] so that a malformed
// cu_seqlens array can only produce wrong numbers, never an access outside the buffers.
__device__ __forceinline__ void sequence_range(const int32_t* cu_seqlens, int n, int T, int& row,
                                               int& t0, int& t1) {
    if (cu_seqlens) {
        int a = cu_seqlens[n], b = cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        row = 0;
        t0 = a;
        t1 = b;
    } else {
        row = n;
        t0 = 0;
        t1 = T;
    }
}

}  // namespace gdn
