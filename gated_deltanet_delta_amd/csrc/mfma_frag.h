// mfma_frag.h -- bf16 matrix-core operands on gfx950 shared by the chunked kernels: the vector
// types, one v_mfma_f32_16x16x32_bf16, hi + lo splits of fp32 values, shared-memory accessors, and
// the swizzled row layout of a chunk's K (or Q) rows in shared memory with its two fragment reads.
//
// v_mfma_f32_16x16x32_bf16 (checked on the device with an in-bounds probe): lane 16 g + c holds
// A[c][8 g .. 8 g + 7] and B[8 g .. 8 g + 7][c]; the result D[4 g + r][c] sits in element r of
// lane 16 g + c.  ds_read_b64_tr_b16: within a 16-lane group, lane i receives element i % 4 of the
// 4-element vectors addressed by lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4.
#pragma once

#include "common.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 cat44(const bf16x4& a, const bf16x4& b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

typedef __attribute__((address_space(1))) void glb_void;   // for global_load_lds (memory -> LDS)
typedef __attribute__((address_space(3))) void lds_void;
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

// K ring rows: unpadded (pitch DK elements: 256 or 128 bytes), the 16-byte chunk q of row t stored at
// chunk q ^ kswz<DK>(t).  The rows are read two ways, each 16 lanes at a time, and with 64 four-byte
// banks both are free of bank conflicts:
//   row fragments: 16 consecutive rows (aligned), one chunk each at the same logical q -- the swizzle
//     restricted to 16 such rows (to the 8 rows of one parity at DK = 64, whose rows alternate
//     between the two halves of the banks) is a bijection, so the 16 chunks are distinct;
//   transposed fragments: 4 consecutive rows (aligned) x 4 consecutive logical chunks (an aligned
//     quad), 8 bytes each -- the swizzle's quad bits differ between those rows (between the two rows
//     of one parity at DK = 64), so each row's quad lands on its own 4 physical chunks.
template <int DK>
__host__ __device__ constexpr int kswz(int t) {
    return DK == 128 ? (((t & 3) << 2) | ((t >> 2) & 3)) : ((((t >> 1) & 1) << 2) | ((t >> 2) & 3));
}

// index (token or key) that accumulator row m of tile a stands for
__device__ __forceinline__ int rho(int a, int m) {
    return 32 * (a >> 1) + 8 * (m >> 2) + 4 * (a & 1) + (m & 3);
}

// Lane parts of the K ring addresses (elements).  Row fragment of row 16 a + c (any a) at the
// logical chunk 4 blk + g of 32-key block blk:
template <int DK>
__device__ __forceinline__ int kf_lane(int c, int g, int blk) {
    return c * DK + 8 * ((4 * blk + g) ^ kswz<DK>(c));
}
// K^T fragment for the state update: lane (g, c) receives K[32 kb + 4 g + e][rho(kt, c)] (e < 4)
// and K[32 kb + 16 + 4 g + e - 4][rho(kt, c)] (e >= 4): keys in the state tiles' row order, tokens
// as in the chain's D fragments.  Each half is a transposed read of row 32 kb + 4 g (+ 16) + c / 4
// at logical chunk 4 (kt / 2) + c % 4, half kt % 2 of the chunk.  kt_lane gives the lane's part for
// the quad kt / 2 (the rows' swizzle depends only on 4 g + c / 4); kt_frag adds the rest.
template <int DK>
__device__ __forceinline__ int kt_lane(int c, int g, int quad) {
    const int r = 4 * g + (c >> 2);
    return r * DK + 8 * ((4 * quad + (c & 3)) ^ kswz<DK>(r));
}
template <int KR>
__device__ __forceinline__ bf16x8 kt_frag(lds_u8* k0, int half, int kb) {
    const int off = 2 * (32 * kb * KR + 4 * half);
    return cat44(read_tr(k0, off), read_tr(k0, off + 2 * 16 * KR));
}

}  // namespace
}  // namespace gdn
