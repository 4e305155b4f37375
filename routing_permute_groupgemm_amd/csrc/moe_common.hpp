// Shared device/host helpers of the HIP library (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "moe.h"

namespace moe {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

#define MOE_LDS __attribute__((address_space(3)))

// Exact widening of a bf16 bit pattern.
__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Low / high bf16 of a packed pair, widened.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint32_t f2bf(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return f2bf(lo) | (f2bf(hi) << 16);
}

// The same pair converted by one packed conversion instruction (identical
// rounding on each half).
__device__ __forceinline__ uint32_t pack_bf2x(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) float f32x2_t;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

// Buffer resource for raw (unstructured) buffer loads: `bytes` bounds the
// valid range; loads at or past it return zero (and write zero to LDS for
// LDS-direct loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// An offset that is always outside any resource built by make_rsrc here.
constexpr uint32_t kOOB = 0x80000000u;
// The same for the one resource that covers all tokens of the zero-copy
// gate/up GEMM, which may be up to this many bytes (3.75 GiB): its in-range
// offsets stay below it, and this plus any column offset of a row still fits
// in 32 bits.
constexpr uint32_t kOOB_GATHER = 0xF0000000u;

}  // namespace moe

// Host-side helpers shared by the entry points.
namespace moe_host {

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int num_cus();  // compute units of the current device (cached per device)

// Elementwise passes of the router (router.hip).  n and stride count floats;
// n, stride and period are multiples of 4 (n of 8 for the cast).
int sum_partials(const float* part, int S, int64_t n, int64_t stride, const float* bias, int period, float* out,
                 hipStream_t s);
int cast_f32_bf16(const float* in, int64_t n, uint16_t* out, hipStream_t s);

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe_host
