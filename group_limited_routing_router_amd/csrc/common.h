// common.h -- device-side helpers shared by the libmoe kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: workgroups go round-robin over 8 XCDs
// Intermediate buffers larger than the Infinity Cache (256 MB on MI355X) that
// are written once and read once stream past the caches.
constexpr int64_t kStreamBytes = static_cast<int64_t>(256) << 20;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even.  Adding 0x7fff
// plus the lowest kept bit carries into the kept half exactly when the dropped
// half is above one half, or equal to it with an odd kept half.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float sigmoid_f32(float z) { return 1.0f / (1.0f + expf(-z)); }

// silu(z) = z * sigmoid(z) in fp32 with the hardware exp2 and reciprocal
// (about 1 ulp each); the result is rounded to bf16 right after, so the
// difference to correctly rounded fp32 shows only at bf16 rounding ties.
__device__ __forceinline__ float silu_f32(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// One 16x16x32 bf16 MFMA step: acc += A(16x32) * B(32x16).  Lane l supplies
// row (l % 16) of A and column (l % 16) of B, both for the 8 consecutive k of
// chunk (l / 16); it receives rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One 32x32x16 bf16 MFMA step: acc += A(32x16) * B(16x32).  Lane l supplies
// row (l % 32) of A and column (l % 32) of B, both for the 8 consecutive k of
// half (l / 32); for i = 0..15 it receives row 8*(i/4) + 4*(l/32) + (i%4) of
// column (l % 32).  Twice the work of the 16x16x32 form per issue: on gfx950
// it is the shape that reaches the bf16 peak.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
    return __builtin_bit_cast(bf16x8, v);
}

// 16-byte global load that bypasses nothing special; kept in one place so the
// load width is explicit.
__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace moe
