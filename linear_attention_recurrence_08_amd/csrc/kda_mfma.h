// Matrix-core fragment helpers shared by the bf16 KDA kernels (gfx950): vector types, the two
// v_mfma_f32_16x16x{32,16}_bf16 products, float32 <-> bf16 conversions, the LDS transpose read,
// buffer-resource loads and the LDS-only workgroup barrier.
//
// Fragment conventions for a 16 x 16 block, lane l = ln + 16 lg (ln = l % 16, lg = l / 16):
//   accumulator acc(X): register r holds X[4 lg + r][ln];
//   the A operand of Z = X Y is acc(X^T) (as bf16), the B operand acc(Y).
// For the K = 32 products, slot j of lane group lg stands for index 16 (j / 4) + 4 lg + (j % 4)
// of the 32-long contraction; A and B operands always use this order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float L2E_HI = 1.4453125f;          // bf16(log2 e)
constexpr float L2E_LO = -0.00262451171875f;  // bf16(log2 e - L2E_HI)

// Raw buffer resource word 3 for gfx9 (32-bit data format, no swizzle, no thread-id offset);
// loads past the record count return zero.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// float32 -> bf16, round to nearest even, two values per v_cvt_pk_bf16_f32.  Going through 32-bit
// integers keeps the conversions paired when the result feeds a matrix-core operand.
__device__ __forceinline__ uint32_t pk2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ bf16x4 bf4(f32x4 x) {
    const u32x2 u = {pk2(x[0], x[1]), pk2(x[2], x[3])};
    return __builtin_bit_cast(bf16x4, u);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 zero4() { return (f32x4){0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ bf16x4 as_bf4(uint2 u) { return __builtin_bit_cast(bf16x4, u); }
__device__ __forceinline__ uint2 as_u2(bf16x4 b) { return __builtin_bit_cast(uint2, b); }
__device__ __forceinline__ bf16x4 zb4() { return as_bf4(make_uint2(0u, 0u)); }
__device__ __forceinline__ bf16x4 neg4(bf16x4 b) {   // exact sign flip of four bf16 values
    const uint2 u = as_u2(b);
    return as_bf4(make_uint2(u.x ^ 0x80008000u, u.y ^ 0x80008000u));
}
__device__ __forceinline__ f32x4 unpack4(uint2 u) {  // bf16 x4 -> float32 x4 (exact)
    return (f32x4){__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                   __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}
// LDS transpose read (ds_read_b64_tr_b16): in each group of 16 lanes, lane i receives, as
// element e, element i % 4 of the four 16-bit values that lane 4e + i / 4 of the group addresses.
// With lane 16q + 4r + a addressing the four values (row 4q + r, columns 4a .. 4a+3) of a
// row-major 16 x 16 block, lane 16q + i receives column i of rows 4q .. 4q+3: the accumulator
// layout of the block (the transpose of its row-major operand fragment).
__device__ __forceinline__ bf16x4 lds_tr16(const void* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}
__device__ __forceinline__ uint2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Workgroup barrier that orders LDS only: global loads issued before it stay in flight (a full
// __syncthreads() would also wait for the prefetched tiles).  The scheduling fences keep the
// compiler from hoisting the next step's arithmetic above the barrier, where it would consume
// registers whose loads were issued only one step ago.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace mfma
}  // namespace kda
