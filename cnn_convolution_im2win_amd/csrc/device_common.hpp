// device_common.hpp -- element types and conversions used by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ciw {

typedef _Float16 half_t;

// bf16 is carried as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(half_t v) { return (float)v; }
__device__ __forceinline__ float to_f32(bf16_t v) {
    return __uint_as_float(((uint32_t)v.bits) << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float v);

template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }

// fp32 -> fp16, round to nearest even (the hardware conversion's default mode).
template <>
__device__ __forceinline__ half_t from_f32<half_t>(float v) { return (half_t)v; }

// fp32 -> bf16, round to nearest even (the hardware conversion, two values
// per instruction); NaN stays NaN.
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
    bf16_t r;
    r.bits = __builtin_bit_cast(uint16_t, (__bf16)v);
    return r;
}

// The 16-bit pattern of from_f32<T>(v), for the 16-bit element types.
template <typename T>
__device__ __forceinline__ uint16_t f32_bits(float v);

template <>
__device__ __forceinline__ uint16_t f32_bits<half_t>(float v) {
    return __builtin_bit_cast(uint16_t, from_f32<half_t>(v));
}

template <>
__device__ __forceinline__ uint16_t f32_bits<bf16_t>(float v) {
    return from_f32<bf16_t>(v).bits;
}

template <typename T>
__device__ __forceinline__ T zero_elem() {
    return from_f32<T>(0.0f);
}

// Stores marked non-temporal (the nt bit: the lines are not kept in the
// caches for reuse).  Whether they pay is measured per kernel: the band
// kernel's output stores (whole 64-byte runs; its input rows are re-read
// from L2 by the neighbouring band) are faster this way.  The few-channel
// and depthwise in-LDS kernels' stores and the repack's window-tensor
// stores (read again right after) were much slower, and the materialised
// row kernel's faster in one layer's full call but slower on its own, so
// those keep plain stores.
typedef uint32_t u32x4_vec __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_vec __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store_stream(void* p, uint4 v) {
    const u32x4_vec t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_vec*>(p));
}
__device__ __forceinline__ void store_stream(void* p, uint2 v) {
    const u32x2_vec t = {v.x, v.y};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2_vec*>(p));
}
__device__ __forceinline__ void store_stream(void* p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}
__device__ __forceinline__ void store_stream(void* p, uint16_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint16_t*>(p));
}

}  // namespace ciw
