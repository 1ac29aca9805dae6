// Device-side element types shared by the kernel sources of the library:
// the storage type of each dtype and its exact conversions to and from fp32
// (rounding to nearest even on the way down). Included by .hip files only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msda {
namespace {

constexpr int kBlock = 256;
constexpr int kXcds = 8;

// ------------------------------------------------------------ element types

struct F32T {
    using S = float;
};
struct F16T {
    using S = uint16_t;
};
struct BF16T {
    using S = uint16_t;
};

__device__ __forceinline__ float to_f32(F32T, float v) { return v; }
__device__ __forceinline__ float to_f32(F16T, uint16_t v) {
    return (float)__builtin_bit_cast(_Float16, v);
}
__device__ __forceinline__ float to_f32(BF16T, uint16_t v) {
    return __uint_as_float((uint32_t)v << 16);
}
__device__ __forceinline__ float from_f32(F32T, float v) { return v; }
__device__ __forceinline__ uint16_t from_f32(F16T, float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}
__device__ __forceinline__ uint16_t from_f32(BF16T, float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

}  // namespace
}  // namespace msda
