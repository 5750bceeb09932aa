// sage_device.hpp -- device-side types and helpers shared by the gfx950 kernels.
//
// Operand layouts of the two matrix instructions the mainloop uses (measured
// on gfx950 and fixed by the library's byte layouts):
//   v_mfma_i32_32x32x32_i8 and v_mfma_scale_f32_32x32x64_f8f6f4:
//     A: lane l holds row l%32, k-bytes [K/2 * (l/32), K/2 * (l/32) + K/2)
//     B: lane l holds column l%32, the same k-bytes
//     C/D: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kHD = 128;          // head dimension
constexpr int kQG = 32;           // Q scale group (rows)
constexpr int kBQ = 128;          // Q padding block (rows)
constexpr int kBK = 64;           // K/V tile (rows)
constexpr int kQGroupBytes = 32 * 128;   // 4096
constexpr int kTileBytes = 64 * 128;     // 8192
// Groups, tiles or channels whose absolute maximum is below this get scale 0.
constexpr float kAmaxFloor = 0x1p-100f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two FP32 -> E4M3FN codes (round to nearest even, gfx950 OCP FP8) packed into
// the low (hi_word = false) or high 16 bits of `old`.
template <bool kHiWord>
__device__ __forceinline__ int cvt_pk_e4m3(float a, float b, int old) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, kHiWord);
}

// Nearest-even integer code in [-127, 127] of x * inv.
__device__ __forceinline__ int int8_code(float x, float inv) {
    float y = x * inv;
    float r = __builtin_rintf(y);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Value held by lane l^32 (the other half of the wave).
__device__ __forceinline__ float other_half(float v) { return __shfl_xor(v, 32, 64); }
__device__ __forceinline__ int other_half(int v) { return __shfl_xor(v, 32, 64); }

}  // namespace sage
