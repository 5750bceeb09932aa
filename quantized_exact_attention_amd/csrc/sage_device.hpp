// sage_device.hpp -- device-side types and helpers shared by the gfx950 kernels.
//
// Operand layouts of the two matrix instructions the mainloop uses (measured
// on gfx950 and fixed by the library's byte layouts):
//   v_mfma_i32_32x32x32_i8 and v_mfma_(scale_)f32_32x32x64_f8f6f4:
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

// 8 BF16 values (one 16-byte load) -> 8 FP32.
__device__ __forceinline__ void unpack8(const uint4 w, float* f) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}

// 16 INT8 codes of x[0..15] * inv, packed little-endian into a uint4.
__device__ __forceinline__ uint4 pack16_int8(const float* x, float inv) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t acc = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc |= ((uint32_t)int8_code(x[4 * j + i], inv) & 0xffu) << (8 * i);
        w[j] = acc;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// INT8 quantization of one 32-row Q group by one wavefront ("Sage2 Blackwell
// Mainloop", Existing Contract: per-warp INT8 Q in 32-row groups).  Lane l
// passes `row` = its row 32g + l%32 at channel 16*(l/32) (valid = row < N);
// it loads channels 32kk + 16*(l/32) + 0..15 for kk = 0..3, which are exactly
// the 16 codes it owns in the operand layout of the QK instruction.  The
// group scale is amax/127 and each code rne(x * (127/amax)) clamped to
// +-127; a group with amax < 2^-100 gets scale 0 and zero codes.
__device__ __forceinline__ float quant_q_values(const float (&x)[64], uint4 (&codes)[4]) {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) am = fmaxf(am, fabsf(x[i]));
    am = wave_max(am);
    float scale = 0.0f, inv = 0.0f;
    if (am >= kAmaxFloor) {
        scale = am / 127.0f;
        inv = 127.0f / am;
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) codes[kk] = pack16_int8(x + 16 * kk, inv);
    return scale;
}

// quant_q_values on a row kept as packed BF16 words w[8] (w[2kk + e] holds
// the lane's channels 32kk + 16*(l/32) + 8e + 0..7): the words are widened
// twice, once for the maximum and once for the codes, so that no 64-float
// copy of the row stays live.  Same results as quant_q_values.
__device__ __forceinline__ float quant_q_words(const uint4 (&w)[8], uint4 (&codes)[4]) {
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float x[8];
        unpack8(w[j], x);
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(x[i]));
    }
    am = wave_max(am);
    float scale = 0.0f, inv = 0.0f;
    if (am >= kAmaxFloor) {
        scale = am / 127.0f;
        inv = 127.0f / am;
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        float x[16];
        unpack8(w[2 * kk], x);
        unpack8(w[2 * kk + 1], x + 8);
        codes[kk] = pack16_int8(x, inv);
    }
    return scale;
}

__device__ __forceinline__ float quant_q_group(const uint16_t* row, bool valid, uint4 (&codes)[4]) {
    float x[64];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        uint4 w0 = make_uint4(0, 0, 0, 0), w1 = make_uint4(0, 0, 0, 0);
        if (valid) {
            w0 = *(const uint4*)(row + 32 * kk);
            w1 = *(const uint4*)(row + 32 * kk + 8);
        }
        unpack8(w0, x + 16 * kk);
        unpack8(w1, x + 16 * kk + 8);
    }
    return quant_q_values(x, codes);
}

// FP32 -> BF16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
    const v2bf t = v2bf{(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, t);
}

// Bijection from dispatch order to work items such that the items dispatched
// to one XCD (dispatch index mod 8; each XCD has its own L2) are consecutive.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
    const int q = nwg >> 3, r = nwg & 7;
    const int xcd = wg & 7, slot = wg >> 3;
    const int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return base + slot;
}

__device__ __forceinline__ uint32_t& word_of(uint4& w, int m) {
    return m == 0 ? w.x : m == 1 ? w.y : m == 2 ? w.z : w.w;
}

// Optional upstream producer ("Sage2 Blackwell Mainloop", Completed P1 And
// P2): per-head RMSNorm of one Q or K row, then split-half rotary embedding,
// each result rounded to BF16, in place on the row's BF16 words.  The row is
// held by lanes l%32 and l%32 + 32 of a wave in the QK operand split: on the
// lane with hf = l/32, w[2kk + e] holds channels 32kk + 16hf + 8e + 0..7.
//   ss  = sum over channels 0..127 in order of fl(x*x), from +0 (the running
//         sum passes between the row's two lanes segment by segment, and both
//         end with the same value)
//   r   = fl(1 / fl(sqrt(fl(fl(ss / 128) + eps))))
//   y_c = bf16(fl(fl(x_c * r) * g[c]))
//   o_i = bf16(fl(fl(y_i * cos_i) - fl(y_{i+64} * sin_i))),
//   o_{i+64} = bf16(fl(fl(y_{i+64} * cos_i) + fl(y_i * sin_i))), i < 64,
// with the angle row (cos_row, sin_row: 64 FP32 each) of the row's token.
// Channel i and i + 64 sit on the same lane (kk and kk + 2).  kLowRegs: the
// channel values are unpacked again for the normalisation rather than kept
// from the squares (an empty asm per word hides that they are the same), for
// callers that are short of registers; the results are identical.
template <bool kLowRegs = false>
__device__ __forceinline__ void norm_rope_row(uint4 (&w)[8], int hf, const float* g, const float* cos_row,
                                              const float* sin_row, float eps) {
    // ss in channel order: 16-channel segment s = c/16 is block kk = s/2 of
    // the lanes with hf = s%2.  Each lane squares its own 64 channels once;
    // the running sum then alternates between the row's two lanes: at
    // segment s every lane adds its block s/2 onto the running sum (the
    // result is the sum's next value on the lanes that hold segment s), and
    // v_permlane32_swap gives that value to both lanes for the next segment.
    float ss = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        float sq[16];
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t u = word_of(w[2 * kk + e], m);
                const float a = __uint_as_float(u << 16), b = __uint_as_float(u & 0xffff0000u);
                sq[8 * e + 2 * m] = a * a;
                sq[8 * e + 2 * m + 1] = b * b;
            }
#pragma unroll
        for (int owner = 0; owner < 2; ++owner) {
            float t = ss;
#pragma unroll
            for (int i = 0; i < 16; ++i) t = t + sq[i];
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
            ss = __uint_as_float(r[owner]);
        }
    }
    if (kLowRegs) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            asm volatile("" : "+v"(w[i].x), "+v"(w[i].y), "+v"(w[i].z), "+v"(w[i].w));
    }
    const float ms = ss / 128.0f;
    const float t = ms + eps;
    const float rt = sqrtf(t);
    const float r = 1.0f / rt;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        // channels c = 32kk + 16hf + j (first half) and c + 64 (second half)
        float y0[16], y1[16];
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int j = 8 * e + 2 * m;
                const int c = 32 * kk + 16 * hf + j;
                const uint32_t u0 = word_of(w[2 * kk + e], m), u1 = word_of(w[2 * kk + 4 + e], m);
                const float x00 = __uint_as_float(u0 << 16), x01 = __uint_as_float(u0 & 0xffff0000u);
                const float x10 = __uint_as_float(u1 << 16), x11 = __uint_as_float(u1 & 0xffff0000u);
                float p;
                p = x00 * r; p = p * g[c];          y0[j] = (float)(__bf16)p;
                p = x01 * r; p = p * g[c + 1];      y0[j + 1] = (float)(__bf16)p;
                p = x10 * r; p = p * g[c + 64];     y1[j] = (float)(__bf16)p;
                p = x11 * r; p = p * g[c + 65];     y1[j + 1] = (float)(__bf16)p;
            }
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int j = 8 * e + 2 * m;
                const int i = 32 * kk + 16 * hf + j;
                float o0[2], o1[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float c = cos_row[i + q], s = sin_row[i + q];
                    const float ac = y0[j + q] * c, bs = y1[j + q] * s;
                    const float bc = y1[j + q] * c, as = y0[j + q] * s;
                    o0[q] = ac - bs;
                    o1[q] = bc + as;
                }
                word_of(w[2 * kk + e], m) = bf16x2_bits(o0[0], o0[1]);
                word_of(w[2 * kk + 4 + e], m) = bf16x2_bits(o1[0], o1[1]);
            }
    }
}

// Maximum of the 32 int32 values of two accumulator tiles (two chains, so
// the compiler can form three-input maxima).  Kept in plain C++: the inputs
// are matrix-instruction results, and only compiler-visible code gets the
// wait states the hardware needs before reading them.
__device__ __forceinline__ int max_of_32(const v16i& s0, const v16i& s1) {
    int ma = max(s0[0], s0[1]);
    int mb = max(s1[0], s1[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
        ma = max(ma, max(s0[r], s0[r + 1]));
        mb = max(mb, max(s1[r], s1[r + 1]));
    }
    return max(ma, mb);
}

// Combine a value across the two 32-lane halves of the wave without an LDS
// round trip: v_permlane32_swap(x, x) yields, on every lane l, the values of
// lanes l%32 and l%32 + 32, so both halves get bit-identical results.
__device__ __forceinline__ int halves_max(int v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float halves_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace sage
