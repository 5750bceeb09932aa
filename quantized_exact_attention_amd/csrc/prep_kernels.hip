// prep_kernels.hip -- the quantization prepass on gfx950.
//
// "Sage2 Blackwell Mainloop", section "Decision": K mean/smoothing, Q
// quantization, K subtract-mean quantization, V scale/FP8 quantization;
// section "Existing Contract": per-warp INT8 Q (32-row groups), per-block INT8
// K (64-row blocks), FP8 V with per-channel scales.  "State-Ownership
// Architecture Decision", "Non-Negotiable Dataflow": the exact global K mean
// and V-scale prepasses are kept.
//
// Every kernel here is HBM-bound.  The arithmetic is FP32 with no contraction
// (the library is built with -ffp-contract=off), in the order the C-ABI header
// states, so the outputs are bit-identical to a plain sequential evaluation.
//
// Launch sequence (one stream):
//   1. tile_stats    per 64-row tile: FP32 in-order channel sums of K and
//                    channel absolute maxima of V          (reads K, V)
//   2. finalize      per (b,h): k_mean from the tile sums in tile order; V
//                    channel amax, v_scale = a/448, v_inv = 448/a
//   3. quant_q       per 32-row group: amax, scale, INT8 codes (reads Q)
//   4. quant_k       per 64-row tile: K - k_mean, amax, scale, codes (reads K)
//   5. quant_v       per 64-row tile: E4M3 codes in the mainloop's V layout
//                    (reads V)
#include "sage_device.hpp"
#include "sage_launch.hpp"

namespace sage {

namespace {

// 16 threads per (b, h, tile); thread c8 owns channels 8*c8 .. 8*c8+7.
__global__ __launch_bounds__(256) void tile_stats_kernel(StatsArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t unit = gid >> 4;
    const int c8 = (int)(gid & 15);
    if (unit >= a.units) return;
    const int bh = (int)(unit / a.T);
    const int t = (int)(unit % a.T);
    const int b = bh / a.H, h = bh % a.H;
    const uint16_t* kp = a.k + b * a.k_sb + h * a.k_sh + 8 * c8;
    const uint16_t* vp = a.v + b * a.v_sb + h * a.v_sh + 8 * c8;
    float sum[8], amax[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { sum[i] = 0.0f; amax[i] = 0.0f; }
    const int n0 = t * kBK;
    const int n1 = min(n0 + kBK, a.N);
#pragma unroll 4
    for (int n = n0; n < n1; ++n) {
        float kf[8], vf[8];
        unpack8(*(const uint4*)(kp + (int64_t)n * a.k_sn), kf);
        unpack8(*(const uint4*)(vp + (int64_t)n * a.v_sn), vf);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sum[i] = sum[i] + kf[i];
            amax[i] = fmaxf(amax[i], fabsf(vf[i]));
        }
    }
    float* ks = a.k_tile_sum + ((int64_t)bh * a.T + t) * kHD + 8 * c8;
    float* va = a.v_tile_amax + ((int64_t)bh * a.T + t) * kHD + 8 * c8;
    *(v4f*)(ks) = v4f{sum[0], sum[1], sum[2], sum[3]};
    *(v4f*)(ks + 4) = v4f{sum[4], sum[5], sum[6], sum[7]};
    *(v4f*)(va) = v4f{amax[0], amax[1], amax[2], amax[3]};
    *(v4f*)(va + 4) = v4f{amax[4], amax[5], amax[6], amax[7]};
}

// One block of 128 threads per (b, h); thread d owns channel d.
__global__ __launch_bounds__(128) void finalize_kernel(FinalizeArgs a) {
    const int bh = blockIdx.x;
    const int d = threadIdx.x;
    const float* ks = a.k_tile_sum + (int64_t)bh * a.T * kHD + d;
    const float* va = a.v_tile_amax + (int64_t)bh * a.T * kHD + d;
    float total = 0.0f, amax = 0.0f;
    int t = 0;
    for (; t + 8 <= a.T; t += 8) {
        float s[8], m[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) { s[i] = ks[(int64_t)(t + i) * kHD]; m[i] = va[(int64_t)(t + i) * kHD]; }
#pragma unroll
        for (int i = 0; i < 8; ++i) { total = total + s[i]; amax = fmaxf(amax, m[i]); }
    }
    for (; t < a.T; ++t) {
        total = total + ks[(int64_t)t * kHD];
        amax = fmaxf(amax, va[(int64_t)t * kHD]);
    }
    a.k_mean[(int64_t)bh * kHD + d] = total / (float)a.N;
    float scale = 0.0f, inv = 0.0f;
    if (amax >= kAmaxFloor) {
        scale = amax / 448.0f;
        inv = 448.0f / amax;
    }
    a.v_scale[(int64_t)bh * kHD + d] = scale;
    a.v_inv[(int64_t)bh * kHD + d] = inv;
}

// One wave per (b, h, 32-row group g).  Lane l reads row 32g + l%32, channels
// 32kk + 16*(l/32) + 0..15, which is exactly the 16 bytes it writes for kk.
__global__ __launch_bounds__(256) void quant_q_kernel(QuantQArgs a) {
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= a.waves) return;
    const int lane = threadIdx.x & 63;
    const int bh = (int)(w / a.G);
    const int g = (int)(w % a.G);
    const int b = bh / a.H, h = bh % a.H;
    const int n = g * kQG + (lane & 31);
    const uint16_t* qp = a.q + b * a.sb + (int64_t)n * a.sn + h * a.sh + 16 * (lane >> 5);
    uint4 codes[4];
    const float scale = quant_q_group(qp, n < a.N, codes);
    int8_t* out = a.q_i8 + ((int64_t)bh * a.G + g) * kQGroupBytes + lane * 16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) *(uint4*)(out + kk * 64 * 16) = codes[kk];
    if (lane == 0) a.q_scale[(int64_t)bh * a.G + g] = scale;
}

// One wave per (b, h, 64-row tile t).  Lane l handles rows 64t + 32*half + l%32
// and channels 32kk + 16*(l/32) + 0..15 for half in 0..1, kk in 0..3.
__global__ __launch_bounds__(256) void quant_k_kernel(QuantKArgs a) {
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= a.waves) return;
    const int lane = threadIdx.x & 63;
    const int bh = (int)(w / a.T);
    const int t = (int)(w % a.T);
    const int b = bh / a.H, h = bh % a.H;
    const int c0 = 16 * (lane >> 5);
    const float* kmp = a.k_mean + (int64_t)bh * kHD + c0;
    uint4 raw[2][4][2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int n = t * kBK + 32 * half + (lane & 31);
        const bool valid = n < a.N;
        const uint16_t* kp = a.k + b * a.sb + (int64_t)n * a.sn + h * a.sh + c0;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            raw[half][kk][0] = valid ? *(const uint4*)(kp + 32 * kk) : make_uint4(0, 0, 0, 0);
            raw[half][kk][1] = valid ? *(const uint4*)(kp + 32 * kk + 8) : make_uint4(0, 0, 0, 0);
        }
    }
    float am = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        float km[16];
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            v4f m4 = *(const v4f*)(kmp + 32 * kk + i);
            km[i] = m4[0]; km[i + 1] = m4[1]; km[i + 2] = m4[2]; km[i + 3] = m4[3];
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int n = t * kBK + 32 * half + (lane & 31);
            if (n < a.N) {
                float x[16];
                unpack8(raw[half][kk][0], x);
                unpack8(raw[half][kk][1], x + 8);
#pragma unroll
                for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(x[i] - km[i]));
            }
        }
    }
    am = wave_max(am);
    float scale = 0.0f, inv = 0.0f;
    if (am >= kAmaxFloor) {
        scale = am / 127.0f;
        inv = 127.0f / am;
    }
    int8_t* out = a.k_i8 + ((int64_t)bh * a.T + t) * kTileBytes + lane * 16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        float km[16];
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            v4f m4 = *(const v4f*)(kmp + 32 * kk + i);
            km[i] = m4[0]; km[i + 1] = m4[1]; km[i + 2] = m4[2]; km[i + 3] = m4[3];
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int n = t * kBK + 32 * half + (lane & 31);
            float x[16];
            unpack8(raw[half][kk][0], x);
            unpack8(raw[half][kk][1], x + 8);
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = x[i] - km[i];
            uint4 codes = pack16_int8(x, inv);
            if (n >= a.N) codes = make_uint4(0, 0, 0, 0);
            *(uint4*)(out + (half * 4 + kk) * 64 * 16) = codes;
        }
    }
    if (lane == 0) a.k_scale[(int64_t)bh * a.T + t] = scale;
}

// One block of 256 threads per (b, h, 64-row tile t).  The BF16 tile is staged
// in LDS row-major; each output chunk gathers 16 rows of one channel.
constexpr int kVRow = kHD + 8;   // LDS row pitch in BF16 elements (272 bytes)

__global__ __launch_bounds__(256) void quant_v_kernel(QuantVArgs a) {
    __shared__ uint16_t tile[kBK * kVRow];
    const int64_t blk = blockIdx.x;
    const int bh = (int)(blk / a.T);
    const int t = (int)(blk % a.T);
    const int b = bh / a.H, h = bh % a.H;
    {
        const int row = threadIdx.x >> 2;
        const int seg = threadIdx.x & 3;                 // 32 channels each
        const int n = t * kBK + row;
        const uint16_t* vp = a.v + b * a.sb + (int64_t)n * a.sn + h * a.sh + 32 * seg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 w = n < a.N ? *(const uint4*)(vp + 8 * i) : make_uint4(0, 0, 0, 0);
            *(uint4*)(&tile[row * kVRow + 32 * seg + 8 * i]) = w;
        }
    }
    __syncthreads();
    uint8_t* out = a.v_fp8 + ((int64_t)bh * a.T + t) * kTileBytes;
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
        const int c = threadIdx.x + 256 * rep;          // 16-byte chunk index
        const int db = c >> 7;
        const int half = (c >> 6) & 1;
        const int l = c & 63;
        const int d = 32 * db + (l & 31);
        const int hh = l >> 5;
        const float inv = a.v_inv[(int64_t)bh * kHD + d];
        const bool zero = a.v_scale[(int64_t)bh * kHD + d] == 0.0f;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = 32 * half + 8 * (i >> 2) + 4 * hh + (i & 3);
            x[i] = bf16_bits_to_f32(tile[key * kVRow + d]) * inv;
        }
        uint32_t wd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int p = cvt_pk_e4m3<false>(x[4 * j], x[4 * j + 1], 0);
            p = cvt_pk_e4m3<true>(x[4 * j + 2], x[4 * j + 3], p);
            wd[j] = zero ? 0u : (uint32_t)p;
        }
        *(uint4*)(out + c * 16) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
}

}  // namespace

hipError_t launch_prepass(const PrepassArgs& p, hipStream_t stream) {
    const int64_t BH = (int64_t)p.B * p.H;
    {
        StatsArgs a;
        a.k = p.k; a.k_sb = p.k_sb; a.k_sn = p.k_sn; a.k_sh = p.k_sh;
        a.v = p.v; a.v_sb = p.v_sb; a.v_sn = p.v_sn; a.v_sh = p.v_sh;
        a.H = p.H; a.N = p.N; a.T = p.T; a.units = BH * p.T;
        a.k_tile_sum = p.k_tile_sum; a.v_tile_amax = p.v_tile_amax;
        const int64_t threads = a.units * 16;
        hipLaunchKernelGGL(tile_stats_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
    }
    {
        FinalizeArgs a;
        a.k_tile_sum = p.k_tile_sum; a.v_tile_amax = p.v_tile_amax;
        a.T = p.T; a.N = p.N;
        a.k_mean = p.k_mean; a.v_scale = p.v_scale; a.v_inv = p.v_inv;
        hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)BH), dim3(128), 0, stream, a);
    }
    if (p.with_q) {
        QuantQArgs a;
        a.q = p.q; a.sb = p.q_sb; a.sn = p.q_sn; a.sh = p.q_sh;
        a.H = p.H; a.N = p.N; a.G = p.G; a.waves = BH * p.G;
        a.q_i8 = p.q_i8; a.q_scale = p.q_scale;
        hipLaunchKernelGGL(quant_q_kernel, dim3((unsigned)((a.waves + 3) / 4)), dim3(256), 0, stream, a);
    }
    {
        QuantKArgs a;
        a.k = p.k; a.sb = p.k_sb; a.sn = p.k_sn; a.sh = p.k_sh;
        a.H = p.H; a.N = p.N; a.T = p.T; a.waves = BH * p.T;
        a.k_mean = p.k_mean; a.k_i8 = p.k_i8; a.k_scale = p.k_scale;
        hipLaunchKernelGGL(quant_k_kernel, dim3((unsigned)((a.waves + 3) / 4)), dim3(256), 0, stream, a);
    }
    {
        QuantVArgs a;
        a.v = p.v; a.sb = p.v_sb; a.sn = p.v_sn; a.sh = p.v_sh;
        a.H = p.H; a.N = p.N; a.T = p.T;
        a.v_inv = p.v_inv; a.v_scale = p.v_scale; a.v_fp8 = p.v_fp8;
        hipLaunchKernelGGL(quant_v_kernel, dim3((unsigned)(BH * p.T)), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

// FP32 -> E4M3FN through the same conversion the kernels use.
namespace {
__global__ __launch_bounds__(256) void cvt_e4m3_kernel(const float* x, uint8_t* y, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (i + j < n) ? x[i + j] : 0.0f;
    int p = cvt_pk_e4m3<false>(v[0], v[1], 0);
    p = cvt_pk_e4m3<true>(v[2], v[3], p);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (i + j < n) y[i + j] = (uint8_t)((uint32_t)p >> (8 * j));
}
}  // namespace

hipError_t launch_cvt_e4m3(const float* x, uint8_t* y, int64_t n, hipStream_t stream) {
    const int64_t blocks = (n + 1023) / 1024;
    hipLaunchKernelGGL(cvt_e4m3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y, n);
    return hipGetLastError();
}

}  // namespace sage
