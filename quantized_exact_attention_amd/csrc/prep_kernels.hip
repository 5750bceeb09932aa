// prep_kernels.hip -- the quantization prepass on gfx950.
//
// "Sage2 Blackwell Mainloop", section "Decision": K mean/smoothing, Q
// quantization, K subtract-mean quantization, V scale/FP8 quantization;
// section "Existing Contract": per-warp INT8 Q (32-row groups), per-block INT8
// K (64-row blocks), FP8 V with per-channel scales.  "State-Ownership
// Architecture Decision", "Non-Negotiable Dataflow": the exact global K mean
// and V-scale prepasses are kept.
//
// Every kernel here streams HBM (the RMSNorm + RoPE variants add about a
// thousand vector instructions per row pair).  The arithmetic is FP32 with no
// contraction (the library is built with -ffp-contract=off), in the order the
// C-ABI header states, so the outputs are bit-identical to a plain sequential
// evaluation.
//
// Launch sequence (one stream):
//   1. tile_stats    per 64-row tile: FP32 in-order channel sums of K and
//                    channel absolute maxima of V          (reads K, V)
//                    (tile_stats_nr when the optional RMSNorm + RoPE
//                    producer is applied to Q and K: the normalised rows are
//                    recomputed in launches 1 and 3 and never stored)
//   2. finalize      per (b,h): k_mean from the tile sums in tile order; V
//                    channel amax, v_scale = a/448, v_inv = 448/a
//   3. quant_qkv     per 64-row tile, one pass over its Q, K and V rows:
//                    INT8 Q per 32-row group, INT8 K - k_mean per tile,
//                    E4M3 V in the mainloop's layout (Q is skipped when the
//                    mainloop quantizes it itself)
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

constexpr int kVRow = kHD + 8;   // LDS row pitch in BF16 elements (272 bytes)

// tile_stats with the RMSNorm + RoPE producer applied to K: one block of 256
// threads per (b, h, 64-row tile).  Waves 0-1 load 32 K rows each in the QK
// operand split, normalise and rotate them (norm_rope_row) and stage the BF16
// results in LDS; waves 2-3 take channel absolute maxima of V (thread u owns
// channels 8*(u%16)..+7 of rows u/16, u/16 + 8, ...).  Then thread d sums
// channel d of the staged rows in row order and threads 128+d combine the
// eight V partial maxima of channel d.
__global__ __launch_bounds__(256) void tile_stats_nr_kernel(StatsArgs a) {
    __shared__ uint16_t tile[kBK * kVRow];
    __shared__ float vam[8][kHD];
    const int64_t blk = blockIdx.x;
    const int bh = (int)(blk / a.T);
    const int t = (int)(blk % a.T);
    const int b = bh / a.H, h = bh % a.H;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n0 = t * kBK;
    const int rows = min(kBK, a.N - n0);
    if (wave < 2) {
        const int hf = lane >> 5;
        const int row = 32 * wave + (lane & 31);
        const int n = n0 + row;
        const bool valid = row < rows;
        const uint16_t* kp = a.k + b * a.k_sb + (int64_t)n * a.k_sn + h * a.k_sh + 16 * hf;
        uint4 w[8];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            w[2 * kk] = valid ? *(const uint4*)(kp + 32 * kk) : make_uint4(0, 0, 0, 0);
            w[2 * kk + 1] = valid ? *(const uint4*)(kp + 32 * kk + 8) : make_uint4(0, 0, 0, 0);
        }
        const int na = valid ? n : 0;
        norm_rope_row(w, hf, a.nr.k_weight, a.nr.cos + (int64_t)na * (kHD / 2), a.nr.sin + (int64_t)na * (kHD / 2),
                      a.nr.eps);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                *(uint4*)(&tile[row * kVRow + 32 * kk + 16 * hf + 8 * e]) = w[2 * kk + e];
    } else {
        const int u = threadIdx.x - 128;
        const int c8 = u & 15;
        const int rp = u >> 4;
        const uint16_t* vp = a.v + b * a.v_sb + h * a.v_sh + 8 * c8;
        float am[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) am[i] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = rp + 8 * i;
            if (row < rows) {
                float vf[8];
                unpack8(*(const uint4*)(vp + (int64_t)(n0 + row) * a.v_sn), vf);
#pragma unroll
                for (int c = 0; c < 8; ++c) am[c] = fmaxf(am[c], fabsf(vf[c]));
            }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) vam[rp][8 * c8 + c] = am[c];
    }
    __syncthreads();
    const int d = threadIdx.x & 127;
    if (threadIdx.x < 128) {
        float sum = 0.0f;
        if (rows == kBK) {
            // all 64 LDS reads in flight before the ordered adds
            float x[kBK];
#pragma unroll
            for (int row = 0; row < kBK; ++row) x[row] = bf16_bits_to_f32(tile[row * kVRow + d]);
#pragma unroll
            for (int row = 0; row < kBK; ++row) sum = sum + x[row];
        } else {
            for (int row = 0; row < rows; ++row) sum = sum + bf16_bits_to_f32(tile[row * kVRow + d]);
        }
        a.k_tile_sum[((int64_t)bh * a.T + t) * kHD + d] = sum;
    } else {
        float m = vam[0][d];
#pragma unroll
        for (int i = 1; i < 8; ++i) m = fmaxf(m, vam[i][d]);
        a.v_tile_amax[((int64_t)bh * a.T + t) * kHD + d] = m;
    }
}

// One block of 128 threads per (b, h); thread d owns channel d.
__global__ __launch_bounds__(128) void finalize_kernel(FinalizeArgs a) {
    const int bh = blockIdx.x;
    const int d = threadIdx.x;
    const float* ks = a.k_tile_sum + (int64_t)bh * a.T * kHD + d;
    const float* va = a.v_tile_amax + (int64_t)bh * a.T * kHD + d;
    // Sequential in tile order; loads are issued 32 tiles ahead of the adds.
    constexpr int kBatch = 32;
    float total = 0.0f, amax = 0.0f;
    int t = 0;
    for (; t + kBatch <= a.T; t += kBatch) {
        float s[kBatch], m[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) { s[i] = ks[(int64_t)(t + i) * kHD]; m[i] = va[(int64_t)(t + i) * kHD]; }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) { total = total + s[i]; amax = fmaxf(amax, m[i]); }
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

// Absolute maximum of K - k_mean over one lane's 64 channels of a row held as
// BF16 words (kraw[kk][e]: channels 32kk + 16*(l/32) + 8e + 0..7); kmp points
// at the lane's first k_mean channel.
__device__ __forceinline__ float k_row_amax(const uint4 (&kraw)[4][2], const float* kmp) {
    float am = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        float x[16];
        unpack8(kraw[kk][0], x);
        unpack8(kraw[kk][1], x + 8);
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            const v4f m4 = *(const v4f*)(kmp + 32 * kk + i);
            am = fmaxf(am, fabsf(x[i] - m4[0]));
            am = fmaxf(am, fabsf(x[i + 1] - m4[1]));
            am = fmaxf(am, fabsf(x[i + 2] - m4[2]));
            am = fmaxf(am, fabsf(x[i + 3] - m4[3]));
        }
    }
    return am;
}

// One block of 256 threads per (b, h, 64-row tile t) quantizes everything the
// tile's rows hold, so each projection row segment is read once:
//   waves 0, 1  Q groups 2t and 2t+1 (when Q is quantized here): lane l reads
//               row 32g + l%32, channels 32kk + 16*(l/32) + 0..15, exactly the
//               16 bytes it writes for kk
//   waves 2, 3  K rows 64t + 32*(w-2) + l%32, same channel split; the tile's
//               absolute maximum of K - k_mean is combined through LDS, then
//               each wave writes the codes of its 32 rows
//   all waves   the BF16 V tile is staged row-major in LDS; each 16-byte
//               output chunk then gathers 16 rows of one channel in the PV
//               operand order
// Blocks past the last K/V tile (t >= T, only when Q is quantized: the Q
// padding reaches 64*Tq >= 64*T rows) write the all-padding Q groups.
template <bool kNormRope>
__global__ __launch_bounds__(256) void quant_qkv_kernel(QuantArgs a) {
    __shared__ uint16_t tile[kBK * kVRow];
    __shared__ float k_amax[2];
    const int64_t blk = blockIdx.x;
    const int bh = (int)(blk / a.Tq);
    const int t = (int)(blk % a.Tq);
    const int b = bh / a.H, h = bh % a.H;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const bool kv = t < a.T;   // uniform over the block

    // V rows: thread (row, seg) loads 32 channels of one row.
    const int vrow = threadIdx.x >> 2;
    const int vseg = threadIdx.x & 3;
    const int half = wave - 2;
    const int c0 = 16 * (lane >> 5);
    const float* kmp = a.k_mean + (int64_t)bh * kHD + c0;
    const int kn = t * kBK + 32 * half + (lane & 31);
    uint4 kraw[4][2];
    if constexpr (kNormRope) {
        // This wave's Q or K row words are loaded first, then the V rows,
        // which go to LDS at once so that no V registers stay live through
        // the normalisation.
        const bool do_q = wave < 2 && a.q != nullptr;
        const bool do_k = wave >= 2 && kv;
        const int g = 2 * t + wave;
        const int n = do_q ? g * kQG + (lane & 31) : kn;
        const bool valid = (do_q || do_k) && n < a.N;
        const uint16_t* rp = do_q ? a.q + b * a.q_sb + (int64_t)n * a.q_sn + h * a.q_sh + c0
                                  : a.k + b * a.k_sb + (int64_t)n * a.k_sn + h * a.k_sh + c0;
        uint4 w[8];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            w[2 * kk] = valid ? *(const uint4*)(rp + 32 * kk) : make_uint4(0, 0, 0, 0);
            w[2 * kk + 1] = valid ? *(const uint4*)(rp + 32 * kk + 8) : make_uint4(0, 0, 0, 0);
        }
        if (kv) {
            const int nv = t * kBK + vrow;
            const uint16_t* vp = a.v + b * a.v_sb + (int64_t)nv * a.v_sn + h * a.v_sh + 32 * vseg;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(uint4*)(&tile[vrow * kVRow + 32 * vseg + 8 * i]) =
                    nv < a.N ? *(const uint4*)(vp + 8 * i) : make_uint4(0, 0, 0, 0);
        }
        if (do_q || do_k) {
            const int na = valid ? n : 0;
            norm_rope_row(w, lane >> 5, do_q ? a.nr.q_weight : a.nr.k_weight, a.nr.cos + (int64_t)na * (kHD / 2),
                          a.nr.sin + (int64_t)na * (kHD / 2), a.nr.eps);
        }
        if (do_q) {
            uint4 codes[4];
            const float scale = quant_q_words(w, codes);
            int8_t* out = a.q_i8 + ((int64_t)bh * a.G + g) * kQGroupBytes + lane * 16;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) *(uint4*)(out + kk * 64 * 16) = codes[kk];
            if (lane == 0) a.q_scale[(int64_t)bh * a.G + g] = scale;
        } else if (do_k) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) { kraw[kk][0] = w[2 * kk]; kraw[kk][1] = w[2 * kk + 1]; }
            const float am = wave_max(valid ? k_row_amax(kraw, kmp) : 0.0f);
            if (lane == 0) k_amax[half] = am;
        }
    } else {
        uint4 vraw[4];
        if (kv) {
            const int n = t * kBK + vrow;
            const uint16_t* vp = a.v + b * a.v_sb + (int64_t)n * a.v_sn + h * a.v_sh + 32 * vseg;
#pragma unroll
            for (int i = 0; i < 4; ++i) vraw[i] = n < a.N ? *(const uint4*)(vp + 8 * i) : make_uint4(0, 0, 0, 0);
        }
        if (wave < 2) {
            if (a.q != nullptr) {
                const int g = 2 * t + wave;
                const int n = g * kQG + (lane & 31);
                const uint16_t* qp = a.q + b * a.q_sb + (int64_t)n * a.q_sn + h * a.q_sh + c0;
                uint4 codes[4];
                const float scale = quant_q_group(qp, n < a.N, codes);
                int8_t* out = a.q_i8 + ((int64_t)bh * a.G + g) * kQGroupBytes + lane * 16;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) *(uint4*)(out + kk * 64 * 16) = codes[kk];
                if (lane == 0) a.q_scale[(int64_t)bh * a.G + g] = scale;
            }
        } else if (kv) {
            // this wave's share of the tile's absolute maximum of K - k_mean
            const bool valid = kn < a.N;
            const uint16_t* kp = a.k + b * a.k_sb + (int64_t)kn * a.k_sn + h * a.k_sh + c0;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                kraw[kk][0] = valid ? *(const uint4*)(kp + 32 * kk) : make_uint4(0, 0, 0, 0);
                kraw[kk][1] = valid ? *(const uint4*)(kp + 32 * kk + 8) : make_uint4(0, 0, 0, 0);
            }
            const float am = wave_max(valid ? k_row_amax(kraw, kmp) : 0.0f);
            if (lane == 0) k_amax[half] = am;
        }
        if (kv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) *(uint4*)(&tile[vrow * kVRow + 32 * vseg + 8 * i]) = vraw[i];
        }
    }
    __syncthreads();
    if (!kv) return;

    if (wave >= 2) {
        const float am = fmaxf(k_amax[0], k_amax[1]);
        float scale = 0.0f, inv = 0.0f;
        if (am >= kAmaxFloor) {
            scale = am / 127.0f;
            inv = 127.0f / am;
        }
        int8_t* out = a.k_i8 + ((int64_t)bh * a.T + t) * kTileBytes + lane * 16;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float x[16];
            unpack8(kraw[kk][0], x);
            unpack8(kraw[kk][1], x + 8);
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                const v4f m4 = *(const v4f*)(kmp + 32 * kk + i);
                x[i] = x[i] - m4[0];
                x[i + 1] = x[i + 1] - m4[1];
                x[i + 2] = x[i + 2] - m4[2];
                x[i + 3] = x[i + 3] - m4[3];
            }
            uint4 codes = pack16_int8(x, inv);
            if (kn >= a.N) codes = make_uint4(0, 0, 0, 0);
            *(uint4*)(out + (half * 4 + kk) * 64 * 16) = codes;
        }
        if (wave == 2 && lane == 0) a.k_scale[(int64_t)bh * a.T + t] = scale;
    }

    uint8_t* out = a.v_fp8 + ((int64_t)bh * a.T + t) * kTileBytes;
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
        const int c = threadIdx.x + 256 * rep;          // 16-byte chunk index
        const int db = c >> 7;
        const int vhalf = (c >> 6) & 1;
        const int l = c & 63;
        const int d = 32 * db + (l & 31);
        const int hh = l >> 5;
        const float inv = a.v_inv[(int64_t)bh * kHD + d];
        const bool zero = a.v_scale[(int64_t)bh * kHD + d] == 0.0f;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = 32 * vhalf + 8 * (i >> 2) + 4 * hh + (i & 3);
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
        a.nr = p.nr;
        if (p.norm_rope) {
            hipLaunchKernelGGL(tile_stats_nr_kernel, dim3((unsigned)a.units), dim3(256), 0, stream, a);
        } else {
            const int64_t threads = a.units * 16;
            hipLaunchKernelGGL(tile_stats_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
        }
    }
    {
        FinalizeArgs a;
        a.k_tile_sum = p.k_tile_sum; a.v_tile_amax = p.v_tile_amax;
        a.T = p.T; a.N = p.N;
        a.k_mean = p.k_mean; a.v_scale = p.v_scale; a.v_inv = p.v_inv;
        hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)BH), dim3(128), 0, stream, a);
    }
    {
        QuantArgs a;
        a.q = p.with_q ? p.q : nullptr; a.q_sb = p.q_sb; a.q_sn = p.q_sn; a.q_sh = p.q_sh;
        a.k = p.k; a.k_sb = p.k_sb; a.k_sn = p.k_sn; a.k_sh = p.k_sh;
        a.v = p.v; a.v_sb = p.v_sb; a.v_sn = p.v_sn; a.v_sh = p.v_sh;
        a.H = p.H; a.N = p.N; a.T = p.T; a.G = p.G;
        a.Tq = p.with_q ? p.G / 2 : p.T;
        a.k_mean = p.k_mean; a.v_inv = p.v_inv; a.v_scale = p.v_scale;
        a.q_i8 = p.q_i8; a.q_scale = p.q_scale; a.k_i8 = p.k_i8; a.k_scale = p.k_scale; a.v_fp8 = p.v_fp8;
        a.nr = p.nr;
        if (p.norm_rope)
            hipLaunchKernelGGL(quant_qkv_kernel<true>, dim3((unsigned)(BH * a.Tq)), dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL(quant_qkv_kernel<false>, dim3((unsigned)(BH * a.Tq)), dim3(256), 0, stream, a);
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
