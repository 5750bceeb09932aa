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
//   2. finalize      per (b,h): k_mean from the tile sums in tile order; V
//                    channel amax, v_scale = a/448, v_inv = 448/a
//   3. quant_qkv     per 64-row tile, one pass over its Q, K and V rows:
//                    INT8 Q per 32-row group, INT8 K - k_mean per tile,
//                    E4M3 V in the mainloop's layout (Q is skipped when the
//                    mainloop quantizes it itself)
// With the optional RMSNorm + RoPE producer on Q and K, launch 1 is
// tile_stats_nr, which also normalises and quantizes Q (needing neither
// k_mean nor the V scales), and launch 3 is quant_kv_nr: the normalised K
// rows are recomputed in launches 1 and 3 and never stored.
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

// The RMSNorm + RoPE kernels give each block two heads (bh0 and bh0 + 1) of
// one 64-row tile, so that all four waves do the same normalisation work, and
// take these items tile-major with the head pairs minor, through the XCD
// remap: each XCD then works through its own range of tiles with every head
// of a tile in flight together, so the tile's 64 angle rows (32 KiB) come
// from HBM once per XCD instead of once per head.
__device__ __forceinline__ void pair_item(int BH, int& t, int& bh0) {
    const int pairs = (BH + 1) >> 1;
    const int u = xcd_remap(blockIdx.x, gridDim.x);
    t = u / pairs;
    bh0 = 2 * (u - t * pairs);
}

// One row of 128 BF16 channels of the lane's share in the QK operand split
// (lane l: row l%32, channels 32kk + 16*(l/32) + 0..15 in w[2kk], w[2kk+1]);
// rows that are not valid read as zeros.  `p` points at a readable row in
// every lane (callers substitute a row that exists for one that does not),
// so the eight loads are issued together, outside any branch; the lanes
// whose row is not valid then clear their words.
__device__ __forceinline__ void load_row_words(const uint16_t* p, bool valid, uint4 (&w)[8]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        w[2 * kk] = *(const uint4*)(p + 32 * kk);
        w[2 * kk + 1] = *(const uint4*)(p + 32 * kk + 8);
    }
    if (!valid) {
        // a real branch (taken only in a tile's last rows), not 32 selects
        asm volatile("");
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = make_uint4(0, 0, 0, 0);
    }
}

// tile_stats with the RMSNorm + RoPE producer.  Wave w serves head bh0 + w/2
// and rows 32*(w%2) .. +31 of tile t:
//   * it loads those K rows and, with those loads still in flight, the V
//     rows: lane (c8 = l%16, rp = l/16) takes the absolute maxima of V
//     channels 8c8 .. 8c8+7 over its rows rp, rp+4, ..., rp+28 of the wave's
//     32; the four lanes of one c8 combine across the wave and leave the
//     wave's 128 channel maxima in LDS;
//   * it normalises and rotates the K rows (norm_rope_row) and stages the
//     BF16 results in LDS;
//   * when Q is quantized in this pass, it does the same normalisation for
//     Q group 2t + w%2 of its head and writes that group's INT8 codes and
//     scale (blocks past the last K/V tile, t >= T, do only this: the Q
//     padding reaches 64 * G/2 >= 64 * T rows).
// Then thread (s = u/128, d = u%128) sums channel d of head bh0 + s's staged
// rows in row order and combines the two halves' V maxima of channel d.
__global__ __launch_bounds__(256) void tile_stats_nr_kernel(StatsArgs a) {
    __shared__ uint16_t tile[2][kBK * kVRow];
    __shared__ float vam[2][2][kHD];
    // the RMSNorm weights of K and Q, read from LDS by every row: 64 fewer
    // global loads per lane and row
    __shared__ float wts[2][kHD];
    wts[threadIdx.x >> 7][threadIdx.x & 127] = (threadIdx.x < 128 ? a.nr.k_weight : a.nr.q_weight)[threadIdx.x & 127];
    __syncthreads();
    int t, bh0;
    pair_item(a.BH, t, bh0);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int hs = wave >> 1, half = wave & 1;
    const int bh = bh0 + hs;
    const bool head = bh < a.BH;     // uniform per wave
    const int b = bh / a.H, h = bh - b * a.H;
    const bool kv = t < a.T;         // uniform per block
    const int n0 = t * kBK;
    const int hf = lane >> 5;
    if (kv && head) {
        const int rows = min(kBK, a.N - n0);
        const int row = 32 * half + (lane & 31);
        const int n = n0 + row;
        const bool valid = row < rows;
        uint4 w[8];
        load_row_words(a.k + b * a.k_sb + (int64_t)(valid ? n : n0) * a.k_sn + h * a.k_sh + 16 * hf, valid, w);

        // V maxima first, with all eight row loads in flight together
        // alongside the K row's: a row past the tile's end reads the tile's
        // last row instead, which leaves the tile's maximum unchanged (the
        // two halves' maxima are only used combined).
        const int c8 = lane & 15, rp = lane >> 4;
        const uint16_t* vp = a.v + b * a.v_sb + h * a.v_sh + 8 * c8;
        uint4 vraw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            vraw[i] = *(const uint4*)(vp + (int64_t)(n0 + min(32 * half + rp + 4 * i, rows - 1)) * a.v_sn);
        float am[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) am[c] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float vf[8];
            unpack8(vraw[i], vf);
#pragma unroll
            for (int c = 0; c < 8; ++c) am[c] = fmaxf(am[c], fabsf(vf[c]));
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            am[c] = fmaxf(am[c], __shfl_xor(am[c], 16, 64));
            am[c] = fmaxf(am[c], __shfl_xor(am[c], 32, 64));
        }
        if (lane < 16) {
#pragma unroll
            for (int c = 0; c < 8; ++c) vam[hs][half][8 * c8 + c] = am[c];
        }

        const int na = valid ? n : 0;
        norm_rope_row(w, hf, wts[0], a.nr.cos + (int64_t)na * (kHD / 2), a.nr.sin + (int64_t)na * (kHD / 2),
                      a.nr.eps);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                *(uint4*)(&tile[hs][row * kVRow + 32 * kk + 16 * hf + 8 * e]) = w[2 * kk + e];
    }
    if (a.q != nullptr && head) {
        const int g = 2 * t + half;
        const int n = g * kQG + (lane & 31);
        const bool valid = n < a.N;
        uint4 w[8];
        load_row_words(a.q + b * a.q_sb + (int64_t)min(n, a.N - 1) * a.q_sn + h * a.q_sh + 16 * hf, valid, w);
        const int na = valid ? n : 0;
        norm_rope_row(w, hf, wts[1], a.nr.cos + (int64_t)na * (kHD / 2), a.nr.sin + (int64_t)na * (kHD / 2),
                      a.nr.eps);
        uint4 codes[4];
        const float scale = quant_q_words(w, codes);
        int8_t* out = a.q_i8 + ((int64_t)bh * a.G + g) * kQGroupBytes + lane * 16;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) *(uint4*)(out + kk * 64 * 16) = codes[kk];
        if (lane == 0) a.q_scale[(int64_t)bh * a.G + g] = scale;
    }
    if (!kv) return;                 // uniform per block: no wave reaches the barrier
    __syncthreads();
    const int sl = threadIdx.x >> 7, d = threadIdx.x & 127;
    const int bhs = bh0 + sl;
    if (bhs >= a.BH) return;
    const int rows = min(kBK, a.N - n0);
    const uint16_t* col = &tile[sl][d];
    float sum = 0.0f;
    if (rows == kBK) {
        // all 64 LDS reads in flight before the ordered adds
        float x[kBK];
#pragma unroll
        for (int row = 0; row < kBK; ++row) x[row] = bf16_bits_to_f32(col[row * kVRow]);
#pragma unroll
        for (int row = 0; row < kBK; ++row) sum = sum + x[row];
    } else {
        for (int row = 0; row < rows; ++row) sum = sum + bf16_bits_to_f32(col[row * kVRow]);
    }
    const int64_t o = ((int64_t)bhs * a.T + t) * kHD + d;
    a.k_tile_sum[o] = sum;
    a.v_tile_amax[o] = fmaxf(vam[sl][0][d], vam[sl][1][d]);
}

// One block of 128 threads per (b, h); thread d owns channel d.
__global__ __launch_bounds__(128) void finalize_kernel(FinalizeArgs a) {
    const int bh = blockIdx.x;
    const int d = threadIdx.x;
    const float* ks = a.k_tile_sum + (int64_t)bh * a.T * kHD + d;
    const float* va = a.v_tile_amax + (int64_t)bh * a.T * kHD + d;
    // Sequential in tile order; loads are issued 64 tiles ahead of the adds.
    constexpr int kBatch = 64;
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
    if (d == 0) a.k_scale_max[bh] = 0.0f;    // the quantizer raises it tile by tile
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

// INT8 codes of one wave's 32 K rows minus k_mean at scale am/127 (am: the
// tile's absolute maximum of K - k_mean; below 2^-100 the scale is 0 and the
// codes are zero), in the QK operand order of tile half `half`: lane l holds
// row 32*half + l%32 as kraw (see k_row_amax); rows at or beyond N get zero
// codes.  Returns the scale.
__device__ __forceinline__ float k_codes(const uint4 (&kraw)[4][2], const float* kmp, float am, bool row_valid,
                                         int8_t* tile_out, int half, int lane) {
    float scale = 0.0f, inv = 0.0f;
    if (am >= kAmaxFloor) {
        scale = am / 127.0f;
        inv = 127.0f / am;
    }
    int8_t* out = tile_out + lane * 16;
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
        if (!row_valid) codes = make_uint4(0, 0, 0, 0);
        *(uint4*)(out + (half * 4 + kk) * 64 * 16) = codes;
    }
    return scale;
}

// E4M3 codes of one BF16 V tile staged row-major in LDS (pitch kVRow), in
// the PV operand order: each 16-byte output chunk gathers 16 rows of one
// channel; the block's 256 threads write the tile's 512 chunks.
__device__ __forceinline__ void v_codes(const uint16_t* tile, const float* v_inv, const float* v_scale,
                                        uint8_t* out) {
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
        const int c = threadIdx.x + 256 * rep;          // 16-byte chunk index
        const int db = c >> 7;
        const int vhalf = (c >> 6) & 1;
        const int l = c & 63;
        const int d = 32 * db + (l & 31);
        const int hh = l >> 5;
        const float inv = v_inv[d];
        const bool zero = v_scale[d] == 0.0f;
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

// One block of 256 threads per (b, h, 64-row tile t) quantizes everything the
// tile's rows hold, so each projection row segment is read once:
//   waves 0, 1  Q groups 2t and 2t+1 (when Q is quantized here): lane l reads
//               row 32g + l%32, channels 32kk + 16*(l/32) + 0..15, exactly
//               the 16 bytes it writes for kk
//   waves 2, 3  K rows 64t + 32*(w-2) + l%32, same channel split; the tile's
//               absolute maximum of K - k_mean is combined through LDS, then
//               each wave writes the codes of its 32 rows
//   all waves   the BF16 V tile is staged row-major in LDS, then v_codes
// Blocks past the last K/V tile (t >= T, only when Q is quantized: the Q
// padding reaches 64*Tq >= 64*T rows) write the all-padding Q groups.
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
    __syncthreads();
    if (!kv) return;

    if (wave >= 2) {
        const float scale = k_codes(kraw, kmp, fmaxf(k_amax[0], k_amax[1]), kn < a.N,
                                    a.k_i8 + ((int64_t)bh * a.T + t) * kTileBytes, half, lane);
        if (wave == 2 && lane == 0) {
            a.k_scale[(int64_t)bh * a.T + t] = scale;
            // the head's largest K scale: scales are >= 0, so their bit
            // patterns order as the values do
            atomicMax((unsigned int*)a.k_scale_max + bh, __float_as_uint(scale));
        }
    }
    v_codes(tile, a.v_inv + (int64_t)bh * kHD, a.v_scale + (int64_t)bh * kHD,
            a.v_fp8 + ((int64_t)bh * a.T + t) * kTileBytes);
}

// K and V quantization with the RMSNorm + RoPE producer applied to K (Q is
// quantized by tile_stats_nr or by the mainloop): one block of 256 threads
// per (tile t, heads bh0 and bh0 + 1), see pair_item.  Wave w loads K rows
// 32*(w%2) + l%32 of head bh0 + w/2, normalises and rotates them, and takes
// their share of the tile's absolute maximum of K - k_mean; every thread
// stages 32 channels of one V row of each head in LDS.  After the barrier
// each wave writes the codes of its 32 K rows and the block writes both V
// tiles (v_codes).
__global__ __launch_bounds__(256) void quant_kv_nr_kernel(QuantArgs a) {
    __shared__ uint16_t tile[2][kBK * kVRow];
    __shared__ float k_amax[2][2];
    __shared__ float wts[kHD];         // the RMSNorm weights of K, read from LDS by every row
    if (threadIdx.x < kHD) wts[threadIdx.x] = a.nr.k_weight[threadIdx.x];
    __syncthreads();
    int t, bh0;
    pair_item(a.BH, t, bh0);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int hs = wave >> 1, half = wave & 1;
    const int bh = bh0 + hs;
    const bool head = bh < a.BH;     // uniform per wave
    const int b = bh / a.H, h = bh - b * a.H;
    const int c0 = 16 * (lane >> 5);
    const int kn = t * kBK + 32 * half + (lane & 31);
    const bool valid = head && kn < a.N;
    uint4 w[8];
    {
        // waves of a missing second head read the first head's row
        const int bl = head ? bh : bh0;
        const int bb = bl / a.H, hh = bl - bb * a.H;
        load_row_words(a.k + bb * a.k_sb + (int64_t)min(kn, a.N - 1) * a.k_sn + hh * a.k_sh + c0, valid, w);
    }
    {
        const int vrow = threadIdx.x >> 2;
        const int vseg = threadIdx.x & 3;
        const int n = t * kBK + vrow;
        // all eight loads in flight together: rows past the end read row
        // N - 1 and stage zeros; the second head of a pair past the last
        // head reads the first head's row and stages nothing
        const int nl = min(n, a.N - 1);
        uint4 vraw[2][4];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            const int bv = min(bh0 + sl, a.BH - 1);
            const int vb = bv / a.H, vh = bv - vb * a.H;
            const uint16_t* vp = a.v + vb * a.v_sb + (int64_t)nl * a.v_sn + vh * a.v_sh + 32 * vseg;
#pragma unroll
            for (int i = 0; i < 4; ++i) vraw[sl][i] = *(const uint4*)(vp + 8 * i);
        }
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            if (bh0 + sl >= a.BH) break;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(uint4*)(&tile[sl][vrow * kVRow + 32 * vseg + 8 * i]) =
                    n < a.N ? vraw[sl][i] : make_uint4(0, 0, 0, 0);
        }
    }
    const float* kmp = a.k_mean + (int64_t)bh * kHD + c0;
    uint4 kraw[4][2];
    if (head) {
        const int na = valid ? kn : 0;
        norm_rope_row(w, lane >> 5, wts, a.nr.cos + (int64_t)na * (kHD / 2),
                      a.nr.sin + (int64_t)na * (kHD / 2), a.nr.eps);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) { kraw[kk][0] = w[2 * kk]; kraw[kk][1] = w[2 * kk + 1]; }
        const float am = wave_max(valid ? k_row_amax(kraw, kmp) : 0.0f);
        if (lane == 0) k_amax[hs][half] = am;
    }
    __syncthreads();
    if (head) {
        const float scale = k_codes(kraw, kmp, fmaxf(k_amax[hs][0], k_amax[hs][1]), kn < a.N,
                                    a.k_i8 + ((int64_t)bh * a.T + t) * kTileBytes, half, lane);
        if (half == 0 && lane == 0) {
            a.k_scale[(int64_t)bh * a.T + t] = scale;
            atomicMax((unsigned int*)a.k_scale_max + bh, __float_as_uint(scale));
        }
    }
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
        const int bv = bh0 + sl;
        if (bv >= a.BH) break;
        v_codes(tile[sl], a.v_inv + (int64_t)bv * kHD, a.v_scale + (int64_t)bv * kHD,
                a.v_fp8 + ((int64_t)bv * a.T + t) * kTileBytes);
    }
}

}  // namespace

hipError_t launch_prepass(const PrepassArgs& p, hipStream_t stream) {
    const int64_t BH = (int64_t)p.B * p.H;
    const int64_t pairs = (BH + 1) / 2;    // head pairs of the RMSNorm + RoPE kernels
    {
        StatsArgs a;
        a.k = p.k; a.k_sb = p.k_sb; a.k_sn = p.k_sn; a.k_sh = p.k_sh;
        a.v = p.v; a.v_sb = p.v_sb; a.v_sn = p.v_sn; a.v_sh = p.v_sh;
        a.H = p.H; a.N = p.N; a.T = p.T; a.BH = (int)BH; a.units = BH * p.T;
        a.k_tile_sum = p.k_tile_sum; a.v_tile_amax = p.v_tile_amax;
        a.nr = p.nr;
        a.q = p.with_q ? p.q : nullptr; a.q_sb = p.q_sb; a.q_sn = p.q_sn; a.q_sh = p.q_sh;
        a.G = p.G; a.q_i8 = p.q_i8; a.q_scale = p.q_scale;
        if (p.norm_rope) {
            const int64_t tiles = p.with_q ? p.G / 2 : p.T;
            hipLaunchKernelGGL(tile_stats_nr_kernel, dim3((unsigned)(pairs * tiles)), dim3(256), 0, stream, a);
        } else {
            const int64_t threads = a.units * 16;
            hipLaunchKernelGGL(tile_stats_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
        }
    }
    {
        FinalizeArgs a;
        a.k_tile_sum = p.k_tile_sum; a.v_tile_amax = p.v_tile_amax;
        a.T = p.T; a.N = p.N;
        a.k_mean = p.k_mean; a.v_scale = p.v_scale; a.v_inv = p.v_inv; a.k_scale_max = p.k_scale_max;
        hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)BH), dim3(128), 0, stream, a);
    }
    {
        QuantArgs a;
        a.q = p.with_q && !p.norm_rope ? p.q : nullptr; a.q_sb = p.q_sb; a.q_sn = p.q_sn; a.q_sh = p.q_sh;
        a.k = p.k; a.k_sb = p.k_sb; a.k_sn = p.k_sn; a.k_sh = p.k_sh;
        a.v = p.v; a.v_sb = p.v_sb; a.v_sn = p.v_sn; a.v_sh = p.v_sh;
        a.H = p.H; a.N = p.N; a.T = p.T; a.G = p.G; a.BH = (int)BH;
        a.Tq = a.q != nullptr ? p.G / 2 : p.T;
        a.k_mean = p.k_mean; a.v_inv = p.v_inv; a.v_scale = p.v_scale;
        a.q_i8 = p.q_i8; a.q_scale = p.q_scale; a.k_i8 = p.k_i8; a.k_scale = p.k_scale; a.v_fp8 = p.v_fp8;
        a.k_scale_max = p.k_scale_max;
        a.nr = p.nr;
        if (p.norm_rope)
            hipLaunchKernelGGL(quant_kv_nr_kernel, dim3((unsigned)(pairs * p.T)), dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL(quant_qkv_kernel, dim3((unsigned)(BH * a.Tq)), dim3(256), 0, stream, a);
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
