// sage_launch.hpp -- kernel argument blocks and host launchers (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

// Optional RMSNorm + RoPE producer parameters (device pointers).
struct NormRopeArgs {
    const float* q_weight;   // [128]
    const float* k_weight;   // [128]
    const float* cos;        // [N][64], row n = token n
    const float* sin;        // [N][64]
    float eps;
};

struct StatsArgs {
    const uint16_t* k; int64_t k_sb, k_sn, k_sh;
    const uint16_t* v; int64_t v_sb, v_sn, v_sh;
    int H, N, T;
    int BH;              // B * H
    int64_t units;
    float* k_tile_sum;
    float* v_tile_amax;
    NormRopeArgs nr;
    // RMSNorm + RoPE pass only: the Q groups it quantizes as well (q null: none)
    const uint16_t* q; int64_t q_sb, q_sn, q_sh;
    int G;
    int8_t* q_i8; float* q_scale;
};

struct FinalizeArgs {
    const float* k_tile_sum;
    const float* v_tile_amax;
    int T, N;
    float* k_mean;
    float* v_scale;
    float* v_inv;
    float* k_scale_max;   // zeroed here, then raised by the quantizer
};

struct QuantArgs {
    const uint16_t* q; int64_t q_sb, q_sn, q_sh;   // null: Q is not quantized here
    const uint16_t* k; int64_t k_sb, k_sn, k_sh;
    const uint16_t* v; int64_t v_sb, v_sn, v_sh;
    int H, N, T, G;
    int BH;              // B * H
    int Tq;              // 64-row tiles per (b, h) this launch covers (>= T)
    const float* k_mean;
    const float* v_inv;
    const float* v_scale;
    int8_t* q_i8; float* q_scale;
    int8_t* k_i8; float* k_scale;
    float* k_scale_max;  // per (b, h): maximum of k_scale over the tiles
    uint8_t* v_fp8;
    NormRopeArgs nr;
};

struct PrepassArgs {
    int B, N, H, T, G;
    bool with_q;         // false: Q is quantized by the mainloop instead
    const uint16_t* q; int64_t q_sb, q_sn, q_sh;
    const uint16_t* k; int64_t k_sb, k_sn, k_sh;
    const uint16_t* v; int64_t v_sb, v_sn, v_sh;
    int8_t* q_i8; float* q_scale;
    int8_t* k_i8; float* k_scale; float* k_mean; float* k_scale_max;
    uint8_t* v_fp8; float* v_scale;
    float* k_tile_sum; float* v_tile_amax; float* v_inv;
    bool norm_rope;      // apply the RMSNorm + RoPE producer to Q and K first
    NormRopeArgs nr;
};

// Query groups (32 rows, one wavefront each) per mainloop workgroup.
constexpr int kMainloopWaves = 4;

struct MainloopArgs {
    const int8_t* q_i8; const float* q_scale;
    const int8_t* k_i8; const float* k_scale; const float* k_scale_max;
    const uint8_t* v_fp8; const float* v_scale;
    const uint16_t* q_bf16; int64_t q_sb, q_sn, q_sh;  // non-null: quantize Q from BF16 here
    NormRopeArgs nr;     // nr.q_weight non-null: RMSNorm + RoPE the BF16 Q rows first
    uint16_t* o; int64_t o_sb, o_sn, o_sh;   // output view of the range
    int B, N, H, T, G;
    int q_start, q_end;  // query rows [q_start, q_end) are written
    int h_start, h_count;
    int g_begin, g_end;  // 32-row groups overlapping the rows
    int n_qblk;          // workgroup Q blocks per (b, h) of the range
    int n_items;         // B * h_count * n_qblk
    float c;             // sm_scale * log2(e), rounded to FP32
};

struct DebugQkArgs {
    const int8_t* q_i8;
    const int8_t* k_i8;
    int32_t* s_out;
    int B, N, H, T, G;
};

hipError_t launch_prepass(const PrepassArgs& p, hipStream_t stream);
hipError_t launch_mainloop(const MainloopArgs& p, hipStream_t stream);
hipError_t launch_debug_qk(const DebugQkArgs& p, hipStream_t stream);
hipError_t launch_cvt_e4m3(const float* x, uint8_t* y, int64_t n, hipStream_t stream);

// Instruction streams of the issue probe (issue_probe.hip).
enum IssueProbeKind { kIssueMix = 0, kIssueMixMfma = 1, kIssueMfma = 2 };
hipError_t launch_issue_probe(int kind, int waves_per_simd, int blocks, int iters, uint64_t* ticks,
                              hipStream_t stream);

// Device address of this device's allocation-free workspace array
// (sage_noalloc.hip): resolved on the first call per device, then cached.
hipError_t noalloc_scratch(void** out);

}  // namespace sage
