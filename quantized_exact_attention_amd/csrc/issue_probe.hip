// issue_probe.hip -- measures what the mainloop's tile step costs to issue on
// this GPU, for the vector roofline the benchmark reports next to the matrix
// one.  Each wave of one or more workgroups of 4*w waves (w waves per SIMD)
// runs `iters` iterations of one instruction stream and writes the shader
// clock cycles it took (s_memtime before and after).  The streams:
//
//   kIssueMix       the vector work of one 32-query x 64-key wave tile under
//                   the contract's per-score arithmetic (fused form): 32
//                   float(S) subtractions, 32 score FMAs, 32 exp2, 32
//                   denominator adds, 16 E4M3 pair conversions, 16
//                   three-input maxima -- 160 instructions, no memory
//   kIssueMixMfma   the same, then the tile's matrix work in one burst: 4
//                   FP8 32x32x64 and 8 INT8 32x32x32 instructions
//   kIssueMfma      the 12 matrix instructions alone
//
// The operands are registers that never change; results are discarded (a
// value is stored only so that the compiler keeps the work).  The vector
// streams are inline assembly of ALU instructions only, so their order and
// count are exactly as written.
#include <hip/hip_runtime.h>

#include "sage_device.hpp"
#include "sage_launch.hpp"

namespace sage {
namespace {

#define SAGE_R8 "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
// two scores' worth of the tile step's vector work (ten instructions)
#define SAGE_MIX2                                                        \
    "v_add_f32 %0, 0xcb400000, %0\n v_add_f32 %1, 0xcb400000, %1\n"      \
    "v_fma_f32 %2, %2, %8, %9\n v_fma_f32 %3, %3, %8, %9\n"              \
    "v_exp_f32 %4, %4\n v_exp_f32 %5, %5\n"                              \
    "v_add_f32 %6, %6, %8\n v_add_f32 %7, %7, %8\n"                      \
    "v_cvt_pk_fp8_f32 %0, %8, %9\n v_max3_i32 %1, %1, %8, %9\n"

__device__ __forceinline__ void mix_tile(float& a0, float& a1, float& a2, float& a3, float& a4, float& a5,
                                         float& a6, float& a7, float b, float c) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        asm volatile(SAGE_MIX2 SAGE_MIX2 SAGE_MIX2 SAGE_MIX2 : SAGE_R8 : "v"(b), "v"(c));
}

template <int kKind>
__global__ __launch_bounds__(1024) void issue_probe_kernel(uint64_t* ticks, int iters) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float a0 = lane * 1e-3f, a1 = a0 + 1.0f, a2 = a0 + 2.0f, a3 = a0 + 3.0f, a4 = a0 + 4.0f, a5 = a0 + 5.0f,
          a6 = a0 + 6.0f, a7 = a0 + 7.0f;
    const float b = 0.999f + lane * 1e-6f, c = 1e-3f;
    v16i s0 = {}, s1 = {};
    v16f f0 = {}, f1 = {}, f2 = {}, f3 = {};
    const v4i qa = {lane, 1, 2, 3}, qb = {3, 2, 1, lane};
    const v8i pa = {lane, 1, 2, 3, 4, 5, 6, 7}, pb = {7, 6, 5, 4, 3, 2, 1, lane};
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
        if (kKind != kIssueMfma) mix_tile(a0, a1, a2, a3, a4, a5, a6, a7, b, c);
        __builtin_amdgcn_sched_barrier(0);
        if (kKind != kIssueMix) {
            f0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, pb, f0, 0, 0, 0, 0, 0, 0);
            f1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pb, pa, f1, 0, 0, 0, 0, 0, 0);
            f2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, pa, f2, 0, 0, 0, 0, 0, 0);
            f3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pb, pb, f3, 0, 0, 0, 0, 0, 0);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(kk & 1 ? qa : qb, qa, s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(kk & 1 ? qb : qa, qb, s1, 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    float keep = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
    int ikeep = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        keep += f0[r] + f1[r] + f2[r] + f3[r];
        ikeep += s0[r] + s1[r];
    }
    uint64_t* out = ticks + (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
    if (lane == 0) *out = t1 - t0;
    // never true for these operands; keeps every result live
    if (keep == 1234.5f || ikeep == 7) *out = 0;
}

}  // namespace

hipError_t launch_issue_probe(int kind, int waves_per_simd, int blocks, int iters, uint64_t* ticks,
                              hipStream_t stream) {
    const dim3 grid((unsigned)blocks), block((unsigned)(256 * waves_per_simd));
    switch (kind) {
        case kIssueMix: hipLaunchKernelGGL(issue_probe_kernel<kIssueMix>, grid, block, 0, stream, ticks, iters); break;
        case kIssueMixMfma:
            hipLaunchKernelGGL(issue_probe_kernel<kIssueMixMfma>, grid, block, 0, stream, ticks, iters);
            break;
        default: hipLaunchKernelGGL(issue_probe_kernel<kIssueMfma>, grid, block, 0, stream, ticks, iters); break;
    }
    return hipGetLastError();
}

}  // namespace sage
