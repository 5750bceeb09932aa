// attn_mainloop.hip -- fused INT8-QK / FP8-PV online-softmax mainloop for gfx950.
//
// "State-Ownership Architecture Decision", section "Non-Negotiable Dataflow":
// every K64/V64 tile in strictly increasing order; per tile QK, score
// scaling, max update, denominator update, FP8 probability conversion, PV
// and the FP32 RO addition; no N-by-N score tensor; no split of the KV walk;
// at the end the FP32 reciprocal of d, then normalisation, V scale and BF16
// into token-major NHD rows.  "Sage2 SM89 Temporal Pair Experiment", section
// "Candidate": each query row's per-tile sequence is QK -> update_mdo ->
// accumulate_d -> RS_32_to_8 -> PV, with private RS, RS_f8, RO, m and d.
//
// gfx950 design (not the pages' GB10 one):
//   * A workgroup of 8 wavefronts owns 256 query rows of one (b, h); wave w
//     owns the 32-row group g = 8*qb + w, so its Q scale is wave-uniform.
//   * Scores are computed transposed, S^T = K . Q^T, with
//     v_mfma_i32_32x32x32_i8: lane l then holds 32 keys of the single query
//     row l%32 (lanes l and l^32 share a row), so the row max and sum are
//     in-lane plus one exchange with lane l^32, and the FP8 probabilities
//     are already in the B-operand layout of the PV instruction.
//   * PV is O^T = V^T . P^T with v_mfma_scale_f32_32x32x64_f8f6f4 (scales
//     1.0), accumulating straight into the FP32 RO rows after the alpha
//     rescale, tile by tile in increasing order.
//   * K and V tiles (8 KiB each, already in operand order) are double
//     buffered in LDS; the next tile's 16-byte global loads are in flight
//     while the current tile is computed.
//   * The workgroup-to-(b, h, Q block) map keeps the workgroups that one XCD
//     runs on the same head, so that head's K/V stream is shared in its L2.
#include "sage_device.hpp"
#include "sage_launch.hpp"

namespace sage {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStageBytes = 2 * kTileBytes;       // K tile + V tile
constexpr float kLog2Of448 = 8.8073549220576041f;  // log2(448)

// Bijection from dispatch order to work items such that the items dispatched
// to one XCD (dispatch index mod 8) are consecutive.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
    const int q = nwg >> 3, r = nwg & 7;
    const int xcd = wg & 7, slot = wg >> 3;
    const int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return base + slot;
}

// QK of one wave against one staged K tile: s0 = S^T for keys 0..31, s1 for
// keys 32..63 (register r of lane l: key 8*(r/4) + 4*(l/32) + r%4 of its
// block, query row l%32 of the wave's group).  Exact int32.
__device__ __forceinline__ void qk_tile(const int8_t* ktile, const v4i (&qf)[4], int lane,
                                        v16i& s0, v16i& s1) {
    s0 = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    s1 = s0;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const v4i a0 = *(const v4i*)(ktile + ((0 * 4 + kk) * 64 + lane) * 16);
        const v4i a1 = *(const v4i*)(ktile + ((1 * 4 + kk) * 64 + lane) * 16);
        s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, qf[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, qf[kk], s1, 0, 0, 0);
    }
}

// Key index within the tile of accumulator register r (block blk) on lane l.
__device__ __forceinline__ int key_of(int blk, int r, int lane) {
    return 32 * blk + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

__global__ __launch_bounds__(kThreads, 1) void mainloop_kernel(MainloopArgs a) {
    __shared__ __attribute__((aligned(16))) int8_t lds[2 * kStageBytes];

    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = item / a.n_qblk;
    const int qb = item - bh * a.n_qblk;
    const int b = bh / a.H, h = bh - b * a.H;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = qb * kWaves + wave;
    const bool active = g < a.G && g * kQG < a.N;

    v4i qf[4];
    float qs = 0.0f;
    if (active) {
        const int8_t* qp = a.q_i8 + ((int64_t)bh * a.G + g) * kQGroupBytes + lane * 16;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[kk] = *(const v4i*)(qp + kk * 1024);
        qs = a.q_scale[(int64_t)bh * a.G + g];
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[kk] = v4i{0, 0, 0, 0};
    }

    const int8_t* kg = a.k_i8 + (int64_t)bh * a.T * kTileBytes + threadIdx.x * 16;
    const int8_t* vg = (const int8_t*)a.v_fp8 + (int64_t)bh * a.T * kTileBytes + threadIdx.x * 16;
    const float* ksc = a.k_scale + (int64_t)bh * a.T;

    v4i kr = *(const v4i*)kg;
    v4i vr = *(const v4i*)vg;
    *(v4i*)(lds + threadIdx.x * 16) = kr;
    *(v4i*)(lds + kTileBytes + threadIdx.x * 16) = vr;
    __syncthreads();

    float m = -INFINITY;
    float dpart = 0.0f;    // this lane's share of the row denominator
    v16f ro[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) ro[db][r] = 0.0f;

    const int tail = a.N - (a.T - 1) * kBK;   // valid keys in the last tile, 1..64

    for (int j = 0; j < a.T; ++j) {
        const int8_t* st = lds + (j & 1) * kStageBytes;
        const bool more = j + 1 < a.T;
        if (more) {
            kr = *(const v4i*)(kg + (int64_t)(j + 1) * kTileBytes);
            vr = *(const v4i*)(vg + (int64_t)(j + 1) * kTileBytes);
        }
        if (active) {
            v16i s0, s1;
            qk_tile(st, qf, lane, s0, s1);
            const bool last = (j == a.T - 1) && tail < kBK;
            if (last) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (key_of(0, r, lane) >= tail) s0[r] = INT32_MIN;
                    if (key_of(1, r, lane) >= tail) s1[r] = INT32_MIN;
                }
            }
            // Row max on the exact int32 sums (the score scale is positive).
            int mx = max(s0[0], s1[0]);
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = max(mx, max(s0[r], s1[r]));
            mx = max(mx, other_half(mx));
            const float sj = (qs * ksc[j]) * a.c;
            const float m_new = fmaxf(m, (float)mx * sj);
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            if (__any(m_new != m)) {
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) ro[db][r] *= alpha;
            }
            dpart *= alpha;
            m = m_new;
            // p = 448 * 2^(t - m) with 448 folded into the exponent offset.
            const float off = kLog2Of448 - m_new;
            float p[32];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s0[r], sj, off));
                p[16 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s1[r], sj, off));
            }
            if (last) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (key_of(0, r, lane) >= tail) p[r] = 0.0f;
                    if (key_of(1, r, lane) >= tail) p[16 + r] = 0.0f;
                }
            }
#pragma unroll
            for (int r = 0; r < 32; ++r) dpart += p[r];
            v8i pk;
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                int w = cvt_pk_e4m3<false>(p[4 * v], p[4 * v + 1], 0);
                pk[v] = cvt_pk_e4m3<true>(p[4 * v + 2], p[4 * v + 3], w);
            }
            const int8_t* vt = st + kTileBytes;
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const v4i lo = *(const v4i*)(vt + ((db * 2 + 0) * 64 + lane) * 16);
                const v4i hi = *(const v4i*)(vt + ((db * 2 + 1) * 64 + lane) * 16);
                const v8i vf = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                ro[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pk, ro[db], 0, 0, 0, 127, 0, 127);
            }
        }
        if (more) {
            int8_t* nx = lds + ((j + 1) & 1) * kStageBytes;
            *(v4i*)(nx + threadIdx.x * 16) = kr;
            *(v4i*)(nx + kTileBytes + threadIdx.x * 16) = vr;
        }
        __syncthreads();
    }

    if (!active) return;
    const float dtot = dpart + other_half(dpart);
    const float rcp = 1.0f / dtot;
    const int n = g * kQG + (lane & 31);
    if (n >= a.N) return;
    uint16_t* op = a.o + b * a.o_sb + (int64_t)n * a.o_sn + h * a.o_sh;
    const float* vs = a.v_scale + (int64_t)bh * kHD;
    const int h4 = 4 * (lane >> 5);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int d0 = 32 * db + 8 * rr + h4;
            const v4f s4 = *(const v4f*)(vs + d0);
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (ro[db][4 * rr + i] * rcp) * s4[i];
            const v2bf lo = v2bf{(__bf16)o[0], (__bf16)o[1]};
            const v2bf hi = v2bf{(__bf16)o[2], (__bf16)o[3]};
            uint2 wv;
            wv.x = __builtin_bit_cast(uint32_t, lo);
            wv.y = __builtin_bit_cast(uint32_t, hi);
            *(uint2*)(op + d0) = wv;
        }
    }
}

// One wave per (b, h, group g, tile t): the same QK tile routine as the
// mainloop, written out as int32 for inspection.
__global__ __launch_bounds__(64) void debug_qk_kernel(DebugQkArgs a) {
    __shared__ __attribute__((aligned(16))) int8_t kt[kTileBytes];
    const int g = blockIdx.x, t = blockIdx.y, bh = blockIdx.z;
    const int lane = threadIdx.x;
    const int8_t* kg = a.k_i8 + ((int64_t)bh * a.T + t) * kTileBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *(v4i*)(kt + (i * 64 + lane) * 16) = *(const v4i*)(kg + (i * 64 + lane) * 16);
    __syncthreads();
    v4i qf[4];
    const int8_t* qp = a.q_i8 + ((int64_t)bh * a.G + g) * kQGroupBytes + lane * 16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = *(const v4i*)(qp + kk * 1024);
    v16i s0, s1;
    qk_tile(kt, qf, lane, s0, s1);
    const int64_t Nq = (int64_t)a.G * kQG, Nk = (int64_t)a.T * kBK;
    int32_t* out = a.s_out + ((int64_t)bh * Nq + g * kQG + (lane & 31)) * Nk + (int64_t)t * kBK;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        out[key_of(0, r, lane)] = s0[r];
        out[key_of(1, r, lane)] = s1[r];
    }
}

}  // namespace

hipError_t launch_mainloop(const MainloopArgs& p, hipStream_t stream) {
    hipLaunchKernelGGL(mainloop_kernel, dim3((unsigned)p.n_items), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_debug_qk(const DebugQkArgs& p, hipStream_t stream) {
    hipLaunchKernelGGL(debug_qk_kernel, dim3((unsigned)p.G, (unsigned)p.T, (unsigned)(p.B * p.H)), dim3(64), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace sage
