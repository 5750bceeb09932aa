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
//   * A workgroup of kMainloopWaves (4) wavefronts owns 128 query rows of one
//     (b, h); wave w owns the 32-row group g = 4*qb + w, so its Q scale is
//     wave-uniform.  Three workgroups share a CU (three waves per SIMD, at
//     most 168 VGPRs each) and synchronise independently of each other, so
//     one wave's vector work overlaps the other waves' matrix instructions.
//   * Scores are computed transposed, S^T = K . Q^T, with
//     v_mfma_i32_32x32x32_i8: lane l then holds 32 keys of the single query
//     row l%32 (lanes l and l^32 share a row), so the row max and sum are
//     in-lane plus one exchange with lane l^32, and the FP8 probabilities
//     are already in the B-operand layout of the PV instruction.
//   * PV is O^T = V^T . P^T with the unscaled v_mfma_f32_32x32x64_f8f6f4,
//     accumulating straight into the FP32 RO rows after the alpha rescale,
//     tile by tile in increasing order.
//   * Per iteration a wave issues the previous tile's PV (four matrix
//     instructions), runs the vector phase (the softmax of one tile) and
//     then the next tile's QK; the PV runs under the wave's own softmax, and
//     the three waves of a SIMD overlap each other's phases.  (Workgroups
//     that take the stepwise score form keep each tile's PV after its own
//     softmax.)
//   * K and V tiles (8 KiB each, already in operand order) stream through
//     three-slot LDS rings (48 KiB per workgroup) filled by direct
//     global-to-LDS loads issued two tiles ahead of their use.
//   * The workgroup-to-(b, h, Q block) map keeps the workgroups that one XCD
//     runs on the same head, so that head's K/V stream is shared in its L2.
#include "sage_device.hpp"
#include "sage_launch.hpp"

namespace sage {
namespace {

constexpr int kWaves = kMainloopWaves;
constexpr int kThreads = kWaves * 64;
// Workgroups per CU = waves per SIMD: the register budget (512 / 3 -> 168
// VGPRs per wave) the compiler is held to, and 3 x 48 KiB of LDS.
constexpr int kWavesPerSimd = 3;
// 1 KiB DMA instructions per wave per 8 KiB tile
constexpr int kTileLoads = kTileBytes / (kWaves * 1024);
static_assert(kTileLoads * kWaves * 1024 == kTileBytes, "tile split");
constexpr float kLog2Of448 = 8.8073549220576041f;  // log2(448)

// Scheduling fence: the compiler moves no instruction across it.
#define SAGE_FENCE() __builtin_amdgcn_sched_barrier(0)

// Score accumulators start at the bit pattern of 1.5 * 2^23 instead of 0.
// Every |S| <= 128 * 127 * 127 < 2^22, so the int32 result 0x4B400000 + S is
// the FP32 number 1.5 * 2^23 + S (fixed exponent, S in the mantissa): one
// exact FP32 subtraction gives float(S) without a conversion instruction,
// and the integer maximum of the biased words is the biased maximum of S.
constexpr int kScoreBias = 0x4B400000;
constexpr float kScoreBiasF = 12582912.0f;

__device__ __forceinline__ float unbias(int s) { return __int_as_float(s) - kScoreBiasF; }

// QK of one wave against one staged K tile: s0 = S^T for keys 0..31, s1 for
// keys 32..63 (register r of lane l: key 8*(r/4) + 4*(l/32) + r%4 of its
// block, query row l%32 of the wave's group), exact int32 plus the initial
// accumulator `init` (the mainloop passes the score bias below).
__device__ __forceinline__ void qk_tile(const int8_t* ktile, const v4i (&qf)[4], int lane, v16i& s0, v16i& s1,
                                        const v16i& init) {
    s0 = init;
    s1 = init;
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

// E4M3 x E4M3 -> FP32, 32x32x64 without block scales: zero scale operands
// select the unscaled v_mfma_f32_32x32x64_f8f6f4 (same products as unit
// scales).  The unscaled form also has no scale VGPR operand, whose value
// the scaled form reads with a latency that a write a few instructions
// earlier does not meet.
__device__ __forceinline__ v16f mfma_pv(const v8i& vf, const v8i& pk, const v16f& acc) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pk, acc, 0, 0, 0, 0, 0, 0);
}

// PV of one wave against one staged V tile: ro[db] += V^T(rows 32db..) . P^T,
// accumulated straight into the FP32 output rows.
__device__ __forceinline__ void pv_tile(const int8_t* vtile, const v8i& pk, int lane, v16f (&ro)[4]) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const v4i lo = *(const v4i*)(vtile + ((db * 2 + 0) * 64 + lane) * 16);
        const v4i hi = *(const v4i*)(vtile + ((db * 2 + 1) * 64 + lane) * 16);
        const v8i vf = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        ro[db] = mfma_pv(vf, pk, ro[db]);
    }
}

// Online softmax of one tile for this lane's query row (32 of the tile's keys
// here, the other 32 on lane l^32), on biased sums (kScoreBias): max update on
// the exact int32 sums (the score scale sj is positive, so the largest sum
// gives the largest score), alpha = 2^(m - m_new), p = 448 * 2^(t - m_new),
// this lane's part of the denominator, and the FP8 codes packed in the
// B-operand order of the PV instruction.  kLast masks keys at or beyond
// `tail` in the final, partial tile.  `moved` reports that some row maximum
// of the wave moved, which is also exactly when RO needs the alpha rescale.
//
// Two forms of the score step (kStepwise), one per workgroup for the whole
// loop:
//   * stepwise, the definition's roundings one by one: t = fl(S * sj),
//     x = fl(t - m), p = fl(448 * 2^x);
//   * fused, two vector instructions fewer per score: p = 2^fma(S, sj, off)
//     with off = log2(448) - m, kept across tiles and recomputed when a row
//     maximum moves.  It rounds once where the stepwise form rounds three
//     times; the two differ by about one unit in the last place of m,
//     relative, in p.  The fused form is taken only by workgroups whose
//     scores are all bounded by 2^12 in magnitude (in log2 units, see
//     kStepwiseFrom), where that difference is below 2^-11 of p, a small
//     fraction of an E4M3 step; real attention has |m| of a few units.
template <bool kStepwise, bool kLast>
__device__ __forceinline__ void softmax_tile(v16i& s0, v16i& s1, float sj, int tail, int lane, float& m,
                                             float& off, float& dpart, float& alpha, bool& moved, v8i& pk) {
    if (kLast) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (key_of(0, r, lane) >= tail) s0[r] = INT32_MIN;
            if (key_of(1, r, lane) >= tail) s1[r] = INT32_MIN;
        }
    }
    int ma = max(s0[0], s0[1]);
    int mb = max(s1[0], s1[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
        ma = max(max(ma, s0[r]), s0[r + 1]);
        mb = max(max(mb, s1[r]), s1[r + 1]);
    }
    // the tile's largest score of the row, t = fl(S * sj) of the largest S
    // (unbias is exact); a compare and a select rather than fmaxf, which
    // would add a NaN-quieting instruction (m and t are never NaN here)
    const float tmax = unbias(halves_max(max(ma, mb))) * sj;
    const bool up = tmax > m;
    const float m_new = up ? tmax : m;
    moved = __any(up);
    alpha = 1.0f;           // 2^(m - m_new) is exactly 1 where m does not move
    if (moved) {
        // A real branch: the empty volatile asm keeps the compiler from
        // turning this block into selects, which would run its exp2 on every
        // tile (about 80% of tiles move no maximum).
        asm volatile("");
        alpha = __builtin_amdgcn_exp2f(m - m_new);
        dpart *= alpha;
        if (!kStepwise) off = kLog2Of448 - m_new;
    }
    m = m_new;
    float p[32];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        if (kStepwise) {
            const float t0 = unbias(s0[r]) * sj, t1 = unbias(s1[r]) * sj;
            p[r] = 448.0f * __builtin_amdgcn_exp2f(t0 - m);
            p[16 + r] = 448.0f * __builtin_amdgcn_exp2f(t1 - m);
        } else {
            p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(unbias(s0[r]), sj, off));
            p[16 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(unbias(s1[r]), sj, off));
        }
    }
    if (kLast) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (key_of(0, r, lane) >= tail) p[r] = 0.0f;
            if (key_of(1, r, lane) >= tail) p[16 + r] = 0.0f;
        }
    }
    // this lane's share of the denominator (four chains over the 32 values,
    // three of them started from a value rather than from zero)
    float d0 = dpart, d1 = p[1], d2 = p[2], d3 = p[3];
    d0 += p[0];
#pragma unroll
    for (int r = 4; r < 32; r += 4) {
        d0 += p[r];
        d1 += p[r + 1];
        d2 += p[r + 2];
        d3 += p[r + 3];
    }
    dpart = (d0 + d1) + (d2 + d3);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int w = cvt_pk_e4m3<false>(p[4 * v], p[4 * v + 1], __float_as_int(p[4 * v]));
        pk[v] = cvt_pk_e4m3<true>(p[4 * v + 2], p[4 * v + 3], w);
    }
}

// Scores of magnitude at or above this (log2 units) take the stepwise form.
// A workgroup takes the fused form only when a bound on all of its waves'
// scores lies below it (see the kernel's prologue).
constexpr float kStepwiseFrom = 4096.0f;   // 2^12

__device__ __forceinline__ void rescale(v16f (&ro)[4], float alpha) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) ro[db][r] *= alpha;
}

// LDS rings: K and V tiles in 3 slots each, filled straight from global
// memory by global_load_lds_dwordx4 (no VGPR staging).  In iteration j a
// wave runs the softmax of tile j (scores computed in the previous
// iteration), the PV of tile j-1 (fused score form; tile j in the stepwise
// form) and the QK of tile j+1, while the workgroup's loads of K(j+3) and of
// V(j+1) (V(j+2) in the stepwise form) are in flight; the loads issued one
// iteration earlier are waited for before the barrier that ends the
// iteration.  The fused form runs three iterations per loop pass, so that
// every slot is a constant LDS offset (fused_step); the stepwise form
// rotates slot pointers.  RO receives every tile's PV in increasing tile
// order, each after the rescale by that tile's alpha.
constexpr int kKSlots = 3;
constexpr int kVSlots = 3;

// Each wave copies its share (kTileLoads KiB) of an 8 KiB tile from global
// memory into an LDS slot; lane l's 16 bytes of each KiB land at that KiB's
// base + 16*l (LDS address taken from M0, which is restored afterwards; the
// instruction reads it at issue, one wait state after the SALU write).
// The global address is the tile base in an SGPR pair (wave-uniform, formed
// by scalar instructions) plus the lane's fixed 32-bit byte offset `voff`
// (+1 KiB per further load), so the loads cost no vector instructions.
// Issued as inline assembly so that the compiler does not make every later
// LDS read wait for these loads: the instruction writes no
// VGPR, and the only consumer synchronisation is the explicit vmcnt wait
// before the block barrier that publishes the tile.
__device__ __forceinline__ void tile_to_lds(const int8_t* gtile, int8_t* slot, uint32_t voff, int wave) {
#pragma unroll
    for (int i = 0; i < kTileLoads; ++i) {
        const int part = wave * kTileLoads + i;
        // wave-uniform (wave is), so the compiler forms it in an SGPR
        const uint32_t dst = (uint32_t)(uintptr_t)(slot + part * 1024);
        uint32_t saved_m0;
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %3\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %2\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved_m0)
            : "v"(voff + i * 1024), "s"(gtile), "s"(dst)
            : "memory");
    }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8, the other counters left at their maxima): wait
// until no vector-memory operation of this wave is outstanding, or until at
// most the 2 * kTileLoads tile loads issued in the current iteration are.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVmIter = 0x0F70 | (2 * kTileLoads);
static_assert(2 * kTileLoads < 16, "vmcnt field");

// Workgroup barrier without the memory fence of __syncthreads() (whose
// vmcnt(0) would also wait for the tile loads still meant to be in flight).
// The loop reaches it only after every LDS read of the iteration has been
// consumed and after the explicit wait for the tiles the next iteration
// reads; the memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wave-uniform loads of data the kernel never writes go through the scalar
// cache (constant address space), so they do not join the vector-memory
// counter that tracks the tile loads in flight.
typedef const float __attribute__((address_space(4)))* const_f32_ptr;

// What the prologue hands to the tile loop of one wave.
struct WaveCtx {
    const int8_t* kg;      // the head's K tiles
    const int8_t* vg;      // the head's V tiles
    const_f32_ptr ksc;     // the head's K scales (scalar loads)
    int8_t* lds_k;
    int8_t* lds_v;
    uint32_t voff;         // this lane's byte offset for the tile loads
    int wave, lane;
    bool active;           // the wave's 32-row group holds rows < N of the range
    float qs;              // the group's Q scale
    int g, b, hl, bh;      // group, batch entry, head within the range, b*H + h
};

// Fused score form: LDS slot of K tile i is i % 3; V tile i sits in slot
// (3 - i % 3) % 3 (tile 0 in slot 0 from the prologue, then each iteration j
// loads V(j+1) into the slot that V(j-2) has left).
__device__ __forceinline__ int fused_v_slot(int i) { return (3 - i % 3) % 3; }

// Iteration j of the fused-form tile loop, j % 3 == kPhase: the loads of
// K(j+3) and V(j+1), the PV of tile j-1, the softmax of tile j with the alpha
// rescale of RO, the QK of tile j+1, then the wait for this iteration's loads
// and the workgroup barrier.  The phase fixes every ring slot at compile
// time, so the LDS reads address their slots through the instruction's
// offset field (no per-iteration address arithmetic).
template <int kPhase>
__device__ __forceinline__ void fused_step(const MainloopArgs& a, const WaveCtx& w, const v4i (&qf)[4],
                                           const v16i& bias, int j, v16i& s0, v16i& s1, float& m, float& off,
                                           float& dpart, v16f (&ro)[4], v8i& pkprev) {
    constexpr int kKFill = kPhase;                          // receives K(j+3)
    constexpr int kKRead = (kPhase + 1) % 3;                // holds K(j+1)
    constexpr int kVFill = (3 - (kPhase + 1) % 3) % 3;      // receives V(j+1)
    constexpr int kVRead = (3 - (kPhase + 2) % 3) % 3;      // holds V(j-1)
    tile_to_lds(w.kg + (int64_t)min(j + 3, a.T - 1) * kTileBytes, w.lds_k + kKFill * kTileBytes, w.voff, w.wave);
    tile_to_lds(w.vg + (int64_t)(j + 1) * kTileBytes, w.lds_v + kVFill * kTileBytes, w.voff, w.wave);
    if (w.active) {
        float alpha;
        v8i pk;
        bool moved;
        if (j > 0) pv_tile(w.lds_v + kVRead * kTileBytes, pkprev, w.lane, ro);   // tile j-1
        softmax_tile<false, false>(s0, s1, (w.qs * w.ksc[j]) * a.c, 0, w.lane, m, off, dpart, alpha, moved, pk);
        if (moved) rescale(ro, alpha);
        SAGE_FENCE();
        qk_tile(w.lds_k + kKRead * kTileBytes, qf, w.lane, s0, s1, bias);
        pkprev = pk;
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmIter);   // K(j+2), V(j) have landed
    block_barrier();
    SAGE_FENCE();
}

// One wave from the QK of tile 0 to its stored output rows, in one form of
// the score step: the tile loop, the last (partial) tile, then 1/d, the V
// scale and BF16 into token-major rows.  Inactive waves (query groups beyond
// the rows) issue their share of every tile load and take every barrier, and
// compute nothing.
//
// Ring slots by role, rotated each iteration: kq holds K(j+1) for this
// iteration's QK, kn K(j+2), and kf receives K(j+3); vc holds V(j) for this
// iteration's PV, vn V(j+1), and vf receives V(j+2).
template <bool kStepwise>
__device__ __forceinline__ void attend(const MainloopArgs& a, const WaveCtx& w, const v4i (&qf)[4],
                                       const v16i& bias) {
    const int T = a.T;
    const float c = a.c;
    const int lane = w.lane;
    v16i s0, s1;
    if (w.active) qk_tile(w.lds_k, qf, lane, s0, s1, bias);
    __syncthreads();   // K slot 0 is refilled in iteration 0

    float m = -INFINITY;
    float off = 0.0f;      // fused form: log2(448) - m, set when m first moves
    float dpart = 0.0f;    // this lane's share of the row denominator
    v16f ro[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) ro[db][r] = 0.0f;
    int8_t* kq = w.lds_k + kTileBytes;
    int8_t* kn = w.lds_k + 2 * kTileBytes;
    int8_t* kf = w.lds_k;
    int8_t* vc = w.lds_v;
    int8_t* vn = w.lds_v + kTileBytes;
    int8_t* vf = w.lds_v + 2 * kTileBytes;
    if constexpr (kStepwise) {
        for (int j = 0; j < T - 1; ++j) {
            tile_to_lds(w.kg + (int64_t)min(j + 3, T - 1) * kTileBytes, kf, w.voff, w.wave);
            tile_to_lds(w.vg + (int64_t)min(j + 2, T - 1) * kTileBytes, vf, w.voff, w.wave);
            if (w.active) {
                // softmax of tile j, the alpha rescale of RO (skipped when no
                // row of the wave changed its max), PV of tile j, QK of tile j+1
                float alpha;
                v8i pk;
                bool moved;
                softmax_tile<kStepwise, false>(s0, s1, (w.qs * w.ksc[j]) * c, 0, lane, m, off, dpart, alpha, moved,
                                               pk);
                if (moved) rescale(ro, alpha);
                SAGE_FENCE();
                pv_tile(vc, pk, lane, ro);
                qk_tile(kq, qf, lane, s0, s1, bias);
            }
            __builtin_amdgcn_s_waitcnt(kWaitVmIter);   // K(j+2), V(j+1) have landed
            block_barrier();
            int8_t* t = kf;  kf = kq;  kq = kn;  kn = t;
            t = vf;  vf = vc;  vc = vn;  vn = t;
        }
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        if (!w.active) return;
        {
            const int j = T - 1;
            float alpha;
            v8i pk;
            bool moved;
            softmax_tile<kStepwise, true>(s0, s1, (w.qs * w.ksc[j]) * c, a.N - j * kBK, lane, m, off, dpart, alpha,
                                          moved, pk);
            if (moved) rescale(ro, alpha);
            pv_tile(vc, pk, lane, ro);                   // V(T-1)
        }
    } else {
        // Fused form: each tile's PV moves to the start of the next
        // iteration, ahead of that tile's softmax, so that the matrix pipe
        // works through the softmax's vector instructions.  RO still
        // receives every tile's PV in tile order, each after its own tile's
        // alpha rescale and before the next tile's.  Iteration j loads
        // V(j+1), the V tile of iteration j+2's PV (as far ahead as the
        // stepwise form).  The loop runs three iterations (the rings'
        // period) per pass, so that each has its slots fixed (fused_step).
        v8i pkprev;
        int j = 0;
        for (; j + 3 <= T - 1; j += 3) {
            fused_step<0>(a, w, qf, bias, j, s0, s1, m, off, dpart, ro, pkprev);
            fused_step<1>(a, w, qf, bias, j + 1, s0, s1, m, off, dpart, ro, pkprev);
            fused_step<2>(a, w, qf, bias, j + 2, s0, s1, m, off, dpart, ro, pkprev);
        }
        if (j < T - 1) fused_step<0>(a, w, qf, bias, j++, s0, s1, m, off, dpart, ro, pkprev);
        if (j < T - 1) fused_step<1>(a, w, qf, bias, j++, s0, s1, m, off, dpart, ro, pkprev);
        // V(T-1), loaded in the last iteration, has landed for every wave
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        block_barrier();
        if (!w.active) return;
        {
            const int jl = T - 1;
            float alpha;
            v8i pk;
            bool moved;
            if (T > 1) pv_tile(w.lds_v + fused_v_slot(T - 2) * kTileBytes, pkprev, lane, ro);   // tile T-2
            softmax_tile<false, true>(s0, s1, (w.qs * w.ksc[jl]) * c, a.N - jl * kBK, lane, m, off, dpart, alpha,
                                      moved, pk);
            if (moved) rescale(ro, alpha);
            pv_tile(w.lds_v + fused_v_slot(T - 1) * kTileBytes, pk, lane, ro);   // V(T-1)
        }
    }

    const float dtot = halves_sum(dpart);
    const float rcp = 1.0f / dtot;
    const int n = w.g * kQG + (lane & 31);
    if (n < a.q_start || n >= a.q_end) return;
    uint16_t* op = a.o + w.b * a.o_sb + (int64_t)(n - a.q_start) * a.o_sn + w.hl * a.o_sh;
    const float* vs = a.v_scale + (int64_t)w.bh * kHD;
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

__global__ __launch_bounds__(kThreads, kWavesPerSimd) void mainloop_kernel(MainloopArgs a) {
    __shared__ __attribute__((aligned(16))) int8_t lds_k[kKSlots * kTileBytes];
    __shared__ __attribute__((aligned(16))) int8_t lds_v[kVSlots * kTileBytes];
    __shared__ int form_flags[kWaves];   // per wave: its group needs the stepwise form

    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int bhl = item / a.n_qblk;              // (b, head within the range)
    const int qb = item - bhl * a.n_qblk;
    const int b = bhl / a.h_count, hl = bhl - b * a.h_count;
    const int h = a.h_start + hl;
    const int bh = b * a.H + h;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    // the lane index from v_mbcnt (no inputs), which the compiler can recompute
    // where it is needed instead of holding the work-item id for the whole loop
    const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    // this lane's byte offset in a tile for its first 1 KiB tile load
    const uint32_t voff = (uint32_t)((wave * kTileLoads * 64 + lane) * 16);
    const int g = a.g_begin + qb * kWaves + wave;
    const bool active = g < a.g_end && g * kQG < a.N;
    const int T = a.T;

    const int8_t* kg = a.k_i8 + (int64_t)bh * T * kTileBytes;
    const int8_t* vg = (const int8_t*)a.v_fp8 + (int64_t)bh * T * kTileBytes;
    const const_f32_ptr ksc = (const_f32_ptr)(a.k_scale + (int64_t)bh * T);
    const float c = a.c;

    // Prologue: K(0..2) and V(0..1) to LDS (issued first, so that they are in
    // flight while the wave loads, or quantizes, its Q group), then QK of
    // tile 0.  Loads past the last tile are clamped to it and land in slots
    // that are never read again.
    tile_to_lds(kg, lds_k, voff, wave);
    tile_to_lds(vg, lds_v, voff, wave);
    tile_to_lds(kg + (int64_t)min(1, T - 1) * kTileBytes, lds_k + kTileBytes, voff, wave);
    tile_to_lds(kg + (int64_t)min(2, T - 1) * kTileBytes, lds_k + 2 * kTileBytes, voff, wave);
    tile_to_lds(vg + (int64_t)min(1, T - 1) * kTileBytes, lds_v + kTileBytes, voff, wave);
    v4i qf[4];
    float qs = 0.0f;
    if (a.q_bf16) {
        // The one-call path quantizes the wave's Q group here, from BF16, with
        // the prepass's own group routine: identical codes and scale.  With
        // the RMSNorm + RoPE producer, the rows are normalised and rotated
        // first by the prepass's own row routine.
        const int nq = g * kQG + (lane & 31);
        const bool valid = active && nq < a.N;
        const uint16_t* qp = a.q_bf16 + b * a.q_sb + (int64_t)nq * a.q_sn + h * a.q_sh + 16 * (lane >> 5);
        uint4 codes[4];
        if (a.nr.q_weight) {
            uint4 w[8];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                w[2 * kk] = valid ? *(const uint4*)(qp + 32 * kk) : make_uint4(0, 0, 0, 0);
                w[2 * kk + 1] = valid ? *(const uint4*)(qp + 32 * kk + 8) : make_uint4(0, 0, 0, 0);
            }
            const int na = valid ? nq : 0;
            norm_rope_row<true>(w, lane >> 5, a.nr.q_weight, a.nr.cos + (int64_t)na * (kHD / 2),
                          a.nr.sin + (int64_t)na * (kHD / 2), a.nr.eps);
            qs = quant_q_words(w, codes);
        } else {
            qs = quant_q_group(qp, valid, codes);
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qf[kk] = v4i{(int)codes[kk].x, (int)codes[kk].y, (int)codes[kk].z, (int)codes[kk].w};
    } else if (active) {
        const int8_t* qp = a.q_i8 + ((int64_t)bh * a.G + g) * kQGroupBytes + lane * 16;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[kk] = *(const v4i*)(qp + kk * 1024);
        qs = a.q_scale[(int64_t)bh * a.G + g];
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[kk] = v4i{0, 0, 0, 0};
    }

    // the initial QK accumulator, kept in registers for the whole loop (the
    // empty asm hides the constant from the compiler, which would otherwise
    // rebuild it every iteration)
    v16i bias = v16i{kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias,
                     kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias,
                     kScoreBias, kScoreBias};
    asm volatile("" : "+v"(bias));

    // The score step's form for this workgroup.  Every code has
    // |code| <= 127, so |S| <= 127 * ||q||_1 for each query row q of a
    // group and every key, and |t| = |S| * sj <= 127 * max ||q||_1 * qs *
    // max_t k_scale[t] * c over every tile of the head.  A wave's group may
    // take the fused form when that bound is below kStepwiseFrom; the
    // workgroup takes it when all four may (the waves share the K/V rings,
    // and the two forms load and wait for them on different schedules), else
    // the stepwise form, which is the definition's own rounding.  ||q||_1
    // comes from the codes in registers (v_sad_u8 on the codes shifted to
    // offset binary), the head's largest K scale from the prepass.
    uint32_t l1 = 0;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) l1 = __builtin_amdgcn_sad_u8((uint32_t)qf[kk][e] ^ 0x80808080u, 0x80808080u, l1);
    l1 += (uint32_t)__shfl_xor((int)l1, 32, 64);            // the row's other 64 channels
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) l1 = max(l1, (uint32_t)__shfl_xor((int)l1, o, 64));
    const float ksmax = ((const_f32_ptr)a.k_scale_max)[bh];
    const float bound = ((127.0f * (float)l1) * qs) * (ksmax * c);
    if (lane == 0) form_flags[wave] = !(bound < kStepwiseFrom);

    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    bool stepwise = false;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) stepwise = stepwise || form_flags[i] != 0;
    // Each form runs from here to the stored output in its own copy of the
    // code, which keeps the register allocation of the two loops apart.
    const WaveCtx w{kg, vg, ksc, lds_k, lds_v, voff, wave, lane, active, qs, g, b, hl, bh};
    if (stepwise)
        attend<true>(a, w, qf, bias);
    else
        attend<false>(a, w, qf, bias);
}

// One wave per (b, h, group g, tile t): the mainloop's QK tile routine with
// the mainloop's initial accumulator, written out as int32 (bias removed)
// for inspection.
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
    const v16i bias = v16i{kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias,
                           kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias, kScoreBias,
                           kScoreBias, kScoreBias};
    v16i s0, s1;
    qk_tile(kt, qf, lane, s0, s1, bias);
    const int64_t Nq = (int64_t)a.G * kQG, Nk = (int64_t)a.T * kBK;
    int32_t* out = a.s_out + ((int64_t)bh * Nq + g * kQG + (lane & 31)) * Nk + (int64_t)t * kBK;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        out[key_of(0, r, lane)] = s0[r] - kScoreBias;
        out[key_of(1, r, lane)] = s1[r] - kScoreBias;
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
