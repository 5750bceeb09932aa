/*
 * sage_mi355x.h -- C ABI of SageAttention2-style quantized non-causal
 * attention for AMD Instinct MI355X (gfx950).
 *
 * The operation (sources: page titles and sections):
 *   "Sage2 Blackwell Mainloop", sections "Decision" and "Existing Contract":
 *     an exact K channel-mean (smoothing) prepass; INT8 Q with one scale per
 *     32-row group inside 128-row blocks; INT8 K, mean subtracted, with one
 *     scale per 64-row block; FP8 V with per-channel scales; a fused mainloop
 *     that takes the INT8 Q/K, FP8 V and the Q/K/V scales and emits the final
 *     BF16 attention output, contiguous token-major NHD; batch, 56 heads,
 *     head dimension 128, non-causal, projection-strided BF16 NHD inputs.
 *   "State-Ownership Architecture Decision", sections "Non-Negotiable
 *     Dataflow" and "Interface And Future Ulysses Layout": all K64/V64 tiles
 *     in strictly increasing order; per tile QK, score scaling, max update,
 *     denominator update, FP8 probability conversion and PV added into FP32
 *     output rows; never an N-by-N score tensor; never a split of the KV walk;
 *     the FP32 reciprocal of d then normalisation, V scale and BF16; strided
 *     NHD inputs consumed directly (no transpose or contiguous copy), output
 *     rows at [token, head*128 + d].
 *
 * Conventions for every entry point:
 *   - Data pointers are DEVICE pointers (HIP device memory of the current
 *     device); shapes, strides and descriptors are host values.
 *   - The caller owns every buffer.  The library allocates no memory and keeps
 *     no state except a thread-local error message.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising.  A kernel fault surfaces at
 *     the caller's next synchronisation of that stream.  Nothing but kernels
 *     on `stream` is issued (no copies, fills or host waits), so the calls
 *     can be captured in a HIP graph.
 *   - Arguments are validated on the host before anything is launched; on
 *     error nothing is launched and a status other than SAGE_OK is returned,
 *     with detail in sage_last_error_message().  No exception crosses the ABI.
 *   - Inputs must be finite BF16 values; non-finite inputs give unspecified
 *     (but memory-safe) results.  Outputs follow the step-by-step definition
 *     below up to the hardware exp2 and the order of FP32 sums, which can move
 *     a probability to the adjacent E4M3 code at a rounding midpoint.  Where
 *     each of the four 32-row query groups of a 128-row block has its scores
 *     bounded by 2^12 in log2 units (score * sm_scale * log2(e); the bound is
 *     127 * the largest L1 norm of the group's Q codes * q_scale * the head's
 *     largest k_scale * sm_scale * log2(e)), the block forms each probability
 *     as 2^(S*sj + log2(448) - m) with a single rounding; every other block
 *     takes the definition's three roundings one by one, for any finite input.  Where an intermediate of the definition
 *     overflows FP32 (input magnitudes near the BF16 range), the outputs do
 *     too.
 */
#ifndef SAGE_MI355X_H
#define SAGE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: adds sage_quantize_qkv_norm_rope and sage_attn_fwd_norm_rope (additions only).
 * 3: sage_quantized gains k_scale_max (the struct grows; rebuild callers). */
#define SAGE_ABI_VERSION 3
#define SAGE_HEAD_DIM 128

typedef enum sage_status {
    SAGE_OK = 0,
    SAGE_ERR_INVALID_ARGUMENT = 1,  /* null pointer, bad shape, bad scale     */
    SAGE_ERR_UNSUPPORTED = 2,       /* legal but unsupported stride/alignment */
    SAGE_ERR_WORKSPACE = 3,         /* workspace null, misaligned or too small */
    SAGE_ERR_HIP = 4                /* a HIP launch failed                    */
} sage_status;

/* Problem shape.  D must be 128; 1 <= B, H; 1 <= N <= 2^24; B*H <= 2^24 and
 * B*H*2*ceil(N/128) < 2^31 (launch grid limit). */
typedef struct sage_shape {
    int32_t B, N, H, D;
} sage_shape;

/* A BF16 [B, N, H, 128] input view with unit stride along D.  Element
 * (b, n, h, d) is at data + b*stride_b + n*stride_n + h*stride_h + d
 * (strides in elements).  Supported: strides >= 0 and multiples of 8, data
 * 16-byte aligned.  Q, K and V may be column slices of one projection buffer
 * [B, N, 3*H*128] (stride_n = 3*H*128). */
typedef struct sage_bf16_in {
    const void* data;
    int64_t stride_b, stride_n, stride_h;
} sage_bf16_in;

/* A BF16 [B, N, H, 128] output view, same addressing.  Supported: strides
 * >= 0 and multiples of 4, data 8-byte aligned.  Only rows n < N are
 * written. */
typedef struct sage_bf16_out {
    void* data;
    int64_t stride_b, stride_n, stride_h;
} sage_bf16_out;

/* Quantized operands, carved from one caller-owned workspace by
 * sage_quantized_carve().  With T = ceil(N/64), Nq = 128*ceil(N/128),
 * G = Nq/32 and bh = b*H + h, the layouts are:
 *
 *   q_i8    INT8 codes, 4096 bytes per (bh, group g):
 *           byte ((bh*G + g)*4096 + (kk*64 + l)*16 + i)
 *             = code of Q[b, 32g + l%32, h, 32kk + 16*(l/32) + i]
 *           for kk in 0..3, l in 0..63, i in 0..15.  Rows >= N hold 0.
 *   q_scale FP32 [B][H][G]; groups with no row < N hold 0.
 *   k_i8    INT8 codes of K - k_mean, 8192 bytes per (bh, tile t):
 *           byte ((bh*T + t)*8192 + ((half*4 + kk)*64 + l)*16 + i)
 *             = code of K[b, 64t + 32*half + l%32, h, 32kk + 16*(l/32) + i]
 *           for half in 0..1.  Rows >= N hold 0.
 *   k_scale FP32 [B][H][T]
 *   k_mean  FP32 [B][H][128]
 *   v_fp8   E4M3FN bytes, 8192 bytes per (bh, tile t):
 *           byte ((bh*T + t)*8192 + ((db*2 + half)*64 + l)*16 + i)
 *             = code of V[b, 64t + 32*half + 8*(i/4) + 4*(l/32) + i%4, h,
 *                         32db + l%32]
 *           for db in 0..3.  Rows >= N hold 0x00.
 *   v_scale FP32 [B][H][128]
 *   k_tile_sum, v_tile_amax  FP32 [B][H][T][128], v_inv FP32 [B][H][128]:
 *           scratch of the prepass (per-tile K channel sums, per-tile V
 *           channel absolute maxima, per-channel 448/amax).
 *   k_scale_max FP32 [B][H]: the largest k_scale of each (b, h), written by
 *           the prepass; the mainloop reads it to bound its scores (see the
 *           conventions above).
 *
 * The INT8 and E4M3 layouts are the operand layouts of the gfx950 matrix
 * instructions the mainloop issues, so every mainloop load is a contiguous
 * 1 KiB row of 16-byte lanes. */
typedef struct sage_quantized {
    sage_shape shape;
    int8_t* q_i8;
    float* q_scale;
    int8_t* k_i8;
    float* k_scale;
    float* k_mean;
    uint8_t* v_fp8;
    float* v_scale;
    float* k_tile_sum;
    float* v_tile_amax;
    float* v_inv;
    float* k_scale_max;
} sage_quantized;

/* Bytes of workspace sage_quantized_carve() and sage_attn_fwd() need for
 * shape s (a pure host function); 0 if s is invalid. */
size_t sage_workspace_bytes(sage_shape s);

/* Lays out the quantized operands of shape s inside ws (device memory,
 * 256-byte aligned, at least sage_workspace_bytes(s) bytes) and fills *out.
 * Host only; touches no device memory.
 * Errors: INVALID_ARGUMENT (bad shape, out == NULL), WORKSPACE. */
sage_status sage_quantized_carve(sage_shape s, void* ws, size_t ws_bytes, sage_quantized* out);

/* The prepass ("Sage2 Blackwell Mainloop", Decision: K mean/smoothing, Q
 * quantization, K subtract-mean quantization, V scale/FP8 quantization):
 *   k_mean[b,h,d]  = (sum over 64-row tiles, in order, of the in-order FP32
 *                     sum of K over the tile's rows) / N
 *   per 32-row group of Q and per 64-row tile of K - k_mean:
 *                    a = max |x|; scale = a/127; code = rne(x * (127/a))
 *                    clamped to [-127, 127]
 *   per channel of V over all N rows: a = max |v|; scale = a/448;
 *                    code = E4M3(v * (448/a)), round to nearest even
 *   (groups, tiles or channels with a < 2^-100 get scale 0 and zero codes).
 * q, k, v share qz->shape.  Writes every field of *qz (including scratch).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, HIP. */
sage_status sage_quantize_qkv(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v,
                              const sage_quantized* qz, void* stream);

/* Parameters of the optional upstream Q/K producer ("Sage2 Blackwell
 * Mainloop", Completed P1 And P2: strided-NHD Q/K RMSNorm and split-half RoPE
 * fused with Q INT8 quantization).  Device pointers, FP32, 16-byte aligned:
 * q_weight, k_weight: the RMSNorm weights [128], shared by every head;
 * cos, sin: the rotary angle tables [N][64], row n for token n of every batch
 * entry and head, column i for the channel pair (i, i + 64).  eps > 0. */
typedef struct sage_norm_rope {
    const float* q_weight;
    const float* k_weight;
    const float* cos;
    const float* sin;
    float eps;
} sage_norm_rope;

/* sage_quantize_qkv applied to Q' and K' instead of Q and K, where for each
 * (b, n, h) row x of Q (weight q_weight) or K (weight k_weight):
 *   ss = sum over channels c = 0..127, in order, of fl(x_c * x_c), from +0
 *   r  = fl(1 / fl(sqrt(fl(fl(ss / 128) + eps))))
 *   y_c = bf16(fl(fl(x_c * r) * weight[c]))                   (RNE)
 *   x'_i = bf16(fl(fl(y_i * cos[n][i]) - fl(y_{i+64} * sin[n][i])))
 *   x'_{i+64} = bf16(fl(fl(y_{i+64} * cos[n][i]) + fl(y_i * sin[n][i])))  (i < 64)
 * V is used as is.  Q' and K' are never stored: the prepass recomputes them
 * from Q and K where it reads them, so the outputs are byte-identical to
 * sage_quantize_qkv on Q', K' and the memory traffic is that of
 * sage_quantize_qkv.  Errors: as sage_quantize_qkv; INVALID_ARGUMENT when nr
 * or one of its pointers is NULL or eps is not finite and > 0; UNSUPPORTED
 * when a table or weight pointer is not 16-byte aligned. */
sage_status sage_quantize_qkv_norm_rope(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v,
                                        const sage_norm_rope* nr, const sage_quantized* qz, void* stream);

/* The fused mainloop and epilogue ("State-Ownership Architecture Decision",
 * Non-Negotiable Dataflow).  For every query row, over K/V tiles t = 0..T-1:
 *   S = q_i8 . k_i8^T (exact int32);  t = S * (q_scale*k_scale*sm_scale*log2 e)
 *   m' = max(m, max t); alpha = 2^(m - m'); RO *= alpha; d *= alpha
 *   p = 448 * 2^(t - m') (keys >= N masked); d += sum p; P8 = E4M3(p)
 *   RO += P8 . v_fp8 (FP32 accumulation, tile by tile in increasing order)
 * then O = BF16((RO * (1/d)) * v_scale).  sm_scale must be finite and > 0
 * (the usual choice is 1/sqrt(128)).  Reads only *qz's operands.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, HIP. */
sage_status sage_attn_fwd_quantized(const sage_quantized* qz, float sm_scale,
                                    const sage_bf16_out* o, void* stream);

/* A sub-range of the attention work ("State-Ownership Architecture Decision",
 * Interface And Future Ulysses Layout: the work descriptor carries a query
 * row range, a head range and destination strides, while every query still
 * walks the whole KV sequence in order).  Rows q_start .. q_start+q_count-1
 * and heads head_start .. head_start+head_count-1 of every batch entry. */
typedef struct sage_range {
    int32_t q_start, q_count;
    int32_t head_start, head_count;
} sage_range;

/* sage_attn_fwd_quantized restricted to *r: output row (b, q_start + i,
 * head_start + j) is stored at o[b, i, j, :], so o is a [B, q_count,
 * head_count, 128] view (it may start at any offset of a larger buffer);
 * nothing outside those rows is written.  Each stored row is bit-identical to
 * the same row of the full call; the work done is whole 32-row groups of the
 * range.  Errors: as sage_attn_fwd_quantized; INVALID_ARGUMENT when r is NULL
 * or a range is empty or leaves [0, N) x [0, H). */
sage_status sage_attn_fwd_quantized_range(const sage_quantized* qz, float sm_scale, const sage_range* r,
                                          const sage_bf16_out* o, void* stream);

/* Whole path in one call, all on `stream`: carve ws, the prepass for K and V,
 * then the mainloop, which quantizes each 32-row Q group itself from the BF16
 * view with the prepass's arithmetic (the Q producer embedded in the
 * mainloop, "State-Ownership Architecture Decision", VEA-B: producers may be
 * embedded to feed the slots).  The codes, scales and output are identical to
 * sage_quantize_qkv + sage_attn_fwd_quantized; the workspace's q_i8 and
 * q_scale regions are left unwritten.  ws must hold sage_workspace_bytes(s)
 * bytes, 256-byte aligned.  Errors: as the calls above, and WORKSPACE. */
sage_status sage_attn_fwd(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v,
                          sage_shape s, float sm_scale, const sage_bf16_out* o,
                          void* ws, size_t ws_bytes, void* stream);

/* sage_attn_fwd with the RMSNorm + split-half RoPE producer of
 * sage_quantize_qkv_norm_rope (same arithmetic, same parameters): K is
 * normalised and rotated inside the prepass and Q inside the mainloop, which
 * normalises, rotates and quantizes each 32-row group in its prologue (the
 * pages' P1 producer embedded to feed the slots: "Sage2 Blackwell Mainloop",
 * Completed P1 And P2; "State-Ownership Architecture Decision", VEA-B).  The
 * output is identical to sage_quantize_qkv_norm_rope +
 * sage_attn_fwd_quantized.  Errors: as sage_attn_fwd and
 * sage_quantize_qkv_norm_rope. */
sage_status sage_attn_fwd_norm_rope(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v,
                                    sage_shape s, const sage_norm_rope* nr, float sm_scale,
                                    const sage_bf16_out* o, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the device array the allocation-free entry point uses as its
 * workspace (one array per GPU, held by the library until the process ends). */
#define SAGE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * sage_attn_fwd without a workspace argument.  Its workspace is a device
 * array of SAGE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU; the
 * call itself allocates nothing.  Shapes whose sage_workspace_bytes() exceed
 * the array are rejected with SAGE_ERR_UNSUPPORTED before anything is
 * launched (64 MiB holds, e.g., B=1, H=8, N=4096 or B=1, H=56, N=2048).  Every
 * call on a GPU uses that GPU's one array, which keeps the last call's
 * contents (nothing in it has to start at zero): calls whose kernels overlap
 * on one GPU (on different streams, or from several host threads) race and
 * give undefined output; calls on one stream are ordered and safe.  The first
 * call on each device resolves the array's device address (a host query, no
 * allocation); make that first call outside stream capture.  Output identical
 * to sage_attn_fwd.  Errors: as sage_attn_fwd; UNSUPPORTED for a shape
 * beyond the array; HIP when the array's address cannot be resolved. */
sage_status sage_attn_fwd_noalloc(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v,
                                  sage_shape s, float sm_scale, const sage_bf16_out* o, void* stream);

/* Static text for a status code. */
const char* sage_status_string(sage_status st);

/* Detail of the last failure on the calling thread ("" if none). */
const char* sage_last_error_message(void);

/* SAGE_ABI_VERSION of the loaded library. */
int32_t sage_abi_version(void);

/* ---- test and inspection entry points (not on the hot path) ---- */

/* The int32 Q.K^T sums the mainloop computes, produced by the mainloop's own
 * tile routine, for every (b, h, query row < Nq, key < 64*T):
 * s_out[((b*H + h)*Nq + r)*(64*T) + n].  Materialises an Nq-by-Nk tensor per
 * head, so N <= 4096 is required.  Errors: INVALID_ARGUMENT, UNSUPPORTED, HIP. */
sage_status sage_debug_qk_s32(const sage_quantized* qz, int32_t* s_out, void* stream);

/* The FP32 -> E4M3FN conversion the kernels use (round to nearest even), on n
 * values; |x| must be below 464 for a finite code.  Errors: INVALID_ARGUMENT, HIP. */
sage_status sage_debug_cvt_e4m3(const float* x, uint8_t* y, int64_t n, void* stream);

/* Measurement support, not an operation of the pages: shader clock cycles of
 * the mainloop's tile step on this GPU (the vector roofline the benchmark
 * reports next to the matrix one; the per-score work it issues is that of
 * "Sage2 Blackwell Mainloop", Existing Contract, as the mainloop does it).  Launches `blocks`
 * workgroups of 4*waves_per_simd waves (waves_per_simd waves on each SIMD of a
 * CU); every wave runs `iters` repetitions of one instruction stream and
 * stores the cycles it took (s_memtime difference) at
 * ticks[block * 4*waves_per_simd + wave] (device memory, blocks *
 * 4*waves_per_simd entries).  The streams (kind):
 *   0  the vector work of one 32-query x 64-key wave tile under the
 *      contract's per-score arithmetic, fused score form (160 instructions:
 *      32 float(S) subtractions, 32 score FMAs, 32 exp2, 32 denominator adds,
 *      16 E4M3 pair conversions, 16 three-input maxima), no memory access
 *   1  stream 0 followed by the tile's matrix work in one burst (4 FP8
 *      32x32x64 and 8 INT8 32x32x32 instructions)
 *   2  the 12 matrix instructions alone
 * A SIMD's cycles per tile = the largest count among its waves /
 * (iters * waves_per_simd).  1 <= waves_per_simd <= 4, 1 <= blocks <= 65536,
 * 1 <= iters <= 2^20.  Errors: INVALID_ARGUMENT, HIP. */
sage_status sage_debug_issue_probe(int32_t kind, int32_t waves_per_simd, int32_t blocks, int32_t iters,
                                   uint64_t* ticks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_MI355X_H */
