// sage_api.cpp -- the C ABI declared in include/sage_mi355x.h: host-side
// validation, workspace carving and kernel launches on the caller's stream.
#include "sage_mi355x.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "sage_launch.hpp"

namespace {

thread_local char g_err[512] = "";

sage_status fail(sage_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

void clear_err() { g_err[0] = '\0'; }

constexpr size_t kAlign = 256;
constexpr int64_t kMaxN = int64_t(1) << 24;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Dims {
    int64_t B, N, H, T, G, Nq, Nk;
};

bool dims_of(const sage_shape& s, Dims* d) {
    if (s.B < 1 || s.N < 1 || s.H < 1 || s.D != SAGE_HEAD_DIM || s.N > kMaxN) return false;
    if ((int64_t)s.B * s.H > (int64_t)1 << 24) return false;
    d->B = s.B;
    d->N = s.N;
    d->H = s.H;
    d->T = (s.N + 63) / 64;
    d->Nq = (s.N + 127) / 128 * 128;
    d->G = d->Nq / 32;
    d->Nk = d->T * 64;
    // every launch grid must fit the 32-bit grid size; the largest is the
    // quantizer's, one block per (b, h, 64 rows of the padded Q length)
    if (d->B * d->H * (d->Nq / 64) > 0x7fffffff) return false;
    return true;
}

// Region sizes in carve order.
constexpr int kRegions = 11;

void region_sizes(const Dims& d, size_t out[kRegions]) {
    const size_t BH = (size_t)(d.B * d.H);
    out[0] = BH * d.Nq * 128;              // q_i8
    out[1] = BH * d.G * sizeof(float);     // q_scale
    out[2] = BH * d.Nk * 128;              // k_i8
    out[3] = BH * d.T * sizeof(float);     // k_scale
    out[4] = BH * 128 * sizeof(float);     // k_mean
    out[5] = BH * d.Nk * 128;              // v_fp8
    out[6] = BH * 128 * sizeof(float);     // v_scale
    out[7] = BH * d.T * 128 * sizeof(float);  // k_tile_sum
    out[8] = BH * d.T * 128 * sizeof(float);  // v_tile_amax
    out[9] = BH * 128 * sizeof(float);     // v_inv
    out[10] = BH * sizeof(float);          // k_scale_max
}

size_t total_bytes(const Dims& d) {
    size_t sz[kRegions];
    region_sizes(d, sz);
    size_t t = 0;
    for (size_t x : sz) t += align_up(x);
    return t;
}

sage_status check_in(const sage_bf16_in* x, const char* name) {
    if (!x) return fail(SAGE_ERR_INVALID_ARGUMENT, "%s descriptor is NULL", name);
    if (!x->data) return fail(SAGE_ERR_INVALID_ARGUMENT, "%s data is NULL", name);
    if (x->stride_b < 0 || x->stride_n < 0 || x->stride_h < 0)
        return fail(SAGE_ERR_UNSUPPORTED, "%s has a negative stride", name);
    if (x->stride_b % 8 || x->stride_n % 8 || x->stride_h % 8)
        return fail(SAGE_ERR_UNSUPPORTED, "%s strides must be multiples of 8 elements", name);
    if ((uintptr_t)x->data % 16)
        return fail(SAGE_ERR_UNSUPPORTED, "%s data must be 16-byte aligned", name);
    return SAGE_OK;
}

sage_status check_out(const sage_bf16_out* o) {
    if (!o) return fail(SAGE_ERR_INVALID_ARGUMENT, "output descriptor is NULL");
    if (!o->data) return fail(SAGE_ERR_INVALID_ARGUMENT, "output data is NULL");
    if (o->stride_b < 0 || o->stride_n < 0 || o->stride_h < 0)
        return fail(SAGE_ERR_UNSUPPORTED, "output has a negative stride");
    if (o->stride_b % 4 || o->stride_n % 4 || o->stride_h % 4)
        return fail(SAGE_ERR_UNSUPPORTED, "output strides must be multiples of 4 elements");
    if ((uintptr_t)o->data % 8) return fail(SAGE_ERR_UNSUPPORTED, "output data must be 8-byte aligned");
    return SAGE_OK;
}

sage_status check_quantized(const sage_quantized* qz, Dims* d) {
    if (!qz) return fail(SAGE_ERR_INVALID_ARGUMENT, "quantized descriptor is NULL");
    if (!dims_of(qz->shape, d))
        return fail(SAGE_ERR_INVALID_ARGUMENT, "invalid shape B=%d N=%d H=%d D=%d (need D=128, 1<=N<=2^24, B,H>=1, B*H<=2^24, B*H*2*ceil(N/128)<2^31)",
                    qz->shape.B, qz->shape.N, qz->shape.H, qz->shape.D);
    if (!qz->q_i8 || !qz->q_scale || !qz->k_i8 || !qz->k_scale || !qz->k_mean || !qz->v_fp8 || !qz->v_scale ||
        !qz->k_tile_sum || !qz->v_tile_amax || !qz->v_inv || !qz->k_scale_max)
        return fail(SAGE_ERR_INVALID_ARGUMENT, "a quantized-operand pointer is NULL");
    const void* p16[] = {qz->q_i8, qz->k_i8, qz->v_fp8, qz->k_mean, qz->v_scale, qz->k_tile_sum, qz->v_tile_amax,
                         qz->v_inv};
    for (const void* p : p16)
        if ((uintptr_t)p % 16) return fail(SAGE_ERR_UNSUPPORTED, "quantized operands must be 16-byte aligned");
    if ((uintptr_t)qz->q_scale % 4 || (uintptr_t)qz->k_scale % 4 || (uintptr_t)qz->k_scale_max % 4)
        return fail(SAGE_ERR_UNSUPPORTED, "scales must be 4-byte aligned");
    return SAGE_OK;
}

sage_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SAGE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return SAGE_OK;
}

sage_status check_norm_rope(const sage_norm_rope* nr) {
    if (!nr) return fail(SAGE_ERR_INVALID_ARGUMENT, "norm/rope descriptor is NULL");
    if (!nr->q_weight || !nr->k_weight || !nr->cos || !nr->sin)
        return fail(SAGE_ERR_INVALID_ARGUMENT, "a norm/rope weight or table pointer is NULL");
    const void* p16[] = {nr->q_weight, nr->k_weight, nr->cos, nr->sin};
    for (const void* p : p16)
        if ((uintptr_t)p % 16) return fail(SAGE_ERR_UNSUPPORTED, "norm/rope weights and tables must be 16-byte aligned");
    if (!std::isfinite(nr->eps) || !(nr->eps > 0.0f))
        return fail(SAGE_ERR_INVALID_ARGUMENT, "eps must be finite and > 0");
    return SAGE_OK;
}

sage_status prepass(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v,
                    const sage_quantized* qz, bool with_q, const sage_norm_rope* nr, void* stream) {
    Dims d;
    sage_status st;
    if ((st = check_quantized(qz, &d)) != SAGE_OK) return st;
    if ((st = check_in(q, "q")) != SAGE_OK) return st;
    if ((st = check_in(k, "k")) != SAGE_OK) return st;
    if ((st = check_in(v, "v")) != SAGE_OK) return st;
    sage::PrepassArgs p;
    p.B = (int)d.B; p.N = (int)d.N; p.H = (int)d.H; p.T = (int)d.T; p.G = (int)d.G;
    p.with_q = with_q;
    p.q = (const uint16_t*)q->data; p.q_sb = q->stride_b; p.q_sn = q->stride_n; p.q_sh = q->stride_h;
    p.k = (const uint16_t*)k->data; p.k_sb = k->stride_b; p.k_sn = k->stride_n; p.k_sh = k->stride_h;
    p.v = (const uint16_t*)v->data; p.v_sb = v->stride_b; p.v_sn = v->stride_n; p.v_sh = v->stride_h;
    p.q_i8 = qz->q_i8; p.q_scale = qz->q_scale;
    p.k_i8 = qz->k_i8; p.k_scale = qz->k_scale; p.k_mean = qz->k_mean; p.k_scale_max = qz->k_scale_max;
    p.v_fp8 = qz->v_fp8; p.v_scale = qz->v_scale;
    p.k_tile_sum = qz->k_tile_sum; p.v_tile_amax = qz->v_tile_amax; p.v_inv = qz->v_inv;
    p.norm_rope = nr != nullptr;
    p.nr = sage::NormRopeArgs{nullptr, nullptr, nullptr, nullptr, 0.0f};
    if (nr) p.nr = sage::NormRopeArgs{nr->q_weight, nr->k_weight, nr->cos, nr->sin, nr->eps};
    return hip_status(sage::launch_prepass(p, (hipStream_t)stream), "prepass launch");
}

// The mainloop over range *r; q_src non-null makes it quantize Q from BF16.
sage_status mainloop(const sage_quantized* qz, float sm_scale, const sage_range* r, const sage_bf16_out* o,
                     const sage_bf16_in* q_src, const sage_norm_rope* nr, void* stream) {
    Dims d;
    sage_status st;
    if ((st = check_quantized(qz, &d)) != SAGE_OK) return st;
    if (!r) return fail(SAGE_ERR_INVALID_ARGUMENT, "range descriptor is NULL");
    if (r->q_start < 0 || r->q_count < 1 || (int64_t)r->q_start + r->q_count > d.N)
        return fail(SAGE_ERR_INVALID_ARGUMENT, "query range [%d, %d + %d) is empty or outside [0, %lld)",
                    r->q_start, r->q_start, r->q_count, (long long)d.N);
    if (r->head_start < 0 || r->head_count < 1 || (int64_t)r->head_start + r->head_count > d.H)
        return fail(SAGE_ERR_INVALID_ARGUMENT, "head range [%d, %d + %d) is empty or outside [0, %lld)",
                    r->head_start, r->head_start, r->head_count, (long long)d.H);
    if ((st = check_out(o)) != SAGE_OK) return st;
    if (q_src && (st = check_in(q_src, "q")) != SAGE_OK) return st;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
        return fail(SAGE_ERR_INVALID_ARGUMENT, "sm_scale must be finite and > 0");
    sage::MainloopArgs p;
    p.q_i8 = qz->q_i8; p.q_scale = qz->q_scale;
    p.k_i8 = qz->k_i8; p.k_scale = qz->k_scale; p.k_scale_max = qz->k_scale_max;
    p.v_fp8 = qz->v_fp8; p.v_scale = qz->v_scale;
    p.q_bf16 = q_src ? (const uint16_t*)q_src->data : nullptr;
    p.q_sb = q_src ? q_src->stride_b : 0; p.q_sn = q_src ? q_src->stride_n : 0; p.q_sh = q_src ? q_src->stride_h : 0;
    p.nr = sage::NormRopeArgs{nullptr, nullptr, nullptr, nullptr, 0.0f};
    if (q_src && nr) p.nr = sage::NormRopeArgs{nr->q_weight, nr->k_weight, nr->cos, nr->sin, nr->eps};
    p.o = (uint16_t*)o->data; p.o_sb = o->stride_b; p.o_sn = o->stride_n; p.o_sh = o->stride_h;
    p.B = (int)d.B; p.N = (int)d.N; p.H = (int)d.H; p.T = (int)d.T; p.G = (int)d.G;
    p.q_start = r->q_start;
    p.q_end = r->q_start + r->q_count;
    p.h_start = r->head_start;
    p.h_count = r->head_count;
    p.g_begin = p.q_start / 32;
    p.g_end = (p.q_end + 31) / 32;
    p.n_qblk = (p.g_end - p.g_begin + sage::kMainloopWaves - 1) / sage::kMainloopWaves;
    const int64_t items = d.B * (int64_t)r->head_count * p.n_qblk;
    if (items > 0x7fffffff) return fail(SAGE_ERR_UNSUPPORTED, "too many work items");
    p.n_items = (int)items;
    const float log2e = 1.4426950408889634f;
    p.c = sm_scale * log2e;
    return hip_status(sage::launch_mainloop(p, (hipStream_t)stream), "mainloop launch");
}

// The whole path in one call; nr non-null adds the RMSNorm + RoPE producer
// (K in the prepass, Q in the mainloop prologue).
sage_status one_call(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v, sage_shape s,
                     const sage_norm_rope* nr, float sm_scale, const sage_bf16_out* o, void* ws, size_t ws_bytes,
                     void* stream) {
    sage_quantized qz;
    sage_status st = sage_quantized_carve(s, ws, ws_bytes, &qz);
    if (st != SAGE_OK) return st;
    if ((st = check_out(o)) != SAGE_OK) return st;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
        return fail(SAGE_ERR_INVALID_ARGUMENT, "sm_scale must be finite and > 0");
    if ((st = check_in(q, "q")) != SAGE_OK) return st;
    // K and V through the prepass; Q is quantized inside the mainloop.
    if ((st = prepass(q, k, v, &qz, false, nr, stream)) != SAGE_OK) return st;
    const sage_range all = {0, s.N, 0, s.H};
    return mainloop(&qz, sm_scale, &all, o, q, nr, stream);
}

}  // namespace

extern "C" {

int32_t sage_abi_version(void) { return SAGE_ABI_VERSION; }

const char* sage_status_string(sage_status st) {
    switch (st) {
        case SAGE_OK: return "ok";
        case SAGE_ERR_INVALID_ARGUMENT: return "invalid argument";
        case SAGE_ERR_UNSUPPORTED: return "unsupported layout";
        case SAGE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case SAGE_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* sage_last_error_message(void) { return g_err; }

size_t sage_workspace_bytes(sage_shape s) {
    Dims d;
    if (!dims_of(s, &d)) return 0;
    return total_bytes(d);
}

sage_status sage_quantized_carve(sage_shape s, void* ws, size_t ws_bytes, sage_quantized* out) {
    clear_err();
    Dims d;
    if (!out) return fail(SAGE_ERR_INVALID_ARGUMENT, "out is NULL");
    if (!dims_of(s, &d))
        return fail(SAGE_ERR_INVALID_ARGUMENT, "invalid shape B=%d N=%d H=%d D=%d (need D=128, 1<=N<=2^24, B,H>=1, B*H<=2^24, B*H*2*ceil(N/128)<2^31)",
                    s.B, s.N, s.H, s.D);
    if (!ws) return fail(SAGE_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)ws % kAlign) return fail(SAGE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const size_t need = total_bytes(d);
    if (ws_bytes < need) return fail(SAGE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    size_t sz[kRegions];
    region_sizes(d, sz);
    char* p = (char*)ws;
    void* r[kRegions];
    for (int i = 0; i < kRegions; ++i) {
        r[i] = p;
        p += align_up(sz[i]);
    }
    out->shape = s;
    out->q_i8 = (int8_t*)r[0];
    out->q_scale = (float*)r[1];
    out->k_i8 = (int8_t*)r[2];
    out->k_scale = (float*)r[3];
    out->k_mean = (float*)r[4];
    out->v_fp8 = (uint8_t*)r[5];
    out->v_scale = (float*)r[6];
    out->k_tile_sum = (float*)r[7];
    out->v_tile_amax = (float*)r[8];
    out->v_inv = (float*)r[9];
    out->k_scale_max = (float*)r[10];
    return SAGE_OK;
}

sage_status sage_quantize_qkv(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v,
                              const sage_quantized* qz, void* stream) {
    clear_err();
    return prepass(q, k, v, qz, true, nullptr, stream);
}

sage_status sage_quantize_qkv_norm_rope(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v,
                                        const sage_norm_rope* nr, const sage_quantized* qz, void* stream) {
    clear_err();
    sage_status st;
    if ((st = check_norm_rope(nr)) != SAGE_OK) return st;
    return prepass(q, k, v, qz, true, nr, stream);
}

sage_status sage_attn_fwd_quantized_range(const sage_quantized* qz, float sm_scale, const sage_range* r,
                                          const sage_bf16_out* o, void* stream) {
    clear_err();
    return mainloop(qz, sm_scale, r, o, nullptr, nullptr, stream);
}

sage_status sage_attn_fwd_quantized(const sage_quantized* qz, float sm_scale, const sage_bf16_out* o,
                                    void* stream) {
    clear_err();
    Dims d;
    sage_status st;
    if ((st = check_quantized(qz, &d)) != SAGE_OK) return st;
    const sage_range all = {0, (int32_t)d.N, 0, (int32_t)d.H};
    return sage_attn_fwd_quantized_range(qz, sm_scale, &all, o, stream);
}

sage_status sage_attn_fwd(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v, sage_shape s,
                          float sm_scale, const sage_bf16_out* o, void* ws, size_t ws_bytes, void* stream) {
    clear_err();
    return one_call(q, k, v, s, nullptr, sm_scale, o, ws, ws_bytes, stream);
}

sage_status sage_attn_fwd_norm_rope(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v,
                                    sage_shape s, const sage_norm_rope* nr, float sm_scale, const sage_bf16_out* o,
                                    void* ws, size_t ws_bytes, void* stream) {
    clear_err();
    sage_status st;
    if ((st = check_norm_rope(nr)) != SAGE_OK) return st;
    return one_call(q, k, v, s, nr, sm_scale, o, ws, ws_bytes, stream);
}

sage_status sage_attn_fwd_noalloc(const sage_bf16_in* q, const sage_bf16_in* k, const sage_bf16_in* v,
                                  sage_shape s, float sm_scale, const sage_bf16_out* o, void* stream) {
    clear_err();
    Dims d;
    if (!dims_of(s, &d))
        return fail(SAGE_ERR_INVALID_ARGUMENT, "invalid shape B=%d N=%d H=%d D=%d (need D=128, 1<=N<=2^24, B,H>=1, B*H<=2^24, B*H*2*ceil(N/128)<2^31)",
                    s.B, s.N, s.H, s.D);
    const size_t need = total_bytes(d);
    if (need > SAGE_NOALLOC_SCRATCH_BYTES)
        return fail(SAGE_ERR_UNSUPPORTED,
                    "shape B=%d N=%d H=%d needs %zu workspace bytes; the allocation-free path holds %zu "
                    "(use sage_attn_fwd with a caller workspace)",
                    s.B, s.N, s.H, need, (size_t)SAGE_NOALLOC_SCRATCH_BYTES);
    sage_status st;
    if ((st = check_in(q, "q")) != SAGE_OK) return st;
    if ((st = check_in(k, "k")) != SAGE_OK) return st;
    if ((st = check_in(v, "v")) != SAGE_OK) return st;
    if ((st = check_out(o)) != SAGE_OK) return st;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
        return fail(SAGE_ERR_INVALID_ARGUMENT, "sm_scale must be finite and > 0");
    void* ws = nullptr;
    if ((st = hip_status(sage::noalloc_scratch(&ws), "allocation-free workspace address")) != SAGE_OK) return st;
    return one_call(q, k, v, s, nullptr, sm_scale, o, ws, need, stream);
}

sage_status sage_debug_qk_s32(const sage_quantized* qz, int32_t* s_out, void* stream) {
    clear_err();
    Dims d;
    sage_status st;
    if ((st = check_quantized(qz, &d)) != SAGE_OK) return st;
    if (!s_out) return fail(SAGE_ERR_INVALID_ARGUMENT, "s_out is NULL");
    if (d.N > 4096) return fail(SAGE_ERR_UNSUPPORTED, "debug QK dump needs N <= 4096");
    if (d.B * d.H > 65535) return fail(SAGE_ERR_UNSUPPORTED, "debug QK dump needs B*H <= 65535");
    sage::DebugQkArgs p;
    p.q_i8 = qz->q_i8; p.k_i8 = qz->k_i8; p.s_out = s_out;
    p.B = (int)d.B; p.N = (int)d.N; p.H = (int)d.H; p.T = (int)d.T; p.G = (int)d.G;
    return hip_status(sage::launch_debug_qk(p, (hipStream_t)stream), "debug QK launch");
}

sage_status sage_debug_cvt_e4m3(const float* x, uint8_t* y, int64_t n, void* stream) {
    clear_err();
    if (!x || !y) return fail(SAGE_ERR_INVALID_ARGUMENT, "x or y is NULL");
    if (n < 0) return fail(SAGE_ERR_INVALID_ARGUMENT, "n < 0");
    if (n == 0) return SAGE_OK;
    if (n > ((int64_t)1 << 40)) return fail(SAGE_ERR_UNSUPPORTED, "n too large");
    return hip_status(sage::launch_cvt_e4m3(x, y, n, (hipStream_t)stream), "cvt launch");
}

sage_status sage_debug_issue_probe(int32_t kind, int32_t waves_per_simd, int32_t blocks, int32_t iters,
                                   uint64_t* ticks, void* stream) {
    clear_err();
    if (kind < 0 || kind > 2) return fail(SAGE_ERR_INVALID_ARGUMENT, "kind must be 0, 1 or 2");
    if (waves_per_simd < 1 || waves_per_simd > 4) return fail(SAGE_ERR_INVALID_ARGUMENT, "waves_per_simd must be 1..4");
    if (blocks < 1 || blocks > 65536) return fail(SAGE_ERR_INVALID_ARGUMENT, "blocks must be 1..65536");
    if (iters < 1 || iters > (1 << 20)) return fail(SAGE_ERR_INVALID_ARGUMENT, "iters must be 1..2^20");
    if (!ticks) return fail(SAGE_ERR_INVALID_ARGUMENT, "ticks is NULL");
    return hip_status(sage::launch_issue_probe(kind, waves_per_simd, blocks, iters, ticks, (hipStream_t)stream),
                      "issue probe launch");
}

}  // extern "C"
