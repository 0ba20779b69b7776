// kda_api.cpp -- C ABI of libkda.so (declared in include/kda.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so invalid calls return a status and launch nothing.  Kernels
// live in kda_decode.hip (recurrent step) and kda_prefill.hip (chunkwise form).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"
#include "kda_common.hpp"

#define KDA_EXPORT extern "C" __attribute__((visibility("default")))

namespace kda {
int launch_decode(const void *q, const void *k, const void *v, bool f32io, const float *z, const float *beta,
                  const float *A, float *S, int N, int H, float *o, const Layer &ly, hipStream_t stream);
int launch_prefill(const void *q, const void *k, const void *v, bool f32io, const float *z, const float *beta,
                   const float *A, const float *S0, const int32_t *cu, int B, int64_t T, int H, int N,
                   float *o, float *S_final, const Ckpt &ck, const Layer &ly, void *ws, hipStream_t stream,
                   hipEvent_t *ev);
size_t prefill_workspace_bytes(int64_t T_total, int N, int H, bool f32io);
int set_prefill_attributes();
}  // namespace kda

namespace {

constexpr int kD = 128;

bool misaligned(const void *p) { return p && ((uintptr_t)p & 15u) != 0; }

// [a, a + na) and [b, b + nb) share a byte
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

std::once_flag g_attr_once;
int g_attr_status = 0;

// Device-resident workspace of kda_chunk_fwd_noalloc, one copy per GPU (the
// code object holds it for as long as the process runs).  In host code the
// array's name is only a stand-in: its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[KDA_NOALLOC_WORKSPACE_BYTES];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Passed as `workspace` by kda_chunk_fwd_noalloc: "use the array above".
void *const kStaticWorkspace = (void *)&g_scratch_ptr;

// The device address of `scratch` on `dev`, or nullptr if it cannot be had.
void *scratch_on(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev] {
        int cur = -1;
        hipError_t rc = hipGetDevice(&cur);
        if (rc == hipSuccess && cur != dev) rc = hipSetDevice(dev);
        void *ptr = nullptr;
        if (rc == hipSuccess) rc = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev && hipSetDevice(cur) != hipSuccess && rc == hipSuccess) rc = hipErrorUnknown;
        g_scratch_status[dev] = rc;
        g_scratch_ptr[dev] = rc == hipSuccess ? ptr : nullptr;
    });
    return g_scratch_ptr[dev];
}

}  // namespace

KDA_EXPORT const char *kda_status_str(int status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: dk and dv must be 128 and sizes non-negative";
        case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: qkv_dtype must be KDA_BF16 or KDA_F32";
        case KDA_ERR_SEQLENS: return "KDA_ERR_SEQLENS: cu_seqlens needs B == 1 and n_seqs >= 1";
        case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: pointers must be 16-byte aligned";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP launch failed";
        case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: o overlaps an input";
        default: return "KDA_ERR_UNKNOWN";
    }
}

KDA_EXPORT int kda_version(void) { return 100; }

KDA_EXPORT size_t kda_chunk_fwd_workspace_bytes(int64_t T_total, int32_t n_seqs, int32_t H, kda_dtype qkv_dtype) {
    if (T_total < 0 || n_seqs < 0 || H < 0 || H > KDA_MAX_HEADS) return 0;
    if (qkv_dtype != KDA_BF16 && qkv_dtype != KDA_F32) return 0;
    if (T_total == 0 && n_seqs == 0) return 0;
    return kda::prefill_workspace_bytes(T_total, n_seqs, H, qkv_dtype == KDA_F32);
}

namespace {

// Shared body of the prefill entry points.
int chunk_fwd(const void *q, const void *k, const void *v, kda_dtype qkv_dtype, const float *g_raw,
              const float *beta, const float *A, const float *S0, const int32_t *cu_seqlens, int32_t B, int64_t T,
              int32_t H, int32_t n_seqs, int32_t dk, int32_t dv, float *o, float *S_final, void *workspace,
              size_t workspace_bytes, void *stream, void *const *stage_events, float *S_ckpt, int64_t ckpt_stride,
              int64_t ckpt_capacity, const kda_layer_opts *lo) {
    if (dk != kD || dv != kD) return KDA_ERR_SHAPE;
    if (B < 0 || T < 0 || H < 0 || H > KDA_MAX_HEADS || n_seqs < 0) return KDA_ERR_SHAPE;
    if (qkv_dtype != KDA_BF16 && qkv_dtype != KDA_F32) return KDA_ERR_DTYPE;
    if (cu_seqlens) {
        if (B != 1 || n_seqs < 1) return KDA_ERR_SEQLENS;
    } else if (n_seqs != B) {
        return KDA_ERR_SEQLENS;
    }
    if (S_ckpt && (ckpt_stride <= 0 || ckpt_stride % 64 != 0 || ckpt_stride / 64 > INT32_MAX || ckpt_capacity < 0))
        return KDA_ERR_SHAPE;
    const float *out_gate = lo ? lo->out_gate : nullptr, *norm_weight = lo ? lo->norm_weight : nullptr;
    if (lo && (!(lo->qk_eps >= 0.f) || !(lo->norm_eps >= 0.f))) return KDA_ERR_SHAPE;  // NaN fails too
    if (lo && lo->gate_kind != KDA_GATE_K3 && lo->gate_kind != KDA_GATE_SOFTPLUS) return KDA_ERR_SHAPE;
    if (lo && lo->reverse_order != 0) return KDA_ERR_SHAPE;  // a decode option
    const bool lrz = lo && lo->gate_u;
    if (lrz && (lo->gate_rank < 32 || lo->gate_rank > 256 || lo->gate_rank % 32 != 0 || lo->gate_per_head))
        return KDA_ERR_SHAPE;
    const size_t z_row = lrz ? 0 : (lo && lo->gate_per_head ? 1 : kD);  // g_raw values per (token, head)
    const int64_t T_total = (int64_t)B * T;
    if (T_total > INT32_MAX - 64 || (int64_t)n_seqs * H > INT32_MAX / 64) return KDA_ERR_SHAPE;
    if (S_ckpt && ckpt_capacity > (int64_t)(SIZE_MAX / 2) / ((int64_t)(H > 0 ? H : 1) * kD * kD * 4))
        return KDA_ERR_SHAPE;
    if (n_seqs == 0 || H == 0) return KDA_OK;  // nothing to compute
    if (!A) return KDA_ERR_NULL;
    if (T_total > 0 && (!q || !k || !v || (!g_raw && !lrz) || !beta || !o)) return KDA_ERR_NULL;
    if (out_gate && !norm_weight) return KDA_ERR_NULL;
    if (lrz && !lo->gate_w) return KDA_ERR_NULL;
    const void *gu = lrz ? lo->gate_u : nullptr, *gw = lrz ? lo->gate_w : nullptr;
    const void *ptrs[] = {q,      k,        v,           g_raw, beta, A, S0, o, S_final,
                          workspace == kStaticWorkspace ? nullptr : workspace, S_ckpt, out_gate, norm_weight, gu, gw};
    for (const void *p : ptrs)
        if (misaligned(p)) return KDA_ERR_ALIGN;
    const size_t need = kda_chunk_fwd_workspace_bytes(T_total, n_seqs, H, qkv_dtype);
    // kda_chunk_fwd_noalloc passes kStaticWorkspace: the library's own array,
    // whose address is looked up only once every other check has passed.
    const bool own_ws = workspace == kStaticWorkspace;
    if (own_ws ? need > (size_t)KDA_NOALLOC_WORKSPACE_BYTES : (!workspace || workspace_bytes < need))
        return KDA_ERR_WORKSPACE;
    if (own_ws) workspace = nullptr;
    const size_t esz = qkv_dtype == KDA_F32 ? 4 : 2;
    const size_t tok = (size_t)T_total * H;
    const size_t o_bytes = tok * kD * 4;
    const size_t st_bytes = (size_t)n_seqs * H * kD * kD * 4;
    if (overlap(o, o_bytes, q, tok * kD * esz) || overlap(o, o_bytes, k, tok * kD * esz) ||
        overlap(o, o_bytes, v, tok * kD * esz) || overlap(o, o_bytes, g_raw, tok * z_row * 4) ||
        overlap(o, o_bytes, beta, tok * 4) || overlap(o, o_bytes, A, (size_t)H * 4) ||
        overlap(o, o_bytes, S0, st_bytes) || overlap(o, o_bytes, S_final, st_bytes) ||
        overlap(o, o_bytes, workspace, need) || overlap(o, o_bytes, out_gate, o_bytes) ||
        overlap(o, o_bytes, norm_weight, (size_t)kD * 4) ||
        (lrz && (overlap(o, o_bytes, gu, (size_t)T_total * lo->gate_rank * 2) ||
                 overlap(o, o_bytes, gw, (size_t)H * kD * lo->gate_rank * 2))))
        return KDA_ERR_ALIAS;
    if (S_ckpt) {
        const size_t ck_bytes = (size_t)ckpt_capacity * H * kD * kD * 4;
        const void *others[] = {q, k, v, g_raw, beta, A, S0, o, S_final, workspace};
        const size_t sizes[] = {tok * kD * esz, tok * kD * esz, tok * kD * esz, tok * z_row * 4, tok * 4,
                                (size_t)H * 4, st_bytes, o_bytes, st_bytes, need};
        for (int i = 0; i < 10; ++i)
            if (overlap(S_ckpt, ck_bytes, others[i], sizes[i])) return KDA_ERR_ALIAS;
    }

    if (own_ws) {
        int dev = -1;
        if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return KDA_ERR_HIP;
        workspace = scratch_on(dev);  // the array of the stream's GPU
        if (!workspace) return KDA_ERR_HIP;
        if (overlap(o, o_bytes, workspace, need) || overlap(S_ckpt, (size_t)ckpt_capacity * H * kD * kD * 4, workspace, need))
            return KDA_ERR_ALIAS;
    }
    std::call_once(g_attr_once, [] { g_attr_status = kda::set_prefill_attributes(); });
    if (g_attr_status != 0) return KDA_ERR_HIP;
    const kda::Ckpt ck{S_ckpt && ckpt_capacity > 0 ? S_ckpt : nullptr, nullptr, (int)(S_ckpt ? ckpt_stride / 64 : 1),
                       ckpt_capacity};
    const kda::Layer ly{lo && lo->qk_l2norm != 0, lo ? lo->qk_eps : 0.f, out_gate, norm_weight,
                        lo ? lo->norm_eps : 0.f, lo ? lo->gate_kind : KDA_GATE_K3, lo && lo->gate_per_head != 0,
                        false, (const __bf16 *)gu, (const __bf16 *)gw, lrz ? lo->gate_rank : 0};
    const int rc = kda::launch_prefill(q, k, v, qkv_dtype == KDA_F32, g_raw, beta, A, S0, cu_seqlens, B, T, H,
                                       n_seqs, o, S_final, ck, ly, workspace, (hipStream_t)stream,
                                       (hipEvent_t *)stage_events);
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

KDA_EXPORT int kda_chunk_fwd_timed(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                                   const float *g_raw, const float *beta, const float *A, const float *S0,
                                   const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t n_seqs,
                                   int32_t dk, int32_t dv, float *o, float *S_final, void *workspace,
                                   size_t workspace_bytes, void *stream, void *const *stage_events) {
    return chunk_fwd(q, k, v, qkv_dtype, g_raw, beta, A, S0, cu_seqlens, B, T, H, n_seqs, dk, dv, o, S_final,
                     workspace, workspace_bytes, stream, stage_events, nullptr, 0, 0, nullptr);
}

KDA_EXPORT int kda_chunk_fwd(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                             const float *g_raw, const float *beta, const float *A, const float *S0,
                             const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t n_seqs,
                             int32_t dk, int32_t dv, float *o, float *S_final, void *workspace,
                             size_t workspace_bytes, void *stream) {
    return chunk_fwd(q, k, v, qkv_dtype, g_raw, beta, A, S0, cu_seqlens, B, T, H, n_seqs, dk, dv, o, S_final,
                     workspace, workspace_bytes, stream, nullptr, nullptr, 0, 0, nullptr);
}

KDA_EXPORT int kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                                     const float *g_raw, const float *beta, const float *A, const float *S0,
                                     const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t n_seqs,
                                     int32_t dk, int32_t dv, float *o, float *S_final, void *stream) {
    return chunk_fwd(q, k, v, qkv_dtype, g_raw, beta, A, S0, cu_seqlens, B, T, H, n_seqs, dk, dv, o, S_final,
                     kStaticWorkspace, 0, stream, nullptr, nullptr, 0, 0, nullptr);
}

KDA_EXPORT int kda_chunk_fwd_ckpt(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                                  const float *g_raw, const float *beta, const float *A, const float *S0,
                                  const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t n_seqs,
                                  int32_t dk, int32_t dv, float *o, float *S_final, float *S_ckpt,
                                  int64_t ckpt_stride, int64_t ckpt_capacity, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    if (!S_ckpt) return KDA_ERR_NULL;
    return chunk_fwd(q, k, v, qkv_dtype, g_raw, beta, A, S0, cu_seqlens, B, T, H, n_seqs, dk, dv, o, S_final,
                     workspace, workspace_bytes, stream, nullptr, S_ckpt, ckpt_stride, ckpt_capacity, nullptr);
}

KDA_EXPORT int kda_chunk_fwd_layer(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                                   const float *g_raw, const float *beta, const float *A, const float *S0,
                                   const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t n_seqs,
                                   int32_t dk, int32_t dv, const kda_layer_opts *opts, float *o, float *S_final,
                                   float *S_ckpt, int64_t ckpt_stride, int64_t ckpt_capacity, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    if (!opts) return KDA_ERR_NULL;
    return chunk_fwd(q, k, v, qkv_dtype, g_raw, beta, A, S0, cu_seqlens, B, T, H, n_seqs, dk, dv, o, S_final,
                     workspace, workspace_bytes, stream, nullptr, S_ckpt, ckpt_stride, ckpt_capacity, opts);
}

namespace {

// Shared body of the decode entry points.
int decode_step(const void *q, const void *k, const void *v, kda_dtype qkv_dtype, const float *g_raw,
                const float *beta, const float *A, float *S, int32_t N, int32_t H, int32_t dk, int32_t dv, float *o,
                void *stream, const kda_layer_opts *lo) {
    if (dk != kD || dv != kD) return KDA_ERR_SHAPE;
    if (N < 0 || H < 0) return KDA_ERR_SHAPE;
    if (qkv_dtype != KDA_BF16 && qkv_dtype != KDA_F32) return KDA_ERR_DTYPE;
    if ((int64_t)N * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (lo && (!(lo->qk_eps >= 0.f) || !(lo->norm_eps >= 0.f))) return KDA_ERR_SHAPE;  // NaN fails too
    if (lo && lo->gate_kind != KDA_GATE_K3 && lo->gate_kind != KDA_GATE_SOFTPLUS) return KDA_ERR_SHAPE;
    const bool lrz = lo && lo->gate_u;
    if (lrz && (lo->gate_rank < 32 || lo->gate_rank > 256 || lo->gate_rank % 32 != 0 || lo->gate_per_head))
        return KDA_ERR_SHAPE;
    if (N == 0 || H == 0) return KDA_OK;
    if (!q || !k || !v || (!g_raw && !lrz) || !beta || !A || !S || !o) return KDA_ERR_NULL;
    const float *out_gate = lo ? lo->out_gate : nullptr, *norm_weight = lo ? lo->norm_weight : nullptr;
    if (out_gate && !norm_weight) return KDA_ERR_NULL;
    if (lrz && !lo->gate_w) return KDA_ERR_NULL;
    const void *gu = lrz ? lo->gate_u : nullptr, *gw = lrz ? lo->gate_w : nullptr;
    const void *ptrs[] = {q, k, v, g_raw, beta, A, S, o, out_gate, norm_weight, gu, gw};
    for (const void *p : ptrs)
        if (misaligned(p)) return KDA_ERR_ALIGN;
    const size_t esz = qkv_dtype == KDA_F32 ? 4 : 2;
    const size_t nh = (size_t)N * H;
    const size_t o_bytes = nh * kD * 4;
    const size_t z_row = lrz ? 0 : (lo && lo->gate_per_head ? 1 : kD);
    if ((lrz && (overlap(o, o_bytes, gu, (size_t)N * lo->gate_rank * 2) ||
                 overlap(o, o_bytes, gw, (size_t)H * kD * lo->gate_rank * 2))) ||
        overlap(o, o_bytes, S, nh * kD * kD * 4) || overlap(o, o_bytes, q, nh * kD * esz) ||
        overlap(o, o_bytes, k, nh * kD * esz) || overlap(o, o_bytes, v, nh * kD * esz) ||
        overlap(o, o_bytes, g_raw, nh * z_row * 4) || overlap(o, o_bytes, beta, nh * 4) ||
        overlap(o, o_bytes, A, (size_t)H * 4) || overlap(o, o_bytes, out_gate, o_bytes) ||
        overlap(o, o_bytes, norm_weight, (size_t)kD * 4))
        return KDA_ERR_ALIAS;
    const kda::Layer ly{lo && lo->qk_l2norm != 0, lo ? lo->qk_eps : 0.f, out_gate, norm_weight,
                        lo ? lo->norm_eps : 0.f, lo ? lo->gate_kind : KDA_GATE_K3, lo && lo->gate_per_head != 0,
                        lo && lo->reverse_order != 0, (const __bf16 *)gu, (const __bf16 *)gw, lrz ? lo->gate_rank : 0};
    const int rc = kda::launch_decode(q, k, v, qkv_dtype == KDA_F32, g_raw, beta, A, S, N, H, o, ly,
                                      (hipStream_t)stream);
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

KDA_EXPORT int kda_decode_step(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                               const float *g_raw, const float *beta, const float *A, float *S, int32_t N,
                               int32_t H, int32_t dk, int32_t dv, float *o, void *stream) {
    return decode_step(q, k, v, qkv_dtype, g_raw, beta, A, S, N, H, dk, dv, o, stream, nullptr);
}

KDA_EXPORT int kda_decode_step_layer(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                                     const float *g_raw, const float *beta, const float *A, float *S, int32_t N,
                                     int32_t H, int32_t dk, int32_t dv, const kda_layer_opts *opts, float *o,
                                     void *stream) {
    if (!opts) return KDA_ERR_NULL;
    return decode_step(q, k, v, qkv_dtype, g_raw, beta, A, S, N, H, dk, dv, o, stream, opts);
}
