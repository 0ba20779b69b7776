// kda_common.hpp -- shared device helpers for the gfx950 KDA kernels.
//
// MFMA fragment conventions (v_mfma_f32_16x16x32_bf16, wave64):
//   A operand (16 x 32): lane l holds row (l & 15) and the 8 consecutive k
//                        indices 8 * (l >> 4) + e, e = 0..7;
//   B operand (32 x 16): lane l holds column (l & 15), same 8 k indices;
//   C / D     (16 x 16): lane l holds column (l & 15), rows 4 * (l >> 4) + i.
// Because the k index is summed, any permutation of k is allowed as long as
// the A and B fragments use the same one.  The fp32 path feeds the same
// 8-element fragments to eight v_mfma_f32_16x16x4_f32 (one per element e),
// which again pairs equal k on both sides.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int D = 128;      // d_k = d_v (Kimi Linear summary, sections 4 and 6.3)
constexpr int CH = 64;      // chunk length (section 6.3, appendix C)
constexpr int SUB = 16;     // sub-chunk length (Kimi K3: 16-token tiles)
constexpr float GMIN = -5.f;  // Kimi K3 lower bound of the log-decay

__host__ __device__ constexpr size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// State snapshots at a chunk-aligned stride, for a KDA-aware prefix cache
// (Kimi K3 paper review, Significance and Limitations paragraphs: the recurrent
// state is kept only at sparse checkpoint boundaries).  Snapshot m of sequence
// n is the state after its first (m + 1) * stride tokens, stored at slot
// off[n] + m of S, where off is the exclusive prefix sum of floor(len / stride)
// over the sequences; slots at or past `cap` are not written.  S == nullptr
// turns snapshots off.
struct Ckpt {
    float *S;
    const int64_t *off;  // [N + 1], built on the device by ckpt_prep_kernel
    int stride_chunks;   // stride / 64
    int64_t cap;
};

// The KDA layer's steps on either side of the operator (Kimi Linear summary,
// section 4), fused into the prefill: unit-length queries and keys
// (x / sqrt(sum x^2 + qk_eps) per token and head), and the output's per-head
// RMSNorm followed by the sigmoid output gate,
// o <- o / sqrt(mean o^2 + norm_eps) * weight * sigmoid(gate).
struct Layer {
    bool qk_norm;
    float qk_eps;
    const float *gate;    // [tokens, H, 128] fp32 pre-activation, or nullptr: no output step
    const float *weight;  // [128]
    float norm_eps;
    int gate_kind;        // GATE_K3 or GATE_SOFTPLUS
    bool gate_per_head;   // z is [tokens, H]: one gate value per (token, head)
    bool reverse_order;   // decode: visit (sequence, head) pairs last to first
    // Low-rank forget gate: z[t, h, c] = sum_j zu[t, j] zw[h, c, j] (zu == nullptr: z is given).
    const __bf16 *zu;     // [tokens, zrank]
    const __bf16 *zw;     // [H, 128, zrank]
    int zrank;            // a multiple of 32, at most 256
};

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Eight fp32 values of one lane's 32-deep k slice.
struct F8 {
    float v[8];
};
// The same values as an unevaluated sum hi + lo of two bf16 vectors.
struct S8 {
    bf16x8 hi, lo;
};

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
// hi = RNE bf16 of each value; lo = RNE bf16 of the remainder.  Pairs are
// rounded with one packed conversion and widened back with shifts/masks.
__device__ __forceinline__ S8 split8(const F8 &x) {
    S8 s;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float a = x.v[2 * p], b = x.v[2 * p + 1];
        const bf16x2 hp = {(__bf16)a, (__bf16)b};
        uint32_t u = __builtin_bit_cast(uint32_t, hp);
        asm("" : "+v"(u));  // keep the packed pair: widen it instead of converting a again
        const float fa = __builtin_bit_cast(float, u << 16), fb = __builtin_bit_cast(float, u & 0xffff0000u);
        const bf16x2 lp = {(__bf16)(a - fa), (__bf16)(b - fb)};
        s.hi[2 * p] = hp[0];
        s.hi[2 * p + 1] = hp[1];
        s.lo[2 * p] = lp[0];
        s.lo[2 * p + 1] = lp[1];
    }
    return s;
}
__device__ __forceinline__ bf16x8 round8(const F8 &x) {
    bf16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (__bf16)x.v[e];
    return h;
}

// Products of fragments.  "s" = split (hi + lo), "1" = single bf16.
// hi*lo and lo*hi are kept, lo*lo is dropped (below fp32 rounding of the sum).
__device__ __forceinline__ f32x4 mma_ss(f32x4 c, const S8 &a, const S8 &b) {
    c = mfma_bf16(a.lo, b.hi, c);
    c = mfma_bf16(a.hi, b.lo, c);
    return mfma_bf16(a.hi, b.hi, c);
}
__device__ __forceinline__ f32x4 mma_s1(f32x4 c, const S8 &a, bf16x8 b) {
    c = mfma_bf16(a.lo, b, c);
    return mfma_bf16(a.hi, b, c);
}
__device__ __forceinline__ f32x4 mma_1s(f32x4 c, bf16x8 a, const S8 &b) {
    c = mfma_bf16(a, b.lo, c);
    return mfma_bf16(a, b.hi, c);
}
__device__ __forceinline__ f32x4 mma_11(f32x4 c, bf16x8 a, bf16x8 b) { return mfma_bf16(a, b, c); }
// exact fp32 products (fp32 I/O build)
__device__ __forceinline__ f32x4 mma_ff(f32x4 c, const F8 &a, const F8 &b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = mfma_f32(a.v[e], b.v[e], c);
    return c;
}

__device__ __forceinline__ F8 ld_f8(const float *p) {  // 32-byte aligned
    F8 r;
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
    r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
    return r;
}
__device__ __forceinline__ bf16x8 ld_b8(const __bf16 *p) { return *(const bf16x8 *)p; }

// load 8 consecutive inputs of type IO as fp32
__device__ __forceinline__ F8 ld_io8(const float *p) { return ld_f8(p); }
__device__ __forceinline__ F8 ld_io8(const __bf16 *p) {
    bf16x8 b = ld_b8(p);
    F8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.v[e] = (float)b[e];
    return r;
}
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }

// Kimi K3 gate: g = g_min * Sigmoid(e^A z) with Sigmoid(x) = 1 / (1 + e^-x)
// evaluated as v_rcp(1 + v_exp): x = +inf gives exactly g_min, x = -inf gives
// e^-x = inf and exactly 0, NaN propagates.  v_rcp_f32 is accurate to 1 ulp.
__device__ __forceinline__ float kda_gate(float expA, float z) {
    const float x = expA * z;
    return GMIN * __builtin_amdgcn_rcpf(1.f + __expf(-x));
}
// Kimi Linear's unbounded negative-softplus decay, the parameterisation the K3
// gate replaces (Kimi K3 architecture, sequence-bottleneck section; K3 paper
// review, Method): g = -e^A softplus(z), softplus(z) = max(z, 0) + log(1 + e^-|z|).
// z = -inf gives 0 (alpha = 1).  A step's log-decay is floored at SP_G_FLOOR:
// e^-104 lies below fp32's smallest subnormal (e^-103.3), so alpha is zero in
// fp32 either way, and the floor keeps the chunk form's running sums finite
// (z = +inf would otherwise give differences -inf - (-inf)).  NaN propagates.
constexpr float SP_G_FLOOR = -104.f;
__device__ __forceinline__ float softplus_gate(float expA, float z) {
    const float g = -expA * (fmaxf(z, 0.f) + __logf(1.f + __expf(-fabsf(z))));
    return g < SP_G_FLOOR ? SP_G_FLOOR : g;
}
// Decay parameterisations (kda_layer_opts::gate_kind).
enum { GATE_K3 = 0, GATE_SOFTPLUS = 1 };
template <int GK>
__device__ __forceinline__ float gate_of(float expA, float z) {
    if constexpr (GK == GATE_K3)
        return kda_gate(expA, z);
    else
        return softplus_gate(expA, z);
}

}  // namespace kda
