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

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt), not for its global loads in flight, which __syncthreads' fence
// would also wait for.  The empty asm statements with a memory clobber keep
// the compiler from moving memory accesses across the barrier: s_barrier
// itself is not a memory operation to it, and a single-thread fence did not
// stop it from sinking an LDS read past the barrier into a later branch that
// uses the value.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// largest n in [0, N) with off[n] <= x (for off[0] <= x < off[N], the owner of x)
__device__ inline int off_find(const int32_t *off, int N, int x) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= x)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// The packed sequences of a prefill.  Sequence n spans tokens
// [start(n), end(n)); its chunks are chunk0(n) .. chunk0(n + 1) - 1 of the
// per-chunk operand blocks; its segments (L chunks each, the last one
// shorter) are seg0(n) .. seg0(n + 1) - 1; and those with a successor, whose
// transitions the scan composes, are numbered segA0(n) .. segA0(n + 1) - 1.
// With cu_seqlens the offsets are arrays that seq_table_kernel builds on the
// device (cu_seqlens is never read on the host).  Without, the call holds B
// sequences of Tper tokens: every entry is arithmetic and nothing is built.
struct SeqTable {
    int32_t *seg_off, *segA_off, *chunk_off;  // [N + 1] (cu_seqlens only)
    int64_t *seq_start, *seq_end;             // [N]     (cu_seqlens only)
    int L;                                    // chunks per segment
    int64_t Tper;                             // >= 0: fixed-length sequences; < 0: the arrays
    int nchp, segp;                           // fixed length: chunks and segments per sequence

    __device__ int64_t start(int n) const { return Tper >= 0 ? (int64_t)n * Tper : seq_start[n]; }
    __device__ int64_t end(int n) const { return Tper >= 0 ? (int64_t)(n + 1) * Tper : seq_end[n]; }
    __device__ int chunk0(int n) const { return Tper >= 0 ? n * nchp : chunk_off[n]; }
    __device__ int seg0(int n) const { return Tper >= 0 ? n * segp : seg_off[n]; }
    __device__ int segA0(int n) const { return Tper >= 0 ? n * max(segp - 1, 0) : segA_off[n]; }
    // owners, for an index below the total (chunk0(N), seg0(N), segA0(N))
    __device__ int seq_of_chunk(int c, int N) const { return Tper >= 0 ? c / nchp : off_find(chunk_off, N, c); }
    __device__ int seq_of_seg(int x, int N) const { return Tper >= 0 ? x / segp : off_find(seg_off, N, x); }
    __device__ int seq_of_segA(int a, int N) const {
        return Tper >= 0 ? a / max(segp - 1, 1) : off_find(segA_off, N, a);
    }
};
// Bytes of the table's arrays in a workspace, and their placement at p.
__host__ inline size_t seq_table_bytes(int N) {
    return 3 * align_up(4 * (size_t)(N + 1)) + 2 * align_up(8 * (size_t)N);
}
__host__ inline SeqTable seq_table_at(char *p, int N, int L) {
    SeqTable t{};
    t.seg_off = (int32_t *)p;
    p += align_up(4 * (size_t)(N + 1));
    t.segA_off = (int32_t *)p;
    p += align_up(4 * (size_t)(N + 1));
    t.chunk_off = (int32_t *)p;
    p += align_up(4 * (size_t)(N + 1));
    t.seq_start = (int64_t *)p;
    p += align_up(8 * (size_t)N);
    t.seq_end = (int64_t *)p;
    t.L = L;
    t.Tper = -1;
    return t;
}
// Fill the table for a call: fixed-length sequences of T tokens (cu == nullptr)
// set the arithmetic fields; with cu_seqlens seq_table_kernel is launched.
int launch_seq_table(const int32_t *cu, int N, int64_t T_total, int64_t T, SeqTable &t, hipStream_t stream);
// off[n] = sum over sequences m < n of floor(len_m / stride), n = 0 .. N.
int launch_ckpt_prep(const SeqTable &t, int N, int64_t stride, int64_t *off, hipStream_t stream);

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

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp16 hi/lo split of a pair of floats: hi = fp16(a), fp16(b), lo = fp16 of the
// remainders.  a - fp32(hi) is exact in fp32, so one mixed-precision FMA per
// element (fp16 hi and fp32 a as sources, fp16 result) gives the same lo as a
// subtraction in fp32 followed by a conversion, in one instruction.
__device__ __forceinline__ void split_f16_pair(float a, float b, uint32_t &hi, uint32_t &lo) {
    const f16x2 h = {(_Float16)a, (_Float16)b};
    hi = __builtin_bit_cast(uint32_t, h);
    asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, -%1, 1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(lo)
        : "v"(hi), "v"(a), "v"(b));
}

// Unsigned maximum over one DPP row (16 lanes with equal lane / 16), in every lane.
__device__ __forceinline__ uint32_t row_umax16(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false));
    return x;
}
// Unsigned maximum over the whole wave, wave-uniform (so the compiler keeps it
// in a scalar register and branches on it without divergence).
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
    x = row_umax16(x);
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16),
                   c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
    return max(max(a, b), max(c, d));
}
// Buffer resource word 3 for raw (untyped) buffer access on gfx9-family chips:
// 32-bit data format, so accesses past num_records read 0 and drop writes.
constexpr int BUF_RSRC3 = 0x00020000;
typedef __attribute__((address_space(3))) void lds_void;

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
        const uint32_t u = __builtin_bit_cast(uint32_t, hp);
        const float fa = __builtin_bit_cast(float, u << 16), fb = __builtin_bit_cast(float, u & 0xffff0000u);
        const bf16x2 lp = {(__bf16)(a - fa), (__bf16)(b - fb)};
        s.hi[2 * p] = hp[0];
        s.hi[2 * p + 1] = hp[1];
        s.lo[2 * p] = lp[0];
        s.lo[2 * p + 1] = lp[1];
    }
    return s;
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
// 2^x (v_exp_f32: 2^-inf = 0, 2^inf = inf, NaN propagates).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float LOG2E = 1.44269504088896341f;
// The log-decay in base 2, g log2 e: the K3 gate as g_min log2 e * Sigmoid(x)
// with e^-x = 2^{-x log2 e} (same limits as kda_gate), the softplus decay scaled.
template <int GK>
__device__ __forceinline__ float gate_log2(float expA, float z) {
    if constexpr (GK == GATE_K3)
        return (GMIN * LOG2E) * __builtin_amdgcn_rcpf(1.f + ex2(-(expA * LOG2E) * z));
    else
        return softplus_gate(expA, z) * LOG2E;
}

}  // namespace kda
