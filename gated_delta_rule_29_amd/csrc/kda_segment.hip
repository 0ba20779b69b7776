// kda_segment.hip -- chunkwise KDA prefill for bf16 q/k/v on gfx950.
//
// Pages: "Kimi Linear: An Expressive, Efficient Attention Architecture" summary
// (sections 2.1, 3.1, 6.3, appendix C: chunk size 64, WY / UT transform with a
// forward-substitution inverse, inter-chunk recurrence) and "Kimi K3
// architecture" (sequence-bottleneck section: g = -5 Sigmoid(e^A z), 16-token
// tiles; KDA context parallelism merges local state updates with a prefix scan).
//
// Within a chunk of n <= 64 tokens with incoming state S (rows = key channel):
//   G_t      inclusive cumulative log-decay per key channel, Gam_t = e^{G_t}
//   Akk[r,c] = beta_r sum_j k_rj k_cj e^{G_rj - G_cj}   (c < r)
//   Aqk[r,c] = sum_j q_rj k_cj e^{G_rj - G_cj}          (c <= r)
//   T = (I + Akk)^{-1},  W = T diag(beta) (K * Gam),  U = T diag(beta) V
//   Delta = U - W S,  O = (Q * Gam) S + Aqk Delta,
//   S' = Diag(gamma) S + K~^T Delta,  K~ = K * e^{G_n - G},  gamma = e^{G_n}.
// So each chunk maps the state affinely, S' = M S + B with
// M = Diag(gamma) - K~^T W and B = K~^T U.
//
// Kernels, in stream order:
//   seq_table_kernel  (with cu_seqlens; kda_prefill.hip) sequence bounds, per-sequence first chunk and first
//                     segment (a segment = L consecutive chunks of a sequence);
//   wy_kernel         one workgroup per (chunk, head), all chunks in parallel:
//                     gate and cumulative sums, the two decay-scaled Gram
//                     tiles, the blocked forward-substitution inverse and the
//                     WY / UT products; writes one block of chain operands
//                     (W, Q~, K~^T, Aqk, U, gamma) per (chunk, head);
//   seg_chain_kernel<A>  per (segment, head): from X = [I | 0] runs the chain
//                     on the 256 columns of X and writes the segment map
//                     (M_p, B_p);
//   seg_scan_kernel   per (sequence, head): S_in[0] = S0,
//                     S_in[p+1] = M_p S_in[p] + B_p;
//   seg_chain_kernel<B>  per (segment, head): from S_in[p] runs the chain with
//                     outputs, writes o (and S_final for the last segment).
//
// Operand blocks are stored fragment-major: an MFMA operand tile is 64 lanes x
// 16 B, stored lane after lane, so a wave moves it with one coalesced 16 B
// access per lane, in global memory and in LDS alike.
//
// The chain step is wave-local: wave w owns a slice of state columns, keeps it
// in MFMA C-layout registers and feeds those registers back as the B operand
// of the next product.  That works because the k index of an MFMA is summed:
// pairing the C tiles 2s and 2s+1 gives k slot e -> row
// 32s + 16*(e>>2) + 4*(lane>>4) + (e&3), and the A operands (W, Q~ over key
// channels; Aqk, K~^T over tokens) are stored with that permutation (perm32).
//
// Operand precision (chosen against the fp64 oracle): W, Q~, K~ and the state
// enter the chain as single fp16; Delta as fp16 hi + lo; Aqk as fp16 hi + lo;
// the Gram tiles and T diag(beta) as bf16 hi + lo (their column factors reach
// e^80, beyond fp16 range).  U is stored in 16-bit fixed point with a
// power-of-two scale per 4 x 16 block (error <= 2^-14 of the block's largest
// value): U enters the state, so its rounding accumulates along the chain, and
// single fp16 (relative 2^-11 per value) doubled the error of o; the block
// format costs the bytes of fp16 and keeps the error of fp32 U.
#include <utility>

#include "kda_common.hpp"

namespace kda {


// Byte layout of the chain-operand block of one (chunk, head).
constexpr int BO_W = 0;        // -W   A tiles (token tile rt 0..3, key block s 0..3), fp16, k = perm32(channel)
constexpr int BO_QT = 16384;   // Q~   same layout as W
constexpr int BO_KT = 32768;   // K~^T A tiles (key tile rt 0..7, token block s 0..1), fp16, k = perm32(token)
constexpr int BO_AQ = 49152;   // Aqk  A tiles (rt, s <= rt/2): fp16 hi tile then lo tile, k = perm32(token)
constexpr int BO_U = 61440;    // U    C tiles (token tile rt 0..3, value tile ct 0..7), 16-bit fixed point (UBlk)
constexpr int U_TILE = 512;    // bytes of one U tile: 8 per lane
constexpr int BO_US = 77824;   // U scales: fp32 per (tile, lane group g), each for 4 rows x 16 columns
constexpr int BO_GM = 78336;   // gamma = e^{G_n}, 128 fp32
constexpr size_t BLK = 78848;  // multiple of 256

__device__ __forceinline__ int aq_tile(int rt, int s) { return rt < 2 ? rt : 2 * rt - 2 + s; }
__device__ __forceinline__ int frag(int tile, int lane) { return (tile * 64 + lane) * 16; }

__device__ __forceinline__ bf16x4 ld_bf16x4(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

constexpr int PTT = 68;  // pitch (floats) of T [64][64]

// max |u| over a lane's four values as the bits of a non-negative float: as
// unsigned integers these order like the values, and NaN orders above inf, so
// a NaN is kept (fmaxf would drop it).
__device__ __forceinline__ uint32_t abs_max_bits(f32x4 u) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x = u[i];  // a value: a bit-cast of the element expression reads element 0
        m = max(m, __builtin_bit_cast(uint32_t, x) & 0x7FFFFFFFu);
    }
    return m;
}

// U in 16-bit fixed point: each block of 4 rows x 16 columns (one lane group of
// a C tile) shares a power-of-two scale sc with max|u| / sc < 2^14, so a value
// is stored to within sc / 2 <= 2^-14 max|u| of the block, and |q| <= 2^14
// needs no clamp.  Decoding, q * sc, is exact.  A block holding inf or NaN
// gets that value as its scale and q = 0, so all of it decodes to NaN.
struct UBlk {
    uint32_t q01, q23;
    float sc;
};
__device__ __forceinline__ UBlk u_encode(f32x4 u, uint32_t bmax_bits) {
    const float bmax = __builtin_bit_cast(float, bmax_bits);
    const uint32_t eb = bmax_bits >> 23;  // bmax < 2^(eb - 126); 0xFF: inf or NaN
    const uint32_t e2 = max(eb, 14u) - 13;                                   // sc = 2^(e2 - 127)
    const bool fin = eb != 0xFF;
    const float sc = fin ? __builtin_bit_cast(float, e2 << 23) : bmax;
    const float inv = fin ? __builtin_bit_cast(float, (254 - e2) << 23) : 0.f;
    int qv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) qv[m] = (int)rintf(u[m] * inv);
    return {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(qv[0], qv[1])),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(qv[2], qv[3])), sc};
}
// Decoded and multiplied by 2^e (exact unless the result leaves fp32's normal range).
__device__ __forceinline__ f32x4 u_decode(UBlk b, int e) {
    const float sc = __builtin_amdgcn_ldexpf(b.sc, e);
    f32x4 u;
    u[0] = (float)(int)(int16_t)(b.q01 & 0xFFFF) * sc;
    u[1] = (float)((int)b.q01 >> 16) * sc;
    u[2] = (float)(int)(int16_t)(b.q23 & 0xFFFF) * sc;
    u[3] = (float)((int)b.q23 >> 16) * sc;
    return u;
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

struct SegTable {
    SeqTable sq;         // the sequences, their chunks and segments (pass A: those with a successor)
    char *blocks;        // chain operands, block (c, h) at (c * H + h) * BLK
    float *Mseg;         // [nseg][H][128][128] segment transitions
    float *Bseg;         // [nseg][H][128][128] segment offsets
    float *Sin;          // [nseg][H][128][128] state entering each segment
    Ckpt ck;             // state snapshots (ck.S == nullptr: none)
    Layer ly;            // fused layer steps around the operator
};

// -------------------------------------------------------------- WY / UT --

constexpr int PEH = 68;  // pitch (floats) of the half-width arrays [64 tokens][64 channels]

template <int GK>
struct WySmem {
    union {
        float E1[CH * PEH];  // e^{G_t - R_s}, s = sub-chunk of t, one 64-channel half (phases 1-2)
        float T[CH * PTT];   // Akk, then T = (I + Akk)^{-1} (phases 2-4)
    } a;
    float CB[CH * PEH];      // k_t e^{R_{s+1} - G_t}, in [e^-80, 1] |k_t|, same half (phases 1-2)
    // K3 gate: e^{R_i - R_{j+1}} for j <= i, row i(i+1)/2 + j.  Softplus decay:
    // R_s, s = 0..3, as logs (the factors are formed when used, and the smaller
    // table lets four workgroups share a CU).
    float F[(GK == GATE_K3 ? 10 : 4) * D];
    float eR[4 * D];         // e^{R_s}
    float beta[CH];
    float nk[CH], nq[CH];    // 1 / |k_t|, 1 / |q_t| (or 1: inputs already unit length)
};
static_assert(PTT <= PEH, "T lives in the E1 region");

// One workgroup (4 waves) per (chunk, head); blockIdx.x = chunk * H + head.
//
// Phase 1 runs with wave w on key channels 32w .. 32w+31: lane (lr, g) holds,
// for c2 = 0, 1 and token blocks ks = 0, 1, channel 32w + 16 c2 + lr and the
// eight tokens 32 ks + 16 hh + 4 g + m (slot 4 hh + m).  That is the perm32
// token order of an MFMA operand whose rows are channels, so K~^T leaves as
// finished fragments and (K * Gam)^T and V stay in registers as the operands
// of the W and U products.  The 16-token cumulative sums run in-lane over m
// and across the lanes g = 0..3 by shuffles.  E1 is passed through LDS to the
// Gram phase, which works on token rows (wave i = sub-chunk i).
#ifndef WY_WPE
#define WY_WPE 3
#endif
#ifndef WY_ROT
#define WY_ROT 1
#endif
#ifndef WY_WPE_SP
#define WY_WPE_SP 3
#endif
// QKN: q and k arrive raw and are normalised to unit length here (the layer's
// step fused in); a separate instantiation, so the plain path carries none of it.
// GK: the decay parameterisation.  With the K3 gate every factor of a 16-token
// tile lies in [e^-80, e^80] and the diagonal Gram tiles are dense MFMA
// products like the others.  With the unbounded softplus decay a factor
// e^{G_r - G_c} of a diagonal tile cannot be split into a row and a column part
// without overflow, so those tiles are formed position pair by position pair
// on the VALU, in the log domain (the cost the K3 bound removes).
template <bool QKN, int GK, bool LRZ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(GK == GATE_K3 ? WY_WPE : WY_WPE_SP))) void wy_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ z, const float *__restrict__ beta, const float *__restrict__ A, int N, int H,
    SegTable tab) {
    __shared__ WySmem<GK> sm;
    const int c = (int)(blockIdx.x / (unsigned)H), h = (int)(blockIdx.x % (unsigned)H);
    if (c >= tab.sq.chunk0(N)) return;
    const int n = tab.sq.seq_of_chunk(c, N);
    const int64_t t0 = tab.sq.start(n) + (int64_t)(c - tab.sq.chunk0(n)) * CH;
    const int len = (int)min((int64_t)CH, tab.sq.end(n) - t0);
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, lr = l & 15;
    // Row-block role of this wave in the Gram and inverse phases, whose work
    // grows with the row block: rotated from workgroup to workgroup.
    const int wr = WY_ROT ? (w + (int)(blockIdx.x & 3u)) & 3 : w;
    const size_t HD = (size_t)H * D;
    const size_t base = (size_t)t0 * HD + (size_t)h * D;  // element (t, ch) at base + t * HD + ch
    char *blk = tab.blocks + ((size_t)c * H + h) * BLK;
    const float eA = __expf(A[h]);
    if (w == 0) sm.beta[l] = l < len ? beta[(size_t)(t0 + l) * H + h] : 0.f;
    // Log-decays are carried in base 2 (g log2 e) from the gate on, so every
    // factor e^{G_a - G_b} is one v_exp_f32 of a difference, with no multiply.

    // Phases 1 and 2 run twice, once per 64-channel half hf, so E1 and CB only
    // ever hold half the channels (that keeps three workgroups on a CU).
    //
    // ---- phase 1: gate, cumulative sums, E1 and CB (to LDS), K~^T (to the
    // block), (K * Gam)^T (kept as an MFMA operand).  Wave w takes key
    // channels 64 hf + 16 w + lr.  Buffer loads: the resource of each input
    // covers this chunk's rows, so a row past the end reads as 0 and the row
    // part of every offset is a scalar.
    // z is [tokens, H, 128], or [tokens, H] with one gate value per (token, head).
    const bool zh = tab.ly.gate_per_head;
    const uint32_t pz = zh ? (uint32_t)(H * 4) : (uint32_t)(HD * 4), ph = (uint32_t)(HD * 2);  // row pitches, bytes
    const int zcs = zh ? 0 : 4;                                                                // channel pitch
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(z + (zh ? (size_t)t0 * H + h : base)), 0, len * pz, BUF_RSRC3);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)(k + base), 0, len * ph, BUF_RSRC3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)(v + base), 0, len * ph, BUF_RSRC3);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)(q + base), 0, len * ph, BUF_RSRC3);
    bf16x8 kga[2][2];  // [hf][ks]: channel tile 4 hf + w
    // Gram accumulators of sub-chunk i = wr against sub-chunks j <= i; tiles come
    // out transposed: lane (lr, g) holds row r = 16i + lr against columns
    // 16j + 4g + m.
    f32x4 a1[4], a2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a1[j] = a2[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Phase-1 inputs of one half, as loaded: z and k of channel 64 hf + 16 w + lr
    // at the eight tokens of each token block ks.
    uint32_t zin[2][8];
    uint16_t kin[2][8];
    auto load_half = [&](int hf) __attribute__((always_inline)) {
        const int ch = 64 * hf + 16 * w + lr;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tl = 4 * g + (e & 3), tu = 32 * ks + 16 * (e >> 2);  // row = tu (scalar) + tl
                if constexpr (!LRZ) zin[ks][e] = __builtin_amdgcn_raw_buffer_load_b32(rz, tl * pz + zcs * ch, tu * pz, 0);
                kin[ks][e] = __builtin_amdgcn_raw_buffer_load_b16(rk, tl * ph + 2 * ch, tu * ph, 0);
            }
    };
    // Low-rank forget gate: the z tiles of both channel halves on MFMA before
    // phase 1, Z (64 tokens x the wave's 16 channels of a half) = U (tokens x r)
    // W_h^T (r x channels).  A operand: token rows of U, from a copy in LDS
    // shared by the waves; B operand: the wave's channel rows of W_h.  The C tile
    // zc[hf][rt] holds tokens 16 rt + 4 g + m of channel 64 hf + 16 w + lr: the
    // phase-1 layout.  The rank goes in blocks of 128 whose W loads are all
    // issued before the first product; k-steps past the rank re-read the last
    // one and enter the products as zeros.
    const int zr = LRZ ? tab.ly.zrank : 0, zr2 = 2 * zr;  // rank, bytes per row
    const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(tab.ly.zu + (LRZ ? (size_t)t0 * zr : 0)), 0, LRZ ? len * zr2 : 0, BUF_RSRC3);
    const __amdgpu_buffer_rsrc_t rwz = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(tab.ly.zw + (LRZ ? (size_t)h * D * zr : 0)), 0, LRZ ? D * zr2 : 0, BUF_RSRC3);
    f32x4 zc[2][4];
    // A wave issues its global loads at raised priority (s_setprio 3, back to 0
    // after the issue), so the arbiter lets it get its loads out ahead of the
    // other waves' VALU work: 0.547 -> 0.537 ms at 64K x 16.
    __builtin_amdgcn_s_setprio(3);
    load_half(0);  // the first half's k loads are in flight during the projection
    __builtin_amdgcn_s_setprio(0);
    if constexpr (LRZ) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) zc[hf][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int nit = zr / 32;  // k-steps of 32: 1 .. 8
        const bf16x8 zero8 = {};
        // The chunk's u tile is copied once into LDS (the E1 and CB arrays, free
        // until phase 1 writes them): 16-byte slot s holds row t = s / nch at
        // chunk (s - t) mod nch, so the 16 rows one A-operand read touches fall
        // in different banks.
        const int nch = zr / 8;  // 16-byte chunks per row
        char *ulds = (char *)&sm;
        static_assert(sizeof(sm.a) + sizeof(sm.CB) >= 64 * 512, "u tile fits E1 and CB");
        for (int s0 = 64 * w; s0 < 64 * nch; s0 += 256) {
            const int sl = s0 + l, t = sl / nch, c = (sl % nch - t % nch + nch) % nch;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (lds_void *)(ulds + 16 * s0), 16, t * zr2 + 16 * c, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
        __syncthreads();
        for (int kb = 0; kb < nit; kb += 4) {
            bf16x8 wb[2][4], ua[4][4];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int kc = min(kb + s4, nit - 1), ko = 2 * (32 * kc + 8 * g);
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    wb[hf][s4] = __builtin_bit_cast(
                        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rwz, (64 * hf + 16 * w + lr) * zr2 + ko, 0, 0));
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int t = 16 * rt + lr;
                    ua[s4][rt] = *(const bf16x8 *)(ulds + t * zr2 + 16 * ((4 * kc + g + t) % nch));
                }
            }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const bool live = kb + s4 < nit;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const bf16x8 a = live ? ua[s4][rt] : zero8;
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) zc[hf][rt] = mfma_bf16(a, wb[hf][s4], zc[hf][rt]);
                }
            }
        }
        __syncthreads();  // every wave has read the u tile before phase 1 writes E1 and CB
    }

    // (Issuing the second half's loads during the first half's Gram phase was
    // slower: 0.62 against 0.57 ms at 64K x 16.)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        if (hf) {
            __syncthreads();  // the Gram half before is done with E1 and CB
            __builtin_amdgcn_s_setprio(3);
            load_half(1);
            __builtin_amdgcn_s_setprio(0);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int ch = 64 * hf + 16 * w + lr, chl = 16 * w + lr;
        float Rs[5], eRs[4];
        {
            float gv[2][8];
            bf16x8 kb[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int tl = 4 * g + (e & 3), tu = 32 * ks + 16 * (e >> 2);
                    const bool ok = tu + tl < len;
                    float zv;
                    if constexpr (LRZ) {
                        const f32x4 zt = zc[hf][2 * ks + (e >> 2)];
                        zv = zt[e & 3];
                    } else {
                        const uint32_t zu = zin[ks][e];
                        zv = __builtin_bit_cast(float, zu);
                    }
                    const uint16_t ku = kin[ks][e];
                    gv[ks][e] = gate_log2<GK>(eA, ok ? zv : -__builtin_inff());  // -inf: g = 0
                    kb[ks][e] = __builtin_bit_cast(__bf16, ku);
                }
            // ---- phase 0 (QKN, first half only): the inverse L2 norms of the
            // chunk's key and query rows (wave w: rows 16 w .. 16 w + 15, four
            // lanes of 32 channels per row), issued after this phase's own loads
            // and exchanged through LDS behind a bare barrier, so those loads
            // stay in flight meanwhile.
            if constexpr (QKN) {
                if (hf == 0) {
                    const int tr = 16 * w + (l >> 2), cq = 32 * (l & 3);
                    float sk = 0.f, sq = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int off = tr * (int)ph + 2 * (cq + 8 * i);  // rows past the end read as 0
                        const bf16x8 kx =
                            __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
                        const bf16x8 qx =
                            __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float a = (float)kx[e], b = (float)qx[e];
                            sk += a * a;
                            sq += b * b;
                        }
                    }
                    sk += __shfl_xor(sk, 1);
                    sk += __shfl_xor(sk, 2);
                    sq += __shfl_xor(sq, 1);
                    sq += __shfl_xor(sq, 2);
                    if ((l & 3) == 0) {  // rows past the end: 0 (1 / sqrt(0) would make NaN with qk_eps = 0)
                        sm.nk[tr] = tr < len ? 1.f / __fsqrt_rn(sk + tab.ly.qk_eps) : 0.f;
                        sm.nq[tr] = tr < len ? 1.f / __fsqrt_rn(sq + tab.ly.qk_eps) : 0.f;
                    }
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    __builtin_amdgcn_s_barrier();
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                }
            }

            float st[4];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    float a = 0.f;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        a += gv[ks][4 * hh + m];
                        gv[ks][4 * hh + m] = a;
                    }
                    // inclusive sum over the lanes g' <= g holding the same channel
                    float x = a;
                    float y = __shfl_up(x, 16);
                    if (g >= 1) x += y;
                    y = __shfl_up(x, 32);
                    if (g >= 2) x += y;
                    const float ex = x - a;
#pragma unroll
                    for (int m = 0; m < 4; ++m) gv[ks][4 * hh + m] += ex;  // G_t - R_s
                    st[2 * ks + hh] = __shfl(x, 48 + lr);                   // sub-chunk total
                }
            Rs[0] = 0.f;
#pragma unroll
            for (int s = 0; s < 4; ++s) Rs[s + 1] = Rs[s] + st[s];
            float eN[4];  // e^{G_n - R_{s+1}}
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                eRs[s] = ex2(Rs[s]);
                eN[s] = ex2(Rs[4] - Rs[s + 1]);
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                f16x8 kt;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = 2 * ks + (e >> 2);
                    const int t = 32 * ks + 16 * (e >> 2) + 4 * g + (e & 3);
                    const float cs = gv[ks][e];
                    const float e1 = ex2(cs);
                    const float kf = QKN ? (float)kb[ks][e] * sm.nk[t] : (float)kb[ks][e];
                    const float cb = kf * ex2(st[s] - cs);  // k e^{R_{s+1} - G_t}
                    // softplus decay: the log G_t - R_s and raw k instead (phase 2)
                    sm.a.E1[t * PEH + chl] = GK == GATE_K3 ? e1 : cs;
                    sm.CB[t * PEH + chl] = GK == GATE_K3 ? cb : kf;
                    kt[e] = (_Float16)(cb * eN[s]);             // k e^{G_n - G_t}
                    kga[hf][ks][e] = (__bf16)(kf * (eRs[s] * e1));
                }
                *(f16x8 *)(blk + BO_KT + frag((4 * hf + w) * 2 + ks, l)) = kt;
                // K * Gam formed here and kept (else the compiler defers it to
                // phase 4 and spills its inputs instead)
                {
                    const bf16x8 kv = kga[hf][ks];
                    u32x4 kg = __builtin_bit_cast(u32x4, kv);
                    __asm__ volatile("" : "+v"(kg));
                    kga[hf][ks] = __builtin_bit_cast(bf16x8, kg);
                }
            }
        }
        if (g == 0) {
#pragma unroll
            for (int s = 0; s < 4; ++s) sm.eR[s * D + ch] = eRs[s];
            if constexpr (GK == GATE_K3) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jj = 0; jj <= i; ++jj)
                        sm.F[(i * (i + 1) / 2 + jj) * D + ch] = ex2(Rs[i] - Rs[jj + 1]);
            } else {  // the references R_s themselves, as logs
#pragma unroll
                for (int s = 0; s < 4; ++s) sm.F[s * D + ch] = Rs[s];
            }
            ((float *)(blk + BO_GM))[ch] = ex2(Rs[4]);
        }
        __syncthreads();

        // ---- phase 2 (this half): Gram tiles of sub-chunk i = wr against j <= i, and Q~.
        // Row operands x_r e^{G_r - R_i} (x = k, q) are formed once per 32-channel
        // block; the column operand k_c e^{R_i - G_c} is CB_c e^{R_i - R_{j+1}}: CB
        // lies in [e^-80, 1] |k|, the factor is <= 1 for j < i (an underflow drops
        // only terms below e^-87) and in [1, e^80] for j = i.  The channel order
        // inside each 32-block is perm32, shared by both operands and by Q~.
        {
            const int i = wr, r = 16 * i + lr;
            const float nkr = QKN ? sm.nk[r] : 1.f, nqr = QKN ? sm.nq[r] : 1.f;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                __builtin_amdgcn_sched_barrier(0);  // one 32-channel block at a time
                const int ks = 2 * hf + kh;
                const int c0 = 32 * ks + 4 * g, cl = 32 * kh + 4 * g;  // global / in-half channel
                const int ro = r * ph + 2 * c0;                         // rows past the end read as 0
                __builtin_amdgcn_s_setprio(3);
                const bf16x4 k0 = ld_bf16x4(rk, ro), k1 = ld_bf16x4(rk, ro + 32);
                const bf16x4 q0 = ld_bf16x4(rq, ro), q1 = ld_bf16x4(rq, ro + 32);
                __builtin_amdgcn_s_setprio(0);
                f32x4 ea = *(const f32x4 *)&sm.a.E1[r * PEH + cl], eb = *(const f32x4 *)&sm.a.E1[r * PEH + cl + 16];
                const f32x4 la = ea, lb = eb;  // softplus decay: logs G_r - R_i
                if constexpr (GK != GATE_K3)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        ea[m] = ex2(la[m]);
                        eb[m] = ex2(lb[m]);
                    }
                const f32x4 pa = *(const f32x4 *)&sm.eR[i * D + c0], pb = *(const f32x4 *)&sm.eR[i * D + c0 + 16];
                F8 xk, xq;
                f16x8 qt;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    xk.v[m] = (QKN ? (float)k0[m] * nkr : (float)k0[m]) * ea[m];
                    xk.v[4 + m] = (QKN ? (float)k1[m] * nkr : (float)k1[m]) * eb[m];
                    xq.v[m] = (QKN ? (float)q0[m] * nqr : (float)q0[m]) * ea[m];
                    xq.v[4 + m] = (QKN ? (float)q1[m] * nqr : (float)q1[m]) * eb[m];
                    qt[m] = (_Float16)(xq.v[m] * pa[m]);
                    qt[4 + m] = (_Float16)(xq.v[4 + m] * pb[m]);
                }
                *(f16x8 *)(blk + BO_QT + frag(4 * i + ks, l)) = qt;
                const S8 rks = split8(xk), rqs = split8(xq);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (j > i) break;
                    if (GK != GATE_K3 && j == i) break;  // position pairs, below
                    const int cc = 16 * j + lr;
                    const float *cb = &sm.CB[cc * PEH + cl];
                    const f32x4 ca = *(const f32x4 *)cb, cbv = *(const f32x4 *)(cb + 16);
                    F8 xc;
                    if constexpr (GK == GATE_K3) {  // CB_c e^{R_i - R_{j+1}}
                        const float *fij = &sm.F[(i * (i + 1) / 2 + j) * D + c0];
                        const f32x4 fa = *(const f32x4 *)fij, fb = *(const f32x4 *)(fij + 16);
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            xc.v[m] = ca[m] * fa[m];
                            xc.v[4 + m] = cbv[m] * fb[m];
                        }
                    } else {  // k_c e^{R_i - G_c} = k_c e^{(R_i - R_j) - (G_c - R_j)} <= |k_c|
                        const f32x4 ri = *(const f32x4 *)&sm.F[i * D + c0], ri2 = *(const f32x4 *)&sm.F[i * D + c0 + 16];
                        const f32x4 rj = *(const f32x4 *)&sm.F[j * D + c0], rj2 = *(const f32x4 *)&sm.F[j * D + c0 + 16];
                        const f32x4 lc = *(const f32x4 *)&sm.a.E1[cc * PEH + cl];
                        const f32x4 lc2 = *(const f32x4 *)&sm.a.E1[cc * PEH + cl + 16];
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            xc.v[m] = ca[m] * ex2(ri[m] - rj[m] - lc[m]);
                            xc.v[4 + m] = cbv[m] * ex2(ri2[m] - rj2[m] - lc2[m]);
                        }
                    }
                    const S8 cs = split8(xc);
                    a1[j] = mma_ss(a1[j], cs, rks);
                    a2[j] = mma_ss(a2[j], cs, rqs);
                }
                if constexpr (GK != GATE_K3) {
                    // Diagonal tile, pairs in different 4-token micro-blocks: for
                    // rows of micro-block m (chain m = 1..3) both factors are
                    // referenced to P_m = L at the token before that block,
                    // x_r e^{L_r - P_m} <= 1 and k_c e^{P_m - L_c} <= 1 for the
                    // columns of earlier micro-blocks.  Rows outside block m and
                    // columns from block m on enter chain m as zeros, so the three
                    // chains add up in one accumulator.
                    const int mr = lr >> 2;  // micro-block of this lane's row (B side) and column (A side)
                    const float *rowP = &sm.a.E1[(16 * i + 4 * max(mr, 1) - 1) * PEH + cl];
                    const f32x4 pr0 = *(const f32x4 *)rowP, pr1 = *(const f32x4 *)(rowP + 16);
                    F8 yk, yq;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float fa = mr ? ex2(la[m] - pr0[m]) : 0.f, fb = mr ? ex2(lb[m] - pr1[m]) : 0.f;
                        yk.v[m] = (QKN ? (float)k0[m] * nkr : (float)k0[m]) * fa;
                        yk.v[4 + m] = (QKN ? (float)k1[m] * nkr : (float)k1[m]) * fb;
                        yq.v[m] = (QKN ? (float)q0[m] * nqr : (float)q0[m]) * fa;
                        yq.v[4 + m] = (QKN ? (float)q1[m] * nqr : (float)q1[m]) * fb;
                    }
                    const S8 yks = split8(yk), yqs = split8(yq);
                    const S8 zero = {};
                    const int cc = 16 * i + lr;
                    const f32x4 kc0 = *(const f32x4 *)&sm.CB[cc * PEH + cl], kc1 = *(const f32x4 *)&sm.CB[cc * PEH + cl + 16];
                    const f32x4 lc0 = *(const f32x4 *)&sm.a.E1[cc * PEH + cl];
                    const f32x4 lc1 = *(const f32x4 *)&sm.a.E1[cc * PEH + cl + 16];
#pragma unroll
                    for (int mb = 1; mb < 4; ++mb) {
                        const float *pm = &sm.a.E1[(16 * i + 4 * mb - 1) * PEH + cl];
                        const f32x4 p0 = *(const f32x4 *)pm, p1 = *(const f32x4 *)(pm + 16);
                        const bool colin = mr < mb;
                        F8 xc;
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            xc.v[m] = colin ? kc0[m] * ex2(p0[m] - lc0[m]) : 0.f;
                            xc.v[4 + m] = colin ? kc1[m] * ex2(p1[m] - lc1[m]) : 0.f;
                        }
                        const S8 cs = split8(xc);
                        const bool rowin = mr == mb;
                        a1[i] = mma_ss(a1[i], cs, rowin ? yks : zero);
                        a2[i] = mma_ss(a2[i], cs, rowin ? yqs : zero);
                    }
                }
            }
            if constexpr (GK != GATE_K3) {
                // Diagonal tile, pairs inside a micro-block, position pair by
                // position pair over this half's 64 channels: lane p forms pair
                // (row 16 i + p / 4, column of the same micro-block 4 (p / 16) + p % 4),
                // sum_ch x_r k_c e^{min(L_r - L_c, 0)} (c > r is masked later), then
                // hands it to the lane that holds that (row, column) of the tile.
                const int prow = 16 * i + (l >> 2), pcol = 16 * i + 4 * (l >> 4) + (l & 3);
                const float *rowl = &sm.a.E1[prow * PEH], *rowk = &sm.CB[prow * PEH];
                const float *coll = &sm.a.E1[pcol * PEH], *colk = &sm.CB[pcol * PEH];
                const float nqp = QKN ? sm.nq[prow] : 1.f;
                float sk = 0.f, sq = 0.f;
#pragma unroll 4
                for (int cg = 0; cg < 64; cg += 4) {
                    const f32x4 l4 = *(const f32x4 *)(rowl + cg), k4 = *(const f32x4 *)(rowk + cg);
                    const f32x4 lc = *(const f32x4 *)(coll + cg), kc = *(const f32x4 *)(colk + cg);
                    const bf16x4 qv = ld_bf16x4(rq, prow * (int)ph + 2 * (64 * hf + cg));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float f = kc[e] * ex2(fminf(l4[e] - lc[e], 0.f));
                        sk += k4[e] * f;
                        sq += (float)qv[e] * f;
                    }
                }
                sq *= nqp;
                // lane (lr, g) holds columns 16 i + 4 g + m of row 16 i + lr: pair 4 lr + m
                // when g is the row's micro-block
                const bool own = g == (lr >> 2);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int src = 4 * (4 * lr + m);
                    const float vk = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, sk)));
                    const float vq = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, sq)));
                    a1[i][m] += own ? vk : 0.f;
                    a2[i][m] += own ? vq : 0.f;
                }
            }
        }
    }
    f32x4 akk[4];
    {
        const int i = wr, r = 16 * i + lr;
        const float br = sm.beta[r];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j > i) break;
            f16x4 hv, lv;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int col = 16 * j + 4 * g + m;
                akk[j][m] = col < r ? br * a1[j][m] : 0.f;
                const float val = col <= r ? a2[j][m] : 0.f;
                hv[m] = (_Float16)val;
                lv[m] = (_Float16)(val - (float)hv[m]);
            }
            char *aq = blk + BO_AQ + aq_tile(i, j >> 1) * 2048 + l * 16 + (j & 1) * 8;
            *(f16x4 *)aq = hv;
            *(f16x4 *)(aq + 1024) = lv;
        }
        if ((i & 1) == 0) {  // the right half of tile (i, i/2) lies above the diagonal
            const f16x4 zh = {(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
            char *aq = blk + BO_AQ + aq_tile(i, i >> 1) * 2048 + l * 16 + 8;
            *(f16x4 *)aq = zh;
            *(f16x4 *)(aq + 1024) = zh;
        }
    }
    __syncthreads();  // E1 is dead: T takes its place
    {
        const int i = wr, r = 16 * i + lr;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j <= i) *(f32x4 *)&sm.a.T[r * PTT + 16 * j + 4 * g] = akk[j];
        // tiles (0,1) and (2,3) lie inside the 32-token blocks the W and U products read
        if (tid < 128) {
            const int tile = tid >> 6, qd = tid & 63;
            *(f32x4 *)&sm.a.T[(32 * tile + (qd >> 2)) * PTT + 32 * tile + 16 + 4 * (qd & 3)] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __syncthreads();

    // ---- phase 3: T = (I + Akk)^{-1}, blocked forward substitution in place.
    // Diagonal 16 x 16 blocks: lane m of wave b solves column m of block b.
    if (l < 16) {
        const int b = wr, m = l;
        const float *blk0 = &sm.a.T[(16 * b) * PTT + 16 * b];
        float tcol[SUB];
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
            f32x4 arow[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                if (4 * q4 < r) arow[q4] = *(const f32x4 *)&blk0[r * PTT + 4 * q4];
            float acc = r == m ? 1.f : 0.f;
#pragma unroll
            for (int cc = 0; cc < r; ++cc) acc -= arow[cc >> 2][cc & 3] * tcol[cc];
            tcol[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < SUB; ++r) sm.a.T[(16 * b + r) * PTT + 16 * b + m] = tcol[r];
    }
    __syncthreads();
    // Off-diagonal blocks, row block i: T_ij = -T_ii sum_{j <= kb < i} A_i,kb T_kb,j (exact fp32 MFMA)
    for (int i = 1; i < 4; ++i) {
        f32x4 Xb = {0.f, 0.f, 0.f, 0.f};
        const int jb = wr;
        if (jb < i) {
            for (int kb = jb; kb < i; ++kb) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float a = sm.a.T[(16 * i + lr) * PTT + 16 * kb + 4 * s + g];
                    const float b = sm.a.T[(16 * kb + 4 * s + g) * PTT + 16 * jb + lr];
                    Xb = mfma_f32(a, b, Xb);
                }
            }
        }
        __syncthreads();
        if (jb < i) {
            f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) Y = mfma_f32(sm.a.T[(16 * i + lr) * PTT + 16 * i + 4 * g + s], Xb[s], Y);
#pragma unroll
            for (int m = 0; m < 4; ++m) sm.a.T[(16 * i + 4 * g + m) * PTT + 16 * jb + lr] = -Y[m];
        }
        __syncthreads();
    }

    // ---- phase 4: W^T = (K * Gam)^T (T diag(beta))^T and U = T diag(beta) V on
    // wave w's channel tiles w and 4 + w.  T diag(beta) rows are read in the
    // perm32 token order of the phase-1 registers.  A W^T tile of channel tile
    // c is, lane for lane, one 8-byte half of W's A tile (rt, s = c / 2).
    // V in the same operand layout as (K * Gam)^T, read again here (it is not
    // kept in registers across the Gram phase, which keeps three workgroups on a CU)
    bf16x8 vb[2][2];
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tl = 4 * g + (e & 3), tu = 32 * ks + 16 * (e >> 2);
                const int ch = 64 * hf + 16 * w + lr;
                vb[hf][ks][e] = __builtin_bit_cast(
                    __bf16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rv, tl * ph + 2 * ch, tu * ph, 0));
            }
    __builtin_amdgcn_s_setprio(0);
    {
        // T diag(beta) as split bf16 fragments, each of the six (token tile rt,
        // token block ks) tiles formed once, by wave p mod 4, into the CB region
        // (dead since phase 2): every wave needs all six.
        char *tbl = (char *)sm.CB;
        static_assert(sizeof(sm.CB) >= 6 * 2048, "T diag(beta) fragments fit the CB region");
#pragma unroll
        for (int p = 0; p < 6; ++p) {
            const int rt = p < 2 ? p : 2 + ((p - 2) >> 1), ks = p < 2 ? 0 : (p & 1);
            if ((p & 3) != w) continue;
            const int r = 16 * rt + lr, c0 = 32 * ks + 4 * g;
            const f32x4 ta = *(const f32x4 *)&sm.a.T[r * PTT + c0], tc = *(const f32x4 *)&sm.a.T[r * PTT + c0 + 16];
            const f32x4 ba = *(const f32x4 *)&sm.beta[c0], bb = *(const f32x4 *)&sm.beta[c0 + 16];
            F8 x;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                x.v[m] = ta[m] * ba[m];
                x.v[4 + m] = tc[m] * bb[m];
            }
            const S8 sp = split8(x);
            *(bf16x8 *)(tbl + 2048 * p + 16 * l) = sp.hi;
            *(bf16x8 *)(tbl + 2048 * p + 1024 + 16 * l) = sp.lo;
        }
        __syncthreads();
        S8 tb[4][2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks > (rt >> 1)) continue;
                const int p = rt < 2 ? rt : 2 + 2 * (rt - 2) + ks;
                tb[rt][ks].hi = *(const bf16x8 *)(tbl + 2048 * p + 16 * l);
                tb[rt][ks].lo = *(const bf16x8 *)(tbl + 2048 * p + 1024 + 16 * l);
            }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int ctile = 4 * hf + w;  // channel tile of this wave's registers
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks <= (rt >> 1)) acc = mma_1s(acc, kga[hf][ks], tb[rt][ks]);
                f16x4 wo;
#pragma unroll
                for (int m = 0; m < 4; ++m) wo[m] = (_Float16)(-acc[m]);  // stored negated
                // W^T tile (channels of ctile) = one half of W's A tile (rt, s = ctile / 2)
                *(f16x4 *)(blk + BO_W + frag(4 * rt + (ctile >> 1), l) + 8 * (ctile & 1)) = wo;
                f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks <= (rt >> 1)) u = mma_s1(u, tb[rt][ks], vb[hf][ks]);
                {
                    const UBlk ub = u_encode(u, row_umax16(abs_max_bits(u)));
                    *(uint2 *)(blk + BO_U + U_TILE * (8 * rt + ctile) + 8 * l) = make_uint2(ub.q01, ub.q23);
                    if (lr == 0) *(float *)(blk + BO_US + 16 * (8 * rt + ctile) + 4 * g) = ub.sc;
                }
                __builtin_amdgcn_sched_barrier(0);  // one tile's encode at a time
            }
        }
    }
}

// ---------------------------------------------------------------- chain --

// LDS image of one chunk's operands in the chain passes (double-buffered).
// Pass A's image also holds U and its block scales, ahead of gamma in the
// block's own order, so that one 1 KB copy moves both (pass B, whose two
// images and output-step buffers fill the LDS, loads U into registers).
template <bool PASS_A>
struct ChainLds {
    static constexpr int W = 0;
    static constexpr int QT = 16384;                 // pass B only
    static constexpr int KT = PASS_A ? 16384 : 32768;
    static constexpr int AQ = 49152;                 // pass B only
    static constexpr int U = 32768;                  // pass A only
    static constexpr int US = 49152;                 // pass A only: U scales, then gamma
    static constexpr int GM = PASS_A ? US + (BO_GM - BO_US) : 61440;
    static constexpr int BYTES = PASS_A ? US + 1024 : GM + 1024;  // gamma, then padding
};
static_assert(BO_GM - BO_US == 512 && BLK == BO_GM + 512, "U scales and gamma end the block");

// The operand stream of one chain step.  Pass A: 16 W tiles (k-step s
// outermost), 8 gamma rows, 16 K~^T tiles; pass B: 16 (W, Q~) tile pairs, the
// 6 (hi, lo) pairs of Aqk, 8 gamma rows, 16 K~^T tiles.  `off` is the byte
// offset in the LDS image of lane 0's fragment (gamma: of row block rt).
enum { CT_W, CT_Q, CT_AQ_HI, CT_AQ_LO, CT_GAMMA, CT_KT };
struct ChainTile {
    int kind, off, rt, s;
};
template <bool PASS_A>
struct ChainTiles {
    using Lo = ChainLds<PASS_A>;
    static constexpr int N = PASS_A ? 40 : 68;
    static constexpr int SPLIT_AFTER = PASS_A ? 15 : 31;  // last tile of Delta = U - W S
    __device__ static constexpr ChainTile at(int i) {
        if (PASS_A) {
            if (i < 16) return {CT_W, Lo::W + 1024 * (4 * (i % 4) + i / 4), i % 4, i / 4};
            if (i < 24) return {CT_GAMMA, Lo::GM + 64 * (i - 16), i - 16, 0};
            const int k = i - 24;
            return {CT_KT, Lo::KT + 1024 * (2 * (k % 8) + k / 8), k % 8, k / 8};
        }
        if (i < 32) {
            const int it = i / 2, rt = it % 4, s = it / 4;
            return {(i & 1) ? CT_Q : CT_W, ((i & 1) ? Lo::QT : Lo::W) + 1024 * (4 * rt + s), rt, s};
        }
        if (i < 44) {
            const int p = (i - 32) / 2, s = p < 4 ? 0 : 1, rt = p < 4 ? p : p - 2;
            const int tile = rt < 2 ? rt : 2 * rt - 2 + s;
            return {(i & 1) ? CT_AQ_LO : CT_AQ_HI, Lo::AQ + 2048 * tile + 1024 * (i & 1), rt, s};
        }
        if (i < 52) return {CT_GAMMA, Lo::GM + 64 * (i - 44), i - 44, 0};
        const int k = i - 52;
        return {CT_KT, Lo::KT + 1024 * (2 * (k % 8) + k / 8), k % 8, k / 8};
    }
};

#ifndef CHAIN_RING_A
#define CHAIN_RING_A 6
#endif
#ifndef CHAIN_RING_B
#define CHAIN_RING_B 6
#endif

// o is written once and never read here: streaming stores leave fewer dirty
// lines in the caches for the work that follows (the decode step after a 64K
// prefill: 197 -> 184 us; the prefill itself unchanged).  The operand blocks,
// which both chain passes read back, stay ordinary stores (streaming them cost
// wy_kernel 5%).
__device__ __forceinline__ void o_store(float *p, float x) { __builtin_nontemporal_store(x, p); }

constexpr int CH_NW = 8;  // waves per chain workgroup
constexpr int CH_NT = 64 * CH_NW;


// Copy one chunk's LDS image straight from its block into LDS
// (buffer_load_dwordx4 ... lds: lane l of a wave lands at dst + 16 l, so each
// instruction moves 1 KB).  Completion is awaited with vmcnt by the caller.
// A buffer load rather than its global twin: the compiler takes the global
// form for an access of both memory and LDS, and while one is in flight it
// waits for every LDS read to complete before the first use of any.
// With `bytes` = 0 nothing is read and the copy writes zeros: issuing it
// anyway keeps the number of copies in flight the same at every step.  AUX is
// the loads' cache policy (2: non-temporal).
template <bool PASS_A, int NW, int AUX = 0>
__device__ __forceinline__ void chain_dma(const char *__restrict__ blk, int bytes, char *lds, int wv, int l) {
    using Lo = ChainLds<PASS_A>;
    constexpr int NKB = PASS_A ? Lo::US / 1024 : Lo::GM / 1024;
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)blk, 0, bytes, BUF_RSRC3);
#pragma unroll
    for (int i = 0; i < (NKB + NW - 1) / NW; ++i) {
        const int kb = wv + NW * i;
        if (kb < NKB) {
            const int x = 1024 * kb;
            // pass A: W, K~^T, U from their block offsets
            const int src = !PASS_A || x < Lo::KT ? x : x < Lo::U ? BO_KT + (x - Lo::KT) : BO_U + (x - Lo::U);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(lds + x), 16, src + 16 * l, 0, 0, AUX);
        }
    }
    // The block's last KB by every wave, so that each issues the same number
    // of copies (the waves write the same values): pass A, U's scales and
    // gamma; pass B, gamma, whose lanes 32-63 read past the block (zeros)
    // into padding.
    if constexpr (PASS_A)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(lds + Lo::US), 16, BO_US + 16 * l, 0, 0, AUX);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(lds + Lo::GM), 16, BO_GM + 16 * l, 0, 0, AUX);
}

// One workgroup (8 waves) per (segment, head).  Pass A: wave w owns columns
// 32w .. 32w+31 of X = [M | B] (waves 0-3: M, from I; waves 4-7: B, from 0, with
// U); pass B: wave w owns value columns 16w .. 16w+15 of the state.
// SPLIT: for inputs with fewer (segment, head) pairs than half the CUs, two
// workgroups per pair, each with half of the columns, so that twice as many
// CUs share the work: pass A's eight waves take 16 columns each of M or of B,
// pass B's four waves 16 value columns each.  The grid is then two halves of
// G2 workgroups (G2 a multiple of 8, so that the two workgroups of a pair land
// on one XCD and share its L2); the fused output step (which needs a row's 128
// values in one workgroup) is not split.
// STREAM (pass B): the block's loads, its last reads, carry the non-temporal
// hint.  The host sets it when the blocks exceed the 256 MB Infinity Cache:
// at 64K x 16 (1.29 GB of blocks) pass B then took 0.312 ms against 0.338,
// while at 2K x 16 (40 MB, served from the cache) the hint cost 3 us.
template <bool PASS_A, bool SPLIT = false, bool STREAM = false>
__global__ __launch_bounds__(CH_NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void seg_chain_kernel(
    int N, int H, SegTable tab, float *__restrict__ o, float *__restrict__ S_final) {
    using Lo = ChainLds<PASS_A>;
    // Two LDS images: the copy of the next chunk's runs during a step.
    // Distinct arrays (not one array indexed by step): a read of one then
    // provably does not alias a copy in flight into the other.  (Pass A with
    // three images, each copy issued two steps ahead, took the same time.)
    constexpr int NBUF = 2;
    __shared__ __align__(16) char buf0[Lo::BYTES];
    __shared__ __align__(16) char buf1[Lo::BYTES];
    // Fused output step of pass B (see store_o): per-row partial sums of
    // squares [parity][wave][row], and each wave's gate tile [wave][row][16].
    __shared__ __align__(16) float opart[PASS_A ? 4 : 2 * CH_NW * CH];
    __shared__ __align__(16) char ogate[PASS_A ? 16 : CH_NW * CH * 64];
    // Column tiles per wave and waves per workgroup: split, pass A keeps its
    // eight waves with one tile each, pass B runs four.
    constexpr int NCT = PASS_A && !SPLIT ? 2 : 1;
    constexpr int NW = SPLIT && !PASS_A ? 4 : CH_NW;
    constexpr int AUX = STREAM ? 2 : 0;  // cache policy of the block's loads

    // Workgroup i takes head i mod H of the pass's (i / H)-th segment: the
    // workgroups with work come first and in one block, so they spread evenly
    // over the XCDs and none waits behind an empty one.  Pass A has no work for
    // a sequence's last segment (its map is not needed).
    const int G2 = (int)gridDim.x / 2;
    const int half = SPLIT ? (int)blockIdx.x / G2 : 0;
    const int bidx = SPLIT ? (int)blockIdx.x - half * G2 : (int)blockIdx.x;
    const int a = bidx / H, h = bidx % H;
    if (a >= (PASS_A ? tab.sq.segA0(N) : tab.sq.seg0(N))) return;
    const int n = PASS_A ? tab.sq.seq_of_segA(a, N) : tab.sq.seq_of_seg(a, N);
    const int j = a - (PASS_A ? tab.sq.segA0(n) : tab.sq.seg0(n));
    const int x = tab.sq.seg0(n) + j;  // segment index of the maps and states
    const int pn = tab.sq.seg0(n + 1) - tab.sq.seg0(n);
    const int L = tab.sq.L;
    const int64_t s0 = tab.sq.start(n), s1 = tab.sq.end(n);
    const int nch = (int)((s1 - s0 + CH - 1) / CH);
    const int cbeg = j * L, cend = min(nch, cbeg + L);
    const size_t bstride = (size_t)H * BLK;
    const char *blk0 = tab.blocks + ((size_t)tab.sq.chunk0(n) * H + h) * BLK;

    const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4,
              lr = l & 15;
    __builtin_assume(wv >= 0 && wv < NW);
    const size_t HD = (size_t)H * D;
    const size_t sblk = ((size_t)x * H + h) * D * D;
    // pass A: columns 0..127 are M, 128..255 are B
    const int colw = 16 * NCT * wv + (SPLIT ? (PASS_A ? 128 : 64) * half : 0);
    // U is read through a buffer resource that covers one block, or nothing for
    // the waves of M (their loads then return 0 without touching memory).
    const int u_records = (!PASS_A || colw >= 128) ? (int)BLK : 0;
    const int utile = PASS_A ? max(colw - 128, 0) / 16 : colw / 16;

    f32x4 X[8][NCT];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 16 * rt + 4 * g + m, col = colw + 16 * ct + lr;
                if constexpr (PASS_A)
                    X[rt][ct][m] = r == col ? 1.f : 0.f;  // [M | B] = [I | 0]
                else
                    X[rt][ct][m] = tab.Sin[sblk + (size_t)r * D + col];
            }
    // X holds this wave's state columns times 2^E.  The state and Delta enter
    // the products as fp16, whose range (2^-14 .. 65504) a state of any other
    // magnitude would leave: the map is linear in (S, U) column by column, so
    // the wave may carry its columns at any power-of-two scale, and it picks E
    // at every step so that the state and the chunk's U stay below 2^11 (and
    // above 2^7).  Then |Delta| = |U - W S| < 2^11 + sqrt(128) 2^11 < 2^15
    // (with unit keys and beta in [0, 1] each row of W S is bounded by the
    // norm of a state column), and values 2^-21 below the largest still get
    // fp16's full precision.  U is decoded, and o and the states leave, at the
    // matching scale; powers of two are exact.
    int E = 0;

    // Past the segment's last chunk the copies read nothing (and U is 0).
    // Pass B loads U into registers one step ahead; pass A reads it from the
    // chunk's LDS image at the start of the step that uses it (with register
    // loads one step ahead, pass A took 0.202 against 0.192 ms at 64K x 16).
    using UReg = UBlk;  // as stored: decoded at the start of the step that uses it
    auto load_u = [&](int chunk, UReg (&u)[4][NCT]) {
        if constexpr (PASS_A) return;
        const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(blk0 + (size_t)chunk * bstride), 0, chunk < cend ? u_records : 0, BUF_RSRC3);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                // lane part as the register offset, the tile part (wave-uniform) as the scalar one
                const int tile = 8 * rt + utile + ct;
                const u32x2 qq = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(ru, 8 * l, BO_U + U_TILE * tile, AUX));
                u[rt][ct].q01 = qq[0];
                u[rt][ct].q23 = qq[1];
                u[rt][ct].sc =
                    __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ru, 4 * g, BO_US + 16 * tile, AUX));
            }
    };
    // A full state (this wave's columns) to dst [128][128]: buffer stores with
    // the row offset as a scalar operand, so the lane offset is one register.
    const int64_t ck_base = (!PASS_A && tab.ck.S) ? tab.ck.off[n] : 0;
    auto store_state = [&](float *dst) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)(dst + colw), 0, D * D * 4, BUF_RSRC3);
        const int lane_off = (4 * g * D + lr) * 4;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    // a value: a bit-cast of the element expression reads element 0
                    const float val = __builtin_amdgcn_ldexpf(X[rt][ct][m], -E);
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), rs, lane_off,
                                                          ((16 * rt + m) * D + 16 * ct) * 4, 0);
                }
    };
    // Output rows of chunk n leave at the start of chain step n + 1 and drain
    // during that whole step.
    //
    // With the layer's output step fused in (pass B, gate != nullptr) a row is
    // scaled by the inverse RMS of its 128 values, by weight and by
    // sigmoid(gate).  A row's values are spread over the eight waves (16
    // columns each): at the end of its step a wave leaves its per-row sum of
    // squares in LDS, and the deferred store adds the eight partials in wave
    // order (so the result does not depend on timing).  The gate tile of the
    // wave's columns is copied into LDS during the step before.
    const bool ep = !PASS_A && !SPLIT && tab.ly.gate != nullptr;  // (the host never splits with it)
    const float wcol = ep ? tab.ly.weight[colw + lr] : 1.f;
    auto store_o = [&](const f32x4 (&O)[4], int64_t t0, int len, int par) {
        f32x4 Y[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) Y[rt] = O[rt];
        if (ep) {
            const float *pp = opart + par * CH_NW * CH;
            const float *gt = (const float *)(ogate + wv * CH * 64);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 ss = *(const f32x4 *)&pp[16 * rt + 4 * g];
#pragma unroll
                for (int ww = 1; ww < CH_NW; ++ww) {
                    const f32x4 p4 = *(const f32x4 *)&pp[ww * CH + 16 * rt + 4 * g];
#pragma unroll
                    for (int m = 0; m < 4; ++m) ss[m] += p4[m];
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float gv = gt[(16 * rt + 4 * g + m) * 16 + lr];
                    const float sig = __builtin_amdgcn_rcpf(1.f + __expf(-gv));
                    Y[rt][m] = O[rt][m] * __builtin_amdgcn_rsqf(ss[m] * (1.f / D) + tab.ly.norm_eps) * wcol * sig;
                }
            }
        }
        float *orow = o + ((size_t)t0 * HD + (size_t)h * D + colw + lr);
        if (len == CH) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int m = 0; m < 4; ++m) o_store(&orow[(size_t)(16 * rt + 4 * g + m) * HD], Y[rt][m]);
        } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int t = 16 * rt + 4 * g + m;
                    if (t < len) o_store(&orow[(size_t)t * HD], Y[rt][m]);
                }
        }
    };
    // The gate rows of a chunk, this wave's 16 columns, into its LDS tile: four
    // copies of 16 rows (lane l: row 16 q + l / 4, columns 4 (l % 4) ..).  Rows
    // past the sequence end read as 0.
    auto dma_gate = [&](int chunk) {
        const int64_t t0c = s0 + (int64_t)chunk * CH;
        const int lenc = (int)min((int64_t)CH, s1 - t0c);
        char *dst = ogate + wv * CH * 64;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t rows = max(0, lenc - 16 * q);
            const int64_t bytes = min(rows * (int64_t)HD * 4, (int64_t)0x7FFFFFFF);
            const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(tab.ly.gate + ((size_t)(t0c + 16 * q) * HD + (size_t)h * D + colw)), 0, (int)bytes,
                BUF_RSRC3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rg, (lds_void *)(dst + 1024 * q), 16,
                                                     ((l >> 2) * (int)HD + 4 * (l & 3)) * 4, 0, 0, 0);
        }
    };
    // A 16-lane sum (one DPP row: lanes with equal g), the result in every lane.
    auto row_sum16 = [](float x) {
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
        return x;
    };

    // U of a chunk is loaded one step ahead, as stored, into one of two register
    // sets; the step that uses it decodes it into its Delta accumulator.
    UReg ua[4][NCT], ub[4][NCT];
    f32x4 O[4];
    int64_t t0_prev = 0;
    int len_prev = 0;
    // Copies in flight during a step: the image of the next chunk (and, in
    // pass B, its U).
    auto dma = [&](int chunk, char *lds) __attribute__((always_inline)) {
        chain_dma<PASS_A, NW, AUX>(blk0 + (size_t)chunk * bstride, chunk < cend ? (int)BLK : 0, lds, wv, l);
    };
    if (cbeg < cend) {
        dma(cbeg, buf0);
        load_u(cbeg, ua);
    }

    // One chain step on the image in `cur` (Delta accumulates into Dl, which
    // holds the chunk's U), prefetching into `nxt` (the image the previous
    // step read) and `un`.
    auto step = [&](int chunk, const char *cur, char *nxt, UReg (&Dcur)[4][NCT], UReg (&un)[4][NCT])
                    __attribute__((always_inline)) {
        // This wave's copies of this chunk (and its U) have landed (waits in
        // a form the compiler sees, so it adds none of its own for them), then
        // every wave's have, and `nxt` is free.  (Pass B also waits for its
        // LDS writes: the output-step partials.)
        __builtin_amdgcn_s_waitcnt(PASS_A ? 0x0F70 : 0x0070);
        // The barrier is a bare s_barrier between compiler-only fences: the
        // waits above are the only memory ordering needed (no wave writes LDS
        // but by these copies, and every LDS read of the previous step has
        // been consumed), and a workgroup fence would also wait for the
        // newest copy.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if constexpr (PASS_A) {  // this chunk's U, from its image (the waves of M have none)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const int tile = 8 * rt + utile + ct;
                    if (colw >= 128) {
                        const u32x2 qq = *(const u32x2 *)(cur + Lo::U + U_TILE * tile + 8 * l);
                        Dcur[rt][ct].q01 = qq[0];
                        Dcur[rt][ct].q23 = qq[1];
                        Dcur[rt][ct].sc = *(const float *)(cur + Lo::US + 16 * tile + 4 * g);
                    } else {
                        Dcur[rt][ct].q01 = Dcur[rt][ct].q23 = 0u;
                        Dcur[rt][ct].sc = 0.f;
                    }
                }
        }
        // The step's scale: e bounds max(|X|, |U 2^E|) by 2^(e - 126) (fp32
        // exponent fields; |U| < 2^14 sc in its block format).  Inf or NaN
        // present: keep E, the result is not finite either way.
        {
            float mx = 0.f, ms = 0.f;
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float xv = X[rt][ct][m];
                        mx = fmaxf(mx, fabsf(xv));
                    }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) ms = fmaxf(ms, Dcur[rt][ct].sc);
            const int es = (int)(__builtin_bit_cast(uint32_t, mx) >> 23), eu = (int)(__builtin_bit_cast(uint32_t, ms) >> 23);
            const int el = (es == 255 || eu == 255) ? 0xFFFF : max(es, eu ? max(eu + 13 + E, 0) : 0);
            const int e = (int)wave_umax((uint32_t)el);
            if (e != 0xFFFF && e != 0 && (e < 134 || e > 137)) {
                const int sh = 136 - e;
                E += sh;
#pragma unroll
                for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int m = 0; m < 4; ++m) X[rt][ct][m] = __builtin_amdgcn_ldexpf(X[rt][ct][m], sh);
            }
        }
        f32x4 Dl[4][NCT];  // Delta = U - W S accumulates onto this chunk's U
        if (!PASS_A || colw >= 128) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) Dl[rt][ct] = u_decode(Dcur[rt][ct], E);
        } else {  // pass A's columns of M: no U (their copies read nothing), nothing to decode
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) Dl[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if constexpr (!PASS_A) {
            if (chunk > cbeg) store_o(O, t0_prev, len_prev, (chunk - 1) & 1);
            if (ep) dma_gate(chunk);
        }
        load_u(chunk + 1, un);
        dma(chunk + NBUF - 1, nxt);

        const int64_t t0 = s0 + (int64_t)chunk * CH;
        const int len = (int)min((int64_t)CH, s1 - t0);
        // The state as B operand: k-step s pairs the C tiles 2s and 2s+1.
        f16x8 sf[NCT][4];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) sf[ct][s][e] = (_Float16)X[2 * s + (e >> 2)][ct][e & 3];
        if constexpr (!PASS_A)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        f16x8 dh[NCT][2], dlo[NCT][2];  // Delta as B operand (tokens), fp16 hi + lo
        auto split_delta = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    uint32_t hw[4], lw[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const f32x4 &d = Dl[2 * s + (p >> 1)][ct];
                        split_f16_pair(d[2 * (p & 1)], d[2 * (p & 1) + 1], hw[p], lw[p]);
                    }
                    dh[ct][s] = __builtin_bit_cast(f16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
                    dlo[ct][s] = __builtin_bit_cast(f16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
                }
        };
        // Every 16-byte LDS operand of the step, in the order the products use
        // them, is read RING tiles ahead of its use; a scheduling fence after
        // every group of tiles keeps the reads there (left alone, the reads sink
        // next to their products and each waits out the LDS latency).
        constexpr int NT = ChainTiles<PASS_A>::N, RING = PASS_A ? CHAIN_RING_A : CHAIN_RING_B, GROUP = 4;
        const char *lane_frag = cur + 16 * l, *lane_gam = cur + 16 * g;
        auto ld = [&](int i) __attribute__((always_inline)) {
            const ChainTile d = ChainTiles<PASS_A>::at(i);
            return *(const u32x4 *)((d.kind == CT_GAMMA ? lane_gam : lane_frag) + d.off);
        };
        u32x4 ring[RING];
#pragma unroll
        for (int i = 0; i < RING; ++i) ring[i] = ld(i);
        static_for<NT>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            constexpr ChainTile d = ChainTiles<PASS_A>::at(i);
            constexpr int rt = d.rt, s = d.s;
            const u32x4 t = ring[i % RING];
            if constexpr (i + RING < NT) ring[i % RING] = ld(i + RING);
            const f16x8 a = __builtin_bit_cast(f16x8, t);
            if constexpr (d.kind == CT_W) {  // Delta = U - W S
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) Dl[rt][ct] = mfma_f16(a, sf[ct][s], Dl[rt][ct]);
            } else if constexpr (d.kind == CT_Q) {  // O = Q~ S
                O[rt] = mfma_f16(a, sf[0][s], O[rt]);
            } else if constexpr (d.kind == CT_AQ_HI) {  // O += (Aqk * Tril) Delta
                O[rt] = mfma_f16(a, dlo[0][s], O[rt]);
                O[rt] = mfma_f16(a, dh[0][s], O[rt]);
            } else if constexpr (d.kind == CT_AQ_LO) {
                O[rt] = mfma_f16(a, dh[0][s], O[rt]);
            } else if constexpr (d.kind == CT_GAMMA) {  // S <- Diag(gamma) S ...
                const f32x4 gm = __builtin_bit_cast(f32x4, t);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int m = 0; m < 4; ++m) X[rt][ct][m] *= gm[m];
            } else {  // ... + K~^T Delta
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) X[rt][ct] = mfma_f16(a, dlo[ct][s], X[rt][ct]);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) X[rt][ct] = mfma_f16(a, dh[ct][s], X[rt][ct]);
            }
            if constexpr (i == ChainTiles<PASS_A>::SPLIT_AFTER) split_delta();
            if constexpr (i % GROUP == GROUP - 1) __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (!PASS_A) {
            t0_prev = t0;
            len_prev = len;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int m = 0; m < 4; ++m) O[rt][m] = __builtin_amdgcn_ldexpf(O[rt][m], -E);  // to o's own scale
            if (ep) {  // this wave's per-row sums of squares of O
                float *pp = opart + (chunk & 1) * CH_NW * CH + wv * CH;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    f32x4 sq;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float x2 = O[rt][m] * O[rt][m];
                        sq[m] = row_sum16(x2);
                    }
                    if (lr == 0) *(f32x4 *)&pp[16 * rt + 4 * g] = sq;
                }
            }
            // Snapshot after a full chunk that ends a stride.
            if (tab.ck.S && len == CH && (chunk + 1) % tab.ck.stride_chunks == 0) {
                const int64_t slot = ck_base + (chunk + 1) / tab.ck.stride_chunks - 1;
                if (slot < tab.ck.cap) store_state(tab.ck.S + ((size_t)slot * H + h) * D * D);
            }
        }
    };
    // Unrolled so that every step's image and U set are fixed arrays.
    constexpr int UNROLL = 2;
    auto buf = [&](auto ic) -> char * {
        if constexpr (decltype(ic)::value % NBUF == 0) return buf0;
        else return buf1;
    };
    for (int chunk = cbeg; chunk < cend; chunk += UNROLL) {
        static_for<UNROLL>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            // Every pass-A segment holds a whole number of unrolled groups (the
            // host picks L so), so its steps need no bound check; a check would
            // also cost the compiler its view of which image each copy writes.
            if (PASS_A || chunk + i < cend) {
                if constexpr (i % 2 == 0)
                    step(chunk + i, buf(ic), buf(std::integral_constant<int, i + NBUF - 1>{}), ua, ub);
                else
                    step(chunk + i, buf(ic), buf(std::integral_constant<int, i + NBUF - 1>{}), ub, ua);
            }
        });
    }
    // The copies issued past the last chunk still write LDS: let them land
    // before the workgroup can end and its LDS be handed on.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if constexpr (!PASS_A) {
        if (ep) __syncthreads();  // every wave's partials of the last chunk
        if (cbeg < cend) store_o(O, t0_prev, len_prev, (cend - 1) & 1);
    }

    // ---- segment end
    if constexpr (PASS_A) {
        float *dst = colw < 128 ? tab.Mseg : tab.Bseg;
        const int cbase = colw < 128 ? colw : colw - 128;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    dst[sblk + (size_t)(16 * rt + 4 * g + m) * D + cbase + 16 * ct + lr] =
                        __builtin_amdgcn_ldexpf(X[rt][ct][m], -E);
    } else {
        if (S_final && j == pn - 1) {
            const size_t fb = ((size_t)n * H + h) * D * D;
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        S_final[fb + (size_t)(16 * rt + 4 * g + m) * D + colw + 16 * ct + lr] =
                            __builtin_amdgcn_ldexpf(X[rt][ct][m], -E);
        }
    }
}

// ------------------------------------------------------------------ scan --

// One workgroup per (sequence, head, 16 value columns): S_in[0] = S0 and
// S_in[p+1] = M_p S_in[p] + B_p over the sequence's segments, with exact fp32
// MFMA products (an identity transition reproduces the state bit for bit).
// An empty sequence gets S_final = S0 here.
//
// Eight compute waves of 16 rows each (a step is 32 products per wave), one
// store wave and one copy wave.  The copy wave moves every map straight into
// LDS: per compute wave its 16 rows of M_p and the 16 x 16 tile of B_p (9 KB),
// into one of two slots, a map ahead, so the compute waves issue no copies and
// wait on no memory counter.  Loads and stores share the in-order vmcnt
// counter; the store wave, which copies S_in[p] out of the exchange buffer,
// keeps the state stores off the copy wave's counter too.  The exchange buffer
// is doubled like the slots, so a step needs one barrier: step p writes
// S_in[p] into exchange buffer p mod 2, passes the barrier, then reads it and
// map p.  Buffer and slot p mod 2 are written again only in step p + 2, after
// the barrier of step p + 1, which no wave passes before every wave has used
// what it read in step p.
constexpr int SCAN_NT = 640;                          // 8 compute waves, a store wave, a copy wave
constexpr int SCAN_WAVE_BYTES = 9216;                 // 16 rows of M (swizzled), then the 16 x 16 tile of B
constexpr int SCAN_SLOT_BYTES = 8 * SCAN_WAVE_BYTES;  // one map
// Exchange buffer: S_in[p]^T, column c (16) by row r (128), the 16-byte granule
// r / 4 of a column at granule (r / 4) ^ c of its LDS row, so that the 16
// columns one access touches fall in different banks with no padding (two
// slots and two buffers fill the 160 KB of LDS exactly).
__device__ __forceinline__ int xs_at(int c, int r) { return 128 * c + 4 * ((r >> 2) ^ c) + (r & 3); }
__global__ __launch_bounds__(SCAN_NT) void seg_scan_kernel(const float *__restrict__ S0, int N, int H, SegTable tab,
                                                           float *__restrict__ S_final) {
    // Distinct arrays: a read of one provably does not alias a copy in flight
    // into the other, or a write of the other exchange buffer.
    __shared__ __align__(16) char slot0[SCAN_SLOT_BYTES];
    __shared__ __align__(16) char slot1[SCAN_SLOT_BYTES];
    __shared__ __align__(16) float xs0[16 * 128];
    __shared__ __align__(16) float xs1[16 * 128];
    const int nh = blockIdx.x, cb = blockIdx.y;
    const int n = nh / H, h = nh % H;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4,
              lr = l & 15;
    __builtin_assume(w >= 0 && w < 10);
    const bool storer = w == 8, copier = w == 9;
    const int col = 16 * cb + lr, r0 = 16 * (w & 7);
    const int first = tab.sq.seg0(n), pn = tab.sq.seg0(n + 1) - first;
    f32x4 Sr;
    const size_t s0b = ((size_t)n * H + h) * D * D;
#pragma unroll
    for (int m = 0; m < 4; ++m) Sr[m] = S0 ? S0[s0b + (size_t)(r0 + 4 * g + m) * D + col] : 0.f;
    if (pn == 0) {
        if (S_final && w < 8)
#pragma unroll
            for (int m = 0; m < 4; ++m) S_final[s0b + (size_t)(r0 + 4 * g + m) * D + col] = Sr[m];
        return;
    }
    // Steps run in pairs (one per slot), pn rounded up to even: an odd count
    // ends with a step whose state nobody stores.  Every wave passes the same
    // number of barriers: one per step.
    const int pe = (pn + 1) & ~1;
    if (storer) {
        // Lane (row group l / 4, column quad l % 4) writes rows 16 k + l / 4,
        // k = 0..7, four columns each; all read before the first store, so the
        // stores issue back to back (and the reads have completed before the
        // wave reaches the next barrier).
        auto store_step = [&](int p, const float *xs) __attribute__((always_inline)) {
            lds_barrier();
            f32x4 x[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[k][i] = xs[xs_at(4 * (l & 3) + i, 16 * k + (l >> 2))];
            if (p < pn) {
                float *sin = tab.Sin + ((size_t)(first + p) * H + h) * D * D + 16 * cb + 4 * (l & 3);
#pragma unroll
                for (int k = 0; k < 8; ++k) *(f32x4 *)(sin + (size_t)(16 * k + (l >> 2)) * D) = x[k];
            }
        };
        for (int p = 0; p < pe; p += 2) {
            store_step(p, xs0);
            store_step(p + 1, xs1);
        }
        return;
    }
    if (copier) {
        // All copies of the maps, for the eight compute waves' regions (a wave
        // that issued its own stalled on the vector memory queue for about 1.4K
        // of its step's 5.5K cycles).  Region r of a slot: M_p rows 16 r + 2 i,
        // 16 r + 2 i + 1 by instruction i (lane l lands at 16 l), 16-byte column
        // granule c of a row at granule c ^ (row & 7) of its LDS row, so the 16
        // rows one operand read touches fall in different banks; then B_p's tile,
        // row 16 r + l / 4, columns 16 cb + 4 (l % 4) ..  From the sequence's first
        // map on: lane offsets fixed, the region and map offsets (below 2^31: a
        // sequence has at most 256 / H + 1 segments per head) scalars.
        const size_t mbase = ((size_t)first * H + h) * D * D;
        const int mbytes = ((max(pn - 2, 0) * H) * D * D + D * D) * 4;
        const __amdgpu_buffer_rsrc_t rM =
            __builtin_amdgcn_make_buffer_rsrc((void *)(tab.Mseg + mbase), 0, mbytes, BUF_RSRC3);
        const __amdgpu_buffer_rsrc_t rB =
            __builtin_amdgcn_make_buffer_rsrc((void *)(tab.Bseg + mbase), 0, mbytes, BUF_RSRC3);
        int vM[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 2 * i + (l >> 5), c = (l & 31) ^ (row & 7);
            vM[i] = row * D * 4 + 16 * c;
        }
        const int vB = ((l >> 2) * D + 16 * cb) * 4 + 16 * (l & 3);
        auto copy_map = [&](int p, char *slot) __attribute__((always_inline)) {
            const int so = p * H * D * D * 4;
#pragma unroll 1
            for (int r = 0; r < 8; ++r) {
                char *dst = slot + SCAN_WAVE_BYTES * r;
                const int sr = so + 16 * r * D * 4;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rM, (lds_void *)(dst + 1024 * i), 16, vM[i], sr, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void *)(dst + 8192), 16, vB, sr, 0, 0);
            }
        };
        // Map p has landed before the barrier of step p; map p + 1 is issued
        // after it, into the other slot, which the compute waves read in step
        // p - 1 (all of them have used those reads before reaching this barrier).
        // Step q reads map q only while q + 1 < pn.
        auto copy_step = [&](int p, char *nxt) __attribute__((always_inline)) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): map p has landed
            lds_barrier();
            if (p + 2 < pn) copy_map(p + 1, nxt);
        };
        if (pn >= 2) copy_map(0, slot0);
        for (int p = 0; p < pe; p += 2) {
            copy_step(p, slot1);
            copy_step(p + 1, slot0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no copy may land after the workgroup ends
        return;
    }
    const int wb = SCAN_WAVE_BYTES * w;
    auto step = [&](int p, const char *slot, float *xs) __attribute__((always_inline)) {
        *(f32x4 *)&xs[xs_at(lr, r0 + 4 * g)] = Sr;  // S_in[p]
        lds_barrier();  // every wave's rows of S_in[p], and map p, are in LDS
        if (p + 1 >= pn) return;  // S_in[pn] is not needed (pass B forms S_final); there is no map p
        F8 sb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const f32x4 lo = *(const f32x4 *)&xs[xs_at(lr, 32 * ks + 8 * g)];
            const f32x4 hi = *(const f32x4 *)&xs[xs_at(lr, 32 * ks + 8 * g + 4)];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sb[ks].v[e] = lo[e];
                sb[ks].v[4 + e] = hi[e];
            }
        }
        const char *mrow = slot + wb + 512 * lr;
        F8 mr[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c0 = 8 * ks + 2 * g;
            const f32x4 lo = *(const f32x4 *)(mrow + 16 * (c0 ^ (lr & 7)));
            const f32x4 hi = *(const f32x4 *)(mrow + 16 * ((c0 + 1) ^ (lr & 7)));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                mr[ks].v[e] = lo[e];
                mr[ks].v[4 + e] = hi[e];
            }
        }
        f32x4 a[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) a[0][m] = ((const float *)(slot + wb + 8192))[(4 * g + m) * 16 + lr];
        // One accumulator per 32-row block of M (chains of 8 products, not 32),
        // added at the end: with M = I exactly one partial is nonzero, so an
        // identity transition still gives the state bit for bit.
#pragma unroll
        for (int ks = 1; ks < 4; ++ks) a[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a[ks] = mma_ff(a[ks], mr[ks], sb[ks]);
#pragma unroll
        for (int m = 0; m < 4; ++m) Sr[m] = (a[0][m] + a[1][m]) + (a[2][m] + a[3][m]);
    };
    for (int p = 0; p < pe; p += 2) {
        step(p, slot0, xs0);
        step(p + 1, slot1, xs1);
    }
}

// ------------------------------------------------------------------ host --

constexpr int SEG_TARGET_WGS = 256;  // chain workgroups in flight: one per CU (LDS-bound)

// Segments of at least 4 chunks: at 2K x 16, 4-chunk segments (8 per head)
// gave 87 us against 103 us with 2-chunk segments (16 per head; the scan's
// steps cost about 2.9 us each) and 91 us with 6.
#ifndef SEG_L_MIN
#define SEG_L_MIN 4
#endif
// Chunks per segment: about SEG_TARGET_WGS (segment, head) pairs in all,
// rounded up to even (a whole number of two-step pass-A loop bodies): at
// 64K x 16, L = 64 (16 equal segments per head).
static inline int seg_len(int64_t T_total, int H) {
    const int64_t nc = (T_total + CH - 1) / CH;
    const int64_t per_head = SEG_TARGET_WGS / (H > 0 ? H : 1) > 0 ? SEG_TARGET_WGS / H : 1;
    int64_t L = (nc + per_head - 1) / per_head;
    L = L < SEG_L_MIN ? SEG_L_MIN : L;
    L = (L + 1) / 2 * 2;
    return (int)L;
}
static inline int64_t seg_chunks_max(int64_t T_total, int N) { return (T_total + CH - 1) / CH + N; }
static inline int64_t seg_max(int64_t T_total, int N, int H) {
    const int L = seg_len(T_total, H);
    return (seg_chunks_max(T_total, N) + L - 1) / L + N;
}

size_t seg_workspace_bytes(int64_t T_total, int N, int H) {
    const size_t tab = seq_table_bytes(N) + align_up(8 * (size_t)(N + 1));
    return tab + (size_t)seg_chunks_max(T_total, N) * H * BLK +
           3 * (size_t)seg_max(T_total, N, H) * H * D * D * sizeof(float);
}

int launch_segment_prefill(const __bf16 *q, const __bf16 *k, const __bf16 *v, const float *z, const float *beta,
                           const float *A, const float *S0, const int32_t *cu, int B, int64_t T, int H, int N,
                           float *o, float *S_final, const Ckpt &ck, const Layer &ly, void *ws,
                           hipStream_t stream, hipEvent_t *ev) {
    const int64_t T_total = (int64_t)B * T;
    const int L = seg_len(T_total, H);
    const int64_t nsm = seg_max(T_total, N, H);
    const int64_t ncm = seg_chunks_max(T_total, N);
    char *p = (char *)ws;
    SegTable tab;
    tab.sq = seq_table_at(p, N, L);
    p += seq_table_bytes(N);
    int64_t *ckpt_off = (int64_t *)p;
    p += align_up(8 * (size_t)(N + 1));
    tab.ck = Ckpt{ck.S, ckpt_off, ck.stride_chunks, ck.cap};
    tab.ly = ly;
    tab.blocks = p;
    p += (size_t)ncm * H * BLK;
    const size_t st = (size_t)nsm * H * D * D;
    tab.Mseg = (float *)p;
    tab.Bseg = tab.Mseg + st;
    tab.Sin = tab.Bseg + st;
    // a launch covers at most 2^32 - 1 work-items (unreachable within a GPU's memory)
    if (ncm * H > (int64_t)(UINT32_MAX / 256) || nsm * H > (int64_t)(UINT32_MAX / CH_NT)) return -1;
    if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return -1;
    if (launch_seq_table(cu, N, T_total, T, tab.sq, stream) != 0) return -1;
    if (ck.S && launch_ckpt_prep(tab.sq, N, (int64_t)ck.stride_chunks * CH, ckpt_off, stream) != 0) return -1;
    if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return -1;
    if (T_total > 0) {
        const dim3 grid((unsigned)(ncm * H)), blk(256);
        auto wy = [&](auto qkn, auto gk, auto lrz) {
            hipLaunchKernelGGL((wy_kernel<decltype(qkn)::value, decltype(gk)::value, decltype(lrz)::value>), grid,
                               blk, 0, stream, q, k, v, z, beta, A, N, H, tab);
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        using K3 = std::integral_constant<int, GATE_K3>;
        using SP = std::integral_constant<int, GATE_SOFTPLUS>;
        const bool sp = ly.gate_kind == GATE_SOFTPLUS, lr = ly.zu != nullptr;
        if (sp) {
            if (ly.qk_norm) lr ? wy(T_{}, SP{}, T_{}) : wy(T_{}, SP{}, F_{});
            else lr ? wy(F_{}, SP{}, T_{}) : wy(F_{}, SP{}, F_{});
        } else {
            if (ly.qk_norm) lr ? wy(T_{}, K3{}, T_{}) : wy(T_{}, K3{}, F_{});
            else lr ? wy(F_{}, K3{}, T_{}) : wy(F_{}, K3{}, F_{});
        }
    }
    if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return -1;
    // (segment, head) pairs of each chain pass: exact for a fixed-length batch,
    // bounded by the table's capacity with cu_seqlens.  A pass whose pairs fill
    // at most half the CUs runs split (two workgroups per pair).
    int ncu = 0;
    {
        int dev = 0;
        if (hipStreamGetDevice(stream, &dev) != hipSuccess ||
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return -1;
    }
    int64_t pairsB = nsm * H, pairsA = nsm * H;
    if (!cu) {
        const int64_t segs = ((T + CH - 1) / CH + L - 1) / L;
        pairsB = (int64_t)B * segs * H;
        pairsA = (int64_t)B * (segs - 1) * H;
    }
    const bool splitA = 2 * pairsA <= ncu, splitB = 2 * pairsB <= ncu && ly.gate == nullptr;
    // Pass B streams the blocks (non-temporal loads) once they exceed the Infinity Cache.
    const bool streamB = (size_t)ncm * H * BLK > ((size_t)256 << 20);
    const dim3 cgrid((unsigned)(nsm * H));
    const dim3 sgrid((unsigned)(2 * ((nsm * H + 7) / 8 * 8)));  // two halves, each a multiple of 8
    if (splitA)
        hipLaunchKernelGGL((seg_chain_kernel<true, true>), sgrid, dim3(CH_NT), 0, stream, N, H, tab, o, S_final);
    else
        hipLaunchKernelGGL((seg_chain_kernel<true>), cgrid, dim3(CH_NT), 0, stream, N, H, tab, o, S_final);
    if (ev && hipEventRecord(ev[3], stream) != hipSuccess) return -1;
    hipLaunchKernelGGL(seg_scan_kernel, dim3((unsigned)(N * H), 8), dim3(SCAN_NT), 0, stream, S0, N, H, tab, S_final);
    if (ev && hipEventRecord(ev[4], stream) != hipSuccess) return -1;
    if (splitB)
        hipLaunchKernelGGL((seg_chain_kernel<false, true>), sgrid, dim3(CH_NT / 2), 0, stream, N, H, tab, o,
                           S_final);
    else if (streamB)
        hipLaunchKernelGGL((seg_chain_kernel<false, false, true>), cgrid, dim3(CH_NT), 0, stream, N, H, tab, o,
                           S_final);
    else
        hipLaunchKernelGGL(seg_chain_kernel<false>, cgrid, dim3(CH_NT), 0, stream, N, H, tab, o, S_final);
    if (hipGetLastError() != hipSuccess) return -1;
    if (ev && hipEventRecord(ev[5], stream) != hipSuccess) return -1;
    return 0;
}

// The scan over segments on its own, for the fp32 path (which has its own
// per-chunk operands and chain passes but the same segment maps).
int launch_seg_scan(const float *S0, int N, int H, const SeqTable &sq, float *Mseg, float *Bseg, float *Sin,
                    float *S_final, hipStream_t stream) {
    if ((int64_t)N * H > (int64_t)(UINT32_MAX / 256)) return -1;
    SegTable tab{};
    tab.sq = sq;
    tab.Mseg = Mseg;
    tab.Bseg = Bseg;
    tab.Sin = Sin;
    hipLaunchKernelGGL(seg_scan_kernel, dim3((unsigned)(N * H), 8), dim3(SCAN_NT), 0, stream, S0, N, H, tab, S_final);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int set_segment_attributes() { return 0; }  // every kernel here uses static LDS only

}  // namespace kda
