// kda_prefill.hip -- chunkwise KDA prefill on gfx950.
//
// Pages: "Kimi Linear: An Expressive, Efficient Attention Architecture" summary
// (sections 2.1, 3.1, 3.2, 6.3, appendix B/C) and "Kimi K3 architecture"
// (sequence-bottleneck section: g = -5 Sigmoid(e^A z), 16-token tiles that keep
// the cumulative log-decay inside (-80, 0)).
//
// Within a chunk of n <= 64 tokens with incoming state S (rows = key channel):
//   G_t      inclusive cumulative log-decay per key channel, Gam_t = e^{G_t}
//   Akk[r,c] = beta_r sum_j k_rj k_cj e^{G_rj - G_cj}   (c < r)
//   Aqk[r,c] = sum_j q_rj k_cj e^{G_rj - G_cj}          (c <= r)
//   T        = (I + Akk)^{-1}            (forward substitution)
//   W = T diag(beta) (K * Gam),  U = T diag(beta) V      (WY / UT vectors)
//   Delta = U - W S,  O = (Q * Gam) S + Aqk Delta,
//   S' = Diag(Gam_n) S + (K * e^{G_n - G})^T Delta.
// Every e^{G_r - G_c} is evaluated through the 16-token sub-chunk of r with
// reference R_i (G just before the sub-chunk): a row factor e^{G_r - R_i} in
// [e^-80, 1] and a column factor e^{R_i - G_c} in [0, e^80], both inside the
// fp32 / bf16 range, so the diagonal tiles are dense MFMA products too.
//
// Kernels (one launch each, in stream order):
//   seq_table_kernel  (cu_seqlens only; shared with the bf16 path) sequence
//                 boundaries (clamped, non-decreasing), the first chunk of
//                 every sequence and its first segment (L chunks); fixed-length
//                 batches need no table kernel;
//   intra_kernel  one workgroup per (chunk, head), all chunks in parallel:
//                 gate + sub-chunk cumsums, the two Gram tiles on MFMA, the
//                 blocked forward substitution, W and U on MFMA; writes the
//                 per-chunk operands of the chain to the workspace;
//   map_kernel    the affine map S -> M S + B of every segment but a
//                 sequence's last, one workgroup of eight waves per
//                 (segment, head), the chunk's operand tiles copied into LDS;
//   seg_scan_kernel (kda_segment.hip)  the state entering each segment;
//   state_kernel  the state pass, one workgroup of eight waves per (segment,
//                 head): keeps the 128 x 128 fp32 state in registers across the
//                 segment's chunks (16 columns per wave), the chunk's operand
//                 tiles copied into LDS, and forms Delta, the output and the
//                 next state with MFMA;
//   gated_rmsnorm_kernel  (with the layer's output step) in place on o.
//
// This file serves fp32 q/k/v (bf16 q/k/v take kda_segment.hip's path).
// intra_kernel computes in fp32 with exact fp32 MFMA products.  The chain
// kernels multiply fp16 hi + lo pairs (x = hi + lo, hi = fp16(x), lo =
// fp16(x - hi): 22 significant bits) with three v_mfma_f32_16x16x32_f16 per
// product, hi*hi + hi*lo + lo*hi, accumulating in fp32; the dropped lo*lo term
// is below 2^-22 of the product.  That is 16 times the fp32 MFMA rate for a
// third of it.  W, Q~, K~ and Aqk are stored as such pairs; under the operator's
// preconditions (unit-length q and k, beta in [0, 1], decay factors <= 1)
// their entries are at most about 1 in magnitude, where fp16 holds them to 22
// bits down to 2^-3 and to 2^-25 absolutely below.  The state and Delta are
// split on the fly, each wave's columns at a power-of-two scale of their own
// that keeps them inside fp16's range.
#include <type_traits>

#include "kda_common.hpp"

namespace kda {

// ----------------------------------------------------------------- layout --

// Per (chunk, head) block of chain operands in the workspace (bytes).  The
// MFMA A operands are stored as fp16 hi + lo tiles, fragment-major: the 16 B
// of lane l = (lr, g) of tile i at 1024 i + 16 l, holding row 16 rt + lr and,
// in slot e = 0..7, k index 32 s + 16 (e >> 2) + 4 g + (e & 3) of the tile's
// k-step s.  Under that permutation of k a pair of C-layout tiles (rows
// 16 (2 s) + 4 g + m and 16 (2 s + 1) + 4 g + m) is a B operand as it stands.
// Each array of hi tiles is followed by the array of its lo tiles.
constexpr size_t OFF_W = 0;            // -W     tile 4 rt + s (rt: tokens, s: channels), lo at +16 KB
constexpr size_t OFF_U = 32768;        // U      [64][128]  fp32
constexpr size_t OFF_KT = 65536;       // K~^T   tile 2 rt + s (rt: channels, s: tokens), lo at +16 KB;
                                       //        K~ = K * e^{G_n - G}
constexpr size_t OFF_QT = 98304;       // Q~     as W, lo at +16 KB; Q~ = Q * Gam
constexpr size_t OFF_AQ = 131072;      // Aqk    tile 2 rt + s (rows and k both tokens), lo at +8 KB;
                                       //        zero above the diagonal
constexpr size_t OFF_GM = 147456;      // gamma  [128]      fp32, e^{G_n}
constexpr int LO_128 = 16384, LO_AQ = 8192;  // offsets of the lo tiles
constexpr size_t BLK_BYTES = 147968;   // multiple of 256

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Table {  // workspace header
    SeqTable sq;         // the sequences, their chunks and segments
    int64_t *ckpt_off;   // [N+1] first snapshot slot of each sequence
    char *blocks;        // chain operands, block (c, h) at (c * H + h) * BLK_BYTES
    float *Mseg;         // [nseg][H][128][128] segment transitions
    float *Bseg;         // [nseg][H][128][128] segment offsets
    float *Sin;          // [nseg][H][128][128] state entering each segment
    int L;               // chunks per segment
    Ckpt ck;
    Layer ly;
};

__host__ inline size_t table_bytes(int N) { return seq_table_bytes(N) + align256(8 * (size_t)(N + 1)); }
__host__ inline Table carve(void *ws, int N) {
    char *p = (char *)ws;
    Table t;
    t.sq = seq_table_at(p, N, 1);
    p += seq_table_bytes(N);
    t.ckpt_off = (int64_t *)p;
    p += align256(8 * (size_t)(N + 1));
    t.blocks = p;
    t.Mseg = t.Bseg = t.Sin = nullptr;
    t.ck = Ckpt{nullptr, t.ckpt_off, 1, 0};
    t.ly = Layer{false, 0.f, nullptr, nullptr, 0.f};
    return t;
}
__host__ inline int64_t max_chunks(int64_t T_total, int N) { return (T_total + CH - 1) / CH + N; }
// Segments of the chain: about SEG32_TARGET (segment, head) pairs in all.  Both
// chain passes run one workgroup (133 / 154 KB of LDS, one per CU) per pair (the
// map pass per pair with a successor): at 64K x 16, 240 and 256 of them fill the
// chip once (the map pass 0.39 ms; with 128 pairs, 112 workgroups took 0.70 ms).
constexpr int SEG32_TARGET = 256;
// The segment length is even: the map pass runs its chain two steps per loop
// iteration (one per LDS image).
__host__ inline int seg32_len(int64_t T_total, int N, int H) {
    const int64_t per_head = SEG32_TARGET / (H > 0 ? H : 1) > 0 ? SEG32_TARGET / H : 1;
    const int L = (int)((max_chunks(T_total, N) + per_head - 1) / per_head);
    return (L + 1) / 2 * 2;
}
__host__ inline int64_t seg32_max(int64_t T_total, int N, int H) {
    const int L = seg32_len(T_total, N, H);
    return (max_chunks(T_total, N) + L - 1) / L + N;
}

// ------------------------------------------------------------------- prep --

// The sequence table of a cu_seqlens call (both I/O paths).  Sequence n spans
// [s_n, s_{n+1}) with s_m = max_{m' <= m} clamp(cu[m'], 0, T), so sequences
// never overlap and the chunk count is at most ceil(T/64) + N.  One workgroup
// walks the N + 1 offsets in tiles of 256 with a running max, and writes the
// exclusive prefix sums of each sequence's chunk count ceil(len / 64), of its
// segment count ceil(chunks / L) and of that count less one.
__global__ __launch_bounds__(256) void seq_table_kernel(const int32_t *__restrict__ cu, int N, int64_t T_total,
                                                        SeqTable tab) {
    __shared__ int64_t s_scan[256], s_seg[256], s_sa[256];
    __shared__ int64_t s_prev_max, s_prev_sum, s_prev_seg, s_prev_sa;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_prev_max = 0;
        s_prev_sum = 0;
        s_prev_seg = 0;
        s_prev_sa = 0;
    }
    __syncthreads();
    for (int base = 0; base <= N; base += 256) {
        const int m = base + tid;
        int64_t c = 0;
        if (m <= N) {
            c = (int64_t)cu[m];
            c = c < 0 ? 0 : (c > T_total ? T_total : c);
        }
        // running max over the tile (Hillis-Steele), then fold in the previous tiles
        s_scan[tid] = c;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int64_t x = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            if (x > s_scan[tid]) s_scan[tid] = x;
            __syncthreads();
        }
        const int64_t pm = s_prev_max;
        const int64_t sm = s_scan[tid] > pm ? s_scan[tid] : pm;            // s_m
        const int64_t sp = tid > 0 ? (s_scan[tid - 1] > pm ? s_scan[tid - 1] : pm) : pm;  // s_{m-1}
        if (m < N) tab.seq_start[m] = sm;
        if (m >= 1 && m <= N) tab.seq_end[m - 1] = sm;
        // chunks of sequence m - 1, inclusive running sum = chunk_off[m]
        const int64_t cnt = (m >= 1 && m <= N) ? (sm - sp + CH - 1) / CH : 0;
        const int64_t ns = (cnt + tab.L - 1) / tab.L;
        __syncthreads();
        s_scan[tid] = cnt;
        s_seg[tid] = ns;
        s_sa[tid] = ns > 0 ? ns - 1 : 0;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int64_t x = tid >= off ? s_scan[tid - off] : 0;
            const int64_t y = tid >= off ? s_seg[tid - off] : 0;
            const int64_t z = tid >= off ? s_sa[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += x;
            s_seg[tid] += y;
            s_sa[tid] += z;
            __syncthreads();
        }
        const int64_t incl = s_scan[tid] + s_prev_sum, sg = s_seg[tid] + s_prev_seg, sa = s_sa[tid] + s_prev_sa;
        if (m <= N) {
            tab.chunk_off[m] = (int32_t)incl;
            tab.seg_off[m] = (int32_t)sg;
            tab.segA_off[m] = (int32_t)sa;
        }
        __syncthreads();
        if (tid == 255) {
            s_prev_max = sm;
            s_prev_sum = incl;
            s_prev_seg = sg;
            s_prev_sa = sa;
        }
        __syncthreads();
    }
}

int launch_seq_table(const int32_t *cu, int N, int64_t T_total, int64_t T, SeqTable &t, hipStream_t stream) {
    if (!cu) {  // B sequences of T tokens: arithmetic, nothing to build
        t.Tper = T;
        t.nchp = (int)((T + CH - 1) / CH);
        t.segp = (t.nchp + t.L - 1) / t.L;
        return 0;
    }
    t.Tper = -1;
    hipLaunchKernelGGL(seq_table_kernel, dim3(1), dim3(256), 0, stream, cu, N, T_total, t);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// off[n] = sum over sequences m < n of floor(len_m / stride), n = 0 .. N: the
// first snapshot slot of each sequence.  One workgroup, tiles of 256 with a
// running sum.
__global__ __launch_bounds__(256) void ckpt_prep_kernel(SeqTable t, int N, int64_t stride,
                                                        int64_t *__restrict__ off) {
    __shared__ int64_t s_scan[256];
    __shared__ int64_t s_prev;
    const int tid = threadIdx.x;
    if (tid == 0) s_prev = 0;
    __syncthreads();
    for (int base = 0; base <= N; base += 256) {
        const int m = base + tid;  // off[m] sums sequences < m: exclusive scan
        s_scan[tid] = (m >= 1 && m <= N) ? (t.end(m - 1) - t.start(m - 1)) / stride : 0;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            const int64_t x = tid >= d ? s_scan[tid - d] : 0;
            __syncthreads();
            s_scan[tid] += x;
            __syncthreads();
        }
        const int64_t incl = s_scan[tid] + s_prev;
        if (m <= N) off[m] = incl;
        __syncthreads();
        if (tid == 255) s_prev = incl;
        __syncthreads();
    }
}

int launch_ckpt_prep(const SeqTable &t, int N, int64_t stride, int64_t *off, hipStream_t stream) {
    hipLaunchKernelGGL(ckpt_prep_kernel, dim3(1), dim3(256), 0, stream, t, N, stride, off);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ----------------------------------------------------------------- intra --

constexpr int PG = 132;  // LDS pitch (floats) of [64][128] token-major arrays
constexpr int PT = 68;   // LDS pitch (floats) of [*][64] arrays

// 77.6 KB, so that two workgroups share a CU.
struct IntraSmem {
    union {
        float E1[CH * PG];   // e^{G_t - R_{s(t)}}: row factor, in [e^-80, 1] (phases 1-2)
        float Akk[CH * PT];  // Akk, then T = (I + Akk)^{-1} in place (phases 2-4)
    } u;
    float KG[D * PT];      // (K * Gam)^T  [channel][token]
    double R[5 * D];       // R_s: cumulative log-decay before sub-chunk s (R_4 = G_n)
    float nk[CH], nq[CH];  // 1 / |k_t|, 1 / |q_t| (or 1: inputs already unit length)
    float PF[6 * D];       // e^{R_i - R_j} for the six sub-chunk pairs j < i
    float beta[CH];
};

__device__ __forceinline__ int pair_index(int i, int j) { return i * (i - 1) / 2 + j; }  // j < i

// store a value quad at element offset e of the fp32 array at base
__device__ __forceinline__ void st4(char *base, size_t e, float a, float b, float c, float d) {
    *(float4 *)((float *)base + e) = make_float4(a, b, c, d);
}
// Four values as fp16 hi + lo into slots 4 h .. 4 h + 3 of lane l of tile
// `tile` of the hi tiles at base (the lo tiles lo bytes further)
__device__ __forceinline__ void st_pair4(char *base, int lo, int tile, int l, int h, float a, float b, float c,
                                         float d) {
    uint32_t h0, l0, h1, l1;
    split_f16_pair(a, b, h0, l0);
    split_f16_pair(c, d, h1, l1);
    char *p = base + 1024 * tile + 16 * l + 8 * h;
    *(u32x2 *)p = u32x2{h0, h1};
    *(u32x2 *)(p + lo) = u32x2{l0, l1};
}

// SP: the unbounded softplus decay; LRZ: the low-rank forget gate (separate
// instantiations, so that the plain path's loops carry none of their branches).
template <bool SP, bool LRZ>
__global__ __launch_bounds__(256) void intra_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                    const float *__restrict__ v, const float *__restrict__ z,
                                                    const float *__restrict__ beta,
                                                    const float *__restrict__ A, int N, int H, Table tab) {
    extern __shared__ __align__(16) char smem_raw[];
    IntraSmem &sm = *reinterpret_cast<IntraSmem *>(smem_raw);

    const int c = blockIdx.x, h = blockIdx.y;
    const int total = tab.sq.chunk0(N);
    if (c >= total) return;
    const int n = tab.sq.seq_of_chunk(c, N);
    const int64_t t0 = tab.sq.start(n) + (int64_t)(c - tab.sq.chunk0(n)) * CH;
    const int len = (int)min((int64_t)CH, tab.sq.end(n) - t0);
    char *blk = tab.blocks + ((size_t)c * H + h) * BLK_BYTES;

    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, g = l >> 4, lr = l & 15;
    // q, k, v and a per-channel z from this chunk's first token and this head
    // on: token t of the chunk starts at t * H * D, a 32-bit offset (the host
    // admits only 64 H D < 2^31).
    const size_t base = (size_t)t0 * H * D + (size_t)h * D;
    q += base;
    k += base;
    v += base;
    const float *zc = z ? z + base : z;
    const int HD = H * D;
    auto tok = [&](int t) -> int { return t * HD; };

    // ---- phase 0: inverse L2 norms of the key and query rows when the layer's
    // normalisation is fused in (wave w: rows 16 w .. 16 w + 15, four lanes of 32
    // channels per row); 1 otherwise.
    {
        const int tr = 16 * wv + (l >> 2), cq = 32 * (l & 3);
        float nk = 1.f, nq = 1.f;
        if (tab.ly.qk_norm) {
            float sk = 0.f, sq = 0.f;
            if (tr < len) {  // all 32 channels of both rows loaded first
                F8 ka[4], qa[4];
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    ka[c4] = ld_f8(k + tok(tr) + cq + 8 * c4);
                    qa[c4] = ld_f8(q + tok(tr) + cq + 8 * c4);
                }
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        sk += ka[c4].v[e] * ka[c4].v[e];
                        sq += qa[c4].v[e] * qa[c4].v[e];
                    }
            }
            sk += __shfl_xor(sk, 1);
            sk += __shfl_xor(sk, 2);
            sq += __shfl_xor(sq, 1);
            sq += __shfl_xor(sq, 2);
            // rows past the end get 0, not 1 / sqrt(0 + eps): with eps = 0 that
            // would be inf, and inf times a zero row is NaN
            nk = tr < len ? 1.f / __fsqrt_rn(sk + tab.ly.qk_eps) : 0.f;
            nq = tr < len ? 1.f / __fsqrt_rn(sq + tab.ly.qk_eps) : 0.f;
        }
        if ((l & 3) == 0) {
            sm.nk[tr] = nk;
            sm.nq[tr] = nq;
        }
        __syncthreads();
    }

    // ---- phase 1: gate, sub-chunk cumulative sums, elementwise operands ----
    const int ch = tid & (D - 1), half = tid >> 7;
    const float eA = __expf(A[h]);
    // Unbounded softplus decay: E1 holds the logs G_t - R_s rather than their
    // exponentials (1 / E1 would overflow), and the diagonal Gram tiles are
    // formed position pair by position pair in phase 2.
    constexpr bool sp = SP;
    const bool zh = tab.ly.gate_per_head;  // z is [tokens, H]
    // The running sums are kept in fp64: a log-decay difference formed from
    // fp32 sums of up to 64 gates (|G| up to 320) loses ~1e-5 absolute, which
    // the exponential turns into relative error of every decay factor.  Only
    // the final argument of each exponential is rounded to fp32.
    double Gl[2][SUB];
    // All of this thread's z values are loaded before the first is used (rows
    // past the end read row 0 and are masked), so their latencies overlap.
    float zr[2][SUB];
#pragma unroll
    for (int si = 0; si < 2; ++si)
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
            const int t = (half + 2 * si) * SUB + u, tc = t < len ? t : 0;
            zr[si][u] = LRZ ? 0.f : (zh ? z[(size_t)(t0 + tc) * H + h] : zc[tok(tc) + ch]);
        }
#pragma unroll
    for (int si = 0; si < 2; ++si) {
        const int s = half + 2 * si;
        double acc = 0.0;
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
            const int t = s * SUB + u;
            float gt = 0.f;
            if (t < len) {
                float zv;
                if constexpr (LRZ) {  // low-rank forget gate: z = sum_j u[t, j] W[h, ch, j]
                    const int r = tab.ly.zrank;
                    const __bf16 *ur = tab.ly.zu + (size_t)(t0 + t) * r, *wr = tab.ly.zw + ((size_t)h * D + ch) * r;
                    float acc = 0.f;
                    for (int j = 0; j < r; ++j) acc += (float)ur[j] * (float)wr[j];
                    zv = acc;
                } else {
                    zv = zr[si][u];
                }
                gt = sp ? softplus_gate(eA, zv) : kda_gate(eA, zv);
            }
            acc += (double)gt;
            Gl[si][u] = acc;
            sm.u.E1[t * PG + ch] = sp ? (float)acc : __expf((float)acc);
        }
        sm.R[(s + 1) * D + ch] = acc;  // sub-chunk total, turned into R below
    }
    if (tid < CH) sm.beta[tid] = tid < len ? beta[(size_t)(t0 + tid) * H + h] : 0.f;
    __syncthreads();
    if (tid < D) {
        double r = 0.0;
        sm.R[tid] = 0.0;
#pragma unroll
        for (int s = 1; s <= 4; ++s) {
            r += sm.R[s * D + tid];
            sm.R[s * D + tid] = r;
        }
    }
    __syncthreads();
    if (tid < D) {
#pragma unroll
        for (int i = 1; i < 4; ++i)
            for (int j = 0; j < i; ++j)
                sm.PF[pair_index(i, j) * D + tid] = __expf((float)(sm.R[i * D + tid] - sm.R[j * D + tid]));
    }
    {
        const double Gn = sm.R[4 * D + ch];
        char *qt = blk + OFF_QT, *kt = blk + OFF_KT;
#pragma unroll
        for (int si = 0; si < 2; ++si) {
            const int s = half + 2 * si;
            const double Rs = sm.R[s * D + ch];
            float kt_vals[SUB], kr[SUB], qr[SUB];
#pragma unroll
            for (int u = 0; u < SUB; ++u) {  // loads first (rows past the end read row 0)
                const int t = s * SUB + u, tc = t < len ? t : 0;
                kr[u] = k[tok(tc) + ch];
                qr[u] = q[tok(tc) + ch];
            }
#pragma unroll
            for (int u = 0; u < SUB; ++u) {
                const int t = s * SUB + u;
                const double Gt = Rs + Gl[si][u];
                const float gam = __expf((float)Gt);
                const bool ok = t < len;
                const float kv = ok ? kr[u] * sm.nk[t] : 0.f;
                const float qv = ok ? qr[u] * sm.nq[t] : 0.f;
                sm.KG[ch * PT + t] = kv * gam;
                // Q~ pairs channels ch, ch ^ 1 (lanes l, l ^ 1, adjacent slots
                // of one fragment lane): the even lane stores the pair's hi
                // values, the odd lane its lo values
                const float qg = qv * gam;
                const float qo = __builtin_bit_cast(
                    float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, qg), 0xB1, 0xF, 0xF, false));
                const bool odd = ch & 1;
                uint32_t hi2, lo2;
                split_f16_pair(odd ? qo : qg, odd ? qg : qo, hi2, lo2);
                const int qoff = 1024 * (4 * s + (ch >> 5)) + 16 * (u + 16 * ((ch >> 2) & 3)) +
                                 2 * (4 * ((ch >> 4) & 1) + (ch & 2));
                *(uint32_t *)(qt + (odd ? LO_128 : 0) + qoff) = odd ? lo2 : hi2;
                kt_vals[u] = kv * __expf((float)(Gn - Gt));
            }
#pragma unroll
            for (int u = 0; u < SUB; u += 4)
                st_pair4(kt, LO_128, 2 * (ch >> 4) + (s >> 1), (ch & 15) + 4 * u, s & 1, kt_vals[u], kt_vals[u + 1],
                         kt_vals[u + 2], kt_vals[u + 3]);
        }
        if (half == 0) ((float *)(blk + OFF_GM))[ch] = __expf((float)Gn);
    }
    // the six 16 x 16 blocks (ti, tj > ti) of Aqk above the diagonal are zero
    for (int e = tid; e < 6 * 64; e += 256) {
        const int blk6 = e >> 6, ln = e & 63;
        const int ti = blk6 < 3 ? 0 : (blk6 < 5 ? 1 : 2);
        const int tj = blk6 < 3 ? blk6 + 1 : (blk6 < 5 ? blk6 - 1 : 3);
        st_pair4(blk + OFF_AQ, LO_AQ, 2 * ti + (tj >> 1), ln, tj & 1, 0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();

    // ---- phase 2: the two decay-scaled Gram matrices on MFMA ----
    // tile list: for mat in {kk, qk}, i in 0..3, j in 0..i (20 tiles), wave wv
    // takes tiles wv, wv+4, ..  The product is formed transposed (column side as
    // the A operand) so that each lane ends up with 4 consecutive columns of a row.
    // Akk shares its LDS with E1: the tiles of Akk wait in registers until every
    // wave is done with E1.
    f32x4 kkv[3];
    // The tile of step it: wave-uniform (mat, i, j), or false past the last.
    auto tile_at = [&](int it, int &mat, int &i, int &j) {
        const int tix = wv + 4 * it;
        if (tix >= 20) return false;
        mat = tix / 10;
        const int rem = tix % 10;
        i = 0;
        while ((i + 1) * (i + 2) / 2 <= rem) ++i;
        j = rem - i * (i + 1) / 2;
        return true;
    };
    // A tile's row fragments for all four k-steps (rows past the end read row 0
    // and are zeroed when used).  The next tile's are loaded while this one is
    // formed, so one load latency is waited out per wave, not one per tile.
    auto fetch = [&](int it, F8 (&kc)[4], F8 (&xr)[4]) __attribute__((always_inline)) {
        int mat, i, j;
        if (!tile_at(it, mat, i, j)) return;
        const float *X = mat == 0 ? k : q;
        const int cr = 16 * j + lr, rr = 16 * i + lr;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            kc[ks] = ld_f8(k + tok(cr < len ? cr : 0) + 32 * ks + 8 * g);
            xr[ks] = ld_f8(X + tok(rr < len ? rr : 0) + 32 * ks + 8 * g);
        }
    };
    F8 kcb[2][4], xrb[2][4];
    fetch(0, kcb[0], xrb[0]);
#pragma unroll
    for (int it = 0; it < 5; ++it) {
        int mat, i, j;
        if (!tile_at(it, mat, i, j)) break;
        fetch(it + 1, kcb[(it + 1) & 1], xrb[(it + 1) & 1]);
        const float *X = mat == 0 ? k : q;
        const int cr = 16 * j + lr;  // column-side token (A operand row)
        const int rr = 16 * i + lr;  // row-side token (B operand column)
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (sp && j == i) {
            // Position pairs (rr, c = 16 i + 4 g + m): sum_ch x_rr k_c e^{L_rr - L_c}
            // with L = G - R_i; the exponent is clamped at 0 (c > rr is masked below).
            const float nr = mat == 0 ? sm.nk[rr] : sm.nq[rr];
            const int c0 = 16 * i + 4 * g;
            for (int e = 0; e < D; ++e) {
                const float xr = rr < len ? X[tok(rr) + e] * nr : 0.f, lrr = sm.u.E1[rr * PG + e];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int cc = c0 + m;
                    const float kc = cc < len ? k[tok(cc) + e] * sm.nk[cc] : 0.f;
                    acc[m] += xr * kc * __expf(fminf(lrr - sm.u.E1[cc * PG + e], 0.f));
                }
            }
        } else {
        const F8(&kcs)[4] = kcb[it & 1];
        const F8(&xrs)[4] = xrb[it & 1];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c0 = 32 * ks + 8 * g;
            F8 a, b;
            const F8 kc = cr < len ? kcs[ks] : F8{};
            const F8 xr = rr < len ? xrs[ks] : F8{};
            const float nc = sm.nk[cr], nr = mat == 0 ? sm.nk[rr] : sm.nq[rr];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float inv, er;
                if (sp) {  // e^{(R_i - R_j) - (G_c - R_j)} <= 1 for j < i
                    inv = __expf((float)(sm.R[i * D + c0 + e] - sm.R[j * D + c0 + e]) - sm.u.E1[cr * PG + c0 + e]);
                    er = __expf(sm.u.E1[rr * PG + c0 + e]);
                } else {
                    inv = __builtin_amdgcn_rcpf(sm.u.E1[cr * PG + c0 + e]);  // e^{R_j - G_c}, within 1 ulp
                    if (j < i) inv *= sm.PF[pair_index(i, j) * D + c0 + e];
                    er = sm.u.E1[rr * PG + c0 + e];
                }
                a.v[e] = kc.v[e] * nc * inv;
                b.v[e] = xr.v[e] * nr * er;
            }
            acc = mma_ff(acc, a, b);
        }
        }
        // acc[m] = M[r = rr][c = 16 j + 4 g + m]
        const int cb = 16 * j + 4 * g;
        float val[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int cc = cb + m;
            if (mat == 0)
                val[m] = cc < rr ? sm.beta[rr] * acc[m] : 0.f;
            else
                val[m] = cc <= rr ? acc[m] : 0.f;
        }
        if (mat == 0) {
            if (it < 3) kkv[it] = f32x4{val[0], val[1], val[2], val[3]};
        } else {
            st_pair4(blk + OFF_AQ, LO_AQ, 2 * i + (j >> 1), l, j & 1, val[0], val[1], val[2], val[3]);
        }
    }
    __syncthreads();  // E1 is dead: Akk takes its place
#pragma unroll
    for (int it = 0; it < 3; ++it) {
        const int tix = wv + 4 * it;
        if (tix >= 10) break;
        int i = 0;
        while ((i + 1) * (i + 2) / 2 <= tix) ++i;
        const int j = tix - i * (i + 1) / 2;
        *(f32x4 *)&sm.u.Akk[(16 * i + lr) * PT + 16 * j + 4 * g] = kkv[it];
    }
    __syncthreads();

    // ---- phase 3: T = (I + Akk)^{-1}, blocked forward substitution (in place) ----
    // diagonal 16 x 16 blocks: lane m < 16 of wave b solves column m of block b
    if (l < 16) {
        const int b = wv, m = l;
        float tcol[SUB];
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
            float acc = r == m ? 1.f : 0.f;
#pragma unroll
            for (int cc = 0; cc < r; ++cc) acc -= sm.u.Akk[(16 * b + r) * PT + 16 * b + cc] * tcol[cc];
            tcol[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < SUB; ++r) sm.u.Akk[(16 * b + r) * PT + 16 * b + m] = tcol[r];
    }
    __syncthreads();
    // off-diagonal blocks: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj (fp32 MFMA, exact products)
    for (int i = 1; i < 4; ++i) {
        f32x4 X = {0.f, 0.f, 0.f, 0.f};
        const int j = wv;
        if (j < i) {
            for (int kb = j; kb < i; ++kb) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float a = sm.u.Akk[(16 * i + lr) * PT + 16 * kb + 4 * s + g];
                    const float b = sm.u.Akk[(16 * kb + 4 * s + g) * PT + 16 * j + lr];
                    X = mfma_f32(a, b, X);
                }
            }
        }
        __syncthreads();
        if (j < i) {
            // X is in C layout (lane holds rows 4g+m of column lr); pair k = 4g + s
            f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float a = sm.u.Akk[(16 * i + lr) * PT + 16 * i + 4 * g + s];
                Y = mfma_f32(a, X[s], Y);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) sm.u.Akk[(16 * i + 4 * g + m) * PT + 16 * j + lr] = -Y[m];
        }
        __syncthreads();
    }

    // ---- phase 4: W = T diag(beta) (K*Gam), U = T diag(beta) V, formed transposed ----
    // wave wv: row tile rt = wv for W and 3 - wv for U; 8 column tiles each.
    // (K * Gam)^T comes from LDS, V^T from global memory: a column tile's V
    // values are loaded one tile ahead (the first during the W products), rows
    // past the end of the sequence read row 0 and are zeroed when used.
    auto fetch_v = [&](int ct, F8 (&vc)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = 32 * ks + 8 * g + e;
                vc[ks].v[e] = v[tok(t < len ? t : 0) + 16 * ct + lr];
            }
    };
    F8 vb[2][2];
    fetch_v(0, vb[0]);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int rt = pass == 0 ? wv : 3 - wv;
        const int nks = rt < 2 ? 1 : 2;
        const int r = 16 * rt + lr;
        F8 tb[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int cc = 32 * ks + 8 * g + e;
                tb[ks].v[e] = (ks < nks && cc <= r) ? sm.u.Akk[r * PT + cc] * sm.beta[cc] : 0.f;
            }
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            if (pass == 1 && ct + 1 < 8) fetch_v(ct + 1, vb[(ct + 1) & 1]);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks >= nks) break;
                F8 xa;
                if (pass == 0) {
                    xa = ld_f8(&sm.KG[(16 * ct + lr) * PT + 32 * ks + 8 * g]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) xa.v[e] = 32 * ks + 8 * g + e < len ? vb[ct & 1][ks].v[e] : 0.f;
                }
                acc = mma_ff(acc, xa, tb[ks]);
            }
            // acc[m] = out[row r][col 16 ct + 4 g + m]
            if (pass == 0)
                st_pair4(blk + OFF_W, LO_128, 4 * rt + (ct >> 1), l, ct & 1, -acc[0], -acc[1], -acc[2], -acc[3]);
            else
                st4(blk + OFF_U, (size_t)r * D + 16 * ct + 4 * g, acc[0], acc[1], acc[2], acc[3]);
        }
    }
}

// ---------------------------------------------------------- chain helpers --

// A fragment as fp16 hi + lo.
struct H8 {
    f16x8 hi, lo;
};
// A lane's fragment at p (hi) and p + lo
__device__ __forceinline__ H8 ld_frag(const char *p, int lo) {
    return {*(const f16x8 *)p, *(const f16x8 *)(p + lo)};
}
// Term t of a b with a, b as hi + lo: t = 0: lo * hi, 1: hi * lo, 2: hi * hi.
// The products below run term by term over several independent accumulators,
// so that no MFMA waits for the result of the one issued just before it.
__device__ __forceinline__ f32x4 mma_term(int t, f32x4 c, const H8 &a, const H8 &b) {
    return mfma_f16(t == 0 ? a.lo : a.hi, t == 1 ? b.lo : b.hi, c);
}
__device__ __forceinline__ uint32_t abs_bits(float x) { return __builtin_bit_cast(uint32_t, x) & 0x7FFFFFFFu; }

// ------------------------------------------------------------- map pass --

// LDS image of one chunk for the map pass, copied straight from its block: the
// -W tiles (hi, then lo), the K~^T tiles (hi, then lo) and gamma.
constexpr int MI_W = 0, MI_KT = 32768, MI_GM = 65536, MI_BYTES = MI_GM + 1024;

// Copy the image of the chunk whose block is blk into img: 64 tiles of 1 KB,
// eight per wave (buffer_load_dwordx4 ... lds: lane l lands at dst + 16 l),
// and gamma by every wave (the same values; lanes 32-63 read past the block,
// which gives zeros, into padding).  Completion is awaited with vmcnt.
__device__ __forceinline__ void map_dma(const char *__restrict__ blk, char *img, int wv, int l) {
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)blk, 0, (int)BLK_BYTES, BUF_RSRC3);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int x = wv + 8 * i;
        const int src = x < 32 ? (int)OFF_W + 1024 * x : (int)OFF_KT + 1024 * (x - 32);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(img + 1024 * x), 16, src + 16 * l, 0, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(img + MI_GM), 16, (int)OFF_GM + 16 * l, 0, 0, 0);
}

// The affine map S -> M S + B of a segment (every segment of a sequence but its
// last), one workgroup of eight waves per (segment, head): from X = [M | B] =
// [I | 0] it runs the chain step X <- Diag(gamma) X + K~^T (U~ - W X) over the
// segment's chunks, where U~ is U in the B columns and 0 in the M columns.
// Wave w owns the 32 columns 32 w .. 32 w + 31 of X (waves 0-3: M, 4-7: B) as
// C-layout tiles, all 128 rows, and feeds them as the B operand of W X by the
// tile pairing of the block's k order; Delta likewise for K~^T Delta.  The
// chunk's -W and K~^T tiles are copied into one of two LDS images a step
// ahead, so each is read from memory once per workgroup; U (fp32) is loaded a
// step ahead into registers.  Products as fp16 hi + lo pairs (three MFMAs),
// with X and U at a power-of-two scale 2^E per wave (re-picked when the largest
// |X| or |U| 2^E leaves [2^7, 2^11), as in the state pass).
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void map_kernel(int N, int H,
                                                                                             Table tab) {
    __shared__ __align__(16) char img0[MI_BYTES];
    __shared__ __align__(16) char img1[MI_BYTES];
    // workgroup i: head i mod H of the (i / H)-th segment with a successor
    const int a = (int)blockIdx.x / H, h = (int)blockIdx.x % H;
    if (a >= tab.sq.segA0(N)) return;
    const int n = tab.sq.seq_of_segA(a, N);
    const int j = a - tab.sq.segA0(n);
    const int x = tab.sq.seg0(n) + j;  // segment index of the maps
    const int cbeg = tab.sq.chunk0(n) + j * tab.sq.L, cend = cbeg + tab.sq.L;  // a full segment: L chunks
    const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4,
              lr = l & 15;
    const bool bcol = wv >= 4;
    const int colw = 32 * (wv & 3);  // first column of the wave within M or B
    auto block = [&](int c) { return tab.blocks + ((size_t)c * H + h) * BLK_BYTES; };

    f32x4 X[8][2];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int m = 0; m < 4; ++m) X[rt][ct][m] = !bcol && 16 * rt + 4 * g + m == colw + 16 * ct + lr ? 1.f : 0.f;
    int E = 0;

    // U of a chunk (B waves; a buffer of no records reads 0 for the M waves and
    // past the segment): tile (rt, ct) rows 16 rt + 4 g + m, columns colw + 16 ct + lr
    f32x4 uv[4][2];
    auto load_u = [&](int c) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(block(c) + OFF_U), 0, bcol && c < cend ? 64 * D * 4 : 0, BUF_RSRC3);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    uv[rt][ct][m] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(ru, 4 * ((4 * g + m) * D + lr),
                                                                    4 * (16 * rt * D + colw + 16 * ct), 0));
    };
    map_dma(block(cbeg), img0, wv, l);
    load_u(cbeg);

    auto step = [&](int c, const char *cur, char *nxt) __attribute__((always_inline)) {
        // This wave's copies of `cur` and its U have landed, then every wave's
        // have, and every wave is done with `nxt` (read in the step before).
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        if (c + 1 < cend) map_dma(block(c + 1), nxt, wv, l);
        // The step's scale: e bounds max(|X|, |U| 2^E) by 2^(e - 126) (fp32
        // exponent fields).  Inf or NaN present: keep E.
        {
            uint32_t mx = 0, mu = 0;
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        mx = max(mx, abs_bits(X[rt][ct][m]));
                        if (rt < 4) mu = max(mu, abs_bits(uv[rt][ct][m]));
                    }
            const int es = (int)(mx >> 23), eu = (int)(mu >> 23);
            const int el = (es == 255 || eu == 255) ? 0xFFFF : max(es, eu ? max(eu + E, 0) : 0);
            const int e = (int)wave_umax((uint32_t)el);
            if (e != 0xFFFF && e != 0 && (e < 134 || e > 137)) {
                const int sh = 136 - e;
                E += sh;
#pragma unroll
                for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                        for (int m = 0; m < 4; ++m) X[rt][ct][m] = __builtin_amdgcn_ldexpf(X[rt][ct][m], sh);
            }
        }
        // Delta = U 2^E - W X (W stored negated, the accumulator starts at U 2^E)
        f32x4 Dl[4][2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int m = 0; m < 4; ++m) Dl[rt][ct][m] = __builtin_amdgcn_ldexpf(uv[rt][ct][m], E);
        load_u(c + 1);
        const char *lane = cur + 16 * l;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            H8 xb[2];  // X rows 32 s .. 32 s + 31 as the B operand: C tiles 2 s and 2 s + 1
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const f32x4 &xv = X[2 * s + (p >> 1)][ct];
                    split_f16_pair(xv[2 * (p & 1)], xv[2 * (p & 1) + 1], hw[p], lw[p]);
                }
                xb[ct] = {__builtin_bit_cast(f16x8, u32x4{hw[0], hw[1], hw[2], hw[3]}),
                          __builtin_bit_cast(f16x8, u32x4{lw[0], lw[1], lw[2], lw[3]})};
            }
#pragma unroll
            for (int r2 = 0; r2 < 4; r2 += 2) {
                H8 wa[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) wa[q] = ld_frag(lane + MI_W + 1024 * (4 * (r2 + q) + s), LO_128);
#pragma unroll
                for (int t = 0; t < 3; ++t)
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct) Dl[r2 + q][ct] = mma_term(t, Dl[r2 + q][ct], wa[q], xb[ct]);
            }
        }
        // Delta as the B operand (tokens 32 s .. 32 s + 31: C tiles 2 s, 2 s + 1)
        H8 db[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const f32x4 &dv = Dl[2 * s + (p >> 1)][ct];
                    split_f16_pair(dv[2 * (p & 1)], dv[2 * (p & 1) + 1], hw[p], lw[p]);
                }
                db[s][ct] = {__builtin_bit_cast(f16x8, u32x4{hw[0], hw[1], hw[2], hw[3]}),
                             __builtin_bit_cast(f16x8, u32x4{lw[0], lw[1], lw[2], lw[3]})};
            }
        // X <- Diag(gamma) X + K~^T Delta
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            const f32x4 gm = *(const f32x4 *)(cur + MI_GM + 64 * rt + 16 * g);  // gamma of rows 16 rt + 4 g + m
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int m = 0; m < 4; ++m) X[rt][ct][m] *= gm[m];
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int r2 = 0; r2 < 8; r2 += 2) {
                H8 ka[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) ka[q] = ld_frag(lane + MI_KT + 1024 * (2 * (r2 + q) + s), LO_128);
#pragma unroll
                for (int t = 0; t < 3; ++t)
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct) X[r2 + q][ct] = mma_term(t, X[r2 + q][ct], ka[q], db[s][ct]);
            }
    };
    for (int c = cbeg; c < cend; c += 2) {
        step(c, img0, img1);
        step(c + 1, img1, img0);
    }
    float *dst = (bcol ? tab.Bseg : tab.Mseg) + ((size_t)x * H + h) * D * D + colw;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                dst[(size_t)(16 * rt + 4 * g + m) * D + 16 * ct + lr] = __builtin_amdgcn_ldexpf(X[rt][ct][m], -E);
}

// ------------------------------------------------------------ state pass --

// LDS images of one chunk for the state pass, copied straight from its block.
// Image A: the -W tiles (hi, then lo) and the Q~ tiles (hi, then lo); read by
// the first products of a step, refilled for the next chunk as soon as every
// wave has read it.  Image B (two of them, alternating by step): the K~^T tiles
// (hi, then lo), the six Aqk tiles on or below the diagonal (hi, then lo) and
// gamma; filled a whole step ahead.
constexpr int SA_W = 0, SA_QT = 32768, SA_BYTES = 65536;
constexpr int SB_KT = 0, SB_AQ = 32768, SB_GM = SB_AQ + 12288, SB_BYTES = SB_GM + 1024;

__device__ __forceinline__ void state_dma_a(const char *__restrict__ blk, char *img, int wv, int l) {
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)blk, 0, (int)BLK_BYTES, BUF_RSRC3);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int x = wv + 8 * i;  // tile 0..63: -W hi, -W lo, Q~ hi, Q~ lo
        const int src = x < 32 ? (int)OFF_W + 1024 * x : (int)OFF_QT + 1024 * (x - 32);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(img + 1024 * x), 16, src + 16 * l, 0, 0, 0);
    }
}
__device__ __forceinline__ void state_dma_b(const char *__restrict__ blk, char *img, int wv, int l) {
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)blk, 0, (int)BLK_BYTES, BUF_RSRC3);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const int x = wv + 8 * i;  // tile 0..43: K~^T hi, K~^T lo, Aqk hi (6), Aqk lo (6)
        if (x < 44) {
            int src;
            if (x < 32) {
                src = (int)OFF_KT + 1024 * x;
            } else {  // slot q of the six Aqk tiles 2 rt + s with s <= rt / 2: tiles 0, 2, 4, 5, 6, 7
                const int q = (x - 32) % 6;
                src = (int)OFF_AQ + (x < 38 ? 0 : LO_AQ) + 1024 * (q < 2 ? 2 * q : q + 2);
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(img + 1024 * x), 16, src + 16 * l, 0, 0, 0);
        }
    }
    // gamma by every wave (the same values; lanes 32-63 read past the block,
    // which gives zeros, into padding)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(img + SB_GM), 16, (int)OFF_GM + 16 * l, 0, 0, 0);
}

// The state pass: the chain over one segment of a sequence from the state the
// scan gave it, one workgroup of eight waves per (segment, head).  Wave w owns
// the value columns 16 w .. 16 w + 15 of the state, all 128 rows, as C-layout
// tiles, and feeds them as the B operand of W S and Q~ S by the tile pairing of
// the block's k order (Delta likewise for Aqk Delta and K~^T Delta).  Each
// chunk's operand tiles are read from memory once per workgroup, into the LDS
// images above; U (fp32) is loaded into registers a step ahead.  Products as
// fp16 hi + lo pairs (three MFMAs), with the wave's columns, U, Delta and O at a
// power-of-two scale 2^E per wave (re-picked when the largest |S| or |U| 2^E
// leaves [2^7, 2^11): then |Delta| < 2^11 (1 + sqrt(128)) < 2^15).  Writes o
// (and snapshots, and S_final after a sequence's last segment).
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void state_kernel(
    int N, int H, Table tab, float *__restrict__ o, float *__restrict__ S_final) {
    __shared__ __align__(16) char imgA[SA_BYTES];
    __shared__ __align__(16) char imgB0[SB_BYTES];
    __shared__ __align__(16) char imgB1[SB_BYTES];
    // workgroup i: head i mod H of the (i / H)-th segment
    const int a = (int)blockIdx.x / H, h = (int)blockIdx.x % H;
    if (a >= tab.sq.seg0(N)) return;
    const int n = tab.sq.seq_of_seg(a, N);
    const int j = a - tab.sq.seg0(n);
    const int x = tab.sq.seg0(n) + j;  // segment index of the states
    const int pn = tab.sq.seg0(n + 1) - tab.sq.seg0(n);
    const int cseq = tab.sq.chunk0(n);
    const int cbeg = cseq + j * tab.sq.L, cend = min(tab.sq.chunk0(n + 1), cbeg + tab.sq.L);
    const int64_t sstart = tab.sq.start(n), send = tab.sq.end(n);
    const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4,
              lr = l & 15;
    const int col = 16 * wv + lr;  // this lane's state column
    const size_t HD = (size_t)H * D;
    auto block = [&](int c) { return tab.blocks + ((size_t)c * H + h) * BLK_BYTES; };

    f32x4 X[8];
    const size_t sblk = ((size_t)x * H + h) * D * D;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int m = 0; m < 4; ++m) X[rt][m] = tab.Sin[sblk + (size_t)(16 * rt + 4 * g + m) * D + col];
    int E = 0;

    // U of a chunk: tile rt rows 16 rt + 4 g + m, column col (a buffer of no
    // records reads 0 past the segment)
    f32x4 uv[4];
    auto load_u = [&](int c) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(block(c) + OFF_U), 0, c < cend ? 64 * D * 4 : 0, BUF_RSRC3);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                uv[rt][m] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(ru, 4 * ((4 * g + m) * D + col), 4 * 16 * rt * D, 0));
    };
    auto store_state = [&](float *dst) __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                dst[(size_t)(16 * rt + 4 * g + m) * D + col] = __builtin_amdgcn_ldexpf(X[rt][m], -E);
    };
    const int64_t ck_base = tab.ck.S ? tab.ck.off[n] : 0;
    if (cbeg < cend) {
        state_dma_b(block(cbeg), imgB0, wv, l);
        state_dma_a(block(cbeg), imgA, wv, l);
        load_u(cbeg);
    }
    // Outstanding VMEM operations a step may leave behind the copy of image A
    // for the next chunk: its 16 output stores (and the 32 snapshot stores of a
    // step that ends a stride, after which the next step waits for everything).
    bool drain = true;  // the first step waits for everything

    auto step = [&](int c, const char *bcur, char *bnxt) __attribute__((always_inline)) {
        // Image A and U of this chunk (and image B, issued a step earlier) have
        // landed for this wave, then for every wave; every wave is done with
        // the step before, so `bnxt` may be refilled.
        if (drain)
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        else
            __builtin_amdgcn_s_waitcnt(0x0F70 | 0x4000);  // vmcnt(16): all but the last step's output stores
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        if (c + 1 < cend) state_dma_b(block(c + 1), bnxt, wv, l);
        // the step's scale (as in the map pass)
        {
            uint32_t mx = 0, mu = 0;
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    mx = max(mx, abs_bits(X[rt][m]));
                    if (rt < 4) mu = max(mu, abs_bits(uv[rt][m]));
                }
            const int es = (int)(mx >> 23), eu = (int)(mu >> 23);
            const int el = (es == 255 || eu == 255) ? 0xFFFF : max(es, eu ? max(eu + E, 0) : 0);
            const int e = (int)wave_umax((uint32_t)el);
            if (e != 0xFFFF && e != 0 && (e < 134 || e > 137)) {
                const int sh = 136 - e;
                E += sh;
#pragma unroll
                for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                    for (int m = 0; m < 4; ++m) X[rt][m] = __builtin_amdgcn_ldexpf(X[rt][m], sh);
            }
        }
        // Delta = U 2^E - W S (W stored negated, the accumulator starts at U 2^E);  O = Q~ S
        f32x4 Dl[4], O[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int m = 0; m < 4; ++m) Dl[rt][m] = __builtin_amdgcn_ldexpf(uv[rt][m], E);
            O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        load_u(c + 1);
        const char *la = imgA + 16 * l;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            H8 xb;  // S rows 32 s .. 32 s + 31 as the B operand: C tiles 2 s and 2 s + 1
            {
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const f32x4 &xv = X[2 * s + (p >> 1)];
                    split_f16_pair(xv[2 * (p & 1)], xv[2 * (p & 1) + 1], hw[p], lw[p]);
                }
                xb = {__builtin_bit_cast(f16x8, u32x4{hw[0], hw[1], hw[2], hw[3]}),
                      __builtin_bit_cast(f16x8, u32x4{lw[0], lw[1], lw[2], lw[3]})};
            }
#pragma unroll
            for (int r2 = 0; r2 < 4; r2 += 2) {
                H8 wa[2], qa[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    wa[q] = ld_frag(la + SA_W + 1024 * (4 * (r2 + q) + s), LO_128);
                    qa[q] = ld_frag(la + SA_QT + 1024 * (4 * (r2 + q) + s), LO_128);
                }
#pragma unroll
                for (int t = 0; t < 3; ++t)
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        Dl[r2 + q] = mma_term(t, Dl[r2 + q], wa[q], xb);
                        O[r2 + q] = mma_term(t, O[r2 + q], qa[q], xb);
                    }
            }
        }
        // every wave has read image A: refill it with the next chunk's
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        if (c + 1 < cend) state_dma_a(block(c + 1), imgA, wv, l);
        // Delta as the B operand (tokens 32 s .. 32 s + 31: C tiles 2 s, 2 s + 1)
        H8 db[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const f32x4 &dv = Dl[2 * s + (p >> 1)];
                split_f16_pair(dv[2 * (p & 1)], dv[2 * (p & 1) + 1], hw[p], lw[p]);
            }
            db[s] = {__builtin_bit_cast(f16x8, u32x4{hw[0], hw[1], hw[2], hw[3]}),
                     __builtin_bit_cast(f16x8, u32x4{lw[0], lw[1], lw[2], lw[3]})};
        }
        const char *lb = bcur + 16 * l;
        // O += (Aqk * Tril) Delta: tiles (rt, s), s <= rt / 2, image slot q
#pragma unroll
        for (int q = 0; q < 6; ++q) {
            const int rt = q < 2 ? q : (q < 4 ? 2 : 3), s = q < 2 ? 0 : (q & 1);
            const H8 aa = ld_frag(lb + SB_AQ + 1024 * q, 6144);
#pragma unroll
            for (int t = 0; t < 3; ++t) O[rt] = mma_term(t, O[rt], aa, db[s]);
        }
        // S <- Diag(gamma) S + K~^T Delta
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            const f32x4 gm = *(const f32x4 *)(bcur + SB_GM + 64 * rt + 16 * g);  // gamma of rows 16 rt + 4 g + m
#pragma unroll
            for (int m = 0; m < 4; ++m) X[rt][m] *= gm[m];
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int r4 = 0; r4 < 8; r4 += 4) {
                H8 ka[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) ka[q] = ld_frag(lb + SB_KT + 1024 * (2 * (r4 + q) + s), LO_128);
#pragma unroll
                for (int t = 0; t < 3; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q) X[r4 + q] = mma_term(t, X[r4 + q], ka[q], db[s]);
            }
        // output rows of this chunk, and a snapshot after a full chunk that ends a stride
        const int64_t t0 = sstart + (int64_t)(c - cseq) * CH;
        const int len = (int)min((int64_t)CH, send - t0);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int t = 16 * rt + 4 * g + m;
                if (t < len) o[(size_t)(t0 + t) * HD + (size_t)h * D + col] = __builtin_amdgcn_ldexpf(O[rt][m], -E);
            }
        drain = false;
        if (tab.ck.S && len == CH && (c - cseq + 1) % tab.ck.stride_chunks == 0) {
            const int64_t slot = ck_base + (c - cseq + 1) / tab.ck.stride_chunks - 1;
            if (slot < tab.ck.cap) {
                store_state(tab.ck.S + ((size_t)slot * H + h) * D * D);
                drain = true;
            }
        }
    };
    for (int c = cbeg; c < cend; c += 2) {
        step(c, imgB0, imgB1);
        if (c + 1 < cend) step(c + 1, imgB1, imgB0);
    }
    if (S_final && j == pn - 1) store_state(S_final + ((size_t)n * H + h) * D * D);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no copy may land after the workgroup ends
}

// ------------------------------------------------------------ output step --

// The layer's output step on fp32 rows of 128 values, in place (one wave per
// (token, head) row; lane l holds values 2l, 2l+1):
// o <- o / sqrt(mean o^2 + eps) * weight * sigmoid(gate).
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(float *__restrict__ o, const float *__restrict__ gate,
                                                            const float *__restrict__ weight, float eps,
                                                            int64_t rows) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int l = threadIdx.x & 63;
    float2 *orow = (float2 *)(o + row * D);
    const float2 x = orow[l];
    const float2 gv = ((const float2 *)(gate + row * D))[l];
    const float2 wv = ((const float2 *)weight)[l];
    float s = x.x * x.x + x.y * x.y;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    const float r = 1.f / __fsqrt_rn(s * (1.f / D) + eps);
    const float sa = 1.f / (1.f + __expf(-gv.x)), sb = 1.f / (1.f + __expf(-gv.y));
    orow[l] = make_float2(x.x * r * wv.x * sa, x.y * r * wv.y * sb);
}

// ------------------------------------------------------------------ host --

size_t seg_workspace_bytes(int64_t T_total, int N, int H);
int launch_segment_prefill(const __bf16 *q, const __bf16 *k, const __bf16 *v, const float *z, const float *beta,
                           const float *A, const float *S0, const int32_t *cu, int B, int64_t T, int H, int N,
                           float *o, float *S_final, const Ckpt &ck, const Layer &ly, void *ws,
                           hipStream_t stream, hipEvent_t *ev);
int set_segment_attributes();
int launch_seg_scan(const float *S0, int N, int H, const SeqTable &sq, float *Mseg, float *Bseg, float *Sin,
                    float *S_final, hipStream_t stream);

// bf16 q/k/v run the segment-parallel fused path (kda_segment.hip); fp32 q/k/v
// run the path below with exact fp32 MFMA products: the per-chunk operands,
// the segment maps, the scan over segments (shared with the bf16 path) and the
// chain over each segment.
size_t prefill_workspace_bytes(int64_t T_total, int N, int H, bool f32io) {
    if (!f32io) return seg_workspace_bytes(T_total, N, H);
    return table_bytes(N) + (size_t)max_chunks(T_total, N) * (size_t)H * BLK_BYTES +
           3 * (size_t)seg32_max(T_total, N, H) * H * D * D * sizeof(float);
}

// ck.S == nullptr: no snapshots (ck.off is ignored; the launchers point it at
// their workspace).
int launch_prefill(const void *q, const void *k, const void *v, bool f32io, const float *z, const float *beta,
                   const float *A, const float *S0, const int32_t *cu, int B, int64_t T, int H, int N,
                   float *o, float *S_final, const Ckpt &ck, const Layer &ly, void *ws, hipStream_t stream,
                   hipEvent_t *ev) {
    if (!f32io)
        return launch_segment_prefill((const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, z, beta, A, S0, cu, B,
                                      T, H, N, o, S_final, ck, ly, ws, stream, ev);
    const int64_t T_total = (int64_t)B * T;
    Table tab = carve(ws, N);
    tab.ck = Ckpt{ck.S, tab.ckpt_off, ck.stride_chunks, ck.cap};
    tab.ly = ly;
    tab.sq.L = seg32_len(T_total, N, H);
    const int64_t nsm = seg32_max(T_total, N, H);
    const size_t st = (size_t)nsm * H * D * D;
    tab.Mseg = (float *)(tab.blocks + (size_t)max_chunks(T_total, N) * (size_t)H * BLK_BYTES);
    tab.Bseg = tab.Mseg + st;
    tab.Sin = tab.Bseg + st;
    // grids: one workgroup per (segment, head) slot; a launch covers at most
    // 2^32 - 1 work-items
    if (nsm * H > (int64_t)(UINT32_MAX / 512) || max_chunks(T_total, N) * H > (int64_t)UINT32_MAX ||
        (int64_t)CH * H * D > (int64_t)INT32_MAX)
        return -1;
    if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return -1;
    if (launch_seq_table(cu, N, T_total, T, tab.sq, stream) != 0) return -1;
    if (ck.S && launch_ckpt_prep(tab.sq, N, (int64_t)ck.stride_chunks * CH, tab.ckpt_off, stream) != 0) return -1;
    const int64_t nc = max_chunks(T_total, N);
    if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return -1;
    if (T_total > 0) {
        const size_t smem = sizeof(IntraSmem);
        auto intra = [&](auto sp, auto lrz) {
            hipLaunchKernelGGL((intra_kernel<decltype(sp)::value, decltype(lrz)::value>), dim3((unsigned)nc, (unsigned)H),
                               dim3(256), smem, stream, (const float *)q, (const float *)k, (const float *)v, z, beta,
                               A, N, H, tab);
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        const bool sp = ly.gate_kind == GATE_SOFTPLUS, lr = ly.zu != nullptr;
        if (sp)
            lr ? intra(T_{}, T_{}) : intra(T_{}, F_{});
        else
            lr ? intra(F_{}, T_{}) : intra(F_{}, F_{});
    }
    if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return -1;
    hipLaunchKernelGGL(map_kernel, dim3((unsigned)(nsm * H)), dim3(512), 0, stream, N, H, tab);
    if (ev && hipEventRecord(ev[3], stream) != hipSuccess) return -1;
    if (launch_seg_scan(S0, N, H, tab.sq, tab.Mseg, tab.Bseg, tab.Sin, S_final, stream) != 0) return -1;
    if (ev && hipEventRecord(ev[4], stream) != hipSuccess) return -1;
    hipLaunchKernelGGL(state_kernel, dim3((unsigned)(nsm * H)), dim3(512), 0, stream, N, H, tab, o, S_final);
    if (ly.gate && T_total > 0)
        hipLaunchKernelGGL(gated_rmsnorm_kernel, dim3((unsigned)((T_total * H + 3) / 4)), dim3(256), 0, stream, o,
                           ly.gate, ly.weight, ly.norm_eps, T_total * H);
    if (hipGetLastError() != hipSuccess) return -1;
    if (ev && hipEventRecord(ev[5], stream) != hipSuccess) return -1;
    return 0;
}

int set_prefill_attributes() {
    if (set_segment_attributes() != 0) return -1;
    const int smem = (int)sizeof(IntraSmem);
    const void *fns[4] = {(const void *)intra_kernel<false, false>, (const void *)intra_kernel<false, true>,
                          (const void *)intra_kernel<true, false>, (const void *)intra_kernel<true, true>};
    for (const void *f : fns)
        if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, smem) != hipSuccess) return -1;
    return 0;
}

}  // namespace kda
