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
//   prep_kernel   sequence boundaries (clamped, non-decreasing), the first
//                 chunk of every sequence and its first segment (L chunks);
//   intra_kernel  one workgroup per (chunk, head), all chunks in parallel:
//                 gate + sub-chunk cumsums, the two Gram tiles on MFMA, the
//                 blocked forward substitution, W and U on MFMA; writes the
//                 per-chunk operands of the chain to the workspace;
//   chain_kernel<true>   the affine map S -> M S + B of every segment but a
//                 sequence's last, one workgroup per (segment, head, 32 of
//                 the 256 columns of [M | B]);
//   seg_scan_kernel (kda_segment.hip)  the state entering each segment;
//   chain_kernel<false>  one workgroup per (segment, head, 32 value columns):
//                 keeps its 128 x 32 fp32 state slice in registers across the
//                 segment's chunks and forms Delta, the output and the next
//                 state with MFMA.
//
// This file serves fp32 q/k/v (bf16 q/k/v take kda_segment.hip's path): every
// product is an exact fp32 MFMA.  intra_kernel is written over the I/O type
// (with bf16, fp32 intermediates would enter MFMA as hi + lo bf16 pairs); the
// library instantiates it for fp32 only.
#include "kda_common.hpp"

namespace kda {

// ----------------------------------------------------------------- layout --

// Per (chunk, head) block of chain operands in the workspace (bytes).  "Split"
// arrays hold the bf16 hi part followed by the bf16 lo part in the bf16 build
// and plain fp32 in the fp32 build; both use 4 bytes per element.
constexpr size_t OFF_W = 0;            // W      [64][128]  bf16 (fp32 build: fp32)
constexpr size_t OFF_U = 32768;        // U      [64][128]  fp32
constexpr size_t OFF_KT = 65536;       // K~^T   [128][64]  split, K~ = K * e^{G_n - G}
constexpr size_t OFF_QT = 98304;       // Q~     [64][128]  split, Q~ = Q * Gam
constexpr size_t OFF_AQ = 131072;      // Aqk    [64][64]   split, zero above the diagonal
constexpr size_t OFF_GM = 147456;      // gamma  [128]      fp32, e^{G_n}
constexpr size_t BLK_BYTES = 147968;   // multiple of 256

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Table {  // workspace header
    int32_t *chunk_off;  // [N+1] first chunk of each sequence; chunk_off[N] = total
    int32_t *seg_off;    // [N+1] first segment of each sequence
    int32_t *segA_off;   // [N+1] first map segment (every segment but a sequence's last)
    int64_t *seq_start;  // [N]
    int64_t *seq_end;    // [N]
    int64_t *ckpt_off;   // [N+1] first snapshot slot of each sequence
    char *blocks;        // chain operands, block (c, h) at (c * H + h) * BLK_BYTES
    float *Mseg;         // [nseg][H][128][128] segment transitions
    float *Bseg;         // [nseg][H][128][128] segment offsets
    float *Sin;          // [nseg][H][128][128] state entering each segment
    int L;               // chunks per segment
    Ckpt ck;
    Layer ly;
};

__host__ __device__ inline size_t table_bytes(int N) {
    return 3 * align256(4 * (size_t)(N + 1)) + 2 * align256(8 * (size_t)N) + align256(8 * (size_t)(N + 1));
}
__host__ __device__ inline Table carve(void *ws, int N) {
    char *p = (char *)ws;
    Table t;
    t.chunk_off = (int32_t *)p;
    p += align256(4 * (size_t)(N + 1));
    t.seg_off = (int32_t *)p;
    p += align256(4 * (size_t)(N + 1));
    t.segA_off = (int32_t *)p;
    p += align256(4 * (size_t)(N + 1));
    t.seq_start = (int64_t *)p;
    p += align256(8 * (size_t)N);
    t.seq_end = (int64_t *)p;
    p += align256(8 * (size_t)N);
    t.ckpt_off = (int64_t *)p;
    p += align256(8 * (size_t)(N + 1));
    t.blocks = p;
    t.Mseg = t.Bseg = t.Sin = nullptr;
    t.L = 1;
    t.ck = Ckpt{nullptr, t.ckpt_off, 1, 0};
    t.ly = Layer{false, 0.f, nullptr, nullptr, 0.f};
    return t;
}
__host__ inline int64_t max_chunks(int64_t T_total, int N) { return (T_total + CH - 1) / CH + N; }
// Segments of the chain: about SEG32_TARGET (segment, head) pairs in all, so
// that the chain passes have over a thousand workgroups (8 and 16 per pair).
// Their time at 64K x 16 is the same from 128 to 1,024 pairs (they are bound
// by throughput, not by the length of the chain); fewer pairs shorten the scan.
constexpr int SEG32_TARGET = 128;
__host__ inline int seg32_len(int64_t T_total, int N, int H) {
    const int64_t per_head = SEG32_TARGET / (H > 0 ? H : 1) > 0 ? SEG32_TARGET / H : 1;
    return (int)((max_chunks(T_total, N) + per_head - 1) / per_head);
}
__host__ inline int64_t seg32_max(int64_t T_total, int N, int H) {
    const int L = seg32_len(T_total, N, H);
    return (max_chunks(T_total, N) + L - 1) / L + N;
}

// ------------------------------------------------------------------- prep --

// Sequence n spans [s_n, s_{n+1}) with s_m = max_{m' <= m} clamp(cu[m'], 0, T),
// so sequences never overlap and the chunk count is at most ceil(T/64) + N.
// cu == nullptr means B equal sequences of Tper tokens.  One workgroup walks
// the N + 1 offsets in tiles of 256 with a running max and a running sum.
// It also writes seg_off and segA_off: the exclusive prefix sums of each
// sequence's segment count ceil(chunks / L) and of that count less one.
__global__ __launch_bounds__(256) void prep_kernel(const int32_t *__restrict__ cu, int N, int64_t T_total,
                                                   int64_t Tper, Table tab) {
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
            c = cu ? (int64_t)cu[m] : (int64_t)m * Tper;
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

// off[n] = sum over sequences m < n of floor(len_m / stride), n = 0 .. N: the
// first snapshot slot of each sequence.  One workgroup, tiles of 256 with a
// running sum.
__global__ __launch_bounds__(256) void ckpt_prep_kernel(const int64_t *__restrict__ seq_start,
                                                        const int64_t *__restrict__ seq_end, int N, int64_t stride,
                                                        int64_t *__restrict__ off) {
    __shared__ int64_t s_scan[256];
    __shared__ int64_t s_prev;
    const int tid = threadIdx.x;
    if (tid == 0) s_prev = 0;
    __syncthreads();
    for (int base = 0; base <= N; base += 256) {
        const int m = base + tid;  // off[m] sums sequences < m: exclusive scan
        s_scan[tid] = (m >= 1 && m <= N) ? (seq_end[m - 1] - seq_start[m - 1]) / stride : 0;
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

int launch_ckpt_prep(const int64_t *seq_start, const int64_t *seq_end, int N, int64_t stride, int64_t *off,
                     hipStream_t stream) {
    hipLaunchKernelGGL(ckpt_prep_kernel, dim3(1), dim3(256), 0, stream, seq_start, seq_end, N, stride, off);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// locate chunk c: sequence n with chunk_off[n] <= c < chunk_off[n+1]
__device__ inline int find_seq(const int32_t *chunk_off, int N, int c) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= c)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// ----------------------------------------------------------------- intra --

constexpr int PG = 132;  // LDS pitch (floats) of [64][128] token-major arrays
constexpr int PT = 68;   // LDS pitch (floats) of [*][64] arrays

// 77.6 KB, so that two workgroups share a CU.
template <typename IO>
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

// store a split (hi | lo) or fp32 value quad at element offset e of an array of
// n_elems elements starting at base
template <bool F32>
__device__ __forceinline__ void st_split4(char *base, size_t n_elems, size_t e, float a, float b, float c,
                                          float d) {
    if constexpr (F32) {
        *(float4 *)((float *)base + e) = make_float4(a, b, c, d);
    } else {
        bf16x4 h, l;
        h[0] = (__bf16)a; h[1] = (__bf16)b; h[2] = (__bf16)c; h[3] = (__bf16)d;
        l[0] = (__bf16)(a - (float)h[0]); l[1] = (__bf16)(b - (float)h[1]);
        l[2] = (__bf16)(c - (float)h[2]); l[3] = (__bf16)(d - (float)h[3]);
        *(bf16x4 *)((__bf16 *)base + e) = h;
        *(bf16x4 *)((__bf16 *)base + n_elems + e) = l;
    }
}
template <bool F32>
__device__ __forceinline__ void st_split1(char *base, size_t n_elems, size_t e, float a) {
    if constexpr (F32) {
        ((float *)base)[e] = a;
    } else {
        __bf16 h = (__bf16)a;
        ((__bf16 *)base)[e] = h;
        ((__bf16 *)base)[n_elems + e] = (__bf16)(a - (float)h);
    }
}

template <typename IO>
__global__ __launch_bounds__(256) void intra_kernel(const IO *__restrict__ q, const IO *__restrict__ k,
                                                    const IO *__restrict__ v, const float *__restrict__ z,
                                                    const float *__restrict__ beta,
                                                    const float *__restrict__ A, int N, int H, Table tab) {
    constexpr bool F32 = sizeof(IO) == 4;
    extern __shared__ __align__(16) char smem_raw[];
    IntraSmem<IO> &sm = *reinterpret_cast<IntraSmem<IO> *>(smem_raw);

    const int c = blockIdx.x, h = blockIdx.y;
    const int total = tab.chunk_off[N];
    if (c >= total) return;
    const int n = find_seq(tab.chunk_off, N, c);
    const int64_t t0 = tab.seq_start[n] + (int64_t)(c - tab.chunk_off[n]) * CH;
    const int len = (int)min((int64_t)CH, tab.seq_end[n] - t0);
    char *blk = tab.blocks + ((size_t)c * H + h) * BLK_BYTES;

    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, g = l >> 4, lr = l & 15;
    const size_t HD = (size_t)H * D;
    auto tok = [&](int t) -> size_t { return (size_t)(t0 + t) * HD + (size_t)h * D; };

    // ---- phase 0: inverse L2 norms of the key and query rows when the layer's
    // normalisation is fused in (wave w: rows 16 w .. 16 w + 15, four lanes of 32
    // channels per row); 1 otherwise.
    {
        const int tr = 16 * wv + (l >> 2), cq = 32 * (l & 3);
        float nk = 1.f, nq = 1.f;
        if (tab.ly.qk_norm) {
            float sk = 0.f, sq = 0.f;
            if (tr < len) {
                for (int c2 = 0; c2 < 32; ++c2) {
                    const float a = to_f(k[tok(tr) + cq + c2]), b = to_f(q[tok(tr) + cq + c2]);
                    sk += a * a;
                    sq += b * b;
                }
            }
            sk += __shfl_xor(sk, 1);
            sk += __shfl_xor(sk, 2);
            sq += __shfl_xor(sq, 1);
            sq += __shfl_xor(sq, 2);
            nk = 1.f / __fsqrt_rn(sk + tab.ly.qk_eps);
            nq = 1.f / __fsqrt_rn(sq + tab.ly.qk_eps);
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
    const bool sp = tab.ly.gate_kind == GATE_SOFTPLUS;
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
            zr[si][u] = tab.ly.zu ? 0.f : (zh ? z[(size_t)(t0 + tc) * H + h] : z[tok(tc) + ch]);
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
                if (tab.ly.zu) {  // low-rank forget gate: z = sum_j u[t, j] W[h, ch, j]
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
                kr[u] = to_f(k[tok(tc) + ch]);
                qr[u] = to_f(q[tok(tc) + ch]);
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
                st_split1<F32>(qt, CH * D, (size_t)t * D + ch, qv * gam);
                kt_vals[u] = kv * __expf((float)(Gn - Gt));
            }
#pragma unroll
            for (int u = 0; u < SUB; u += 4)
                st_split4<F32>(kt, D * CH, (size_t)ch * CH + s * SUB + u, kt_vals[u], kt_vals[u + 1],
                               kt_vals[u + 2], kt_vals[u + 3]);
        }
        if (half == 0) ((float *)(blk + OFF_GM))[ch] = __expf((float)Gn);
    }
    // the six tiles of Aqk above the diagonal are zero
    for (int e = tid; e < 6 * 64; e += 256) {
        const int tile = e >> 6, quad = e & 63;
        const int ti = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
        const int tj = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
        const int r = 16 * ti + (quad >> 2), c0 = 16 * tj + 4 * (quad & 3);
        st_split4<F32>(blk + OFF_AQ, CH * CH, (size_t)r * CH + c0, 0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();

    // ---- phase 2: the two decay-scaled Gram matrices on MFMA ----
    // tile list: for mat in {kk, qk}, i in 0..3, j in 0..i (20 tiles), wave wv
    // takes tiles wv, wv+4, ..  The product is formed transposed (column side as
    // the A operand) so that each lane ends up with 4 consecutive columns of a row.
    // Akk shares its LDS with E1: the tiles of Akk wait in registers until every
    // wave is done with E1.
    f32x4 kkv[3];
#pragma unroll
    for (int it = 0; it < 5; ++it) {
        const int tix = wv + 4 * it;
        if (tix >= 20) break;
        const int mat = tix / 10, rem = tix % 10;
        int i = 0;
        while ((i + 1) * (i + 2) / 2 <= rem) ++i;
        const int j = rem - i * (i + 1) / 2;
        const IO *X = mat == 0 ? k : q;
        const int cr = 16 * j + lr;  // column-side token (A operand row)
        const int rr = 16 * i + lr;  // row-side token (B operand column)
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (sp && j == i) {
            // Position pairs (rr, c = 16 i + 4 g + m): sum_ch x_rr k_c e^{L_rr - L_c}
            // with L = G - R_i; the exponent is clamped at 0 (c > rr is masked below).
            const float nr = mat == 0 ? sm.nk[rr] : sm.nq[rr];
            const int c0 = 16 * i + 4 * g;
            for (int e = 0; e < D; ++e) {
                const float xr = rr < len ? to_f(X[tok(rr) + e]) * nr : 0.f, lrr = sm.u.E1[rr * PG + e];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int cc = c0 + m;
                    const float kc = cc < len ? to_f(k[tok(cc) + e]) * sm.nk[cc] : 0.f;
                    acc[m] += xr * kc * __expf(fminf(lrr - sm.u.E1[cc * PG + e], 0.f));
                }
            }
        } else {
        // the tile's row fragments for all four k-steps, loaded before the first
        // product (rows past the end read row 0 and are zeroed)
        F8 kcs[4], xrs[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            kcs[ks] = ld_io8(k + tok(cr < len ? cr : 0) + 32 * ks + 8 * g);
            xrs[ks] = ld_io8(X + tok(rr < len ? rr : 0) + 32 * ks + 8 * g);
        }
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
                    inv = __frcp_rn(sm.u.E1[cr * PG + c0 + e]);  // e^{R_j - G_c}
                    if (j < i) inv *= sm.PF[pair_index(i, j) * D + c0 + e];
                    er = sm.u.E1[rr * PG + c0 + e];
                }
                a.v[e] = kc.v[e] * nc * inv;
                b.v[e] = xr.v[e] * nr * er;
            }
            if constexpr (F32)
                acc = mma_ff(acc, a, b);
            else
                acc = mma_ss(acc, split8(a), split8(b));
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
            st_split4<F32>(blk + OFF_AQ, CH * CH, (size_t)rr * CH + cb, val[0], val[1], val[2], val[3]);
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
    // wave wv: row tile rt = wv for W and 3 - wv for U; 8 column tiles each
    for (int pass = 0; pass < 2; ++pass) {
        const int rt = pass == 0 ? wv : 3 - wv;
        // pass 0: (K * Gam)^T from LDS; pass 1: V^T read from global memory
        // (rows past the end of the sequence as 0)
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
        S8 tbs[2];
        if constexpr (!F32) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) tbs[ks] = split8(tb[ks]);
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            // pass 1: this column tile's V values, all loaded before its products
            // (rows past the end read row 0 and are zeroed)
            F8 vcol[2];
            if (pass == 1) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int t = 32 * ks + 8 * g + e;
                        const float x = to_f(v[tok(t < len ? t : 0) + 16 * ct + lr]);
                        vcol[ks].v[e] = t < len ? x : 0.f;
                    }
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks >= nks) break;
                F8 xa;
                if (pass == 0) {
                    xa = ld_f8(&sm.KG[(16 * ct + lr) * PT + 32 * ks + 8 * g]);
                } else {
                    xa = vcol[ks];
                }
                if constexpr (F32)
                    acc = mma_ff(acc, xa, tb[ks]);
                else
                    acc = mma_1s(acc, round8(xa), tbs[ks]);
            }
            // acc[m] = out[row r][col 16 ct + 4 g + m]
            const size_t e0 = (size_t)r * D + 16 * ct + 4 * g;
            if (pass == 0) {
                if constexpr (F32) {
                    *(float4 *)((float *)(blk + OFF_W) + e0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                } else {
                    bf16x4 hv;
                    hv[0] = (__bf16)acc[0]; hv[1] = (__bf16)acc[1];
                    hv[2] = (__bf16)acc[2]; hv[3] = (__bf16)acc[3];
                    *(bf16x4 *)((__bf16 *)(blk + OFF_W) + e0) = hv;
                }
            } else {
                *(float4 *)((float *)(blk + OFF_U) + e0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }
    }
}

// ----------------------------------------------------------------- chain --

constexpr int NCT = 2;         // 16-column tiles per workgroup
constexpr int NB = 16 * NCT;  // state columns per workgroup

struct ChainSmem {
    float S[NB * 132];  // the state slice, transposed [column][key row]
    float Dl[NB * 68];  // Delta, transposed [column][token]
};

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt), not for its global loads in flight, which __syncthreads' fence
// would also wait for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// largest n in [0, N) with off[n] <= x (for x < off[N] that is the owner of x)
__device__ inline int seq_of(const int32_t *off, int N, int x) {
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

// The chain over one segment of a sequence, 32 state columns per workgroup
// (each operand fragment loaded serves both 16-column tiles), exact fp32 MFMA
// throughout.  The segment map carries a state S entering the segment to
// M S + B; MAP = true computes the columns of X = [M | B] (128 x 256) by
// running the chain step from X = [I | 0], with U entering only the B columns;
// MAP = false runs it from the state the scan gave the segment and writes o
// (and snapshots, and S_final after a sequence's last segment).  Workgroups
// are numbered so that the column blocks of one (segment, head) share an XCD
// (and its L2, which serves their common operand block), and the (segment,
// head) pairs with work come first.
template <bool MAP>
__global__ __launch_bounds__(256) void chain_kernel(int N, int H, Table tab, float *__restrict__ o,
                                                    float *__restrict__ S_final) {
    __shared__ ChainSmem sm;
    constexpr int NCB = (MAP ? 2 * D : D) / NB;  // column blocks per (segment, head)
    const int Lw = blockIdx.x;
    const int p = (Lw & 7) + 8 * (Lw / (8 * NCB)), cb = (Lw >> 3) % NCB;
    const int a = p / H, h = p % H;
    const int32_t *soff = MAP ? tab.segA_off : tab.seg_off;
    if (a >= soff[N]) return;
    const int n = seq_of(soff, N, a);
    const int j = a - soff[n];
    const int x = tab.seg_off[n] + j;  // segment index of the maps and states
    const int pn = tab.seg_off[n + 1] - tab.seg_off[n];
    const bool bcol = MAP && cb >= NCB / 2;              // columns of B (U enters)
    const int col0 = NB * (MAP ? cb % (NCB / 2) : cb);  // first column within M, B or the state
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, lr = l & 15;

    // state slice: wave w owns key rows [32w, 32w+32) as two 16-row tiles (C
    // layout) of each column tile ct (columns col0 + 16 ct + lr)
    f32x4 Sr[NCT][2];
    const size_t sblk = ((size_t)x * H + h) * D * D;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 32 * w + 16 * u + 4 * g + m, cc = col0 + 16 * ct + lr;
                Sr[ct][u][m] = MAP ? (!bcol && r == cc ? 1.f : 0.f) : tab.Sin[sblk + (size_t)r * D + cc];
            }

    const int cseq = tab.chunk_off[n];  // the sequence's first chunk
    const int cbeg = cseq + j * tab.L, cend = min(tab.chunk_off[n + 1], cbeg + tab.L);
    const int64_t sstart = tab.seq_start[n], send = tab.seq_end[n];
    const int nks_aq = w < 2 ? 1 : 2;  // 32-token k-steps of Aqk row tile w
    const int64_t ck_base = tab.ck.S ? tab.ck.off[n] : 0;

    // Operands of one chunk, in registers.  The barriers wait only for LDS
    // traffic, so loads stay in flight across them.  The map pass loads each
    // group for chunk c + 1 as soon as chunk c has used it (the last chunk
    // re-reads itself); the state pass, which has no registers to spare for
    // that, issues all of chunk c's loads at the top of its step.
    constexpr bool PF = MAP;
    const int row = 16 * w + lr;
    F8 wf[4], qf[4], kf[2][2], af[2];
    float uv[NCT][4], gmv[2][4];
    auto load_wq = [&](const char *blk) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            wf[ks] = ld_f8((const float *)(blk + OFF_W) + row * D + 32 * ks + 8 * g);
            if constexpr (!MAP) qf[ks] = ld_f8((const float *)(blk + OFF_QT) + row * D + 32 * ks + 8 * g);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                uv[ct][m] = (!MAP || bcol)
                                ? ((const float *)(blk + OFF_U))[(16 * w + 4 * g + m) * D + col0 + 16 * ct + lr]
                                : 0.f;
    };
    auto load_ka = [&](const char *blk) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int kr = 32 * w + 16 * u;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                kf[u][ks] = ld_f8((const float *)(blk + OFF_KT) + (kr + lr) * CH + 32 * ks + 8 * g);
#pragma unroll
            for (int m = 0; m < 4; ++m) gmv[u][m] = ((const float *)(blk + OFF_GM))[kr + 4 * g + m];
        }
        if constexpr (!MAP)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) af[ks] = ld_f8((const float *)(blk + OFF_AQ) + row * CH + 32 * ks + 8 * g);
    };
    auto block = [&](int cc) { return tab.blocks + ((size_t)cc * H + h) * BLK_BYTES; };
    if (PF && cbeg < cend) {
        load_wq(block(cbeg));
        load_ka(block(cbeg));
    }

    for (int c = cbeg; c < cend; ++c) {
        const char *nblk = block(min(c + 1, cend - 1));
        if (!PF) {
            load_wq(block(c));
            load_ka(block(c));
        }
        const int64_t t0 = sstart + (int64_t)(c - cseq) * CH;
        const int len = (int)min((int64_t)CH, send - t0);

        // (1) publish the state slice as the B operand of W S and Q~ S
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                *(float4 *)&sm.S[(16 * ct + lr) * 132 + 32 * w + 16 * u + 4 * g] =
                    make_float4(Sr[ct][u][0], Sr[ct][u][1], Sr[ct][u][2], Sr[ct][u][3]);
        lds_barrier();

        // (2) Delta rows [16w, 16w+16) = U - W S ;  O = Q~ S
        f32x4 ws[NCT], oacc[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) ws[ct] = oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const F8 sb = ld_f8(&sm.S[(16 * ct + lr) * 132 + 32 * ks + 8 * g]);
                ws[ct] = mma_ff(ws[ct], wf[ks], sb);
                if constexpr (!MAP) oacc[ct] = mma_ff(oacc[ct], qf[ks], sb);
            }
        }
        f32x4 dl[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int m = 0; m < 4; ++m) dl[ct][m] = uv[ct][m] - ws[ct][m];
        if (PF) load_wq(nblk);
        // (3) publish Delta as the B operand of Aqk Delta and K~^T Delta
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            *(float4 *)&sm.Dl[(16 * ct + lr) * 68 + 16 * w + 4 * g] =
                make_float4(dl[ct][0], dl[ct][1], dl[ct][2], dl[ct][3]);
        lds_barrier();
        F8 dF[NCT][2];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) dF[ct][ks] = ld_f8(&sm.Dl[(16 * ct + lr) * 68 + 32 * ks + 8 * g]);
        // (4) O += Aqk Delta  (row tile w; Aqk is zero above the diagonal)
        if constexpr (!MAP)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (ks < nks_aq)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) oacc[ct] = mma_ff(oacc[ct], af[ks], dF[ct][ks]);
        // (5) S <- Diag(gamma) S + K~^T Delta  (key rows [32w, 32w+32))
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 acc[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int m = 0; m < 4; ++m) acc[ct][m] = gmv[u][m] * Sr[ct][u][m];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) acc[ct] = mma_ff(acc[ct], kf[u][ks], dF[ct][ks]);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) Sr[ct][u] = acc[ct];
        }
        if (PF) load_ka(nblk);
        if constexpr (!MAP) {
            // (5b) snapshot after a full chunk that ends a stride
            if (tab.ck.S && len == CH && (c - cseq + 1) % tab.ck.stride_chunks == 0) {
                const int64_t slot = ck_base + (c - cseq + 1) / tab.ck.stride_chunks - 1;
                if (slot < tab.ck.cap) {
                    float *dst = tab.ck.S + ((size_t)slot * H + h) * D * D;
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int u = 0; u < 2; ++u)
#pragma unroll
                            for (int m = 0; m < 4; ++m)
                                dst[(size_t)(32 * w + 16 * u + 4 * g + m) * D + col0 + 16 * ct + lr] = Sr[ct][u][m];
                }
            }
            // (6) output rows of this chunk
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int t = 16 * w + 4 * g + m;
                if (t < len)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) o[((size_t)(t0 + t) * H + h) * D + col0 + 16 * ct + lr] = oacc[ct][m];
            }
        }
    }
    float *dst = nullptr;
    if (MAP)
        dst = (bcol ? tab.Bseg : tab.Mseg) + sblk;
    else if (S_final && j == pn - 1)
        dst = S_final + ((size_t)n * H + h) * D * D;
    if (dst) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    dst[(size_t)(32 * w + 16 * u + 4 * g + m) * D + col0 + 16 * ct + lr] = Sr[ct][u][m];
    }
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
int launch_seg_scan(const float *S0, int N, int H, const int32_t *seg_off, float *Mseg, float *Bseg, float *Sin,
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
    tab.L = seg32_len(T_total, N, H);
    const int64_t nsm = seg32_max(T_total, N, H);
    const size_t st = (size_t)nsm * H * D * D;
    tab.Mseg = (float *)(tab.blocks + (size_t)max_chunks(T_total, N) * (size_t)H * BLK_BYTES);
    tab.Bseg = tab.Mseg + st;
    tab.Sin = tab.Bseg + st;
    // chain grids: 4 (state) or 8 (map) workgroups of 256 per (segment, head)
    // slot; a launch covers at most 2^32 - 1 work-items
    const int64_t slots8 = (nsm * H + 7) / 8;
    if (slots8 * 128 > (int64_t)(UINT32_MAX / 256) || max_chunks(T_total, N) * H > (int64_t)UINT32_MAX) return -1;
    if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return -1;
    hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(256), 0, stream, cu, N, T_total, cu ? (int64_t)0 : T, tab);
    if (ck.S && launch_ckpt_prep(tab.seq_start, tab.seq_end, N, (int64_t)ck.stride_chunks * CH, tab.ckpt_off,
                                 stream) != 0)
        return -1;
    const int64_t nc = max_chunks(T_total, N);
    if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return -1;
    if (T_total > 0) {
        const size_t smem = sizeof(IntraSmem<float>);
        hipLaunchKernelGGL(intra_kernel<float>, dim3((unsigned)nc, (unsigned)H), dim3(256), smem, stream,
                           (const float *)q, (const float *)k, (const float *)v, z, beta, A, N, H, tab);
    }
    if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return -1;
    hipLaunchKernelGGL(chain_kernel<true>, dim3((unsigned)(8 * (2 * D / NB) * slots8)), dim3(256), 0, stream, N, H,
                       tab, o, S_final);
    if (ev && hipEventRecord(ev[3], stream) != hipSuccess) return -1;
    if (launch_seg_scan(S0, N, H, tab.seg_off, tab.Mseg, tab.Bseg, tab.Sin, S_final, stream) != 0) return -1;
    if (ev && hipEventRecord(ev[4], stream) != hipSuccess) return -1;
    hipLaunchKernelGGL(chain_kernel<false>, dim3((unsigned)(8 * (D / NB) * slots8)), dim3(256), 0, stream, N, H,
                       tab, o, S_final);
    if (ly.gate && T_total > 0)
        hipLaunchKernelGGL(gated_rmsnorm_kernel, dim3((unsigned)((T_total * H + 3) / 4)), dim3(256), 0, stream, o,
                           ly.gate, ly.weight, ly.norm_eps, T_total * H);
    if (hipGetLastError() != hipSuccess) return -1;
    if (ev && hipEventRecord(ev[5], stream) != hipSuccess) return -1;
    return 0;
}

int set_prefill_attributes() {
    if (set_segment_attributes() != 0) return -1;
    const int smem = (int)sizeof(IntraSmem<float>);
    if (hipFuncSetAttribute((const void *)intra_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize, smem) !=
        hipSuccess)
        return -1;
    return 0;
}

}  // namespace kda
