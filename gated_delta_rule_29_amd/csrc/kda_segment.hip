// kda_segment.hip -- segment-parallel fused chunkwise KDA prefill (bf16 q/k/v).
//
// Pages: "Kimi Linear: An Expressive, Efficient Attention Architecture" summary
// (sections 2.1, 3.1, 6.3, appendix C: chunk size 64, WY / UT transform with a
// forward-substitution inverse, inter-chunk recurrence) and "Kimi K3
// architecture" (sequence-bottleneck section: g = -5 Sigmoid(e^A z), 16-token
// tiles; KDA context parallelism merges per-rank local state updates with a
// prefix scan).
//
// Each chunk maps the incoming state affinely, S' = M S + B with
// M = Diag(gamma) - K~^T W and B = K~^T U (the chunk algebra is written out in
// kda_prefill.hip).  A sequence is cut into segments of L chunks; one
// workgroup owns one (segment, head):
//   pass A  from X = [I | 0] it runs the chunk recurrence on the 256 columns of
//           X (the segment's transition M_p and offset B_p at once) and writes
//           (M_p, B_p) -- no outputs;
//   scan    per (sequence, head): S_in[0] = S0, S_in[p+1] = M_p S_in[p] + B_p;
//   pass B  from S_in[p] it reruns the segment with outputs and writes o (and
//           S_final for the last segment).
// Inside a workgroup every chunk is processed in LDS: gate and sub-chunk
// cumulative sums, the two decay-scaled Gram tiles (bf16 hi+lo MFMA), the
// blocked forward-substitution inverse, W and U (MFMA), then the chain step.
// The chain step is wave-local: wave w owns a slice of state columns, keeps it
// in MFMA C-layout registers and feeds those registers straight back as the
// B operand of the next product.  That works because the k index of an MFMA is
// summed: pairing the C tiles 2s and 2s+1 gives k slot e -> row
// 32s + 16*(e>>2) + 4*(lane>>4) + (e&3), and the A operands (W, Q~ over key
// channels; Aqk, K~^T over tokens) are stored in LDS with that permutation
// (perm32 below).  No LDS exchange and no barrier sits inside the chain.
//
// Operand precision (chosen against the fp64 oracle): W, Q~, K~ and the state
// enter the chain as single fp16; Delta as fp16 hi+lo; Aqk and Delta as
// fp16 hi+lo pairs (three MFMAs); the Gram tiles and T diag(beta) as bf16
// hi+lo (their column factors reach e^80, beyond fp16 range).
#include "kda_common.hpp"

namespace kda {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// k-slot permutation inside 32-blocks: x = 16h + 4g + m  ->  8g + 4h + m
__device__ __forceinline__ int perm32(int x) {
    const int r = x & 31;
    return (x & ~31) | (((r >> 2) & 3) << 3) | (((r >> 4) & 1) << 2) | (r & 3);
}

constexpr int P16 = 136;  // pitch (halves) of [64][128] 16-bit LDS arrays
constexpr int P64 = 72;   // pitch (halves) of [*][64] 16-bit LDS arrays
constexpr int PE = 132;   // pitch (floats) of E1 [64][128]
constexpr int PTT = 72;   // pitch (floats) of T [64][64]; the region also holds T diag(beta) as bf16 hi / lo

struct SegSmem {
    union {
        float E1[CH * PE];      // e^{G_t - R_s(t)} (phases 1-2.5)
        __bf16 KGt[D * P64];    // (K * Gam)^T [channel][token] (phases 2.5-4)
    } a;
    union {
        __bf16 K[CH * P16];     // k [token][channel] (phases 1-2.5)
        _Float16 W[CH * P16];   // -W [token][perm(channel)] (phase 4 - chain)
    } b;
    union {
        __bf16 Q[CH * P16];     // q [token][channel]
        _Float16 Qt[CH * P16];  // Q~ [token][perm(channel)]
    } c;
    __bf16 Vt[D * P64];         // V^T [channel][token]
    union {
        float T[CH * PTT];        // Akk, then T = (I + Akk)^{-1}
        __bf16 Tb[2 * CH * P64];  // T diag(beta): hi [64][72], then lo [64][72]
    } t;
    _Float16 KtT[D * P64];      // K~^T [channel][perm(token)]
    _Float16 AqH[CH * P64];     // Aqk [token][perm(token)], fp16 hi
    _Float16 AqL[CH * P64];     // fp16 lo
    float R[5 * D];             // R_s, cumulative log-decay before sub-chunk s; R_4 = G_n
    float PF[7 * D];            // e^{R_i - R_j} for the pairs j < i; row 6 is all ones (j = i)
    float beta[CH];
    float gam[D];               // e^{G_n}
};

struct SegTable {
    int32_t *seg_off;    // [N+1] first segment of each sequence
    int64_t *seq_start;  // [N]
    int64_t *seq_end;    // [N]
    float *Mseg;         // [nseg][H][128][128] segment transitions
    float *Bseg;         // [nseg][H][128][128] segment offsets
    float *Sin;          // [nseg][H][128][128] state entering each segment
    int L;               // chunks per segment
};

// ------------------------------------------------------------------ prep --

// Sequences as in the chunk table: s_m = running max of clamped offsets.
// seg_off = exclusive prefix sum of ceil(ceil(len / 64) / L).
__global__ __launch_bounds__(256) void seg_prep_kernel(const int32_t *__restrict__ cu, int N, int64_t T_total,
                                                       int64_t Tper, SegTable tab) {
    __shared__ int64_t s_scan[256];
    __shared__ int64_t s_prev_max, s_prev_sum;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_prev_max = 0;
        s_prev_sum = 0;
    }
    __syncthreads();
    for (int base = 0; base <= N; base += 256) {
        const int m = base + tid;
        int64_t c = 0;
        if (m <= N) {
            c = cu ? (int64_t)cu[m] : (int64_t)m * Tper;
            c = c < 0 ? 0 : (c > T_total ? T_total : c);
        }
        s_scan[tid] = c;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int64_t x = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            if (x > s_scan[tid]) s_scan[tid] = x;
            __syncthreads();
        }
        const int64_t pm = s_prev_max;
        const int64_t sm = s_scan[tid] > pm ? s_scan[tid] : pm;
        const int64_t sp = tid > 0 ? (s_scan[tid - 1] > pm ? s_scan[tid - 1] : pm) : pm;
        if (m < N) tab.seq_start[m] = sm;
        if (m >= 1 && m <= N) tab.seq_end[m - 1] = sm;
        int64_t cnt = 0;
        if (m >= 1 && m <= N) {
            const int64_t nch = (sm - sp + CH - 1) / CH;
            cnt = (nch + tab.L - 1) / tab.L;
        }
        __syncthreads();
        s_scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int64_t x = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += x;
            __syncthreads();
        }
        const int64_t incl = s_scan[tid] + s_prev_sum;
        if (m <= N) tab.seg_off[m] = (int32_t)incl;
        __syncthreads();
        if (tid == 255) {
            s_prev_max = sm;
            s_prev_sum = incl;
        }
        __syncthreads();
    }
}

__device__ inline int seg_find(const int32_t *off, int N, int x) {
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

// --------------------------------------------------------- segment pass --

// Raw input tiles of one chunk as held in registers: q, k, v rows of 256 B in
// 16 B pieces (row = tid / 16 + (threads / 16) p), z rows of 512 B in 16 B
// pieces (row = tid / 32 + (threads / 32) p), and beta (wave 0, lane = row).
template <int NP16, int NPZ>
struct Tiles {
    u32x4 k[NP16], q[NP16], v[NP16];
    f32x4 z[NPZ];
    float b;
};

template <bool PASS_A, int NP16, int NPZ>
__device__ __forceinline__ Tiles<NP16, NPZ> load_tiles(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
                                                       const __bf16 *__restrict__ v, const float *__restrict__ z,
                                                       const float *__restrict__ beta, int64_t s0, int64_t s1,
                                                       int chunk, int h, int H, int tid) {
    constexpr int THREADS = 1024 / NP16;
    static_assert(THREADS * NPZ == 2048, "tile split");
    Tiles<NP16, NPZ> t;
    const size_t HD = (size_t)H * D;
    const int64_t t0 = s0 + (int64_t)chunk * CH;
    const int len = (int)min((int64_t)CH, s1 - t0);
    const int r16 = tid >> 4, o16 = 8 * (tid & 15), r32 = tid >> 5, o32 = 4 * (tid & 31);
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int p = 0; p < NP16; ++p) {
        const int row = r16 + (THREADS / 16) * p;
        const size_t e = (size_t)(t0 + row) * HD + (size_t)h * D + o16;
        const bool ok = row < len;
        t.k[p] = ok ? *(const u32x4 *)(k + e) : zero4;
        t.v[p] = ok ? *(const u32x4 *)(v + e) : zero4;
        t.q[p] = (!PASS_A && ok) ? *(const u32x4 *)(q + e) : zero4;
    }
#pragma unroll
    for (int p = 0; p < NPZ; ++p) {
        const int row = r32 + (THREADS / 32) * p;
        const size_t e = (size_t)(t0 + row) * HD + (size_t)h * D + o32;
        t.z[p] = row < len ? *(const f32x4 *)(z + e) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int l = tid & 63;
    t.b = (tid < 64 && l < len) ? beta[(size_t)(t0 + l) * H + h] : 0.f;
    return t;
}

template <bool PASS_A, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void seg_pass_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ z, const float *__restrict__ beta, const float *__restrict__ A, int N, int H,
    SegTable tab, float *__restrict__ o, float *__restrict__ S_final) {
    extern __shared__ __align__(16) char smem_raw[];
    SegSmem &sm = *reinterpret_cast<SegSmem *>(smem_raw);
    constexpr int NT_ = 64 * NW;  // threads

    const int x = blockIdx.x, h = blockIdx.y;
    const int nseg = tab.seg_off[N];
    if (x >= nseg) return;
    const int n = seg_find(tab.seg_off, N, x);
    const int j = x - tab.seg_off[n];
    const int pn = tab.seg_off[n + 1] - tab.seg_off[n];
    if (PASS_A && j == pn - 1) return;  // the last segment's map is not needed
    const int64_t s0 = tab.seq_start[n], s1 = tab.seq_end[n];
    const int nch = (int)((s1 - s0 + CH - 1) / CH);
    const int cbeg = j * tab.L, cend = min(nch, cbeg + tab.L);

    // NW waves: wave wv, lane l; MFMA lane roles g = l >> 4, lr = l & 15
    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, g = l >> 4, lr = l & 15;
    const size_t HD = (size_t)H * D;
    const float eA = __expf(A[h]);
    const size_t blk = ((size_t)x * H + h) * D * D;

    // ---- the state slice: pass B 128 / NW columns per wave, pass A 256 / NW columns of [M | B]
    constexpr int NCT = (PASS_A ? 16 : 8) / NW;
    const int colw = 16 * NCT * wv;  // pass A: columns 0..127 are M, 128..255 are B
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
                    X[rt][ct][m] = tab.Sin[blk + (size_t)r * D + col];
            }

    // ---- raw input tiles of a chunk, prefetched into registers one chunk ahead:
    // q, k, v rows of 256 B as 16 B pieces, z rows of 512 B as 16 B pieces
    constexpr int NP16 = 1024 / NT_, NPZ = 2048 / NT_;
    Tiles<NP16, NPZ> pf;
    if (cbeg < cend) pf = load_tiles<PASS_A, NP16, NPZ>(q, k, v, z, beta, s0, s1, cbeg, h, H, tid);

    // elementwise mapping: sub-chunk sc = wv & 3, channels ch0 + 64 i (i < NCH)
    constexpr int NCH = 8 / NW;
    const int sc = wv & 3;

    for (int chunk = cbeg; chunk < cend; ++chunk) {
        const int64_t t0 = s0 + (int64_t)chunk * CH;
        const int len = (int)min((int64_t)CH, s1 - t0);
        // Lane indices are re-derived from an opaque zero each chunk, so the
        // many LDS addresses built from them are recomputed (a few VALU ops)
        // instead of being hoisted out of the loop and pinned in registers.
        int zero_v;
        asm volatile("v_mov_b32 %0, 0" : "=v"(zero_v));
        const int tid = threadIdx.x + zero_v, l = tid & 63, g = l >> 4, lr = l & 15;
        const int r16 = tid >> 4, o16 = 8 * (tid & 15), r32 = tid >> 5, o32 = 4 * (tid & 31);
        const int ch0 = 64 * (wv >> 2) + l;
        __syncthreads();  // the previous chain step has finished reading LDS

        // ---- phase 0: raw tiles into LDS (z into the E1 slots it is turned into)
#pragma unroll
        for (int p = 0; p < NP16; ++p) {
            const int row = r16 + (NT_ / 16) * p;
            *(u32x4 *)&sm.b.K[row * P16 + o16] = pf.k[p];
            if constexpr (!PASS_A) *(u32x4 *)&sm.c.Q[row * P16 + o16] = pf.q[p];
            const u32x4 vw = pf.v[p];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sm.Vt[(o16 + e) * P64 + row] = __builtin_bit_cast(__bf16, (uint16_t)(vw[e >> 1] >> (16 * (e & 1))));
        }
#pragma unroll
        for (int p = 0; p < NPZ; ++p) *(f32x4 *)&sm.a.E1[(r32 + (NT_ / 32) * p) * PE + o32] = pf.z[p];
        if (wv == 0) sm.beta[l] = pf.b;
        __syncthreads();
        // the next chunk's raw tiles load while this chunk is processed
        if (chunk + 1 < cend) pf = load_tiles<PASS_A, NP16, NPZ>(q, k, v, z, beta, s0, s1, chunk + 1, h, H, tid);

        // ---- phase 1: gate and sub-chunk cumulative sums (E1 overwrites z in place)
        float gl[NCH][SUB];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int ch = ch0 + 64 * i;
            float a = 0.f;
#pragma unroll
            for (int u = 0; u < SUB; ++u) {
                const int t = sc * SUB + u;
                a += t < len ? kda_gate(eA, sm.a.E1[t * PE + ch]) : 0.f;
                gl[i][u] = a;
                sm.a.E1[t * PE + ch] = __expf(a);
            }
            sm.R[(sc + 1) * D + ch] = a;  // sub-chunk totals, prefix-summed below
        }
        __syncthreads();
        if (tid < D) {
            float r = 0.f;
            sm.R[tid] = 0.f;
#pragma unroll
            for (int s = 1; s <= 4; ++s) {
                r += sm.R[s * D + tid];
                sm.R[s * D + tid] = r;
            }
            sm.gam[tid] = __expf(r);
            sm.PF[6 * D + tid] = 1.f;
#pragma unroll
            for (int i = 1; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < i; ++jj)
                    sm.PF[(i * (i - 1) / 2 + jj) * D + tid] = __expf(sm.R[i * D + tid] - sm.R[jj * D + tid]);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NCH; ++i) {  // K~^T = (K * e^{G_n - G})^T with permuted token order
            const int ch = ch0 + 64 * i;
            const float Rs = sm.R[sc * D + ch], Gn = sm.R[4 * D + ch];
#pragma unroll
            for (int u = 0; u < SUB; u += 4) {
                f16x4 a;
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    a[m] = (_Float16)((float)sm.b.K[(sc * SUB + u + m) * P16 + ch] * __expf(Gn - Rs - gl[i][u + m]));
                *(f16x4 *)&sm.KtT[ch * P64 + perm32(sc * SUB + u)] = a;
            }
        }

        // ---- phase 2: decay-scaled Gram tiles (bf16 hi+lo on both operands).
        // Pair (i, j), j <= i, of 16-token sub-chunks: the column operand
        // k_c e^{R_i - G_c} = k_c / E1_c (* e^{R_i - R_j} for j < i) is shared by
        // Akk and Aqk; the row operands are k_r E1_r and q_r E1_r.
        for (int pix = wv; pix < 10; pix += NW) {
            int i = 0;
            while ((i + 1) * (i + 2) / 2 <= pix) ++i;
            const int jj = pix - i * (i + 1) / 2;
            const int cr = 16 * jj + lr, rr = 16 * i + lr;
            const float *pfac = &sm.PF[(jj < i ? i * (i - 1) / 2 + jj : 6) * D];
            f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int c8 = 32 * ks + 8 * g;
                const bf16x8 kc = *(const bf16x8 *)&sm.b.K[cr * P16 + c8];
                const bf16x8 kr = *(const bf16x8 *)&sm.b.K[rr * P16 + c8];
                const f32x4 ec0 = *(const f32x4 *)&sm.a.E1[cr * PE + c8];
                const f32x4 ec1 = *(const f32x4 *)&sm.a.E1[cr * PE + c8 + 4];
                const f32x4 er0 = *(const f32x4 *)&sm.a.E1[rr * PE + c8];
                const f32x4 er1 = *(const f32x4 *)&sm.a.E1[rr * PE + c8 + 4];
                F8 a, b;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float inv = __builtin_amdgcn_rcpf(e < 4 ? ec0[e] : ec1[e - 4]) * pfac[c8 + e];
                    a.v[e] = (float)kc[e] * inv;
                    b.v[e] = (float)kr[e] * (e < 4 ? er0[e] : er1[e - 4]);
                }
                const S8 as = split8(a);
                akk = mma_ss(akk, as, split8(b));
                if constexpr (!PASS_A) {
                    const bf16x8 qr = *(const bf16x8 *)&sm.c.Q[rr * P16 + c8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) b.v[e] = (float)qr[e] * (e < 4 ? er0[e] : er1[e - 4]);
                    aqk = mma_ss(aqk, as, split8(b));
                }
            }
            const int cb = 16 * jj + 4 * g;  // acc[m] = M[rr][cb + m]
            {
                float val[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) val[m] = cb + m < rr ? sm.beta[rr] * akk[m] : 0.f;
                *(f32x4 *)&sm.t.T[rr * PTT + cb] = f32x4{val[0], val[1], val[2], val[3]};
            }
            if constexpr (!PASS_A) {
                f16x4 hv, lv;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float val = cb + m <= rr ? aqk[m] : 0.f;
                    hv[m] = (_Float16)val;
                    lv[m] = (_Float16)(val - (float)hv[m]);
                }
                *(f16x4 *)&sm.AqH[rr * P64 + perm32(cb)] = hv;
                *(f16x4 *)&sm.AqL[rr * P64 + perm32(cb)] = lv;
            }
        }
        if constexpr (!PASS_A) {  // the six tiles of Aqk above the diagonal are zero
            for (int e = tid; e < 6 * 64; e += NT_) {
                const int tile = e >> 6, quad = e & 63;
                const int ti = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
                const int tj = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
                const int r = 16 * ti + (quad >> 2), cc = 16 * tj + 4 * (quad & 3);
                const f16x4 zero = {0, 0, 0, 0};
                *(f16x4 *)&sm.AqH[r * P64 + perm32(cc)] = zero;
                *(f16x4 *)&sm.AqL[r * P64 + perm32(cc)] = zero;
            }
        }
        __syncthreads();

        // ---- phase 2.5: K * Gam (transposed, bf16) and Q~ = Q * Gam (fp16, permuted)
        {
            float kg[NCH][SUB], qg[NCH][SUB];
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int ch = ch0 + 64 * i;
                const float eR = __expf(sm.R[sc * D + ch]);
#pragma unroll
                for (int u = 0; u < SUB; ++u) {
                    const int t = sc * SUB + u;
                    const float gm = eR * sm.a.E1[t * PE + ch];
                    kg[i][u] = (float)sm.b.K[t * P16 + ch] * gm;
                    if constexpr (!PASS_A) qg[i][u] = (float)sm.c.Q[t * P16 + ch] * gm;
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int ch = ch0 + 64 * i;
#pragma unroll
                for (int u = 0; u < SUB; u += 8) {
                    bf16x8 a;
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = (__bf16)kg[i][u + e];
                    *(bf16x8 *)&sm.a.KGt[ch * P64 + sc * SUB + u] = a;
                }
                if constexpr (!PASS_A) {
                    const int pc = perm32(ch);
#pragma unroll
                    for (int u = 0; u < SUB; ++u) sm.c.Qt[(sc * SUB + u) * P16 + pc] = (_Float16)qg[i][u];
                }
            }
        }

        // ---- phase 3: T = (I + Akk)^{-1}, blocked forward substitution in place
        if (wv < 4 && l < 16) {
            // lane m solves column m of diagonal block b; the block's rows are
            // read four at a time ahead of the dependent updates
            const int b = wv, m = l;
            const float *blk0 = &sm.t.T[(16 * b) * PTT + 16 * b];
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
            for (int r = 0; r < SUB; ++r) sm.t.T[(16 * b + r) * PTT + 16 * b + m] = tcol[r];
        }
        __syncthreads();
        for (int i = 1; i < 4; ++i) {
            f32x4 Xb = {0.f, 0.f, 0.f, 0.f};
            const int jb = wv;
            if (jb < i) {
                for (int kb = jb; kb < i; ++kb) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const float a = sm.t.T[(16 * i + lr) * PTT + 16 * kb + 4 * s + g];
                        const float b = sm.t.T[(16 * kb + 4 * s + g) * PTT + 16 * jb + lr];
                        Xb = mfma_f32(a, b, Xb);
                    }
                }
            }
            __syncthreads();
            if (jb < i) {
                f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) Y = mfma_f32(sm.t.T[(16 * i + lr) * PTT + 16 * i + 4 * g + s], Xb[s], Y);
#pragma unroll
                for (int m = 0; m < 4; ++m) sm.t.T[(16 * i + 4 * g + m) * PTT + 16 * jb + lr] = -Y[m];
            }
            __syncthreads();
        }

        // ---- phase 4: T diag(beta) as bf16 hi / lo (once, in place of T); W (to LDS,
        // fp16 permuted) and U (registers)
        {
            constexpr int PER = CH * CH / NT_;  // elements per thread
            float tv[PER];
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int idx = tid + NT_ * e, r = idx >> 6, cc = idx & 63;
                tv[e] = cc <= r ? sm.t.T[r * PTT + cc] * sm.beta[cc] : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int idx = tid + NT_ * e, r = idx >> 6, cc = idx & 63;
                const __bf16 hi = (__bf16)tv[e];
                sm.t.Tb[r * P64 + cc] = hi;
                sm.t.Tb[CH * P64 + r * P64 + cc] = (__bf16)(tv[e] - (float)hi);
            }
            __syncthreads();
        }
        S8 tb[4][2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int off = (16 * rt + lr) * P64 + 32 * ks + 8 * g;
                tb[rt][ks].hi = *(const bf16x8 *)&sm.t.Tb[off];
                tb[rt][ks].lo = *(const bf16x8 *)&sm.t.Tb[CH * P64 + off];
            }
#pragma unroll
        for (int cq = 0; cq < 8 / NW; ++cq) {  // W^T tiles for key channels 16 ct .. 16 ct + 15
            const int ct = (8 / NW) * wv + cq;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks > (rt >> 1)) break;
                    const bf16x8 kgf = *(const bf16x8 *)&sm.a.KGt[(16 * ct + lr) * P64 + 32 * ks + 8 * g];
                    acc = mma_1s(acc, kgf, tb[rt][ks]);
                }
                f16x4 w4;  // stored negated: the chain accumulates U - W S
#pragma unroll
                for (int m = 0; m < 4; ++m) w4[m] = (_Float16)(-acc[m]);
                *(f16x4 *)&sm.b.W[(16 * rt + lr) * P16 + perm32(16 * ct + 4 * g)] = w4;
            }
        }
        // Delta starts as U = T diag(beta) V on this wave's value columns (C layout, rows = tokens)
        f32x4 Dl[4][NCT];
        const bool has_u = !PASS_A || colw >= 128;
        const int ucol = PASS_A ? colw - 128 : colw;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (has_u) {
                    const int vcol = ucol + 16 * ct + lr;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        if (ks > (rt >> 1)) break;
                        const bf16x8 vv = *(const bf16x8 *)&sm.Vt[vcol * P64 + 32 * ks + 8 * g];
                        acc = mma_s1(acc, tb[rt][ks], vv);
                    }
                }
                Dl[rt][ct] = acc;
            }
        __syncthreads();  // W complete

        // ---- phase 5: the chain step, wave-local
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            __builtin_amdgcn_sched_barrier(0);  // one column tile at a time
            f16x8 sf[4];  // state as B operand: k-step s pairs C tiles 2s, 2s+1
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) sf[s][e] = (_Float16)X[2 * s + (e >> 2)][ct][e & 3];
            f32x4 O[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                __builtin_amdgcn_sched_barrier(0);  // bound the fragments kept in flight
                O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const f16x8 wf = *(const f16x8 *)&sm.b.W[(16 * rt + lr) * P16 + 32 * s + 8 * g];
                    Dl[rt][ct] = mfma_f16(wf, sf[s], Dl[rt][ct]);
                    if constexpr (!PASS_A) {
                        const f16x8 qf = *(const f16x8 *)&sm.c.Qt[(16 * rt + lr) * P16 + 32 * s + 8 * g];
                        O[rt] = mfma_f16(qf, sf[s], O[rt]);
                    }
                }
            }
            f16x8 dh[2], dlo[2];  // Delta as B operand (tokens), fp16 hi + lo
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float d = Dl[2 * s + (e >> 2)][ct][e & 3];
                    const _Float16 hh = (_Float16)d;
                    dh[s][e] = hh;
                    dlo[s][e] = (_Float16)(d - (float)hh);
                }
            if constexpr (!PASS_A) {
                const int col = colw + 16 * ct + lr;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        if (s > (rt >> 1)) break;
                        const f16x8 ah = *(const f16x8 *)&sm.AqH[(16 * rt + lr) * P64 + 32 * s + 8 * g];
                        const f16x8 al = *(const f16x8 *)&sm.AqL[(16 * rt + lr) * P64 + 32 * s + 8 * g];
                        O[rt] = mfma_f16(al, dh[s], O[rt]);
                        O[rt] = mfma_f16(ah, dlo[s], O[rt]);
                        O[rt] = mfma_f16(ah, dh[s], O[rt]);
                    }
                    float *orow = o + ((size_t)t0 * HD + (size_t)h * D + col);
                    const int ostride = H * D;
                    if (len == CH) {
#pragma unroll
                        for (int m = 0; m < 4; ++m) orow[(16 * rt + 4 * g + m) * ostride] = O[rt][m];
                    } else {
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            const int t = 16 * rt + 4 * g + m;
                            if (t < len) orow[t * ostride] = O[rt][m];
                        }
                    }
                }
            }
            // S <- Diag(gamma) S + K~^T Delta
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                __builtin_amdgcn_sched_barrier(0);
                f32x4 acc;
#pragma unroll
                for (int m = 0; m < 4; ++m) acc[m] = sm.gam[16 * rt + 4 * g + m] * X[rt][ct][m];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const f16x8 kf = *(const f16x8 *)&sm.KtT[(16 * rt + lr) * P64 + 32 * s + 8 * g];
                    acc = mfma_f16(kf, dlo[s], acc);
                    acc = mfma_f16(kf, dh[s], acc);
                }
                X[rt][ct] = acc;
            }
        }
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
                    dst[blk + (size_t)(16 * rt + 4 * g + m) * D + cbase + 16 * ct + lr] = X[rt][ct][m];
    } else {
        if (S_final && j == pn - 1) {
            const size_t fb = ((size_t)n * H + h) * D * D;
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        S_final[fb + (size_t)(16 * rt + 4 * g + m) * D + colw + 16 * ct + lr] = X[rt][ct][m];
        }
    }
}

// ------------------------------------------------------------------ scan --

// One workgroup per (sequence, head, 16 value columns): S_in[0] = S0 and
// S_in[p+1] = M_p S_in[p] + B_p over the sequence's segments, with exact fp32
// MFMA products (an identity transition reproduces the state bit for bit).
// An empty sequence gets S_final = S0 here.
__global__ __launch_bounds__(256) void seg_scan_kernel(const float *__restrict__ S0, int N, int H, SegTable tab,
                                                       float *__restrict__ S_final) {
    __shared__ float Ss[16 * 132];  // S^T [column][row]
    const int nh = blockIdx.x, cb = blockIdx.y;
    const int n = nh / H, h = nh % H;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, lr = l & 15;
    const int col = 16 * cb + lr;
    const int first = tab.seg_off[n], pn = tab.seg_off[n + 1] - first;
    f32x4 Sr[2];
    const size_t s0b = ((size_t)n * H + h) * D * D;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int m = 0; m < 4; ++m)
            Sr[u][m] = S0 ? S0[s0b + (size_t)(32 * w + 16 * u + 4 * g + m) * D + col] : 0.f;
    if (pn == 0) {
        if (S_final)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int m = 0; m < 4; ++m) S_final[s0b + (size_t)(32 * w + 16 * u + 4 * g + m) * D + col] = Sr[u][m];
        return;
    }
    for (int p = 0; p < pn; ++p) {
        const size_t b = ((size_t)(first + p) * H + h) * D * D;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int m = 0; m < 4; ++m) tab.Sin[b + (size_t)(32 * w + 16 * u + 4 * g + m) * D + col] = Sr[u][m];
        if (p == pn - 1) break;
#pragma unroll
        for (int u = 0; u < 2; ++u)
            *(f32x4 *)&Ss[lr * 132 + 32 * w + 16 * u + 4 * g] = Sr[u];
        __syncthreads();
        F8 sb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sb[ks] = ld_f8(&Ss[lr * 132 + 32 * ks + 8 * g]);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r0 = 32 * w + 16 * u;
            f32x4 acc;
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = tab.Bseg[b + (size_t)(r0 + 4 * g + m) * D + col];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = mma_ff(acc, ld_f8(&tab.Mseg[b + (size_t)(r0 + lr) * D + 32 * ks + 8 * g]), sb[ks]);
            Sr[u] = acc;
        }
    }
}

// ------------------------------------------------------------------ host --

constexpr int SEG_TARGET_WGS = 256;  // one workgroup per CU (LDS-bound)
#ifndef SEG_NW
#define SEG_NW 8  // waves per segment workgroup (2 per SIMD)
#endif

static inline int seg_len(int64_t T_total, int H) {
    const int64_t nc = (T_total + CH - 1) / CH;
    const int64_t per_head = SEG_TARGET_WGS / (H > 0 ? H : 1) > 0 ? SEG_TARGET_WGS / H : 1;
    int64_t L = (nc + per_head - 1) / per_head;
    return (int)(L < 1 ? 1 : L);
}
static inline int64_t seg_max(int64_t T_total, int N, int H) {
    const int L = seg_len(T_total, H);
    const int64_t nc = (T_total + CH - 1) / CH + N;
    return (nc + L - 1) / L + N;
}

size_t seg_workspace_bytes(int64_t T_total, int N, int H) {
    const size_t tab = align_up(4 * (size_t)(N + 1)) + 2 * align_up(8 * (size_t)N);
    return tab + 3 * (size_t)seg_max(T_total, N, H) * H * D * D * sizeof(float);
}

int launch_segment_prefill(const __bf16 *q, const __bf16 *k, const __bf16 *v, const float *z, const float *beta,
                           const float *A, const float *S0, const int32_t *cu, int B, int64_t T, int H, int N,
                           float *o, float *S_final, void *ws, hipStream_t stream, hipEvent_t *ev) {
    const int64_t T_total = (int64_t)B * T;
    const int L = seg_len(T_total, H);
    const int64_t nsm = seg_max(T_total, N, H);
    char *p = (char *)ws;
    SegTable tab;
    tab.seg_off = (int32_t *)p;
    p += align_up(4 * (size_t)(N + 1));
    tab.seq_start = (int64_t *)p;
    p += align_up(8 * (size_t)N);
    tab.seq_end = (int64_t *)p;
    p += align_up(8 * (size_t)N);
    const size_t st = (size_t)nsm * H * D * D;
    tab.Mseg = (float *)p;
    tab.Bseg = tab.Mseg + st;
    tab.Sin = tab.Bseg + st;
    tab.L = L;
    const size_t smem = sizeof(SegSmem);
    if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return -1;
    hipLaunchKernelGGL(seg_prep_kernel, dim3(1), dim3(256), 0, stream, cu, N, T_total, cu ? (int64_t)0 : T, tab);
    if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return -1;
    hipLaunchKernelGGL((seg_pass_kernel<true, SEG_NW>), dim3((unsigned)nsm, (unsigned)H), dim3(64 * SEG_NW), smem, stream, q, k, v, z,
                       beta, A, N, H, tab, o, S_final);
    if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return -1;
    hipLaunchKernelGGL(seg_scan_kernel, dim3((unsigned)(N * H), 8), dim3(256), 0, stream, S0, N, H, tab, S_final);
    if (ev && hipEventRecord(ev[3], stream) != hipSuccess) return -1;
    hipLaunchKernelGGL((seg_pass_kernel<false, SEG_NW>), dim3((unsigned)nsm, (unsigned)H), dim3(64 * SEG_NW), smem, stream, q, k, v,
                       z, beta, A, N, H, tab, o, S_final);
    if (hipGetLastError() != hipSuccess) return -1;
    if (ev && hipEventRecord(ev[4], stream) != hipSuccess) return -1;
    return 0;
}

int set_segment_attributes() {
    const int smem = (int)sizeof(SegSmem);
    if (hipFuncSetAttribute((const void *)seg_pass_kernel<true, SEG_NW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            smem) != hipSuccess)
        return -1;
    if (hipFuncSetAttribute((const void *)seg_pass_kernel<false, SEG_NW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            smem) != hipSuccess)
        return -1;
    return 0;
}

}  // namespace kda
