// kda_decode.hip -- single-token recurrent KDA update (Kimi Linear summary,
// section 6.3: generation uses the recurrent update; each head keeps a fixed
// 128 x 128 state), with the Kimi K3 lower-bounded gate or one of its variants
// (the unbounded softplus decay, one gate value per head), and optionally the
// KDA layer's q/k normalisation and gated output RMSNorm.
//
// One workgroup of 256 threads per (sequence, head).  The 64 KiB fp32 state is
// streamed from HBM once and written back once, with non-temporal stores:
//   wave w owns key rows [32w, 32w+32); lane l owns columns 4*(l&31)..+3 of the
//   rows 32w + 2m + (l>>5), m = 0..15 (16 float4 per lane, held in registers).
// Per head: alpha = exp(g(z)); S' = Diag(alpha) S; p = S'^T k and r = S'^T q
// (partial sums per lane, reduced across the two row parities by a lane swap
// and across the four waves through LDS); delta = beta (v - p);
// o = r + (k.q) delta (= S_new^T q); S_new = S' + k delta^T.
#include "kda_common.hpp"

namespace kda {

template <typename IO>
__global__ __launch_bounds__(256) void decode_kernel(const IO *__restrict__ q, const IO *__restrict__ k,
                                                     const IO *__restrict__ v, const float *__restrict__ z,
                                                     const float *__restrict__ beta,
                                                     const float *__restrict__ A, float *__restrict__ S,
                                                     int H, float *__restrict__ o, Layer ly) {
    // n * H + h; in reverse order the sweep starts with the states that a
    // forward step before it wrote last (still in the last-level cache)
    const int nh = ly.reverse_order ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
    const int h = nh % H;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int cg = l & 31, rp = l >> 5;

    __shared__ float s_alpha[D], s_k[D], s_q[D], s_v[D];
    __shared__ float s_p[4][D], s_r[4][D];
    __shared__ float s_delta[D];
    __shared__ float s_kq[4];  // k . q, then (qk_norm) the inverse norms of k and q
    __shared__ float s_on[2];  // (output step) the two waves' sums of o^2

    float *Sh = S + (size_t)nh * D * D;
    float4 st[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int i = 32 * w + 2 * m + rp;
        st[m] = *(const float4 *)(Sh + (size_t)i * D + 4 * cg);
    }

    const size_t vec = (size_t)nh * D;
    if (tid < D) {
        const float eA = __expf(A[h]);
        float zv;
        if (ly.zu) {  // low-rank forget gate: z = sum_j u[n, j] W[h, c, j]
            const int r = ly.zrank;
            const __bf16 *ur = ly.zu + (size_t)(nh / H) * r, *wr = ly.zw + ((size_t)h * D + tid) * r;
            float acc = 0.f;
            for (int j = 0; j < r; ++j) acc += (float)ur[j] * (float)wr[j];
            zv = acc;
        } else {
            zv = ly.gate_per_head ? z[nh] : z[vec + tid];
        }
        s_alpha[tid] = __expf(ly.gate_kind == GATE_SOFTPLUS ? softplus_gate(eA, zv) : kda_gate(eA, zv));
        s_k[tid] = to_f(k[vec + tid]);
        s_q[tid] = to_f(q[vec + tid]);
        s_v[tid] = to_f(v[vec + tid]);
    }
    __syncthreads();
    if (w == 0) {  // k . q over the 128 channels (and |k|^2, |q|^2 for the layer's normalisation)
        float kq = s_k[l] * s_q[l] + s_k[l + 64] * s_q[l + 64];
        float kk = s_k[l] * s_k[l] + s_k[l + 64] * s_k[l + 64], qq = s_q[l] * s_q[l] + s_q[l + 64] * s_q[l + 64];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            kq += __shfl_xor(kq, off);
            kk += __shfl_xor(kk, off);
            qq += __shfl_xor(qq, off);
        }
        if (l == 0) {
            // unit-length k and q enter as the scale factors nk, nq: p and r are
            // linear in k and q, and k enters the update as nk k
            const float nk = ly.qk_norm ? 1.f / __fsqrt_rn(kk + ly.qk_eps) : 1.f;
            const float nq = ly.qk_norm ? 1.f / __fsqrt_rn(qq + ly.qk_eps) : 1.f;
            s_kq[0] = kq * nk * nq;
            s_kq[1] = nk;
            s_kq[2] = nq;
        }
    }

    float p[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int i = 32 * w + 2 * m + rp;
        const float a = s_alpha[i], ki = s_k[i], qi = s_q[i];
        st[m].x *= a; st[m].y *= a; st[m].z *= a; st[m].w *= a;
        p[0] += ki * st[m].x; p[1] += ki * st[m].y; p[2] += ki * st[m].z; p[3] += ki * st[m].w;
        r[0] += qi * st[m].x; r[1] += qi * st[m].y; r[2] += qi * st[m].z; r[3] += qi * st[m].w;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        p[c] += __shfl_xor(p[c], 32);
        r[c] += __shfl_xor(r[c], 32);
    }
    if (rp == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s_p[w][4 * cg + c] = p[c];
            s_r[w][4 * cg + c] = r[c];
        }
    }
    __syncthreads();
    float oj = 0.f;
    if (tid < D) {
        const float pj = (s_p[0][tid] + s_p[1][tid] + s_p[2][tid] + s_p[3][tid]) * s_kq[1];
        const float rj = (s_r[0][tid] + s_r[1][tid] + s_r[2][tid] + s_r[3][tid]) * s_kq[2];
        const float dj = beta[nh] * (s_v[tid] - pj);
        s_delta[tid] = dj;
        oj = rj + s_kq[0] * dj;
        if (ly.gate) {
            float s2 = oj * oj;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) s2 += __shfl_xor(s2, off);
            if (l == 0) s_on[w] = s2;
        } else {
            o[vec + tid] = oj;
        }
    }
    __syncthreads();
    if (ly.gate && tid < D) {  // the layer's output step: RMSNorm over the head, then the sigmoid gate
        const float rn = 1.f / __fsqrt_rn((s_on[0] + s_on[1]) * (1.f / D) + ly.norm_eps);
        const float gs = 1.f / (1.f + __expf(-ly.gate[vec + tid]));
        o[vec + tid] = oj * rn * ly.weight[tid] * gs;
    }
    const float4 dl = *(const float4 *)(s_delta + 4 * cg);
    const float nk = s_kq[1];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int i = 32 * w + 2 * m + rp;
        const float ki = s_k[i] * nk;
        float4 x = st[m];
        x.x += ki * dl.x; x.y += ki * dl.y; x.z += ki * dl.z; x.w += ki * dl.w;
        // non-temporal: the state is next read a whole step later, after the
        // other heads' states have passed through the caches
        __builtin_nontemporal_store(f32x4{x.x, x.y, x.z, x.w}, (f32x4 *)(Sh + (size_t)i * D + 4 * cg));
    }
}

int launch_decode(const void *q, const void *k, const void *v, bool f32io, const float *z,
                  const float *beta, const float *A, float *S, int N, int H, float *o, const Layer &ly,
                  hipStream_t stream) {
    const unsigned blocks = (unsigned)N * (unsigned)H;
    if (blocks == 0) return 0;
    if (f32io)
        hipLaunchKernelGGL(decode_kernel<float>, dim3(blocks), dim3(256), 0, stream, (const float *)q,
                           (const float *)k, (const float *)v, z, beta, A, S, H, o, ly);
    else
        hipLaunchKernelGGL(decode_kernel<__bf16>, dim3(blocks), dim3(256), 0, stream, (const __bf16 *)q,
                           (const __bf16 *)k, (const __bf16 *)v, z, beta, A, S, H, o, ly);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kda
