/*
 * kda.h -- C ABI of libkda.so, the MI355X (gfx950) Kimi Delta Attention operator.
 *
 * The operator (pages: "Kimi Linear: An Expressive, Efficient Attention
 * Architecture" summary, section 3; "Kimi K3 architecture", sequence-bottleneck
 * section) updates, per head, a d_k x d_v state
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 *     alpha_t = exp(g_t),  g_t = -5 * Sigmoid(exp(A_h) * z_t)   (per key channel),
 *
 * decaying first and then applying the delta-rule correction.  Prefill uses the
 * chunkwise form (Kimi Linear summary, sections 3.1 and 6.3, appendix C:
 * chunk size 64, WY / UT transform with a forward-substitution inverse, 16-token
 * sub-chunks, inter-chunk state recurrence); generation uses the recurrent
 * single-token update (section 6.3).
 *
 * Conventions shared by every entry point
 *   - Head dims are fixed: d_k = d_v = 128 (Kimi Linear summary, sections 4 and
 *     6.3).  Any other value returns KDA_ERR_SHAPE.
 *   - Every tensor pointer is a device pointer owned by the caller; the library
 *     allocates no device memory.  Its only global state is set once per
 *     process (kernel attributes) or once per GPU (the address of the
 *     workspace array of kda_chunk_fwd_noalloc), thread-safely.
 *   - Layouts are dense, row-major, innermost dimension last:
 *       q, k, z : [tokens, H, 128]   v, o : [tokens, H, 128]
 *       beta    : [tokens, H]        A    : [H]
 *       states  : [N, H, 128, 128] with rows = key channel, columns = value channel.
 *   - q, k and v are bf16 (KDA_BF16) or fp32 (KDA_F32); z, beta, A, the states
 *     and o are always fp32.
 *   - q and k are expected to be L2-normalised by the caller (the KDA layer
 *     normalises them before the operator); the operator does not normalise and
 *     applies no query scale.
 *   - beta is the final delta strength (already squashed into (0, 1)); 0 and 1
 *     are valid.
 *   - Input scale.  With bf16 q/k/v the state and Delta enter the chunk
 *     products as fp16 values; each workgroup carries its state columns at a
 *     power-of-two scale it re-picks every chunk, so o and S_final keep their
 *     accuracy for v and S0 of any magnitude whose states and outputs stay in
 *     fp32's normal range (tested from 2^-60 to 2^60 times unit scale).  That
 *     bound relies on the documented preconditions: unit-length keys and
 *     beta in [0, 1].  With fp32 q/k/v the chunk-local work is fp32 and the
 *     chain's products take fp16 hi + lo pairs (22-bit operands, fp32
 *     accumulation) under the same per-workgroup state scale and the same
 *     preconditions.  The decode step computes in fp32 throughout.
 *   - z = -inf gives alpha = 1 exactly and z = +inf gives alpha = e^-5; both are
 *     valid.  NaN inputs propagate to the outputs.
 *   - Pointers must be 16-byte aligned (KDA_ERR_ALIGN otherwise).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  Arguments are validated on the host before any launch; a
 *     launch failure returns KDA_ERR_HIP; faults during execution surface at the
 *     caller's next synchronisation.  Nothing is thrown across the ABI.
 *   - Calls on different streams are independent as long as they use distinct
 *     outputs and distinct workspaces.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

enum {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,      /* a required pointer is NULL                          */
    KDA_ERR_SHAPE = -2,     /* dk or dv != 128, or a negative / inconsistent size  */
    KDA_ERR_DTYPE = -3,     /* qkv_dtype is not a kda_dtype                        */
    KDA_ERR_SEQLENS = -4,   /* cu_seqlens given with B != 1, or n_seqs < 1         */
    KDA_ERR_ALIGN = -5,     /* a pointer is not 16-byte aligned                    */
    KDA_ERR_WORKSPACE = -6, /* workspace NULL or smaller than required             */
    KDA_ERR_HIP = -7,       /* a HIP launch failed                                 */
    KDA_ERR_ALIAS = -8      /* o overlaps an input                                 */
};

/*
 * Largest head count the prefill entry points accept (KDA_ERR_SHAPE above it;
 * the workspace size is then 0).  A chunk's rows of one input span
 * 64 x H x 512 bytes, which the kernels address with 32-bit buffer offsets.
 */
#define KDA_MAX_HEADS 16384

/* Human-readable name of a status code (static storage, never NULL). */
const char *kda_status_str(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int kda_version(void);

/*
 * Bytes of device workspace kda_chunk_fwd needs for T_total packed tokens in
 * n_seqs sequences, H heads and the given q/k/v dtype (0 for an empty problem
 * or invalid sizes).  It holds a sequence / segment table, the per-chunk
 * operands of the chain (78,848 B per chunk and head with bf16 q/k/v, 147,968 B
 * with fp32) and, per (segment, head), the segment's state transition, its
 * state offset and its incoming state (3 x 64 KiB): about 1.35 GB for 64K
 * tokens x 16 heads with bf16 q/k/v, 2.45 GB with fp32.  Contents are scratch
 * between calls.
 */
size_t kda_chunk_fwd_workspace_bytes(int64_t T_total, int32_t n_seqs, int32_t H, kda_dtype qkv_dtype);

/*
 * Chunkwise KDA prefill (Kimi Linear summary, sections 3.1 and 6.3; appendix C
 * chunk_kda(q, k, v, g, beta, initial_state, chunk_size=64), here with the
 * Kimi K3 gate fused: the operator takes z and A instead of g).
 *
 * Sequences:
 *   cu_seqlens == NULL: B sequences of T tokens each; tensors are [B, T, H, 128]
 *                       and n_seqs must equal B.
 *   cu_seqlens != NULL: B must be 1; the token axis packs n_seqs sequences;
 *                       cu_seqlens is a DEVICE int32 array of n_seqs + 1
 *                       offsets, cu_seqlens[0] = 0, non-decreasing,
 *                       cu_seqlens[n_seqs] = T.  Its contents are not read on
 *                       the host: offsets outside [0, T] are clamped and a
 *                       decreasing entry gives an empty sequence, so malformed
 *                       offsets give wrong results but never out-of-bounds
 *                       accesses.
 *   Each sequence starts from its own initial state and its chunk grid starts
 *   at its first token; its last chunk may be partial.  Zero-length sequences
 *   are allowed (S_final = S0).
 *
 * Arguments:
 *   q, k, v     [B*T, H, 128] of qkv_dtype          (input)
 *   g_raw       [B*T, H, 128] fp32, z of the gate    (input)
 *   beta        [B*T, H] fp32                        (input)
 *   A           [H] fp32, the gate uses exp(A[h])    (input)
 *   S0          [n_seqs, H, 128, 128] fp32 or NULL (= zeros)            (input)
 *   o           [B*T, H, 128] fp32; must not overlap any input         (output)
 *   S_final     [n_seqs, H, 128, 128] fp32 or NULL; may alias S0       (output)
 *   workspace   device scratch of workspace_bytes >=
 *               kda_chunk_fwd_workspace_bytes(B*T, n_seqs, H, qkv_dtype)
 *   stream      hipStream_t
 */
int kda_chunk_fwd(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                  const float *g_raw, const float *beta, const float *A, const float *S0,
                  const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t n_seqs,
                  int32_t dk, int32_t dv, float *o, float *S_final, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * kda_chunk_fwd with stage timing: when stage_events is not NULL it points to
 * six hipEvent_t created by the caller; they are recorded on `stream` at the
 * boundaries of the library's five stages, so the caller can read each
 * stage's duration with hipEventElapsedTime.  bf16 q/k/v: [sequence table,
 * intra-chunk WY / UT operands, segment transitions (pass A), segment scan,
 * segment outputs (pass B)]; fp32 q/k/v: [chunk table, intra-chunk kernel,
 * chain kernel, (empty), (empty)].  Everything else is as kda_chunk_fwd.
 * A failing hipEventRecord returns KDA_ERR_HIP.
 */
int kda_chunk_fwd_timed(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                        const float *g_raw, const float *beta, const float *A, const float *S0,
                        const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t n_seqs,
                        int32_t dk, int32_t dv, float *o, float *S_final, void *workspace,
                        size_t workspace_bytes, void *stream, void *const *stage_events);

/*
 * kda_chunk_fwd without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a device-resident array of
 * KDA_NOALLOC_WORKSPACE_BYTES inside the library, one per GPU, held from the
 * first call on that GPU until the process ends; the call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).  A problem whose
 * kda_chunk_fwd_workspace_bytes exceeds KDA_NOALLOC_WORKSPACE_BYTES returns
 * KDA_ERR_WORKSPACE: with bf16 q/k/v and 16 heads up to 4,544 tokens fit
 * (2,048 tokens x 16 heads need 62 MB).  The GPU is the stream's
 * (hipStreamGetDevice); its first call takes the array's address with
 * hipGetSymbolAddress (KDA_ERR_HIP if that fails).
 *
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (nothing in it needs to start at zero): calls that overlap in time
 * on one GPU, on different streams or from different threads, race and give
 * wrong results.  Serialise them (one stream, or events).  Everything else
 * (arguments, validation, results: the same bits) is as kda_chunk_fwd.
 */
#define KDA_NOALLOC_WORKSPACE_BYTES (128u << 20)
int kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                          const float *g_raw, const float *beta, const float *A, const float *S0,
                          const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t n_seqs,
                          int32_t dk, int32_t dv, float *o, float *S_final, void *stream);

/*
 * kda_chunk_fwd that also keeps state snapshots for a KDA-aware prefix cache
 * (Kimi K3 paper review, Significance and Limitations paragraphs: the KDA
 * recurrent state can be checkpointed only at sparse boundaries, up to 6,144
 * tokens apart, and a unified prefix cache pages these checkpoints beside the
 * MLA KV blocks).
 *
 *   ckpt_stride    tokens between snapshots: a positive multiple of 64 (the
 *                  chunk size), else KDA_ERR_SHAPE.
 *   S_ckpt         [ckpt_capacity, H, 128, 128] fp32 (output; must not overlap
 *                  any other argument, else KDA_ERR_ALIAS; NULL gives
 *                  KDA_ERR_NULL).  Snapshot m of sequence n (m = 0, 1, ...,
 *                  floor(len_n / ckpt_stride) - 1) is the state after the
 *                  sequence's first (m + 1) * ckpt_stride tokens, the state a
 *                  later call would take as S0 to continue from there.  It is
 *                  stored at slot off_n + m, where off_n = sum over sequences
 *                  i < n of floor(len_i / ckpt_stride): sequence after
 *                  sequence, in order.  A sequence shorter than the stride has
 *                  none; one whose length is a multiple of the stride has its
 *                  last snapshot equal to its S_final.
 *   ckpt_capacity  slots in S_ckpt.  Slots at or past it are not written (the
 *                  library does not read cu_seqlens on the host, so the caller,
 *                  who knows the lengths, sizes S_ckpt); 0 writes nothing.
 *
 * o, S_final and everything else are exactly as kda_chunk_fwd (the same bits).
 */
int kda_chunk_fwd_ckpt(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                       const float *g_raw, const float *beta, const float *A, const float *S0,
                       const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t n_seqs,
                       int32_t dk, int32_t dv, float *o, float *S_final, float *S_ckpt, int64_t ckpt_stride,
                       int64_t ckpt_capacity, void *workspace, size_t workspace_bytes, void *stream);
/*
 * The KDA layer's steps on either side of the operator, fused into the prefill
 * (Kimi Linear summary, section 4: queries and keys are normalised to unit
 * length; the output gets a per-head RMSNorm and then a data-dependent sigmoid
 * output gate).  Values are device pointers owned by the caller.
 *
 *   qk_l2norm    nonzero: q and k are raw; each (token, head) row x of 128
 *                values is used as x / sqrt(sum_j x_j^2 + qk_eps).
 *   out_gate     [tokens, H, 128] fp32, the output gate's pre-activation (the
 *                caller's low-rank projection), or NULL for no output step.
 *                With it, each output row becomes
 *                o / sqrt(mean_j o_j^2 + norm_eps) * norm_weight * sigmoid(out_gate).
 *   norm_weight  [128] fp32, the RMSNorm weight shared by all heads (required
 *                with out_gate).
 *   qk_eps, norm_eps  >= 0 (else KDA_ERR_SHAPE); 1e-6 is a usual choice.
 *   gate_kind    the decay parameterisation (else KDA_ERR_SHAPE):
 *                KDA_GATE_K3: g = -5 * Sigmoid(exp(A_h) z), the lower-bounded
 *                  gate of the operator above (Kimi K3 architecture,
 *                  sequence-bottleneck section);
 *                KDA_GATE_SOFTPLUS: g = -exp(A_h) softplus(z), Kimi Linear's
 *                  unbounded negative-softplus decay that the bound replaces
 *                  (Kimi K3 architecture, sequence-bottleneck section; K3 paper review, Method).
 *                  With no lower bound on g the 16 x 16 diagonal Gram tiles
 *                  are formed position pair by position pair instead of on
 *                  MFMA, which costs the prefill time.  z = -inf gives g = 0;
 *                  a step's g is floored at -104 (alpha = e^-104 is below
 *                  fp32's smallest subnormal, so it acts as 0, which z = +inf
 *                  gives); NaN propagates.
 *   gate_per_head  nonzero: g_raw is [tokens, H], one value per (token, head)
 *                applied to all 128 key channels (the scalar per-head gate of
 *                Gated DeltaNet that KDA refines channel-wise, Kimi Linear
 *                summary, section 3).  Zero: g_raw is [tokens, H, 128].
 *   reverse_order  decode only (the prefill rejects nonzero with
 *                KDA_ERR_SHAPE): nonzero visits the (sequence, head) states
 *                last to first.  The results are the same bits either way.
 *                (The state stores are non-temporal, so the order has no
 *                effect on the speed of consecutive steps.)
 *   gate_u, gate_w, gate_rank  the forget gate's low-rank projection (Kimi
 *                Linear summary, section 4), fused in: with gate_u set, z is
 *                not read from g_raw (which may be NULL) but formed as
 *                z[t, h, c] = sum_j gate_u[t, j] * gate_w[h, c, j], with
 *                gate_u [tokens, gate_rank] and gate_w [H, 128, gate_rank],
 *                both bf16 (KDA_ERR_NULL if gate_w is NULL).  gate_rank is a
 *                multiple of 32 in [32, 256] (KDA_ERR_SHAPE otherwise, and
 *                with gate_per_head).  The decay is then gate_kind's, as with
 *                a given z.  Both must be 16-byte aligned and must not overlap o.
 */
enum { KDA_GATE_K3 = 0, KDA_GATE_SOFTPLUS = 1 };
typedef struct kda_layer_opts {
    int32_t qk_l2norm;
    float qk_eps;
    const float *out_gate;
    const float *norm_weight;
    float norm_eps;
    int32_t gate_kind;
    int32_t gate_per_head;
    int32_t reverse_order;
    const void *gate_u;
    const void *gate_w;
    int32_t gate_rank;
} kda_layer_opts;
/*
 * kda_chunk_fwd with the layer's steps fused in (opts, NULL gives KDA_ERR_NULL)
 * and optional state snapshots (S_ckpt may be NULL; otherwise as
 * kda_chunk_fwd_ckpt).  o holds the gated, normalised output when
 * opts->out_gate is set; S_final and the snapshots are the operator's states
 * either way.  out_gate and norm_weight must not overlap o (KDA_ERR_ALIAS) and
 * must be 16-byte aligned.
 */
int kda_chunk_fwd_layer(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                        const float *g_raw, const float *beta, const float *A, const float *S0,
                        const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t n_seqs,
                        int32_t dk, int32_t dv, const kda_layer_opts *opts, float *o, float *S_final,
                        float *S_ckpt, int64_t ckpt_stride, int64_t ckpt_capacity, void *workspace,
                        size_t workspace_bytes, void *stream);
/*
 * One recurrent decode step for N independent sequences (Kimi Linear summary,
 * section 6.3: generation uses the recurrent update; each head keeps a fixed
 * 128 x 128 state).  For every (n, h): alpha from z, S' = Diag(alpha) S,
 * delta = beta (v - S'^T k), S <- S' + k delta^T, o = S^T q.  S is read and
 * written once, in place.
 *
 *   q, k, v  [N, H, 128] of qkv_dtype; g_raw [N, H, 128] fp32; beta [N, H] fp32;
 *   A [H] fp32; S [N, H, 128, 128] fp32 (in/out); o [N, H, 128] fp32 (output,
 *   must not overlap S or an input).
 */
int kda_decode_step(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                    const float *g_raw, const float *beta, const float *A, float *S, int32_t N,
                    int32_t H, int32_t dk, int32_t dv, float *o, void *stream);
/*
 * kda_decode_step with the layer's steps and gate options of kda_layer_opts
 * (opts, NULL gives KDA_ERR_NULL): q and k normalised to unit length inside
 * (qk_l2norm), o returned as RMSNorm(o) * norm_weight * sigmoid(out_gate)
 * (out_gate [N, H, 128] fp32, or NULL), the decay chosen by gate_kind, and
 * g_raw of [N, H] when gate_per_head is set.  The state update is the
 * operator's own either way; the same validation as kda_decode_step, plus the
 * option checks of kda_chunk_fwd_layer.
 */
int kda_decode_step_layer(const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
                          const float *g_raw, const float *beta, const float *A, float *S, int32_t N,
                          int32_t H, int32_t dk, int32_t dv, const kda_layer_opts *opts, float *o,
                          void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
