/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) hot path.
 *
 * What is computed.  Per (sequence, head) a fixed d_k x d_v fp32 state S is carried
 * through the tokens.  Each token t applies a per-channel decay and then a
 * beta-weighted erase-and-write, and reads the output from the updated state:
 *
 *     gt_t = min(0, max(-5, g_t))                 per key channel (floor at -5)
 *     S'   = Diag(exp(gt_t)) S                    decay the key rows of S
 *     u_t  = beta_t (v_t - S'^T k_t)              erase what S' recalls for k_t
 *     S    = S' + k_t u_t^T                       write
 *     o_t  = S^T q_t                              read after the write
 *
 * and optionally  out_t = o_t / sqrt(mean_j o_tj^2 + eps) * w * sigmoid(gate_t).
 *
 * Sources (web pages on Kimi K3; none prints the formulas, see the design notes for
 * the readings taken):
 *   [R] "xhh.club" tag page 结构, entry on KDA's recurrent form: per-channel decay and
 *       erase-and-write into a 128x128 per-head state independent of context length;
 *       per-head RMSNorm and a full-rank sigmoid output gate.
 *   [C] same page, entry on the chunkwise-parallel algorithm: chunks linked by a
 *       state recurrence and computed inside with matrix products; the -5 floor on
 *       each step's log-decay lets the 16-token diagonal tiles run as BF16 matmul;
 *       training/prefill use the chunkwise form, decode the recurrent form.
 *   [S] same page, entry on the structure's system implications: three execution
 *       forms (fast kernel, intra-device context parallelism, state rollback);
 *       context parallelism decomposes by an associative prefix scan, never by
 *       adding states; the prefix cache reuses state at 512-token boundaries.
 *   [G] "nlpx.cn" Kimi K3 reading guide, section 6: KCP passes segment transitions;
 *       why the floor is -5 and why the reciprocal cumulative decay overflows
 *       without it; why per-rank states cannot be summed; why the prefix cache
 *       needs KDA checkpoints.
 *
 * Conventions for every entry point.
 *   - All data pointers are DEVICE pointers on the current HIP device, owned by
 *     the caller.  The library allocates nothing and keeps no pointer after
 *     returning.
 *   - Layouts are dense row-major: activations token-major [B, T, H, d], states
 *     [B, H, d_k, d_v] (row = key channel, column = value channel).
 *   - Argument errors are reported synchronously and nothing is launched.  Work
 *     is enqueued asynchronously on `stream`; faults surface at the caller's
 *     synchronisation.  A launch failure returns KDA_ERR_HIP.  No C++ exception
 *     crosses this boundary.
 *   - Only gfx950 devices are supported (KDA_ERR_DEVICE otherwise).
 *   - Calls are thread-safe; calls that share output buffers must be ordered by
 *     the caller.
 *   - Supported shapes: d_k = d_v = 128.
 *   - NaN/Inf in inputs propagate; the library does not scrub them.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 3

#if defined(__GNUC__) || defined(__clang__)
#define KDA_API __attribute__((visibility("default")))
#else
#define KDA_API
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,         /* a required pointer is NULL */
  KDA_ERR_SHAPE = 2,        /* a size is negative or inconsistent */
  KDA_ERR_UNSUPPORTED = 3,  /* valid but not implemented (d != 128, chunk, dtype) */
  KDA_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required */
  KDA_ERR_ALIAS = 5,        /* an output overlaps an input it must not overlap */
  KDA_ERR_DEVICE = 6,       /* current device is not gfx950 or cannot be queried */
  KDA_ERR_HIP = 7           /* a HIP launch failed */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/*
 * Chunkwise prefill ([C]; the chunkwise form is the prefill form).  Processes T
 * tokens of B independent sequences and H heads from state S0, writing o for
 * every token and the final state.
 *
 * Numerics.  in_dtype = KDA_BF16: the 16-token diagonal tiles of the intra-chunk
 * products run as BF16 MFMA (operands split into bf16 high and low parts), the
 * remaining products as fp16 MFMA, all with fp32 accumulation; the state is kept
 * in fp32.  fp16 ends at 65504 while bf16 values and the fp32 state reach far
 * beyond it: the operands that carry values (v, the state copy and the delta-rule
 * update u) are scaled, per 16 state columns and chunk, by a power of two that
 * keeps their largest magnitude below 2^9 (scale 1, no effect, while everything
 * is already below), and results are scaled back; any finite bf16 v and fp32 S0
 * give finite results with the same relative accuracy (tested up to |v| ~ 3e6 and
 * |S0| ~ 1e6).  The other fp16 operands are built from q, k, g and beta alone and
 * are bounded by 1 when q and k have unit L2 norm per head and token, as the
 * method prescribes (beta in [0, 1]); inputs that violate this are outside the
 * supported range, not detected, and may overflow.
 * in_dtype = KDA_F32: every product runs as fp32 MFMA.
 */
typedef struct kda_prefill_desc {
  int32_t B, T, H;          /* T >= 0; any T (a ragged last chunk is handled) */
  int32_t d_k, d_v;         /* must be 128 */
  int32_t chunk;            /* 16 or 64 tokens per chunk (16 when in_dtype = KDA_F32) */
  int32_t in_dtype;         /* kda_dtype of q, k, v and gate */
  int32_t out_dtype;        /* kda_dtype of o */
  const void *q;            /* [B,T,H,d_k] */
  const void *k;            /* [B,T,H,d_k] */
  const void *v;            /* [B,T,H,d_v] */
  const float *g;           /* [B,T,H,d_k] per-channel log-decay; clamped to [-5, 0] */
  const float *beta;        /* [B,T,H] write strength, used as given */
  const float *S0;          /* [B,H,d_k,d_v] initial state, or NULL for zeros */
  float *S_final;           /* [B,H,d_k,d_v] final state, or NULL; may equal S0 */
  void *o;                  /* [B,T,H,d_v]; must not overlap any input */
  const void *gate;         /* [B,T,H,d_v] gate logits, or NULL: then o is raw S^T q */
  const float *norm_weight; /* [d_v] RMSNorm weight, or NULL for ones (gate only) */
  float norm_eps;           /* RMSNorm epsilon (gate only), e.g. 1e-6 */
  int32_t ckpt_every;       /* 0, or a multiple of chunk: checkpoint period in tokens */
  float *ckpt;              /* [B, T/ckpt_every, H, d_k, d_v]: state after the first
                               m*ckpt_every tokens, m = 1..T/ckpt_every ([S]: 512) */
  int32_t n_segments;       /* 0 = choose; 1 = one pass; >1 = split every sequence into
                               that many segments combined by an associative scan of
                               their state maps ([S], [G]) */
  int32_t v_split;          /* 0 = choose (1); 1 or 2 workgroups per (seq, head)
                               splitting the d_v columns of the state */
  void *workspace;          /* device scratch of kda_prefill_workspace_size() bytes:
                               per-chunk records (61 KiB per 64-token chunk and head),
                               plus segment maps and raw outputs when used */
  size_t workspace_bytes;
} kda_prefill_desc;

/* Bytes of workspace kda_prefill_chunked needs for this descriptor (pointers are
 * not read).  Returns the same argument errors as kda_prefill_chunked. */
KDA_API kda_status kda_prefill_workspace_size(const kda_prefill_desc *d, size_t *bytes);

/* Enqueue the prefill.  Errors: NULL (q/k/v/g/beta/o, or ckpt when ckpt_every > 0,
 * or workspace when one is needed), SHAPE (negative sizes, ckpt_every not a
 * multiple of chunk, n_segments > number of chunks, 2^31 or more (sequence, head,
 * chunk) triples), UNSUPPORTED (d != 128, chunk
 * not 16/64, bad dtype, v_split not 0/1/2), WORKSPACE, ALIAS (o overlapping an
 * input, or S_final overlapping an input other than S0), DEVICE, HIP. */
KDA_API kda_status kda_prefill_chunked(const kda_prefill_desc *d, hipStream_t stream);

/*
 * The prefill for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not allocate, harnesses that forbid it.  The same
 * computation and kernels as kda_prefill_chunked; d->workspace and d->workspace_bytes
 * are ignored.  The workspace is a fixed array of KDA_NOALLOC_WORKSPACE_BYTES in device
 * memory, one per GPU, reserved when the library is loaded and held until the process
 * ends; its device address is looked up on a device's first call.  The call allocates
 * nothing and needs no zeroed memory (every byte of workspace it reads, it first
 * writes).  Calls on one GPU share that array: calls that overlap in time on one GPU
 * (two streams, or two host threads) race and give wrong results; order them.
 * Errors: as kda_prefill_chunked, and KDA_ERR_WORKSPACE when the descriptor needs more
 * workspace than the array holds (kda_prefill_workspace_size() bytes; the records take
 * 61 KiB per 64-token chunk and head).
 */
#define KDA_NOALLOC_WORKSPACE_BYTES (64u << 20)
KDA_API kda_status kda_prefill_chunked_noalloc(const kda_prefill_desc *d, hipStream_t stream);

/*
 * One recurrent decode step ([C]: decode uses the recurrent form; [R]) for N
 * independent sequences and H heads: every state is read and written once, in
 * place.  fp32 arithmetic throughout.
 */
typedef struct kda_decode_desc {
  int32_t N, H;             /* N >= 0 sequences */
  int32_t d_k, d_v;         /* must be 128 */
  int32_t in_dtype;         /* kda_dtype of q, k, v and gate */
  int32_t out_dtype;        /* kda_dtype of o */
  const void *q;            /* [N,H,d_k] */
  const void *k;            /* [N,H,d_k] */
  const void *v;            /* [N,H,d_v] */
  const float *g;           /* [N,H,d_k] log-decay; clamped to [-5, 0] */
  const float *beta;        /* [N,H] */
  float *state;             /* [N,H,d_k,d_v] fp32, updated in place */
  void *o;                  /* [N,H,d_v]; must not overlap any input or the state */
  const void *gate;         /* [N,H,d_v] or NULL (then o is raw S^T q) */
  const float *norm_weight; /* [d_v] or NULL */
  float norm_eps;
} kda_decode_desc;

/* Errors: NULL, SHAPE (negative sizes, N * H of 2^31 or more), UNSUPPORTED, ALIAS,
 * DEVICE, HIP as for the prefill. */
KDA_API kda_status kda_decode_step(const kda_decode_desc *d, hipStream_t stream);

/*
 * Serving: one decode step for a batch whose states live in a pool of slots ([S]:
 * the serving path keeps per-sequence states; this is kda_decode_step with an
 * indirection).  d->state is the pool, [pool_size, H, d_k, d_v] fp32.  Sequence n of
 * the batch (its rows of q, k, v, g, beta, gate and o, laid out [N, H, ...] as in
 * kda_decode_desc) reads and updates, in place, the states of slot slots[n].
 * slots: DEVICE array of N int32, distinct (two sequences on one slot race).  A slot
 * outside [0, pool_size) is not visible to the host: that sequence's o row is NaN
 * and the pool is not touched for it.  Slots no sequence names are not touched.
 * Errors: as kda_decode_step, plus NULL (slots when N * H > 0), SHAPE
 * (pool_size < 0), and ALIAS when the pool overlaps o or an input.
 */
KDA_API kda_status kda_decode_step_pooled(const kda_decode_desc *d, const int32_t *slots,
                                          int32_t pool_size, hipStream_t stream);

/*
 * State checkpoint and rollback ([S]: state rollback is one of KDA's execution
 * forms; the prefix cache keeps checkpoints).  Both copy n_states fp32 states of
 * d_k x d_v on the stream: checkpoint ckpt[i] = state[i], rollback
 * state[i] = ckpt[i].  The two buffers must not overlap (KDA_ERR_ALIAS).
 * n_states = 0 is a no-op.  Errors: NULL, SHAPE (n_states < 0, d_k or d_v < 1),
 * ALIAS, DEVICE, HIP.
 */
KDA_API kda_status kda_state_checkpoint(const float *state, float *ckpt, int64_t n_states, int32_t d_k,
                                int32_t d_v, hipStream_t stream);
KDA_API kda_status kda_state_rollback(float *state, const float *ckpt, int64_t n_states, int32_t d_k,
                              int32_t d_v, hipStream_t stream);

/*
 * Indexed state copy (serving: prefix-cache reuse from 512-token checkpoints, moving
 * states in and out of a pool, write-back to host; [S]).  For i < n:
 *     dst[dst_slots[i]] = src[src_slots[i]]
 * where each element is one state of state_elems fp32 values (for instance
 * H * d_k * d_v, all heads of a sequence; a prefill's checkpoints
 * [B, T/ckpt_every, H, d_k, d_v] are B * T/ckpt_every such states).  A NULL slot
 * array means slot i.  dst holds dst_count states and src holds src_count; a pair
 * with a slot outside its array is skipped.  dst and src are device memory or
 * pinned host memory the device can access (hipHostMalloc), so write-back to host
 * is this call with a host dst.  Slot arrays are DEVICE arrays of n int32.  The
 * copies run in parallel: destinations must be distinct and no destination may be a
 * source of the same call.  Errors: NULL (dst or src when n > 0 and
 * state_elems > 0), SHAPE (a negative size, n above a count whose slot array is
 * NULL, or more than 2^31 workgroups), DEVICE, HIP.
 */
KDA_API kda_status kda_state_copy_indexed(float *dst, const int32_t *dst_slots, int64_t dst_count,
                                          const float *src, const int32_t *src_slots,
                                          int64_t src_count, int64_t n, int64_t state_elems,
                                          hipStream_t stream);

/*
 * Gradients of the chunkwise prefill (training: [C] says the chunkwise form serves
 * training as well as prefill).  Given dO = dL/do for the raw outputs o = S^T q of
 * every token (before any norm or gate) and dS_final = dL/dS_T for the final state,
 * computes dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta and dL/dS0 of the recurrence above.
 * The gradient of g is zero where the clamp to [-5, 0] is active (g < -5 or g > 0)
 * and passes at the two bounds.  fp32 arithmetic throughout (fp32 MFMA); every
 * gradient is fp32.
 */
typedef struct kda_backward_desc {
  int32_t B, T, H;          /* T >= 0; any T (a ragged last chunk is handled) */
  int32_t d_k, d_v;         /* must be 128 */
  int32_t chunk;            /* must be 64 */
  int32_t in_dtype;         /* kda_dtype of q, k, v (as given to the prefill) */
  const void *q;            /* [B,T,H,d_k] */
  const void *k;            /* [B,T,H,d_k] */
  const void *v;            /* [B,T,H,d_v] */
  const float *g;           /* [B,T,H,d_k] log-decay as given to the prefill */
  const float *beta;        /* [B,T,H] */
  const float *S0;          /* [B,H,d_k,d_v] initial state, or NULL for zeros */
  const float *dO;          /* [B,T,H,d_v] fp32 gradient of the raw outputs */
  const float *dS_final;    /* [B,H,d_k,d_v] gradient of the final state, or NULL (zeros) */
  float *dq, *dk;           /* [B,T,H,d_k] */
  float *dv;                /* [B,T,H,d_v] */
  float *dg;                /* [B,T,H,d_k] */
  float *dbeta;             /* [B,T,H] */
  float *dS0;               /* [B,H,d_k,d_v], or NULL when not wanted */
  void *workspace;          /* device scratch of kda_backward_workspace_size() bytes:
                               368.5 KiB per 64-token chunk and head (chunk
                               quantities, the state and its gradient at every chunk
                               boundary, and the chunk's dL/dU) */
  size_t workspace_bytes;
} kda_backward_desc;

/* Bytes of workspace kda_prefill_backward needs (pointers are not read).  Returns the
 * same size errors as kda_prefill_backward. */
KDA_API kda_status kda_backward_workspace_size(const kda_backward_desc *d, size_t *bytes);

/* Enqueue the backward pass.  Errors: NULL (an input, dO or a gradient output when
 * B*T*H > 0; workspace), SHAPE (negative sizes, 2^31 or more (sequence, head, chunk)
 * triples), UNSUPPORTED (d != 128, chunk != 64,
 * bad dtype), WORKSPACE, ALIAS (a gradient output overlapping an input, another
 * output or the workspace), DEVICE, HIP. */
KDA_API kda_status kda_prefill_backward(const kda_backward_desc *d, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
KDA_API const char *kda_status_string(kda_status s);

/* KDA_ABI_VERSION of the built library. */
KDA_API int32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
