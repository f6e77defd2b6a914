/*
 * hils.h -- C ABI of the HiLS (Hierarchical Landmark Sparse) attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * Method: "Hierarchical Sparse Attention Done Right: Toward Infinite Context
 * Modeling" (arXiv 2607.02980v1), source-linked summary page, cited below as
 * [HSADR <section>].  For every query i and query head h of KV group g:
 *
 *   candidates   C_i: complete chunks c (keys [cS, cS+S)) strictly before the
 *                query's own chunk (causal), or all complete chunks
 *                (non-causal)                         [HSADR §2 Preliminary]
 *   score        s_{h,i,c} = scale * <q_{h,i}, lmk_{g,c}> + bias_{g,c}
 *                (one landmark key per chunk; affine surrogate of the chunk's
 *                LogSumExp mass)        [HSADR §3 "Linear surrogate for chunk mass"]
 *   selection    T_{g,i} = top min(K, |C_i|) chunks by the fp32 group score
 *                mean_{h in g} s_{h,i,c}, ties to the lower chunk id; the heads
 *                of a group share it   [HSADR §3 "Sparse training"; §4 GQA]
 *   window       the chunk-aligned local window of w = local_chunks slots: the
 *                query's own chunk (its visible tokens) and the w - 1 complete
 *                chunks before it; candidates are the complete chunks before the
 *                window, so window and retrieval never overlap.  w = 0: no
 *                window; w = 1: the own chunk only  [HSADR §2 Preliminary]
 *   attention    per chunk c in T and per window chunk: l_j = scale*<q, k_j>,
 *                lse_c = log sum exp l_j, o_c = sum_j exp(l_j - lse_c) v_j
 *                                                     [HSADR §3 "Hierarchical softmax"]
 *   fusion       F = T + window chunks; a window chunk's score is its exact
 *                lse_c; LSE = log sum_{c in F} exp s_c;
 *                O = sum_{c in F} exp(s_c - LSE) o_c  [HSADR Abstract; §3]
 *   backward     gradients of <dO, O> for q, k, v, lmk, bias with the selection
 *                held fixed; unselected chunks get none [HSADR §3; §9]
 *
 * Causal queries sit at key positions t_i = seq_kv - seq_q + i (prefill:
 * seq_q == seq_kv; decode: seq_q == 1, t = seq_kv - 1); the own chunk is
 * floor(t_i / chunk_size).  Non-causal: the own slot is the trailing partial
 * chunk (possibly empty) and the window's other chunks precede it.  An empty fusion set gives
 * O = 0 and LSE = -inf.
 *
 * Layouts (all contiguous, row-major):
 *   q, q_ret, out,     [batch, heads_q,  seq_q,  head_dim]
 *   dout, dq, dq_ret
 *   k, v, dk, dv       [batch, heads_kv, seq_kv, head_dim]
 *   lmk, dlmk          [batch, heads_kv, num_landmarks, head_dim]
 *   lmk_bias, dbias    [batch, heads_kv, num_landmarks]          fp32, nullable
 *   sel_idx            [batch, heads_kv, seq_q, top_k]           int32, ascending
 *                                                               chunk ids, -1 padded
 *   lse                [batch, heads_q,  seq_q]                  fp32
 * dtype HILS_BF16: q, q_ret, k, v, lmk, out, dout, dq, dq_ret, dk, dv, dlmk are bf16 (raw 16-bit
 * patterns); arithmetic is fp32. HILS_F32: all of them fp32.
 *
 * Ownership and concurrency: every pointer is a device pointer owned by the
 * caller.  The library allocates nothing and shares no mutable state between
 * threads (the last-error message and the profiling hook are per calling thread);
 * scratch memory is the caller's `ws` buffer of at least
 * hils_workspace_size() bytes (256-byte aligned).  Work is enqueued on
 * `stream` (a hipStream_t; NULL = the default stream) and never synchronised;
 * calls sharing one workspace must be ordered on one stream.
 *
 * Errors: arguments are validated before any launch.  A null required
 * pointer, a negative size, heads_q % heads_kv != 0, chunk_size or top_k < 1,
 * local_chunks outside 0..64,
 * num_landmarks < seq_kv / chunk_size, a causal call with seq_q > seq_kv, a
 * decode call with seq_q != 1, a base pointer not 16-byte aligned, or a
 * workspace that is too small gives HILS_ERR_INVALID_ARG / HILS_ERR_WORKSPACE.
 * Shapes the kernels do not cover (top_k > 64: the selection kernels keep
 * one composite key per lane of a 64-wide wave; head_dim > 256,
 * chunk_size > 256, heads_q / heads_kv > 64, or a backward with
 * chunk_size * head_dim > 8192) give HILS_ERR_UNSUPPORTED.  A failed launch
 * gives HILS_ERR_HIP.  Nothing throws across the ABI; hils_last_error() holds
 * a message for the calling thread.  Empty problems (batch, seq_q or heads
 * equal to 0) are valid; they launch nothing, except that hils_backward
 * zero-fills the key-side gradients.
 */
#ifndef HILS_H_
#define HILS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HILS_OK = 0,
  HILS_ERR_INVALID_ARG = 1,
  HILS_ERR_UNSUPPORTED = 2,
  HILS_ERR_WORKSPACE = 3,
  HILS_ERR_HIP = 4
} hils_status;

typedef enum { HILS_F32 = 0, HILS_BF16 = 1 } hils_dtype;

typedef enum { HILS_OP_FORWARD = 0, HILS_OP_DECODE = 1, HILS_OP_BACKWARD = 2 } hils_op;

typedef struct {
  int32_t batch;           /* B                                                  */
  int32_t heads_q;         /* Hq; a multiple of heads_kv                         */
  int32_t heads_kv;        /* Hkv; G = Hq / Hkv query heads share one chunk set  */
  int32_t head_dim;        /* d                                                  */
  int32_t seq_q;           /* queries per (batch, head)                          */
  int32_t seq_kv;          /* keys per (batch, kv head)                          */
  int32_t chunk_size;      /* S                                                  */
  int32_t top_k;           /* K retrieved chunks per query (fewer if fewer exist)*/
  int32_t num_landmarks;   /* landmark rows per (batch, kv head), >= seq_kv / S  */
  int32_t causal;          /* 0 / 1                                              */
  int32_t local_chunks;    /* chunk slots of the local window, 0..64 (below)     */
  float scale;             /* token-logit and score scale; <= 0 means 1/sqrt(d)  */
  int32_t dtype;           /* hils_dtype                                          */
} hils_params;

/* Bytes of workspace that `op` (hils_op) needs for these parameters; 0 when the
 * parameters are invalid. */
size_t hils_workspace_size(const hils_params* p, int32_t op);

/* Forward pass (prefill or any seq_q): scores, group top-K selection, per-chunk
 * attention and fusion [HSADR §3].  Writes out, sel_idx and (if non-null) lse.
 * q_ret (nullable, layout and dtype of q): a separate retrieval query, e.g. one
 * calibrated by a low-rank query adaptation [HSADR §4 "Architecture"]: the chunk
 * scores, and so the selection and the fusion weights, use q_ret; the token
 * logits inside every chunk use q.  NULL: the scores use q. */
hils_status hils_forward(const hils_params* p, const void* q, const void* q_ret, const void* k,
                         const void* v, const void* lmk, const float* lmk_bias, void* out,
                         int32_t* sel_idx, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Single-token decode over a KV cache: seq_q must be 1 and causal is implied
 * (the query is the newest token, at position seq_kv - 1, its K/V already in
 * the cache).  Same math as hils_forward's last row; candidate scoring and
 * chunk attention are split across the GPU and merged by log-sum-exp. */
hils_status hils_decode(const hils_params* p, const void* q, const void* q_ret, const void* k,
                        const void* v, const void* lmk, const float* lmk_bias, void* out,
                        int32_t* sel_idx, float* lse, void* ws, size_t ws_bytes, void* stream);

/* hils_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, math and results as hils_decode; its
 * scratch memory (per-split top-K lists and per-chunk partial outputs) is a
 * fixed array of hils_decode_noalloc_scratch_bytes() = 16 MiB inside the
 * library, one per GPU, held until the process ends.  Nothing is allocated
 * and nothing needs clearing between calls (every scratch entry a call reads,
 * that call writes first).  Sizes that need more scratch than that
 * (hils_workspace_size(p, HILS_OP_DECODE) > 16 MiB; decode_128k-sized
 * batches need about 9 MB) give HILS_ERR_UNSUPPORTED before any launch.
 * All calls on one GPU share its array: calls that may overlap on one GPU
 * (different streams, or unordered host threads) race and must be serialised
 * by the caller. */
hils_status hils_decode_noalloc(const hils_params* p, const void* q, const void* q_ret,
                                const void* k, const void* v, const void* lmk,
                                const float* lmk_bias, void* out, int32_t* sel_idx, float* lse,
                                void* stream);

/* Size in bytes of hils_decode_noalloc's fixed scratch array. */
size_t hils_decode_noalloc_scratch_bytes(void);

/* Backward pass with the selection `sel_idx` (from hils_forward) held fixed
 * [HSADR §3 "Hierarchical softmax"; §9].  Writes (overwrites) dq, dk, dv,
 * dlmk and, if non-null, dlmk_bias.  `out` and `lse` are the forward's
 * outputs; `lse` must be non-null.  With q_ret (the forward's retrieval query)
 * the score gradients go to dq_ret (layout of dq) and dq holds the
 * token-attention part; q_ret and dq_ret are both given or both NULL.
 * sel_idx is read, never trusted: an entry that is not a candidate of its
 * query (negative, or not a complete chunk before the query's local window)
 * or that repeats an earlier entry of its row is skipped like -1, so any
 * int32 contents are safe; a row hils_forward wrote is used as it is.
 * With no query rows (batch, heads_q or seq_q zero) dk, dv, dlmk and
 * dlmk_bias are still overwritten, with zeros (null allowed where a buffer
 * is empty). */
hils_status hils_backward(const hils_params* p, const void* q, const void* q_ret, const void* k,
                          const void* v, const void* lmk, const float* lmk_bias, const void* out,
                          const void* dout, const int32_t* sel_idx, const float* lse,
                          void* dq, void* dq_ret, void* dk, void* dv, void* dlmk,
                          float* dlmk_bias, void* ws, size_t ws_bytes, void* stream);

/* Landmark formation [HSADR §3 "Linear surrogate for chunk mass"]: for every
 * complete chunk c < seq_kv / chunk_size of each (batch, kv head), the landmark
 * query lq_c induces p = softmax_j(scale * <lq_c, k_j>) over the chunk's keys
 * j in [c*S, c*S + S); the landmark key is lmk_c = sum_j p_j k_j and the bias is
 * the entropy of p, -sum_j p_j log p_j (with these, the retrieval score equals
 * the chunk's exact LogSumExp at q = lq_c and is its first-order expansion
 * around it).
 *   lq, lmk       [batch, heads_kv, num_landmarks, head_dim]   dtype of p
 *   k             [batch, heads_kv, seq_kv, head_dim]          dtype of p
 *   lmk_bias      [batch, heads_kv, num_landmarks]             fp32, nullable
 * Rows c >= seq_kv / chunk_size of lmk and lmk_bias are written as 0; lq's rows
 * there are not read.  Fields used: dtype, batch, heads_kv, head_dim, seq_kv,
 * chunk_size, num_landmarks, scale (heads_q, seq_q, top_k, causal and
 * local_chunks are ignored).  Errors: a null pointer to a non-empty buffer, a negative size,
 * num_landmarks < seq_kv / chunk_size or a base pointer not 16-byte aligned give
 * HILS_ERR_INVALID_ARG; chunk_size or head_dim above 256, or
 * chunk_size * head_dim above 16384, give HILS_ERR_UNSUPPORTED.  No workspace. */
hils_status hils_landmarks(const hils_params* p, const void* lq, const void* k, void* lmk,
                           float* lmk_bias, void* stream);

/* Gradient of hils_landmarks: given dlmk (dtype of p) and dlmk_bias (fp32,
 * nullable = zero), writes (overwrites) dlq [batch, heads_kv, num_landmarks,
 * head_dim] and dk [batch, heads_kv, seq_kv, head_dim]:
 *   dp_j = <dlmk_c, k_j> - dbias_c (log p_j + 1),
 *   dl_j = p_j (dp_j - sum_i p_i dp_i),
 *   dlq_c = scale sum_j dl_j k_j,   dk_j = scale dl_j lq_c + p_j dlmk_c.
 * Rows of dlq past the complete chunks and keys of a trailing partial chunk
 * get 0.  dk is this step's contribution only: a caller that also has the
 * attention's dk adds the two.  Same fields and errors as hils_landmarks. */
hils_status hils_landmarks_backward(const hils_params* p, const void* lq, const void* k,
                                    const void* dlmk, const float* dlmk_bias, void* dlq, void* dk,
                                    void* stream);

/* Kernel families, for hils_profile_kernel. */
typedef enum {
  HILS_KERNEL_GENERIC_SELECT = 1,
  HILS_KERNEL_GENERIC_ATTEND = 2,
  HILS_KERNEL_GENERIC_BWD_ROWS = 3,
  HILS_KERNEL_GENERIC_BWD_CHUNKS = 4,
  HILS_KERNEL_DECODE_SCORE = 5,
  HILS_KERNEL_DECODE_MERGE = 6,
  HILS_KERNEL_DECODE_ATTEND = 7,
  HILS_KERNEL_PREFILL_SELECT = 8,
  HILS_KERNEL_PREFILL_ATTEND = 9,
  HILS_KERNEL_PREFILL_BWD_ROWS = 10,
  HILS_KERNEL_PREFILL_BWD_CHUNKS = 11,
  HILS_KERNEL_LANDMARKS = 12,
  HILS_KERNEL_LANDMARKS_BWD = 13
} hils_kernel_id;

/* Profiling hook (measurement only; not needed for computation).  Until `n`
 * launches of kernel family `kernel` (a hils_kernel_id) have been made by
 * library calls on the calling thread, launch i is bracketed by
 * hipEventRecord(starts[i]) and hipEventRecord(stops[i]) on its stream.  The
 * caller owns the n + n events (hipEvent_t, created with timing enabled) and
 * reads them with hipEventElapsedTime.  n = 0 disarms.  Thread-local state:
 * the only state the library keeps.  Returns HILS_ERR_INVALID_ARG for an
 * unknown kernel id, a negative n, or null arrays with n > 0. */
hils_status hils_profile_kernel(int32_t kernel, void* const* starts, void* const* stops,
                                int32_t n);

/* Number of launches recorded since hils_profile_kernel armed the hook. */
int32_t hils_profile_count(void);

/* Static description of a status code. */
const char* hils_status_string(hils_status s);

/* Message of the last failing call on this thread ("" if none). */
const char* hils_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HILS_H_ */
