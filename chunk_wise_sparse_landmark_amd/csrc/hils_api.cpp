// C ABI of the HiLS library: argument validation, workspace sizing, dispatch.
// All checks run on the host before any launch; nothing throws across the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <string>

#include "hils.h"
#include "hils_kernels.h"
#include "hils_profile.h"

namespace hils {
ProfileSlot& profile_slot() {
  static thread_local ProfileSlot slot;
  return slot;
}
}  // namespace hils

namespace {

thread_local std::string g_last_error;

hils_status fail(hils_status s, const char* fmt, ...) {
  char msg[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof(msg), fmt, ap);
  va_end(ap);
  g_last_error = msg;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_empty(const hils_params* p) {
  return p->batch == 0 || p->heads_q == 0 || p->seq_q == 0;
}

// Shape checks shared by every entry point.  `op` is a hils_op.
hils_status check_params(const hils_params* p, int op) {
  if (!p) return fail(HILS_ERR_INVALID_ARG, "params is null");
  if (p->batch < 0 || p->heads_q < 0 || p->heads_kv < 0 || p->head_dim < 0 || p->seq_q < 0 ||
      p->seq_kv < 0 || p->num_landmarks < 0)
    return fail(HILS_ERR_INVALID_ARG, "negative size");
  if (p->dtype != HILS_F32 && p->dtype != HILS_BF16)
    return fail(HILS_ERR_INVALID_ARG, "dtype %d is not HILS_F32 or HILS_BF16", p->dtype);
  if (p->chunk_size < 1) return fail(HILS_ERR_INVALID_ARG, "chunk_size must be >= 1");
  if (p->top_k < 1) return fail(HILS_ERR_INVALID_ARG, "top_k must be >= 1");
  if (p->causal != 0 && p->causal != 1) return fail(HILS_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->local_chunks < 0 || p->local_chunks > hils::kMaxLocalChunks)
    return fail(HILS_ERR_INVALID_ARG, "local_chunks must be in 0..%d (got %d)",
                hils::kMaxLocalChunks, p->local_chunks);
  if (!std::isfinite(p->scale)) return fail(HILS_ERR_INVALID_ARG, "scale is not finite");
  if (p->heads_kv == 0 && p->heads_q != 0)
    return fail(HILS_ERR_INVALID_ARG, "heads_kv is 0 but heads_q is not");
  if (p->heads_kv > 0 && p->heads_q % p->heads_kv != 0)
    return fail(HILS_ERR_INVALID_ARG, "heads_q (%d) is not a multiple of heads_kv (%d)",
                p->heads_q, p->heads_kv);
  if (p->head_dim < 1) return fail(HILS_ERR_INVALID_ARG, "head_dim must be >= 1");
  if (p->num_landmarks < p->seq_kv / p->chunk_size)
    return fail(HILS_ERR_INVALID_ARG, "num_landmarks (%d) < seq_kv / chunk_size (%d)",
                p->num_landmarks, p->seq_kv / p->chunk_size);
  if (op == HILS_OP_DECODE && p->seq_q != 1 && !is_empty(p))
    return fail(HILS_ERR_INVALID_ARG, "decode needs seq_q == 1 (got %d)", p->seq_q);
  const int causal = op == HILS_OP_DECODE ? 1 : p->causal;
  if (causal && p->seq_q > p->seq_kv)
    return fail(HILS_ERR_INVALID_ARG, "causal call with seq_q (%d) > seq_kv (%d)", p->seq_q,
                p->seq_kv);
  if (p->top_k > hils::kMaxTopK)
    return fail(HILS_ERR_UNSUPPORTED, "top_k %d > %d", p->top_k, hils::kMaxTopK);
  if (p->head_dim > 256) return fail(HILS_ERR_UNSUPPORTED, "head_dim %d > 256", p->head_dim);
  if (p->chunk_size > 256) return fail(HILS_ERR_UNSUPPORTED, "chunk_size %d > 256", p->chunk_size);
  if (p->heads_kv > 0 && p->heads_q / p->heads_kv > 64)
    return fail(HILS_ERR_UNSUPPORTED, "heads_q / heads_kv > 64");
  if (op == HILS_OP_BACKWARD && (int64_t)p->chunk_size * p->head_dim > 8192)
    return fail(HILS_ERR_UNSUPPORTED, "backward needs chunk_size * head_dim <= 8192");
  return HILS_OK;
}

hils::Geometry geometry(const hils_params* p, int op) {
  hils::Geometry g;
  g.B = p->batch;
  g.Hq = p->heads_q;
  g.Hkv = p->heads_kv;
  g.G = p->heads_kv > 0 ? p->heads_q / p->heads_kv : 1;
  g.d = p->head_dim;
  g.Lq = p->seq_q;
  g.Lkv = p->seq_kv;
  g.S = p->chunk_size;
  g.K = p->top_k;
  g.NC = p->seq_kv / p->chunk_size;
  g.NCcap = p->num_landmarks;
  g.causal = op == HILS_OP_DECODE ? 1 : p->causal;
  g.win = p->local_chunks;
  g.keep_own = p->local_chunks > 0;
  g.scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->head_dim);
  return g;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t ws_bytes_for(const hils_params* p, int op) {
  if (is_empty(p)) return 0;
  hils::Geometry g = geometry(p, op);
  const int bf16 = p->dtype == HILS_BF16;
  switch (op) {
    case HILS_OP_FORWARD:
      return hils::prefill_fast_supported(g, bf16) ? round256(hils::prefill_fast_ws(g)) : 0;
    case HILS_OP_DECODE:
      return hils::decode_fast_supported(g, bf16) ? round256(hils::decode_fast_ws(g)) : 0;
    case HILS_OP_BACKWARD:
      // the sanitised selection first, then the kernels' own scratch
      return round256(hils::sanitized_selection_bytes(g)) +
             (hils::prefill_bwd_fast_supported(g, bf16) ? round256(hils::prefill_bwd_fast_ws(g))
                                                        : round256(hils::generic_backward_ws(g)));
    default:
      return 0;
  }
}

hils_status check_ws(const hils_params* p, int op, const void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_for(p, op);
  if (need == 0) return HILS_OK;
  if (!ws) return fail(HILS_ERR_WORKSPACE, "workspace of %zu bytes needed, got null", need);
  if (ws_bytes < need)
    return fail(HILS_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, ws_bytes);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(HILS_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return HILS_OK;
}

hils_status launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(HILS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return HILS_OK;
}

hils_status forward_like(int op, const hils_params* p, const void* q, const void* q_ret,
                         const void* k, const void* v, const void* lmk, const float* lmk_bias,
                         void* out, int32_t* sel_idx, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  hils_status s = check_params(p, op);
  if (s != HILS_OK) return s;
  if (is_empty(p)) return HILS_OK;
  if (!q || !k || !v || !lmk || !out || !sel_idx)
    return fail(HILS_ERR_INVALID_ARG, "a required pointer (q, k, v, lmk, out, sel_idx) is null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(lmk) || !aligned16(out) ||
      !aligned16(sel_idx) || (lse && !aligned16(lse)) || (lmk_bias && !aligned16(lmk_bias)) ||
      (q_ret && !aligned16(q_ret)))
    return fail(HILS_ERR_INVALID_ARG, "base pointers must be 16-byte aligned");
  s = check_ws(p, op, ws, ws_bytes);
  if (s != HILS_OK) return s;
  hils::Geometry g = geometry(p, op);
  const int bf16 = p->dtype == HILS_BF16;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const void* qr = q_ret ? q_ret : q;
  (void)hipGetLastError();   // clear a stale error so it is not reported as ours
  if (op == HILS_OP_DECODE && hils::decode_fast_supported(g, bf16))
    return launch_status(
        hils::launch_decode_fast(g, q, qr, k, v, lmk, lmk_bias, out, sel_idx, lse, ws, st),
        "decode launch");
  if (op == HILS_OP_FORWARD && hils::prefill_fast_supported(g, bf16))
    return launch_status(
        hils::launch_prefill_fast(g, q, qr, k, v, lmk, lmk_bias, out, sel_idx, lse, ws, st),
        "prefill launch");
  return launch_status(
      hils::launch_generic_forward(g, bf16, q, qr, k, v, lmk, lmk_bias, out, sel_idx, lse, st),
      "forward launch");
}

// Checks of the landmark-formation entry points: only the fields they use.  A
// pointer is required when the buffer it names is not empty.
struct Buf {
  const void* ptr;
  bool required;
};

hils_status check_landmarks(const hils_params* p, std::initializer_list<Buf> bufs) {
  if (!p) return fail(HILS_ERR_INVALID_ARG, "params is null");
  if (p->batch < 0 || p->heads_kv < 0 || p->head_dim < 0 || p->seq_kv < 0 || p->num_landmarks < 0)
    return fail(HILS_ERR_INVALID_ARG, "negative size");
  if (p->dtype != HILS_F32 && p->dtype != HILS_BF16)
    return fail(HILS_ERR_INVALID_ARG, "dtype %d is not HILS_F32 or HILS_BF16", p->dtype);
  if (p->chunk_size < 1) return fail(HILS_ERR_INVALID_ARG, "chunk_size must be >= 1");
  if (p->head_dim < 1) return fail(HILS_ERR_INVALID_ARG, "head_dim must be >= 1");
  if (!std::isfinite(p->scale)) return fail(HILS_ERR_INVALID_ARG, "scale is not finite");
  if (p->num_landmarks < p->seq_kv / p->chunk_size)
    return fail(HILS_ERR_INVALID_ARG, "num_landmarks (%d) < seq_kv / chunk_size (%d)",
                p->num_landmarks, p->seq_kv / p->chunk_size);
  if (!hils::landmarks_supported(geometry(p, HILS_OP_FORWARD)))
    return fail(HILS_ERR_UNSUPPORTED,
                "landmark formation needs chunk_size, head_dim <= 256 and their product <= 16384");
  for (const Buf& b : bufs) {
    if (b.required && !b.ptr) return fail(HILS_ERR_INVALID_ARG, "a required pointer is null");
    if (b.ptr && !aligned16(b.ptr))
      return fail(HILS_ERR_INVALID_ARG, "base pointers must be 16-byte aligned");
  }
  return HILS_OK;
}

// hils_backward with no query rows (batch, heads_q or seq_q zero): the key-side
// gradients it promises to overwrite are all zero.
hils_status zero_key_grads(const hils_params* p, void* dk, void* dv, void* dlmk, float* dbias,
                           void* stream) {
  const size_t elem = p->dtype == HILS_BF16 ? 2 : 4;
  const size_t groups = (size_t)p->batch * p->heads_kv;
  const size_t kv = groups * p->seq_kv * p->head_dim * elem;
  const size_t lm = groups * p->num_landmarks * p->head_dim * elem;
  const size_t lb = groups * p->num_landmarks * sizeof(float);
  if ((kv && (!dk || !dv)) || (lm && !dlmk))
    return fail(HILS_ERR_INVALID_ARG, "a required gradient pointer of hils_backward is null");
  if ((dk && !aligned16(dk)) || (dv && !aligned16(dv)) || (dlmk && !aligned16(dlmk)) ||
      (dbias && !aligned16(dbias)))
    return fail(HILS_ERR_INVALID_ARG, "base pointers must be 16-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();   // clear a stale error so it is not reported as ours
  hils_status s = HILS_OK;
  if (kv && s == HILS_OK) s = launch_status(hils::launch_zero_fill(dk, kv, st), "zero fill");
  if (kv && s == HILS_OK) s = launch_status(hils::launch_zero_fill(dv, kv, st), "zero fill");
  if (lm && s == HILS_OK) s = launch_status(hils::launch_zero_fill(dlmk, lm, st), "zero fill");
  if (lb && dbias && s == HILS_OK) s = launch_status(hils::launch_zero_fill(dbias, lb, st), "zero fill");
  return s;
}

bool landmarks_empty(const hils_params* p) {
  return p->batch == 0 || p->heads_kv == 0 || (p->seq_kv == 0 && p->num_landmarks == 0);
}

}  // namespace

namespace hils {

// hils_decode on a scratch buffer the library owns (the allocation-free entry
// point): `ws` is that buffer (null when it could not be found on the current
// device) and `ws_limit` its size; a call that needs more fails before any launch.
hils_status decode_with_scratch(const hils_params* p, const void* q, const void* q_ret,
                                     const void* k, const void* v, const void* lmk,
                                     const float* lmk_bias, void* out, int32_t* sel_idx, float* lse,
                                     void* ws, size_t ws_bytes, size_t ws_limit, void* stream) {
  hils_status s = check_params(p, HILS_OP_DECODE);
  if (s != HILS_OK) return s;
  const size_t need = ws_bytes_for(p, HILS_OP_DECODE);
  if (need > ws_limit)
    return fail(HILS_ERR_UNSUPPORTED,
                "hils_decode_noalloc: these sizes need %zu bytes of scratch, its fixed buffer "
                "holds %zu (use hils_decode with a workspace)", need, ws_limit);
  if (need > 0 && !ws)
    return fail(HILS_ERR_HIP, "hils_decode_noalloc: the scratch buffer of the current device "
                              "could not be located");
  return forward_like(HILS_OP_DECODE, p, q, q_ret, k, v, lmk, lmk_bias, out, sel_idx, lse, ws,
                      ws_bytes, stream);
}

}  // namespace hils

extern "C" {

size_t hils_workspace_size(const hils_params* p, int32_t op) {
  if (op < HILS_OP_FORWARD || op > HILS_OP_BACKWARD) return 0;
  if (check_params(p, op) != HILS_OK) return 0;
  return ws_bytes_for(p, op);
}

hils_status hils_forward(const hils_params* p, const void* q, const void* q_ret, const void* k,
                         const void* v, const void* lmk, const float* lmk_bias, void* out,
                         int32_t* sel_idx, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return forward_like(HILS_OP_FORWARD, p, q, q_ret, k, v, lmk, lmk_bias, out, sel_idx, lse, ws,
                      ws_bytes, stream);
}

hils_status hils_decode(const hils_params* p, const void* q, const void* q_ret, const void* k,
                        const void* v, const void* lmk, const float* lmk_bias, void* out,
                        int32_t* sel_idx, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return forward_like(HILS_OP_DECODE, p, q, q_ret, k, v, lmk, lmk_bias, out, sel_idx, lse, ws,
                      ws_bytes, stream);
}

hils_status hils_backward(const hils_params* p, const void* q, const void* q_ret, const void* k,
                          const void* v, const void* lmk, const float* lmk_bias, const void* out,
                          const void* dout, const int32_t* sel_idx, const float* lse, void* dq,
                          void* dq_ret, void* dk, void* dv, void* dlmk, float* dlmk_bias,
                          void* ws, size_t ws_bytes, void* stream) {
  hils_status s = check_params(p, HILS_OP_BACKWARD);
  if (s != HILS_OK) return s;
  if (is_empty(p)) return zero_key_grads(p, dk, dv, dlmk, dlmk_bias, stream);
  if (!q || !k || !v || !lmk || !out || !dout || !sel_idx || !lse || !dq || !dk || !dv || !dlmk)
    return fail(HILS_ERR_INVALID_ARG, "a required pointer of hils_backward is null");
  const void* ptrs[] = {q, k, v, lmk, out, dout, sel_idx, lse, dq, dk, dv, dlmk};
  for (const void* x : ptrs)
    if (!aligned16(x)) return fail(HILS_ERR_INVALID_ARG, "base pointers must be 16-byte aligned");
  if ((lmk_bias && !aligned16(lmk_bias)) || (dlmk_bias && !aligned16(dlmk_bias)) ||
      (q_ret && !aligned16(q_ret)) || (dq_ret && !aligned16(dq_ret)))
    return fail(HILS_ERR_INVALID_ARG, "base pointers must be 16-byte aligned");
  if ((q_ret != nullptr) != (dq_ret != nullptr))
    return fail(HILS_ERR_INVALID_ARG, "q_ret and dq_ret must be given together");
  s = check_ws(p, HILS_OP_BACKWARD, ws, ws_bytes);
  if (s != HILS_OK) return s;
  hils::Geometry g = geometry(p, HILS_OP_BACKWARD);
  const int bf16 = p->dtype == HILS_BF16;
  const void* qr = q_ret ? q_ret : q;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();   // clear a stale error so it is not reported as ours
  // the kernels read a copy of the selection in which every id the query may not
  // use (not one of its candidates, or a repeat within its row) is -1
  int32_t* sel = reinterpret_cast<int32_t*>(ws);
  void* kws = reinterpret_cast<char*>(ws) + round256(hils::sanitized_selection_bytes(g));
  s = launch_status(hils::launch_sanitize_selection(g, sel_idx, sel, st), "selection check launch");
  if (s != HILS_OK) return s;
  if (hils::prefill_bwd_fast_supported(g, bf16))
    return launch_status(hils::launch_prefill_bwd_fast(g, q, qr, k, v, lmk, lmk_bias, out, dout,
                                                       sel, lse, dq, dq_ret, dk, dv, dlmk,
                                                       dlmk_bias, kws, st),
                         "backward launch");
  return launch_status(hils::launch_generic_backward(g, bf16, q, qr, k, v, lmk, lmk_bias, dout,
                                                     sel, dq, dq_ret, dk, dv, dlmk, dlmk_bias,
                                                     kws, st),
                       "backward launch");
}

hils_status hils_landmarks(const hils_params* p, const void* lq, const void* k, void* lmk,
                           float* lmk_bias, void* stream) {
  hils_status s = check_landmarks(p, {});
  if (s != HILS_OK || landmarks_empty(p)) return s;
  const bool full = p->seq_kv >= p->chunk_size;
  s = check_landmarks(p, {{lq, full}, {k, full}, {lmk, p->num_landmarks > 0}, {lmk_bias, false}});
  if (s != HILS_OK) return s;
  (void)hipGetLastError();   // clear a stale error so it is not reported as ours
  return launch_status(hils::launch_landmarks(geometry(p, HILS_OP_FORWARD), p->dtype == HILS_BF16,
                                              lq, k, lmk, lmk_bias,
                                              reinterpret_cast<hipStream_t>(stream)),
                       "landmark launch");
}

hils_status hils_landmarks_backward(const hils_params* p, const void* lq, const void* k,
                                    const void* dlmk, const float* dlmk_bias, void* dlq, void* dk,
                                    void* stream) {
  hils_status s = check_landmarks(p, {});
  if (s != HILS_OK || landmarks_empty(p)) return s;
  const bool full = p->seq_kv >= p->chunk_size;
  s = check_landmarks(p, {{lq, full}, {k, p->seq_kv > 0}, {dlmk, full}, {dlmk_bias, false},
                          {dlq, p->num_landmarks > 0}, {dk, p->seq_kv > 0}});
  if (s != HILS_OK) return s;
  (void)hipGetLastError();   // clear a stale error so it is not reported as ours
  return launch_status(
      hils::launch_landmarks_backward(geometry(p, HILS_OP_FORWARD), p->dtype == HILS_BF16, lq, k,
                                      dlmk, dlmk_bias, dlq, dk,
                                      reinterpret_cast<hipStream_t>(stream)),
      "landmark backward launch");
}

const char* hils_status_string(hils_status s) {
  switch (s) {
    case HILS_OK: return "HILS_OK";
    case HILS_ERR_INVALID_ARG: return "HILS_ERR_INVALID_ARG";
    case HILS_ERR_UNSUPPORTED: return "HILS_ERR_UNSUPPORTED";
    case HILS_ERR_WORKSPACE: return "HILS_ERR_WORKSPACE";
    case HILS_ERR_HIP: return "HILS_ERR_HIP";
  }
  return "unknown hils_status";
}

const char* hils_last_error(void) { return g_last_error.c_str(); }

hils_status hils_profile_kernel(int32_t kernel, void* const* starts, void* const* stops, int32_t n) {
  hils::ProfileSlot& ps = hils::profile_slot();
  if (n == 0) {
    ps = hils::ProfileSlot();
    return HILS_OK;
  }
  if (kernel < 1 || kernel >= hils::kKernelIdEnd || n < 0 || !starts || !stops)
    return fail(HILS_ERR_INVALID_ARG, "bad profiling request");
  ps.kernel = kernel;
  ps.starts = reinterpret_cast<hipEvent_t const*>(starts);
  ps.stops = reinterpret_cast<hipEvent_t const*>(stops);
  ps.n = n;
  ps.next = 0;
  return HILS_OK;
}

int32_t hils_profile_count(void) { return hils::profile_slot().next; }

}  // extern "C"
