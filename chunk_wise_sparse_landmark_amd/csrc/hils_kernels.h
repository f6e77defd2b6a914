// Host-side launchers of the HiLS kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hils_common.h"

namespace hils {

// shape-generic path (fp32 or bf16)
// qr: the retrieval query the chunk scores use (q itself when none is given);
// dqr: where the score gradients go (null: added into dq)
hipError_t launch_generic_forward(const Geometry& g, int bf16, const void* q, const void* qr,
                                  const void* k, const void* v, const void* lmk, const float* bias,
                                  void* out, int32_t* sel_idx, float* lse, hipStream_t st);
size_t generic_backward_ws(const Geometry& g);
hipError_t launch_generic_backward(const Geometry& g, int bf16, const void* q, const void* qr,
                                   const void* k, const void* v, const void* lmk, const float* bias,
                                   const void* dout, const int32_t* sel_idx, void* dq, void* dqr,
                                   void* dk, void* dv, void* dlmk, float* dbias, void* ws,
                                   hipStream_t st);

// split decode path (bf16, d = 128, S = 64)
bool decode_fast_supported(const Geometry& g, int bf16);
size_t decode_fast_ws(const Geometry& g);
hipError_t launch_decode_fast(const Geometry& g, const void* q, const void* qr, const void* k,
                              const void* v, const void* lmk, const float* bias, void* out,
                              int32_t* sel_idx, float* lse, void* ws, hipStream_t st);

// MFMA prefill path (bf16, d = 128, S = 64, causal, seq_q == seq_kv)
bool prefill_fast_supported(const Geometry& g, int bf16);
size_t prefill_fast_ws(const Geometry& g);
hipError_t launch_prefill_fast(const Geometry& g, const void* q, const void* qr, const void* k,
                               const void* v, const void* lmk, const float* bias, void* out,
                               int32_t* sel_idx, float* lse, void* ws, hipStream_t st);

// MFMA prefill backward (same shapes as the MFMA forward)
bool prefill_bwd_fast_supported(const Geometry& g, int bf16);
size_t prefill_bwd_fast_ws(const Geometry& g);
hipError_t launch_prefill_bwd_fast(const Geometry& g, const void* q, const void* qr, const void* k,
                                   const void* v, const void* lmk, const float* bias,
                                   const void* out, const void* dout, const int32_t* sel_idx,
                                   const float* lse, void* dq, void* dqr, void* dk, void* dv,
                                   void* dlmk, float* dbias, void* ws, hipStream_t st);

// backward service: a copy of a caller's selection with the ids a query may not
// use (not among its candidates, or repeated in its row) set to -1
size_t sanitized_selection_bytes(const Geometry& g);
hipError_t launch_sanitize_selection(const Geometry& g, const int32_t* in, int32_t* out,
                                     hipStream_t st);
// bytes of zeros (a fill kernel, no memset)
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st);

// landmark formation (weighted key sum + entropy bias per chunk) and its backward
bool landmarks_supported(const Geometry& g);
hipError_t launch_landmarks(const Geometry& g, int bf16, const void* lq, const void* k, void* lmk,
                            float* bias, hipStream_t st);
hipError_t launch_landmarks_backward(const Geometry& g, int bf16, const void* lq, const void* k,
                                     const void* dlmk, const float* dbias, void* dlq, void* dk,
                                     hipStream_t st);

}  // namespace hils
