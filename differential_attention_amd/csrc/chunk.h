// chunk.h -- internal to the library: the prefill kernel on query chunks
// against a key/value cache (diffattn_fwd.hip), used by the cache path
// (diffattn_kv.hip) when the chunks are long.  Not part of the C ABI.
#pragma once

#include <stdint.h>

// Estimated duration (microseconds) of diffattn_chunk_prefill on uniform
// sequences of these sizes: launch rounds of the grid times the longest key
// range; infinite for a grid that does not fit.
__attribute__((visibility("hidden"))) double
diffattn_chunk_prefill_us(int32_t nseq, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t H,
                          int32_t Hkv);

// Arguments as validated by diffattn_fwd_kv (bf16, d = 32 or 64); the
// sequences' queries are the last nq of their nk keys, aligned bottom-right.
// Returns a DIFFATTN status.
__attribute__((visibility("hidden"))) int
diffattn_chunk_prefill(const void *q, const void *k, const void *v, const float *lambda_q1,
                       const float *lambda_k1, const float *lambda_q2, const float *lambda_k2,
                       int32_t lambda_stride, float lambda_init, const float *subln_weight,
                       float eps, int causal, const int32_t *cu_seqlens_q,
                       const int32_t *cu_seqlens_k, int32_t nseq, int32_t max_seqlen_q,
                       int32_t Tq, int32_t Tk, int32_t H, int32_t Hkv, int32_t d,
                       const void *rope_cos, const void *rope_sin, int rope_dtype, void *out,
                       void *stream);
