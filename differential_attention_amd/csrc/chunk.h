// chunk.h -- internal to the library: the prefill kernel on query chunks
// against a key/value cache (diffattn_fwd.hip), used by the cache path
// (diffattn_kv.hip) when the chunks are long.  Not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

// How a chunk call runs on the prefill kernel (with sub 32-query
// sub-blocks per wave): unsplit (ck = 0), or with
// each sequence's keys cut into splits of ck keys (nslots slots in all) whose
// partials the cache path's combine kernel merges, through a workspace of
// ws_bytes (fp32 partial O of [nslots][Hkv][rmax][2][2d], then the maxima
// and sums [nslots][Hkv][rmax][4]); est_us is the estimated duration.
struct DiffattnChunkPlan {
    int32_t ck;
    int32_t nslots;
    int32_t rmax;
    int32_t sub;   // 32-query sub-blocks per wave (1 or 2)
    size_t ws_o_bytes, ws_ml_bytes;
    double est_us;
};

// The plan for uniform sequences of these sizes: splits = 1 takes the
// split size (or none) with the lowest estimate, 0 the unsplit plan, 2 the
// cheapest split size; only split sizes whose partials fit in ws_cap bytes
// are candidates.  Returns 0 when the grid does not fit (or, for 2, no
// split size does).
__attribute__((visibility("hidden"))) int
diffattn_chunk_plan(int32_t nseq, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t H,
                    int32_t Hkv, int32_t d, int splits, size_t ws_cap,
                    DiffattnChunkPlan *plan);

// Arguments as validated by diffattn_fwd_kv (bf16, d = 32 or 64); the
// sequences' queries are the last nq of their nk keys, aligned bottom-right.
// With plan->ck > 0, ws_o and ws_ml receive the partials and nothing is
// written to out.  Returns a DIFFATTN status.
__attribute__((visibility("hidden"))) int
diffattn_chunk_prefill(const void *q, const void *k, const void *v, const float *lambda_q1,
                       const float *lambda_k1, const float *lambda_q2, const float *lambda_k2,
                       int32_t lambda_stride, float lambda_init, const float *subln_weight,
                       float eps, int causal, const int32_t *cu_seqlens_q,
                       const int32_t *cu_seqlens_k, int32_t nseq, int32_t max_seqlen_q,
                       int32_t Tq, int32_t Tk, int32_t H, int32_t Hkv, int32_t d,
                       const void *rope_cos, const void *rope_sin, int rope_dtype,
                       const DiffattnChunkPlan *plan, float *ws_o, float *ws_ml, void *out,
                       void *stream);
