/*
 * diffattn.h -- C ABI of the MI355X (gfx950) differential-attention forward.
 *
 * The operation (DiffTransformer.py of Differential-Transformer-PyTorch,
 * MultiHeadDifferentialAttention.forward; LlamaDiffSdpaAttention.py, forward;
 * unilm pull request "Add an isolated implementation of FlashDiffAttention",
 * FlashDiffAttention and alternative_forward):
 *
 *   lambda_h = exp(<lambda_q1_h, lambda_k1_h>) - exp(<lambda_q2_h, lambda_k2_h>)
 *              + lambda_init
 *   for each packed sequence, head h (KV head g = h / (H / Hkv)), query i:
 *     A_m[i, j] = softmax_j( <Qm[i, h], Km[j, g]> / sqrt(d) ),  m = 1, 2,
 *                 over keys j <= i of the same sequence (all of its keys
 *                 when causal == 0)
 *     pre[i]    = sum_j (A_1[i, j] - lambda_h * A_2[i, j]) * V[j, g] (2d wide)
 *     out[i, h] = pre[i] / sqrt(mean(pre[i]^2) + eps) * w * (1 - lambda_init)
 *
 * Memory layout (all device memory, contiguous, token-major; T tokens, H
 * differential heads, Hkv key/value heads, half-head width d):
 *   q   [T, H,   2, d]   q[t, h, 0, :] = Q1, q[t, h, 1, :] = Q2 of head h
 *   k   [T, Hkv, 2, d]   k[t, g, 0, :] = K1, k[t, g, 1, :] = K2 of KV head g
 *   v   [T, Hkv, 2d]
 *   out [T, H,   2d]     equal to [T, H * 2d], the heads concatenated
 * q, k, v and out share one element type (DIFFATTN_BF16 or DIFFATTN_F32)
 * and must be 16-byte aligned.
 *
 * Ownership: the caller owns every buffer.  The library allocates no device
 * or host memory, keeps no state between calls, never synchronises, and is
 * safe to call from several threads.  out must not overlap any input.  The
 * one exception is diffattn_fwd_kv_noalloc, whose static device array (one
 * per GPU, part of the code object) is shared by all of its calls.
 *
 * Errors: every entry point returns a status (DIFFATTN_OK or a negative
 * code) and never aborts or throws.  Argument errors are detected on the host
 * before anything is launched.  Launch errors return DIFFATTN_EHIP; a fault
 * inside the kernel surfaces at the caller's next synchronisation on the
 * stream.
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIFFATTN_ABI_VERSION 11

enum diffattn_status {
    DIFFATTN_OK = 0,
    DIFFATTN_EINVAL = -1,       /* malformed arguments; nothing launched    */
    DIFFATTN_EUNSUPPORTED = -2, /* (dtype, d) pair not compiled in          */
    DIFFATTN_EHIP = -3,         /* HIP runtime error: no device, bad launch */
    DIFFATTN_ETOOLARGE = -4     /* needs more than the static scratch holds */
};

enum diffattn_dtype {
    DIFFATTN_BF16 = 0, /* bfloat16 storage, fp32 accumulation */
    DIFFATTN_F32 = 1   /* fp32 storage, fp32 arithmetic       */
};

/*
 * Differential-attention forward pass, asynchronous on `stream`.
 *
 *   dtype        DIFFATTN_BF16 or DIFFATTN_F32: element type of q, k, v, out.
 *   q, k, v      device inputs in the layout above.
 *   lambda_q1, lambda_k1, lambda_q2, lambda_k2
 *                device fp32 vectors of length d: one set shared by all
 *                heads (the Llama gist and alternative_forward share it), or
 *                one set per head (the DiffTransformer page keeps them so),
 *                head h's vectors starting lambda_stride elements after head
 *                h-1's.
 *   lambda_stride 0 for one shared set, else >= d (e.g. d for [H, d]).
 *   lambda_init  the layer's initial lambda (see diffattn_lambda_init).
 *   subln_weight device fp32 [2d] RMSNorm weight (16-byte aligned), or NULL
 *                for all ones.
 *   eps          RMSNorm epsilon (1e-5 on the DiffTransformer page); >= 0.
 *   causal       1: query i sees keys j <= i of its sequence; 0: all keys of
 *                its sequence.
 *   cu_seqlens   device int32 [nseq + 1] sequence boundaries: cu[0] = 0,
 *                non-decreasing, cu[nseq] = T.  Zero-length sequences are
 *                allowed.  NULL means nseq sequences of T / nseq tokens each.
 *                The contents are a precondition, not checked here (see
 *                diffattn_check_cu_seqlens).
 *   nseq         number of sequences (>= 1 when T > 0).
 *   max_seqlen   an upper bound on every sequence length (>= 1 when T > 0);
 *                sizes the launch grid.  With cu_seqlens == NULL it must be
 *                T / nseq, or <= 0 to let the library take that value.
 *   T, H, Hkv, d sizes; H % Hkv == 0.  Compiled (dtype, d) pairs: see
 *                diffattn_supported.
 *   rope_cos, rope_sin
 *                NULL (both) when q and k are already rotated; otherwise
 *                device tables [rope_len, d/2] of rope_dtype (16-byte
 *                aligned), and the kernel applies the rotary prologue of the
 *                FlashDiffAttention pull request's test (apply_rotary_emb
 *                with interleaved=True on every d-wide half-head of q and k):
 *                the pair (x[2j], x[2j+1]) of a row at position p of its
 *                sequence (0-based, restarting in every packed sequence)
 *                becomes (x0 c - x1 s, x0 s + x1 c) with c = rope_cos[p, j],
 *                s = rope_sin[p, j]; computed in fp32, rounded once to the
 *                storage type.  V is not rotated.
 *   rope_len     rows of the tables; >= max_seqlen when they are given.
 *   rope_dtype   DIFFATTN_F32 or DIFFATTN_BF16: the tables' element type
 *                (the pull request's test caches them in bf16; a bf16 entry
 *                enters the fp32 arithmetic exactly).  Ignored without
 *                tables.
 *   workspace, workspace_bytes
 *                with rotary tables: device scratch of at least
 *                diffattn_fwd_workspace_size(dtype, T, Hkv, d, 1) bytes,
 *                16-byte aligned, owned by the caller, holding the rotated
 *                copy of k during the call (no initialisation needed; calls
 *                in flight at once need separate workspaces).  Without
 *                tables it is not used (NULL, 0).
 *   out          device output [T, H, 2d], same element type as q.
 *   stream       a hipStream_t, or NULL for the null stream.
 *
 * Returns DIFFATTN_OK (also for T == 0, which launches nothing),
 * DIFFATTN_EINVAL, DIFFATTN_EUNSUPPORTED or DIFFATTN_EHIP.
 */
int diffattn_fwd(int dtype, const void *q, const void *k, const void *v,
                 const float *lambda_q1, const float *lambda_k1,
                 const float *lambda_q2, const float *lambda_k2,
                 int32_t lambda_stride, float lambda_init,
                 const float *subln_weight, float eps,
                 int causal, const int32_t *cu_seqlens, int32_t nseq,
                 int32_t max_seqlen, int32_t T, int32_t H, int32_t Hkv,
                 int32_t d, const void *rope_cos, const void *rope_sin,
                 int32_t rope_len, int rope_dtype, void *workspace,
                 size_t workspace_bytes, void *out, void *stream);

/* Bytes of workspace diffattn_fwd needs: the rotated copy of k when rope
 * (rotary tables given) is nonzero, else 0.  Host function. */
size_t diffattn_fwd_workspace_size(int dtype, int32_t T, int32_t Hkv, int32_t d,
                                   int rope);

/*
 * New queries against a key/value cache (decoding), asynchronous on
 * `stream`.  The LlamaDiffSdpaAttention.py gist's forward appends the step's
 * keys and values to the layer's cache and then attends from the new
 * queries to the whole cache; the FlashDiffAttention pull request's
 * alternative_forward aligns the causal mask bottom-right (-inf above
 * diagonal 1 + src_len - tgt_len).  So, per sequence s with nq new queries
 * and nk cached keys (the new tokens' own keys being the last nq of them),
 * query i (0-based) sees keys j <= nk - nq + i when causal == 1 and all nk
 * keys when causal == 0; everything else is as in diffattn_fwd.  With
 * nq == nk this is diffattn_fwd's causal prefill; a prompt cut into chunks
 * (each chunk's keys appended before its queries attend) gives, chunk by
 * chunk, the rows of its one-shot prefill.
 *
 * Three kernel paths, chosen on the host from the sizes (see
 * diffattn_fwd_kv_path): few query rows per sequence (decoding) split the
 * keys over many workgroups and merge the partial results in a second
 * kernel, through the workspace; longer query chunks (4 rows or more, when
 * the library's cost estimate favours it) run on diffattn_fwd's prefill
 * kernel with the keys' own boundaries -- in one kernel and with no
 * workspace, or, when that grid would leave compute units idle, on key
 * splits whose partials the second kernel merges through the workspace.
 *
 *   q            device [Tq, H, 2, d]: the new queries, packed by
 *                cu_seqlens_q.
 *   k, v         device [Tk, Hkv, 2, d] and [Tk, Hkv, 2d]: the caches,
 *                packed by cu_seqlens_k (sequence s owns rows
 *                cu_seqlens_k[s] .. cu_seqlens_k[s+1]-1).
 *   lambda_*, lambda_stride, lambda_init, subln_weight, eps
 *                as for diffattn_fwd.
 *   causal       1: bottom-right causal as above; 0: every cached key.
 *   cu_seqlens_q, cu_seqlens_k
 *                device int32 [nseq + 1] boundaries (cu[0] = 0,
 *                non-decreasing, cu_q[nseq] = Tq, cu_k[nseq] = Tk), both
 *                given or both NULL (NULL: nseq sequences of Tq / nseq
 *                queries and Tk / nseq keys).  Preconditions, not read here:
 *                every sequence with nq > 0 has nk >= 1, and nk >= nq when
 *                causal (see diffattn_check_cu_seqlens_kv).
 *   max_seqlen_q, max_seqlen_k
 *                upper bounds on every nq and nk (ignored when the
 *                boundaries are NULL); with H, Hkv and d they choose the
 *                path, and max_seqlen_q sizes the grid and the workspace.
 *                The split path cuts keys into pieces of one size for all
 *                sequences, chosen from Tk.
 *   Tq, Tk, H, Hkv, d
 *                sizes; H % Hkv == 0.  Compiled (dtype, d) pairs: see
 *                diffattn_supported_kv.
 *   rope_cos, rope_sin, rope_len, rope_dtype
 *                NULL (both) when q is already rotated.  Otherwise tables
 *                as for diffattn_fwd (rope_len >= max_seqlen_k), and each
 *                new query is rotated in the kernel at its absolute
 *                position nk - nq + i, as the gist's forward rotates the
 *                step's queries at their position ids.  The cached keys are
 *                used as they are: a rotated cache holds each key already
 *                rotated at its own position (diffattn_kv_append writes
 *                them so).
 *   workspace, workspace_bytes
 *                device scratch (16-byte aligned, owned by the caller) for
 *                the fp32 partial results passed between the two kernels of
 *                one call; its contents need no initialisation and are
 *                meaningless afterwards.  Two calls in flight at once (on
 *                different streams) need different workspaces.  The call
 *                takes the path and split plan with the lowest estimate
 *                among those whose partials fit workspace_bytes (0 when
 *                workspace is NULL; the prefill kernel alone needs none).
 *                diffattn_fwd_kv_workspace_size(nseq, max_seqlen_q,
 *                max_seqlen_k, H, Hkv, d) bytes are enough for the
 *                library's first choice at these bounds, and a workspace of
 *                that size serves every call within them; with less, a call
 *                may run a slower plan (different rounding order), and one
 *                whose only path does not fit (fewer than 4 query rows in
 *                the longest sequence) returns DIFFATTN_EINVAL.
 *   out          device [Tq, H, 2d], same element type as q.
 *
 * Returns DIFFATTN_OK (also when there is no query row, which launches
 * nothing), DIFFATTN_EINVAL (including a workspace smaller than required),
 * DIFFATTN_EUNSUPPORTED or DIFFATTN_EHIP.
 */
int diffattn_fwd_kv(int dtype, const void *q, const void *k, const void *v,
                    const float *lambda_q1, const float *lambda_k1,
                    const float *lambda_q2, const float *lambda_k2,
                    int32_t lambda_stride, float lambda_init,
                    const float *subln_weight, float eps, int causal,
                    const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                    int32_t nseq, int32_t max_seqlen_q, int32_t max_seqlen_k,
                    int32_t Tq, int32_t Tk, int32_t H, int32_t Hkv, int32_t d,
                    const void *rope_cos, const void *rope_sin, int32_t rope_len,
                    int rope_dtype, void *workspace, size_t workspace_bytes,
                    void *out, void *stream);

/*
 * diffattn_fwd_kv without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The split partials go to a
 * static device array of DIFFATTN_KV_SCRATCH_BYTES that the library owns:
 * one per GPU, created with the code object and held until the process
 * ends.  The call allocates nothing (no hipMalloc or allocating library
 * routine); the first call on a device looks up that device's array.
 *
 * Arguments, results and errors as for diffattn_fwd_kv, minus workspace and
 * workspace_bytes: the call takes the path and plan diffattn_fwd_kv takes
 * with a workspace of DIFFATTN_KV_SCRATCH_BYTES, and its output is bitwise
 * that call's (which is the output with diffattn_fwd_kv_workspace_size
 * bytes whenever that size is no larger than the scratch).  When no path
 * fits the scratch (fewer than 4 query rows in the longest sequence and
 * split-KV partials larger than DIFFATTN_KV_SCRATCH_BYTES) the call returns
 * DIFFATTN_ETOOLARGE before any device work.  On the prefill kernel alone
 * no scratch is used.
 *
 * All calls on one GPU share its array, and it keeps the last call's
 * partials (nothing needs to start at zero: each call writes every partial
 * it reads).  Calls that overlap in time on one GPU (several streams, or
 * several host threads without ordering) race on the array and give wrong
 * results: order them on one stream, or use diffattn_fwd_kv with separate
 * workspaces.
 */
#define DIFFATTN_KV_SCRATCH_BYTES (32u << 20)

int diffattn_fwd_kv_noalloc(int dtype, const void *q, const void *k,
                            const void *v, const float *lambda_q1,
                            const float *lambda_k1, const float *lambda_q2,
                            const float *lambda_k2, int32_t lambda_stride,
                            float lambda_init, const float *subln_weight,
                            float eps, int causal, const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int32_t nseq,
                            int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t Tq, int32_t Tk, int32_t H, int32_t Hkv,
                            int32_t d, const void *rope_cos,
                            const void *rope_sin, int32_t rope_len,
                            int rope_dtype, void *out, void *stream);

/* Bytes of workspace for diffattn_fwd_kv at these bounds: the split-KV
 * plan's, or the prefill kernel's key-split plan's when that is larger and
 * the library may choose it; 0 for sizes it rejects.  A call within these
 * bounds (smaller max_seqlen_q, max_seqlen_k or totals) given this many
 * bytes always finds a path that fits.  Host function. */
size_t diffattn_fwd_kv_workspace_size(int32_t nseq, int32_t max_seqlen_q,
                                      int32_t max_seqlen_k, int32_t H,
                                      int32_t Hkv, int32_t d);

/* The kernels diffattn_fwd_kv runs for these bounds and totals (bf16, the
 * dtype the cache path supports) given a workspace of workspace_bytes
 * (SIZE_MAX: the library's first choice): 0 the split-KV partial kernel and
 * the combine kernel, 1 the prefill kernel alone, 2 the prefill kernel on
 * key splits and the combine kernel; -1 for sizes it rejects (including Tq
 * or Tk < 1).  The split-KV estimate follows the totals, the prefill
 * kernel's the bounds.  workspace_needed (may be NULL) receives the bytes
 * of workspace the chosen plan uses; on path 0 they can exceed
 * workspace_bytes, and the call then returns DIFFATTN_EINVAL.  Host
 * function. */
int diffattn_fwd_kv_path(int32_t nseq, int32_t max_seqlen_q,
                         int32_t max_seqlen_k, int32_t Tq, int32_t Tk,
                         int32_t H, int32_t Hkv, int32_t d,
                         size_t workspace_bytes, size_t *workspace_needed);

/*
 * diffattn_fwd_kv on a path the caller picks (path 0, 1 or 2, numbered as
 * diffattn_fwd_kv_path numbers them) instead of the library's choice, for
 * callers that pin the kernels -- the rounding order, and so the bits of a
 * row, then no longer depend on the rest of the batch -- and for tests of
 * each path.  Path 2 takes the split size with the lowest estimate among
 * those whose partials fit workspace_bytes.  The other arguments, results
 * and errors are diffattn_fwd_kv's; with
 * diffattn_fwd_kv_path_workspace_size(path, ...) bytes path 2 gets its
 * first choice, path 0 needs that many, path 1 none (NULL allowed).
 * Returns DIFFATTN_EINVAL also for a path outside 0..2, and for path 2 when
 * the keys are too few to split or no split's partials fit.
 */
int diffattn_fwd_kv_on_path(int path, int dtype, const void *q, const void *k,
                            const void *v, const float *lambda_q1,
                            const float *lambda_k1, const float *lambda_q2,
                            const float *lambda_k2, int32_t lambda_stride,
                            float lambda_init, const float *subln_weight,
                            float eps, int causal, const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int32_t nseq,
                            int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t Tq, int32_t Tk, int32_t H, int32_t Hkv,
                            int32_t d, const void *rope_cos,
                            const void *rope_sin, int32_t rope_len,
                            int rope_dtype, void *workspace,
                            size_t workspace_bytes, void *out, void *stream);

/* Bytes of workspace diffattn_fwd_kv_on_path needs on `path` for these
 * bounds: 0 for path 1, and for sizes or paths it rejects.  Host
 * function. */
size_t diffattn_fwd_kv_path_workspace_size(int path, int32_t nseq,
                                           int32_t max_seqlen_q,
                                           int32_t max_seqlen_k, int32_t H,
                                           int32_t Hkv, int32_t d);

/*
 * The cache update of a decode step, asynchronous on `stream`: the
 * LlamaDiffSdpaAttention.py gist's forward rotates the step's keys at their
 * position ids and appends them and the values to the layer's cache
 * (past_key_value.update) before it attends.  For every sequence s, its nq
 * new tokens i = 0 .. nq-1 (packed by cu_seqlens_q) go to the last nq rows
 * of its cache region (packed by cu_seqlens_k, nk rows with the new ones
 * counted): cache row cu_seqlens_k[s+1] - nq + i, position nk - nq + i.
 * The key is rotated there as diffattn_fwd rotates keys (interleaved pairs
 * of each d-wide half-head, fp32 arithmetic, rounded once to the storage
 * type) when tables are given, else copied; the value is copied.  Every
 * other cache row is left as it is.
 *
 *   dtype        DIFFATTN_BF16 or DIFFATTN_F32: element type of keys and
 *                values; d = 16, 32 or 64.
 *   k_new, v_new device [Tq, Hkv, 2, d] and [Tq, Hkv, 2d].
 *   cu_seqlens_q, cu_seqlens_k, nseq, max_seqlen_k, Tq, Tk
 *                as for diffattn_fwd_kv (both NULL: nseq sequences of
 *                Tq / nseq new tokens and Tk / nseq cache rows, and
 *                max_seqlen_k ignored).  Precondition, not read here:
 *                nq <= nk for every sequence (a sequence that breaks it is
 *                left unwritten).
 *   rope_cos, rope_sin, rope_len, rope_dtype
 *                as for diffattn_fwd_kv (rope_len >= max_seqlen_k, so the
 *                tables cover every cache position; NULL tables: no
 *                rotation, rope_len and rope_dtype ignored).
 *   k_cache, v_cache
 *                device [Tk, Hkv, 2, d] and [Tk, Hkv, 2d], written in
 *                place; they must not overlap k_new or v_new.
 * All pointers 16-byte aligned.  Returns DIFFATTN_OK (Tq == 0 launches
 * nothing), DIFFATTN_EINVAL, DIFFATTN_EUNSUPPORTED or DIFFATTN_EHIP.
 */
int diffattn_kv_append(int dtype, const void *k_new, const void *v_new,
                       const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                       int32_t nseq, int32_t max_seqlen_k, int32_t Tq, int32_t Tk,
                       int32_t Hkv, int32_t d,
                       const void *rope_cos, const void *rope_sin, int32_t rope_len,
                       int rope_dtype, void *k_cache, void *v_cache, void *stream);

/* 1 if the cache kernel is compiled for (dtype, d), else 0.  Host
 * function. */
int diffattn_supported_kv(int dtype, int d);

/* Host-side check of host copies of cu_seqlens_q and cu_seqlens_k against
 * the preconditions of diffattn_fwd_kv (both well-formed for Tq and Tk,
 * lengths within the bounds, nk >= 1 where nq >= 1, nk >= nq when causal).
 * Returns DIFFATTN_OK or DIFFATTN_EINVAL. */
int diffattn_check_cu_seqlens_kv(const int32_t *host_cu_q,
                                 const int32_t *host_cu_k, int32_t nseq,
                                 int32_t Tq, int32_t Tk, int32_t max_seqlen_q,
                                 int32_t max_seqlen_k, int causal);

/*
 * Training forward: diffattn_fwd (without the rotary prologue) that also
 * saves what diffattn_bwd needs.  Extra outputs, device fp32, written for
 * every row:
 *   lse  [T, H, 2]      per map m, log2 of the sum over the row's visible
 *                       keys of 2^(<Qm, Km[j]> log2(e) / sqrt(d)) (4-byte
 *                       aligned);
 *   o12  [T, H, 2, 2d]  the normalised outputs O_1 and O_2 of the two maps
 *                       (16-byte aligned).  They are kept in fp32 because the
 *                       backward forms O_1 - lambda O_2, which can cancel.
 * Other arguments, return values and errors as for diffattn_fwd.
 */
int diffattn_fwd_train(int dtype, const void *q, const void *k, const void *v,
                       const float *lambda_q1, const float *lambda_k1,
                       const float *lambda_q2, const float *lambda_k2,
                       int32_t lambda_stride, float lambda_init,
                       const float *subln_weight, float eps, int causal,
                       const int32_t *cu_seqlens, int32_t nseq,
                       int32_t max_seqlen, int32_t T, int32_t H, int32_t Hkv,
                       int32_t d, void *out, float *lse, float *o12,
                       void *stream);

/*
 * Backward pass of the prefill (inputs already rotated), asynchronous on
 * `stream`: the gradients of sum(dout * out) for the output `out` of
 * diffattn_fwd_train with the same arguments.  The chain (DiffTransformer
 * page, MultiHeadDifferentialAttention.forward, differentiated), per row
 * (token i, head h) with g = dout * w * (1 - lambda_init) and
 * r = 1 / sqrt(mean(pre^2) + eps):
 *   dpre  = r g - r^3 pre <g, pre> / (2d)
 *   dO_1  = dpre,  dO_2 = -lambda_h dpre,  dlambda_h += -<dpre, O_2>
 *   per map m: dS_m = P_m (dO_m V^T - <dO_m, O_m>)
 *              dQ_m = dS_m K_m / sqrt(d),  dK_m = dS_m^T Q_m / sqrt(d)
 *   dV    = P_1^T dO_1 + P_2^T dO_2
 *   dw    = sum over rows of dout * pre * r * (1 - lambda_init)
 *   lambda = exp(a) - exp(b) + lambda_init, a = <lq1, lk1>, b = <lq2, lk2>:
 *   dlq1 = dlambda e^a lk1, dlk1 = dlambda e^a lq1,
 *   dlq2 = -dlambda e^b lk2, dlk2 = -dlambda e^b lq2
 * (dlambda summed over all heads when the vectors are shared).
 *
 *   dtype        DIFFATTN_BF16 or DIFFATTN_F32, d = 16, 32 or 64 (see
 *                diffattn_supported_bwd).  bf16 at d = 32 and 64 runs the
 *                MFMA kernels (bf16 operands, fp32 accumulation); the other
 *                pairs run exact kernels that keep every intermediate in
 *                fp32 and round only the stored gradients.
 *   q .. max_seqlen, T, H, Hkv, d
 *                exactly as given to diffattn_fwd_train (H <= 256).
 *   dout         device [T, H, 2d], storage type.
 *   lse, o12     device, as written by diffattn_fwd_train.
 *   dq, dk, dv   device outputs in the layouts and storage type of q, k, v
 *                (overwritten, not accumulated).
 *   dlambda_q1 .. dlambda_k2
 *                device fp32 outputs laid out like the lambda vectors
 *                (d elements, or H sets lambda_stride apart).
 *   dsubln_weight device fp32 [2d] output, or NULL to skip it.
 *   workspace    device scratch of diffattn_bwd_workspace_size(dtype, T, H, d)
 *                bytes, 16-byte aligned, owned by the caller; no
 *                initialisation needed; calls in flight at once need
 *                separate workspaces.
 * Every output is a pure function of the inputs: there are no atomics, and
 * repeated calls give bitwise equal results.  Returns DIFFATTN_OK (T == 0
 * launches nothing and writes nothing), DIFFATTN_EINVAL,
 * DIFFATTN_EUNSUPPORTED or DIFFATTN_EHIP.
 */
int diffattn_bwd(int dtype, const void *q, const void *k, const void *v,
                 const float *lambda_q1, const float *lambda_k1,
                 const float *lambda_q2, const float *lambda_k2,
                 int32_t lambda_stride, float lambda_init,
                 const float *subln_weight, float eps, int causal,
                 const int32_t *cu_seqlens, int32_t nseq, int32_t max_seqlen,
                 int32_t T, int32_t H, int32_t Hkv, int32_t d,
                 const void *dout, const float *lse, const float *o12,
                 void *dq, void *dk, void *dv, float *dlambda_q1,
                 float *dlambda_k1, float *dlambda_q2, float *dlambda_k2,
                 float *dsubln_weight, void *workspace, size_t workspace_bytes,
                 void *stream);

/* Bytes of workspace diffattn_bwd needs for (dtype, T, H, d); 0 for sizes
 * or (dtype, d) pairs it rejects.  Host function. */
size_t diffattn_bwd_workspace_size(int dtype, int32_t T, int32_t H, int32_t d);

/* 1 if the backward kernels are compiled for (dtype, d), else 0.  Host
 * function. */
int diffattn_supported_bwd(int dtype, int d);

/* Initial lambda of a layer at 1-based depth: 0.8 - 0.6 * exp(-0.3 *
 * (depth - 1)), the decaying schedule with which DiffTransformer.__init__
 * builds its layers.  Host function; no device work. */
double diffattn_lambda_init(int depth);

/* 1 if the kernel is compiled for (dtype, d), else 0.  Host function. */
int diffattn_supported(int dtype, int d);

/* Host-side check of a host copy of cu_seqlens against the preconditions of
 * diffattn_fwd (cu[0] == 0, non-decreasing, cu[nseq] == T, every length
 * <= max_seqlen).  Returns DIFFATTN_OK or DIFFATTN_EINVAL. */
int diffattn_check_cu_seqlens(const int32_t *host_cu, int32_t nseq, int32_t T,
                              int32_t max_seqlen);

/* Static text for a status code; never NULL. */
const char *diffattn_strerror(int status);

/* DIFFATTN_ABI_VERSION of the built library. */
int diffattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */
