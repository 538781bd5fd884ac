/*
 * msa.h - C ABI of libmsa, the MI355X (gfx950) hot path of MiniMax Sparse
 * Attention (MSA): the index branch (block scoring and exp-free causal top-k)
 * and the main branch (exact softmax attention over the selected blocks) for
 * prefill and paged decode; around it the index projections with RoPE and
 * the training path (gradients of the main branch and the KL-alignment term).
 *
 * Sources:
 *   [P1] "MiniMax Sparse Attention" digest, titansim.online blog:
 *        §2.2 Eq. (1), §3.1 (shapes), §4.2 Eq. (6), §4.3 Eq. (8),
 *        §4.4.1 (exp-free top-k), §4.4.2 (KV-outer traversal, tile chunking
 *        with a two-stage merge), §4.5 (KL alignment, gradient detach),
 *        §5.2 Eq. (12).
 *   [P4] "MiniMax Sparse Attention: Block-Level Top-K for Affordable
 *        Million-Token Contexts", zhichai.net, key points (block size 128,
 *        k = 16, 128-token-aligned memory transfers).
 *   [P5] 163.com commentary on MSA, "Step 1 Index Attention" (one index
 *        query per GQA group, one shared index key, block max-pool).
 *
 * Conventions common to every call
 *   - All tensor pointers are DEVICE pointers owned by the caller; they must
 *     stay valid until the work queued on `hip_stream` has finished.  The
 *     library keeps no pointer after a call returns and allocates no device
 *     memory: scratch space comes from the caller's `workspace`, sized by
 *     msa_workspace_size().  Workspace contents need not be initialised.
 *   - Calls are asynchronous and stream ordered on `hip_stream` (a
 *     hipStream_t; NULL = the null stream).  They never synchronise the host.
 *   - Every float tensor of a call has the dtype `shape->dtype` (bf16 or
 *     fp32), except the caches when `shape->cache_dtype` is MSA_FP8_E4M3 or
 *     MSA_MXFP8_E4M3;
 *     outputs use `shape->dtype`; `lse`, `block_score` and KL values are fp32.
 *   - Arguments are validated on the host before anything is launched.  On
 *     an error the call returns a non-zero msa_status, launches nothing and
 *     leaves every output untouched; msa_last_error() then describes it.
 *     A failed launch returns MSA_ERR_HIP.  Nothing aborts or throws.
 *   - Block b of a sequence is the token range [128 b, 128 b + 127].  The
 *     block size is fixed at 128 ([P1] §3.1; [P4]).
 *   - Query head h belongs to KV group r = h / (h_q / h_kv).
 *   - Block-index lists are ascending, unique, padded with -1 to `top_k`.
 *
 * Layouts
 *   contiguous cache:  k, v   [n_kv, h_kv, d_h]   k_idx [n_kv, d_idx]
 *   paged cache:       k, v   [num_pages, h_kv, 128, d_h]  (head-major page)
 *                      k_idx  [num_pages, 128, d_idx]
 *                      page_table [batch, max_pages] int32: block b of
 *                      sequence s lives in physical page page_table[s*max_pages+b]
 *   All row-major, densely packed, 16-byte aligned base pointers.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 6
#define MSA_BLOCK_SIZE 128
#define MSA_MAX_TOP_K 16

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent shape    */
  MSA_ERR_UNSUPPORTED = 2, /* valid but not built: d_h, d_idx, k, dtype ...  */
  MSA_ERR_WORKSPACE = 3,   /* workspace too small or misaligned              */
  MSA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed     */
} msa_status;

/* MSA_FP8_E4M3: OCP 8-bit float e4m3 ("fn": bias 7, no infinities), one
 * byte per element, used as stored (no scale).  Only for the caches.
 * MSA_MXFP8_E4M3: the OCP microscaling format MXFP8 with e4m3 elements, the
 * 8-bit KV-cache format named on the zhichai.net key points page
 * (Limitations): the same one-byte e4m3 codes, plus one E8M0 scale byte per
 * 32 consecutive elements of a row (value 2^(s - 127); 0xFF is NaN).  An
 * element's value is its e4m3 value times its block's scale.  The scale
 * arrays are separate tensors (msa_kv k_scale, v_scale, k_idx_scale).  Only
 * for the caches. */
typedef enum msa_dtype { MSA_BF16 = 0, MSA_FP32 = 1, MSA_FP8_E4M3 = 2, MSA_MXFP8_E4M3 = 3 } msa_dtype;

/* Block scoring of the index branch.  MSA_POOL_MAX is the method's max-pool
 * ([P1] §4.2 Eq. (6)); MSA_POOL_MEAN averages the visible token scores of a
 * block instead, the block scoring the [P5] commentary ("Step 1 Index
 * Attention") contrasts MSA with (MoBA), kept as an ablation. */
typedef enum msa_pool { MSA_POOL_MAX = 0, MSA_POOL_MEAN = 1 } msa_pool;

/* Head shapes and method hyper-parameters.
 *   h_q, h_kv    query heads and KV heads (GQA groups); h_q % h_kv == 0 and
 *                G = h_q / h_kv in {1, 2, 4, 8, 16}.
 *   d_h          head dim of q/k/v: 64 or 128.
 *   d_idx        index dim of q_idx/k_idx: 32, 64 or 128 (the pages leave it
 *                open; [P1] §4.2 calls it low-dimensional).
 *   block_size   must be 128.
 *   top_k        blocks per (query, group), 1..16 ([P1] §3.1 uses 16).
 *   force_local  1: the query's own (diagonal) block always takes one of the
 *                k slots ([P1] §4.2); 0: plain top-k over visible blocks.
 *   sm_scale     softmax scale of Eq. (8); 0 means 1/sqrt(d_h).
 *   idx_scale    score scale of Eq. (6); 0 means 1/sqrt(d_idx).
 *   dtype        msa_dtype (BF16 or FP32) of every float tensor of the call.
 *   cache_dtype  MSA_FP8_E4M3: the caches k, v and k_idx hold e4m3 codes
 *                (with dtype MSA_BF16; every call except
 *                msa_dense_prefill, msa_sparse_prefill_backward and
 *                msa_index_project); they are widened exactly to bf16
 *                before use.  MSA_MXFP8_E4M3: the same codes times their
 *                block scales (msa_kv), for the same calls; the scaled
 *                values are exact in bf16 whenever they lie in bf16's
 *                range.  Any other value: the caches have type `dtype`.
 *   pool         msa_pool: block scoring of msa_index_topk (other calls
 *                ignore it). */
typedef struct msa_shape {
  int32_t h_q, h_kv, d_h, d_idx, block_size, top_k, force_local;
  float sm_scale, idx_scale;
  int32_t dtype;
  int32_t cache_dtype;
  int32_t pool;
} msa_shape;

/* The KV side of a call.
 *   page_table == NULL: contiguous single-sequence cache of n_kv tokens.
 *   page_table != NULL: paged cache; max_pages = columns of page_table.
 *     seq_lens == NULL: one sequence (batch must be 1) of n_kv tokens.
 *     seq_lens != NULL: device int32 [batch], tokens held per sequence,
 *                       each in [1, 128*max_pages] (decode calls).
 *   k_scale, v_scale, k_idx_scale: with cache_dtype MSA_MXFP8_E4M3, device
 *     uint8 E8M0 scales of k, v and k_idx, each laid out like its cache with
 *     the last dimension divided by 32 (contiguous: [n_kv, h_kv, d_h/32] and
 *     [n_kv, d_idx/32]; paged: [num_pages, h_kv, 128, d_h/32] and
 *     [num_pages, 128, d_idx/32]); scale s of row j covers elements
 *     32 s .. 32 s + 31 of that row.  The index call needs k_idx_scale, the
 *     attention calls k_scale and v_scale; NULL otherwise (ignored for
 *     other cache dtypes).                                              */
typedef struct msa_kv {
  const void* k;
  const void* v;
  const void* k_idx;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int32_t n_kv;
  int32_t max_pages;
  const uint8_t* k_scale;
  const uint8_t* v_scale;
  const uint8_t* k_idx_scale;
} msa_kv;

/* Index branch: [P1] §4.2 Eq. (6) and §4.4.1; shapes from [P5] Step 1.
 * For every query and KV group r:
 *   S_j  = q_idx^(r) . k_idx_j * idx_scale           for keys j <= p
 *   M_b  = max over visible j in block b of S_j      (block max-pool; with
 *          pool == MSA_POOL_MEAN the mean over the same keys)
 *   I    = exp-free top-k of M (ties: lower block wins), diagonal block
 *          kept when force_local.
 * Two modes, chosen by kv->seq_lens:
 *   prefill (seq_lens == NULL): batch must be 1; q_idx [n_q, h_kv, d_idx];
 *     query i sits at position q_start + i; q_start + n_q <= kv->n_kv.
 *   decode  (seq_lens != NULL, paged): n_q must be 1, q_start is ignored;
 *     q_idx [batch, h_kv, d_idx]; the query of sequence s sits at position
 *     seq_lens[s] - 1 and the cache already holds it.
 * Outputs: block_idx int32 [batch*n_q, h_kv, top_k]; block_score (nullable)
 *   fp32, same shape: the pooled score of each listed block (-inf for -1).
 *   Uses k_idx only; k and v may be NULL.                               */
msa_status msa_index_topk(const msa_shape* shape, int32_t batch, int32_t n_q,
                          int32_t q_start, const void* q_idx, const msa_kv* kv,
                          int32_t* block_idx, float* block_score,
                          void* workspace, size_t ws_bytes, void* hip_stream);

/* Main branch, prefill: [P1] §4.3 Eq. (8), run KV-outer (§4.4.2).
 *   q [n_q, h_q, d_h]; query i at position q_start + i; one sequence
 *   (contiguous, or paged with seq_lens == NULL); block_idx int32
 *   [n_q, h_kv, top_k] as produced by msa_index_topk (any ascending -1
 *   padded list of blocks b <= (q_start+i)/128 is accepted).
 *   Each head of group r attends with exact softmax to the causally visible
 *   keys (j <= p) of its group's listed blocks.
 * Outputs: o [n_q, h_q, d_h] (dtype of the call, round-to-nearest-even);
 *   lse (nullable) fp32 [n_q, h_q], natural-log sum of exp of the scaled
 *   scores.  A query with no listed block gets o = 0, lse = -inf.        */
msa_status msa_sparse_prefill(const msa_shape* shape, int32_t n_q, int32_t q_start,
                              const void* q, const msa_kv* kv,
                              const int32_t* block_idx, void* o, float* lse,
                              void* workspace, size_t ws_bytes, void* hip_stream);

/* Main branch, decode: Eq. (8) for the newest token of each sequence.
 *   q [batch, h_q, d_h]; kv must be paged with seq_lens; block_idx int32
 *   [batch, h_kv, top_k] (from msa_index_topk in decode mode).
 * Outputs: o [batch, h_q, d_h]; lse (nullable) fp32 [batch, h_q].        */
msa_status msa_sparse_decode(const msa_shape* shape, int32_t batch, const void* q,
                             const msa_kv* kv, const int32_t* block_idx, void* o,
                             float* lse, void* workspace, size_t ws_bytes,
                             void* hip_stream);

/* Training path: gradients of msa_sparse_prefill ([P1] §4.3 Eq. (8), for
 * the training of §4.5) for one contiguous sequence.  With P the softmax of
 * a (token, head) row over the visible keys of its group's selected blocks
 * (recomputed from the forward's lse), dP = d_o.V^T and D = rowsum(d_o*o):
 *   dS = P*(dP - D),  dq = sm_scale dS.K,  dk = sm_scale dS^T.Q,  dv = P^T.d_o.
 *   q, o, d_o, dq   [n_q, h_q, d_h]      o and lse are the forward's outputs
 *   lse             [n_q, h_q] fp32      (natural log, as msa_sparse_prefill)
 *   kv->k, kv->v    [n_kv, h_kv, d_h]    contiguous (page_table and seq_lens
 *                                        NULL); block_idx as in the forward
 *   dk, dv          [n_kv, h_kv, d_h]    written in full: keys no query
 *                                        attends get 0
 * Built for dtype MSA_BF16 (bf16 caches) and d_h 64/128; other shapes
 * return MSA_ERR_UNSUPPORTED.  Accumulation is fp32 without atomics, so
 * results are bitwise reproducible.
 *
 * kl (nullable): also the KL-alignment term of [P1] §4.5 and the [P4] key
 * points, in the same pass over the selected blocks.  For each query and
 * group over the same visible keys T:
 *   target     p_main(j) = mean over the group's heads of P (detached)
 *   prediction p_idx(j)  = softmax over T of S_idx(j) = q_idx.k_idx_j * idx_scale
 *   KL_row = sum_j p_main(j) (ln p_main(j) - ln p_idx(j));
 *   L = kl_scale * sum over rows of KL_row, differentiated only in q_idx and
 *   k_idx: dq_idx = idx_scale sum_j dS_idx(j) k_idx_j, dk_idx_j = idx_scale
 *   sum over rows of dS_idx(j) q_idx, dS_idx = kl_scale (p_idx - p_main).
 *   kl->q_idx [n_q, h_kv, d_idx], kl->k_idx [n_kv, d_idx] (bf16, contiguous);
 *   kl->kl_out [n_q, h_kv] fp32 (nullable); kl->dq_idx, kl->dk_idx (bf16,
 *   shapes of q_idx, k_idx; dk_idx written in full).  idx_scale comes from
 *   the shape (0 -> 1/sqrt(d_idx)).
 * Workspace: msa_workspace_size(5, ...) without kl, (6, ...) with kl.       */
typedef struct msa_kl {
  const void* q_idx;
  const void* k_idx;
  float kl_scale;
  float* kl_out;
  void* dq_idx;
  void* dk_idx;
} msa_kl;

msa_status msa_sparse_prefill_backward(const msa_shape* shape, int32_t n_q, int32_t q_start,
                                       const void* q, const msa_kv* kv, const int32_t* block_idx,
                                       const void* o, const float* lse, const void* d_o, void* dq,
                                       void* dk, void* dv, const msa_kl* kl, void* workspace,
                                       size_t ws_bytes, void* hip_stream);

/* The steps before the index branch ([P1] §4.2: one index-query projection
 * per GQA group and one shared index-key projection; §3.1: RoPE on 64 dims):
 * for each of n_tok tokens with hidden state x_t at position positions[t],
 *   q_idx[t, r] = RoPE(W_q_idx[r] . x_t, positions[t]),  r < h_kv
 *   k_idx_t     = RoPE(W_k_idx . x_t, positions[t])
 * RoPE turns the pair of dims (i, i + rope_dim/2), i < rope_dim/2, by the
 * angle positions[t] * rope_base^(-2i/rope_dim) (rope_dim 0, 32, 64 or 128,
 * at most d_idx; dims from rope_dim on are left as they are).
 *   x        [n_tok, d_model] bf16; d_model a positive multiple of 16
 *   w_q_idx  [h_kv, d_idx, d_model] bf16; w_k_idx [d_idx, d_model] bf16
 *   positions, seq  device int32 [n_tok]; seq nullable (row 0)
 *   q_idx_out [n_tok, h_kv, d_idx] bf16
 * k_idx_t is appended to the index-key cache kv->k_idx in place: contiguous
 * (page_table NULL) at row positions[t] if it is in [0, n_kv); paged at row
 * positions[t] % 128 of page page_table[seq[t] * max_pages + positions[t] /
 * 128] if positions[t] / 128 < max_pages.  Rows out of range are skipped.
 * bf16 only (dtype MSA_BF16, bf16 cache).
 * Workspace: msa_workspace_size(7, shape, 0, n_tok, 0, d_model, 0) bytes
 *   (d_model passed in the n_kv slot); non-zero only for short calls (fewer
 *   than 256 tokens), which split d_model over workgroups and add the fp32
 *   partial sums in a second kernel.                                      */
msa_status msa_index_project(const msa_shape* shape, int32_t n_tok, int32_t d_model, const void* x,
                             const void* w_q_idx, const void* w_k_idx, int32_t rope_dim, float rope_base,
                             const int32_t* positions, const int32_t* seq, const msa_kv* kv,
                             void* q_idx_out, void* workspace, size_t ws_bytes, void* hip_stream);

/* Dense causal GQA attention, [P1] §2.2 Eq. (1): the comparison kernel.
 *   Same arguments as msa_sparse_prefill without block_idx; contiguous cache
 *   only.  top_k, force_local and the index fields of `shape` are ignored. */
msa_status msa_dense_prefill(const msa_shape* shape, int32_t n_q, int32_t q_start,
                             const void* q, const msa_kv* kv, void* o, float* lse,
                             void* workspace, size_t ws_bytes, void* hip_stream);

/* Workspace bytes a call needs.  op: 0 = msa_index_topk in prefill mode,
 * 1 = msa_sparse_prefill, 2 = msa_sparse_decode, 3 = msa_dense_prefill,
 * 4 = msa_index_topk in decode mode, 5 = msa_sparse_prefill_backward,
 * 6 = msa_sparse_prefill_backward with the KL-alignment term,
 * 7 = msa_index_project (n_q = n_tok, n_kv = d_model).
 * Pass the same shape, batch, n_q,
 * q_start and cache geometry (n_kv; max_pages for decode mode) as the
 * call.  Returns 0 when no workspace is needed or for an invalid request
 * (then msa_last_error() is non-empty).                                 */
size_t msa_workspace_size(int32_t op, const msa_shape* shape, int32_t batch,
                          int32_t n_q, int32_t q_start, int32_t n_kv,
                          int32_t max_pages);

/* Human-readable name of a status.  Static storage.                    */
const char* msa_status_string(msa_status status);

/* Detail of the last error on the calling thread ("" if none).  Valid
 * until the next library call on that thread.                           */
const char* msa_last_error(void);

/* MSA_ABI_VERSION of the built library.                                 */
int32_t msa_abi_version(void);

/* Kernel timing, for measurement (not part of the method).
 * msa_profile_enable(1): from now on every launch of a timed kernel is
 *   bracketed by two HIP events recorded on the call's stream (the library
 *   creates the events on first use and keeps them for reuse; no device
 *   memory is allocated).  msa_profile_enable(0) stops recording.
 * msa_profile_read(kernel, &total_ms, &launches): waits for the recorded
 *   launches of `kernel`, returns their summed GPU time and count, and
 *   forgets them.  Kernel names: "ki_prefill_kernel" (msa_index_topk,
 *   prefill), "kp_kernel" and "km_kernel" (msa_sparse_prefill: the
 *   KV-outer pass, one launch per window of queries, and the merge, one
 *   launch per window or, once a window's partials exceed 256 MB, per span
 *   of consecutive windows),
 *   "ki_decode_scan_kernel" (msa_index_topk, decode), "kd_kernel"
 *   (msa_sparse_decode), "kbq_kernel" (dq pass of msa_sparse_prefill_backward,
 *   one launch per window) and "kbkv_kernel" (its dk/dv pass).  Unknown
 *   names or NULL outputs: MSA_ERR_INVALID_ARG.
 * Not meant to be used while calls are being enqueued from other threads. */
msa_status msa_profile_enable(int32_t on);
msa_status msa_profile_read(const char* kernel, double* total_ms, int64_t* launches);

/* Achievable dense bf16 MFMA rate, for measurement (not part of the method):
 * n_wg workgroups of 4 waves; each wave runs `iters` rounds of 8 independent
 * v_mfma_f32_32x32x16_bf16 chains on register operands, i.e.
 * n_wg * 4 * iters * 8 * 32768 FLOPs, and one float per workgroup is written
 * to `out` (device, n_wg floats, caller-owned) so the work is not removed.
 * Asynchronous on hip_stream; the caller times it.  n_wg or iters < 1, or out
 * NULL: MSA_ERR_INVALID_ARG.                                               */
msa_status msa_probe_mfma(int32_t n_wg, int32_t iters, float* out, void* hip_stream);

/* msa_index_topk in decode mode without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation).  Arguments, outputs and errors as msa_index_topk with
 * kv->seq_lens != NULL and n_q = 1.  The pooled page scores go to a device
 * array of 2^22 floats (16 MiB) that the library holds on each GPU it runs
 * on until the process ends, so batch * h_kv * max_pages must be at most
 * 4194304 (MSA_ERR_UNSUPPORTED otherwise; e.g. 64 sequences x 4 groups x
 * 16384 pages).  Nothing is allocated and nothing needs clearing: every score
 * the call reads is written earlier in the same call.  All calls on one GPU
 * share that array, so calls that may overlap on one GPU (other streams,
 * other threads) race and must be ordered by the caller.                    */
msa_status msa_index_topk_decode_static(const msa_shape* shape, int32_t batch, const void* q_idx,
                                        const msa_kv* kv, int32_t* block_idx, float* block_score,
                                        void* hip_stream);

/* Test hook (not part of the method): the prefill schedule keeps its
 * per-(group, block) counters in LDS while a call has at most a built-in
 * number of KV blocks (16384; 2048 for the backward's ordered schedule) and
 * uses global atomics beyond that.  msa_test_schedule_lds_limit(n), n >= 0,
 * lowers that number to min(n, built-in) for every later call in the process
 * (0 forces the global-atomic path); n < 0 restores the built-in numbers.
 * Results do not depend on the path.  Always MSA_OK.                       */
msa_status msa_test_schedule_lds_limit(int32_t max_blocks);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
