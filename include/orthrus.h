/*
 * orthrus.h -- C ABI of the Orthrus decode-round kernels for AMD Instinct MI355X (gfx950).
 *
 * One Orthrus round (Orthrus paper summary, cjcn.com.cn, sec. 四 "inference"):
 *   (1) the diffusion view drafts a block of K = 32 tokens in one parallel pass from the
 *       anchor plus [MASK] placeholders, attending to the shared AR cache before the anchor
 *       and bidirectionally to its own block      -> orthrus_draft_attn, orthrus_lmhead_argmax
 *   (2) the frozen AR path verifies all K positions in one causal pass
 *                                                  -> orthrus_verify_attn, orthrus_lmhead_argmax
 *   (3) intra-model consensus: accept the longest left-to-right prefix where draft == AR
 *       choice, emit the AR token at the first mismatch, discard the rest, update the cache
 *                                                  -> orthrus_consensus_commit
 *       (temperature > 0: strict rejection sampling) -> orthrus_rejection_accept
 * The support calls (GEMM with fused epilogues, RMSNorm, RoPE + K/V write, block embedding)
 * run the decoder layers of both views so that every step of the round is a kernel here.
 *
 * Conventions shared by every call
 *  - All tensor arguments are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or synchronises.  Scratch memory is a caller-provided workspace sized
 *    by the matching *_workspace_bytes query.
 *  - `stream` is a hipStream_t passed as void*; every call only enqueues work on it.
 *  - Row-major layouts; element type given by an orthrus_dtype_t (bf16 or fp32).
 *  - Arguments are validated on the host before anything is enqueued.  A non-zero
 *    orthrus_status_t means nothing was launched; orthrus_last_error() (thread-local) says why.
 *    ORTHRUS_ERR_HIP means a launch failed; asynchronous device faults surface at the
 *    caller's next synchronisation, as usual for HIP.
 *  - Round state (ctx_len, anchor, out_len, round, done) lives in device memory and is
 *    updated in place by the commit calls, so a round needs no host round-trip.
 *  - No call keeps mutable global state apart from the thread-local error string.
 */
#ifndef ORTHRUS_H_
#define ORTHRUS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORTHRUS_ABI_VERSION 3

typedef enum {
  ORTHRUS_OK = 0,
  ORTHRUS_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent shape          */
  ORTHRUS_ERR_UNSUPPORTED = 2, /* valid but not implemented (head_dim, group, dtype)    */
  ORTHRUS_ERR_WORKSPACE = 3,   /* workspace smaller than the *_workspace_bytes query    */
  ORTHRUS_ERR_HIP = 4          /* a HIP launch returned an error                        */
} orthrus_status_t;

typedef enum { ORTHRUS_BF16 = 0, ORTHRUS_F32 = 1 } orthrus_dtype_t;

/* Philox4x64-10 stream ids (second key word); the first key word is the caller's seed. */
enum { ORTHRUS_STREAM_DRAFT = 1, ORTHRUS_STREAM_ACCEPT = 2, ORTHRUS_STREAM_RESID = 3, ORTHRUS_STREAM_AR = 4 };

int32_t orthrus_abi_version(void);
const char* orthrus_last_error(void);

/* ------------------------------------------------------------------------------------------
 * Dual-view block attention (Orthrus paper summary, sec. 二: the diffusion query attends to
 * concat(K_AR, K_diff) / concat(V_AR, V_diff); sec. 三: draft mask = AR context before the
 * anchor + the whole own block, AR path = causal mask).
 *
 * Shapes (G = q_heads / kv_heads; query head h reads kv head h / G):
 *   q          [batch, block, q_heads, head_dim]          dtype
 *   k_pages,
 *   v_pages    [num_pages, kv_heads, page_size, head_dim]  dtype   (paged AR cache)
 *   page_table [batch, max_pages] int32: logical page p of sequence b -> physical page
 *   ctx_len    [batch] int32: n_b = number of cached keys before the block (= anchor position)
 *   k_blk,
 *   v_blk      [batch, block, kv_heads, head_dim]          dtype   (draft: the block's own keys)
 *   out        [batch, block, q_heads, head_dim]           out_dtype
 * Keys are visited in fixed 32-key tiles at absolute positions and split into fixed chunks
 * of kv_chunk keys that are combined in chunk order, so a query row's result does not depend
 * on block size, batch composition or page order (same inputs -> same bits).
 * Device-side: a sequence with n_b + block > max_ctx writes NaN rows (host cannot see n_b).
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  int32_t batch;
  int32_t q_heads;
  int32_t kv_heads;   /* q_heads % kv_heads == 0, group q_heads/kv_heads in {2, 4} */
  int32_t head_dim;   /* 64 or 128                                                  */
  int32_t block;      /* rows per sequence, 1..32                                   */
  int32_t page_size;  /* keys per page, a divisor of 32 or a multiple of 32         */
  int32_t max_pages;  /* row length of page_table                                   */
  int32_t max_ctx;    /* bound on n_b + block; <= max_pages * page_size             */
  int32_t kv_chunk;   /* keys per split chunk, multiple of 32 (0 = 1024)            */
  int32_t dtype;      /* orthrus_dtype_t of q, pages and block keys/values          */
  int32_t out_dtype;  /* orthrus_dtype_t of out                                     */
  float scale;        /* softmax scale applied to q.k                               */
} orthrus_attn_desc_t;

size_t orthrus_attn_workspace_bytes(const orthrus_attn_desc_t* desc);

/* Draft (diffusion-view) attention: slot i of sequence b attends to cache keys [0, n_b) and to
 * all `block` keys of k_blk/v_blk[b] (bidirectional inside the block). */
int32_t orthrus_draft_attn(const orthrus_attn_desc_t* desc, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* page_table, const int32_t* ctx_len,
                           const void* k_blk, const void* v_blk, void* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Verify (AR-view) attention: the block's own keys are already in the cache at
 * [n_b, n_b + block); slot j attends to cache keys [0, n_b + j] (causal). */
int32_t orthrus_verify_attn(const orthrus_attn_desc_t* desc, const void* q, const void* k_pages,
                            const void* v_pages, const int32_t* page_table, const int32_t* ctx_len,
                            void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * LM head with fused token choice (sec. 四 steps 1-2: each pass yields one token per slot).
 *   h [rows, hidden], w [vocab, hidden] (dtype); z = h w^T accumulated in fp32.
 *   sample == 0: token_out[r] = argmax_x z[r, x], exact ties -> lowest id (any temperature).
 *   sample == 1 (needs temperature > 0): token_out[r] = argmax_x (z[r,x]/T - ln(-ln u[r,x]))
 *     (Gumbel-max, a sample of softmax(z/T)); u from Philox4x64-10 with key (seed, stream_id)
 *     and, for row r = b*block + s, counter (s/4, x, round[b], seq_id[b]) and output word s%4;
 *     the uniform is ((word >> 41) + 0.5) * 2^-23.
 *   logits_out [rows, vocab] fp32 (optional, may be NULL): z.
 *   lse_out [rows] fp32 (optional, may be NULL): logsumexp_x(z[r,x] / T) (T = 1 when
 *     temperature == 0).  Computed only when asked for: each 32-column group's maximum and sum
 *     of exp(z/T - max) are reduced by a fixed lane butterfly, and the groups of a row are merged
 *     in an order set by vocab alone, so a row's lse has the same bits whatever rows share the
 *     call.  Without lse_out the kernel reduces the token choice only.
 *   seq_id, round [rows / block] int32: required when sample == 1, else may be NULL.
 * The rejection accept reads the draft pass's logits and lse of a sampled call (sample == 1) and
 * the verify pass's logits and lse of an argmax call at the same temperature (sample == 0).
 * Supported: dtype bf16 or fp32; hidden % 64 == 0.
 * Workspace: orthrus_lmhead_workspace_bytes() bytes, caller-owned, contents undefined on entry
 * and exit; calls that overlap on one workspace race.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  int32_t rows;
  int32_t hidden;
  int32_t vocab;
  int32_t dtype;
  int32_t block;       /* rows per sequence (RNG counters); rows % block == 0 when sampling */
  int32_t stream_id;   /* ORTHRUS_STREAM_DRAFT or ORTHRUS_STREAM_AR                         */
  float temperature;   /* >= 0; scales the logsumexp and the Gumbel-max key                  */
  uint64_t seed;
  int32_t sample;      /* 1: Gumbel-max sample, 0: argmax                                    */
} orthrus_lmhead_desc_t;

size_t orthrus_lmhead_workspace_bytes(const orthrus_lmhead_desc_t* desc);
int32_t orthrus_lmhead_argmax(const orthrus_lmhead_desc_t* desc, const void* h, const void* w,
                              const int32_t* seq_id, const int32_t* round, int32_t* token_out,
                              float* logits_out, float* lse_out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* orthrus_lmhead_argmax without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * The partials live in a static device array of ORTHRUS_LMHEAD_SCRATCH_BYTES (32 MiB) that each
 * GPU the library runs on holds until the process ends; the call allocates nothing.  It serves
 * calls whose orthrus_lmhead_workspace_bytes() is at most that size (e.g. 512 rows at vocabulary
 * 151936); larger ones return ORTHRUS_ERR_WORKSPACE before anything is launched.  The device is
 * the stream's (the current device for the null stream).  Every call on one GPU shares its array:
 * calls that overlap on one GPU (several streams, several threads) race; calls in stream order do
 * not.  Nothing in the array needs clearing between calls (every partial read is written first
 * by the same call).  Results have the bits of orthrus_lmhead_argmax with the same arguments. */
#define ORTHRUS_LMHEAD_SCRATCH_BYTES (32u << 20)
int32_t orthrus_lmhead_argmax_noalloc(const orthrus_lmhead_desc_t* desc, const void* h,
                                      const void* w, const int32_t* seq_id, const int32_t* round,
                                      int32_t* token_out, float* logits_out, float* lse_out,
                                      void* stream);

/* ------------------------------------------------------------------------------------------
 * Greedy consensus + commit (sec. 四 step 3), one wavefront per sequence, no host round-trip.
 *   draft [batch, block]  = d_1..d_K (diffusion view's choice for positions n+1..n+K)
 *   target [batch, block] = t_1..t_K (AR choice at the same positions)
 * For each sequence b with done[b] == 0:
 *   k = number of leading i with d_i == t_i (0..K); emitted = d_1..d_k, then t_{k+1} if k < K;
 *   the emitted tokens are appended to out_tokens[b, out_len[b] ...] (truncated at max_out);
 *   anchor[b] = last emitted token; ctx_len[b] += min(k + 1, K) (the rollback: cache slots at
 *   and beyond the new ctx_len are dead and get overwritten by the next verify);
 *   accept[b] = k; round[b] += 1; done[b] = 1 once out_len[b] >= max_out, or -1 if the next
 *   round would not fit (ctx_len[b] + K > max_ctx).  Sequences with done[b] != 0 are untouched
 *   except accept[b] = -1.
 * ------------------------------------------------------------------------------------------ */
int32_t orthrus_consensus_commit(int32_t batch, int32_t block, const int32_t* draft,
                                 const int32_t* target, int32_t* ctx_len, int32_t* anchor,
                                 int32_t* accept, int32_t* out_tokens, int32_t* out_len,
                                 int32_t* round, int32_t* done, int32_t max_out, int32_t max_ctx,
                                 void* stream);

/* ------------------------------------------------------------------------------------------
 * Rejection-sampling accept + commit at temperature > 0 (sec. 四: strict rejection sampling
 * keeps the AR distribution; rule of standard speculative sampling).
 *   draft_logits, target_logits [batch, block, vocab] fp32 (z, before the temperature)
 *   draft_lse, target_lse [batch, block] fp32: logsumexp(z / T) as written by the LM head
 *   draft [batch, block]: the sampled drafts d_1..d_K
 * Slot i (in order) accepts d_i iff u_i * q_i(d_i) < p_i(d_i), q = softmax(z_draft/T),
 * p = softmax(z_target/T), u_i from Philox (key (seed, ACCEPT), counter (i/4, 0, round[b],
 * seq_id[b]), word i%4).  At the first rejection j the token is drawn from max(0, p_j - q_j)
 * (from p_j if that has no mass) by exponential race argmax_x r(x) / E_x, E_x = -ln u_x with
 * u_x from (seed, RESID), counter (x/4, 0, round[b], seq_id[b]), word x%4; ties -> lowest id.
 * A draft id outside [0, vocab) is rejected at its slot without reading its logits.
 * Then the same commit as orthrus_consensus_commit.
 * Two launches: the race over the rejected row in 2048-entry vocabulary chunks (one workgroup
 * each, grid batch x chunks), then one wavefront per sequence that takes the maximum over the
 * chunks and commits; the draw does not depend on the chunking (the maximum is exact).
 * Workspace: orthrus_rejection_workspace_bytes(batch, vocab) bytes (16 per chunk per sequence),
 * 16-byte aligned, caller-owned, contents undefined on entry and exit; calls that overlap on one
 * workspace race.
 * ------------------------------------------------------------------------------------------ */
size_t orthrus_rejection_workspace_bytes(int32_t batch, int32_t vocab);
int32_t orthrus_rejection_accept(int32_t batch, int32_t block, int32_t vocab, float temperature,
                                 uint64_t seed, const int32_t* seq_id, const float* draft_logits,
                                 const float* target_logits, const float* draft_lse,
                                 const float* target_lse, const int32_t* draft, int32_t* ctx_len,
                                 int32_t* anchor, int32_t* accept, int32_t* out_tokens,
                                 int32_t* out_len, int32_t* round, int32_t* done, int32_t max_out,
                                 int32_t max_ctx, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ------------------------------------------------------------------------------------------
 * Support kernels for the decoder layers of both views.
 * ------------------------------------------------------------------------------------------ */
typedef enum {
  ORTHRUS_EPI_STORE = 0,    /* c = a w^T                                                     */
  ORTHRUS_EPI_RESIDUAL = 1, /* c = residual + a w^T (c may alias residual)                   */
  ORTHRUS_EPI_SWIGLU = 2    /* w holds gate/up rows interleaved in 32-row groups
                               (see orthrus_pack_gate_up); c[m, j] = silu(g) * u, N/2 columns */
} orthrus_epilogue_t;

/* c [M, N'] = epilogue(a [M, K] . w [N, K]^T), fp32 accumulation.  K % 64 == 0; SwiGLU needs
 * N % 64 == 0.  The summation order of an output element depends on (N, K) only, so a row
 * computed alone has the same bits as the same row inside a larger batch:
 *  - N < 16384 with K a multiple of 256 (bf16) or 128 (fp32): K is cut into S contiguous slices
 *    (S = 8 when K >= 8192 and K is a multiple of 512 (bf16) or 256 (fp32), else S = 4), each
 *    summed in k order into an fp32 partial, and the S partials are added in slice order before
 *    the epilogue;
 *  - other N < 16384: the k-steps of a tile are dealt four ways inside one workgroup and the
 *    four partial sums are added in a fixed order;
 *  - N >= 16384: one k loop in order.
 * Workspace: orthrus_gemm_workspace_bytes() bytes (S * M * N * 4 for the k-split, else 0),
 * 16-byte aligned, caller-owned, contents undefined on entry and exit; a smaller workspace
 * returns ORTHRUS_ERR_WORKSPACE before anything is launched.  Calls that overlap on one
 * workspace race. */
size_t orthrus_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t dtype,
                                    int32_t epilogue);
int32_t orthrus_gemm(int32_t M, int32_t N, int32_t K, int32_t dtype, int32_t out_dtype,
                     int32_t epilogue, const void* a, const void* w, const void* residual, void* c,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The residual GEMM and the RMSNorm that follows it in the layer body, in one call:
 *   x [M, N] = x + a [M, K] . w [N, K]^T   (in place, the residual stream, `dtype`)
 *   y [M, N] = x / sqrt(mean(x^2) + eps) * gain   (gain fp32 [N]; y in `dtype`)
 * The result has exactly the bits of orthrus_gemm(..., ORTHRUS_EPI_RESIDUAL, residual = c = x) followed
 * by orthrus_rmsnorm(M, N, dtype, x, gain, eps, y).  Where the GEMM takes the k-split and a
 * row is at most 1024 16-byte chunks (x, y 16-byte aligned), the slice partials are added, the
 * residual updated and the row normalised in one pass; otherwise the two calls run in sequence.
 * Workspace as orthrus_gemm with ORTHRUS_EPI_RESIDUAL; y must not overlap x. */
int32_t orthrus_gemm_residual_rmsnorm(int32_t M, int32_t N, int32_t K, int32_t dtype, const void* a,
                                      const void* w, void* x, const float* gain, float eps, void* y,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Interleave gate [I, H] and up [I, H] into [2I, H] in 32-row groups: gate 0..31, up 0..31,
 * gate 32..63, ... (I % 32 == 0). */
int32_t orthrus_pack_gate_up(int32_t inter, int32_t hidden, int32_t dtype, const void* gate,
                             const void* up, void* packed, void* stream);

/* The gate/up + SwiGLU GEMM on fragment-packed weights, for rows that are many (the round's 32
 * rows per sequence).  orthrus_pack_gate_up_fragments writes gate [I, H] and up [I, H], interleaved
 * in 32-row groups as orthrus_pack_gate_up does, in an MFMA-fragment order (4 KiB pieces, one
 * per 64-wide k stage and 32-row block, stage-major; 2 * I * H elements, the same size as the
 * row-interleaved packing), from which each wavefront loads its weight fragments straight into
 * registers.  orthrus_gemm_swiglu_fragments then computes c [M, I] = silu(a w_gate^T) * (a w_up^T)
 * with a [M, H], fp32 accumulation in the one-loop k order, so c has exactly the bits of
 * orthrus_gemm(M, 2I, H, dtype, dtype, ORTHRUS_EPI_SWIGLU, a, w) on the row-interleaved packing.
 * Built for bf16 with H = 4096 and 2I >= 16384, a multiple of 192 (128x192 tiles of six
 * wavefronts, and two that load the activations) or else of 256 (128x256 tiles of four); other
 * shapes return
 * ORTHRUS_ERR_UNSUPPORTED (use orthrus_gemm).  Pointers 16-byte aligned; no workspace. */
int32_t orthrus_pack_gate_up_fragments(int32_t inter, int32_t hidden, int32_t dtype,
                                       const void* gate, const void* up, void* packed, void* stream);
int32_t orthrus_gemm_swiglu_fragments(int32_t M, int32_t inter, int32_t hidden, int32_t dtype,
                                      const void* a, const void* w_fragments, void* c, void* stream);

/* y [rows, hidden] = x / sqrt(mean(x^2) + eps) * gain, fp32 math; x and y in `dtype`. */
int32_t orthrus_rmsnorm(int32_t rows, int32_t hidden, int32_t dtype, const void* x,
                        const float* gain, float eps, void* y, void* stream);

/* table [max_pos, head_dim/2, 2] fp32 = (cos, sin) of pos * base^(-2i/D), evaluated in fp64. */
int32_t orthrus_rope_table(int32_t max_pos, int32_t head_dim, double base, float* table,
                           void* stream);

/* The QKV projection and the RoPE + K/V write that follows it in the layer body, in one call:
 * qkv = a [batch*block, hidden] . w [(Hq + 2 Hkv) * D, hidden]^T, then orthrus_rope_kv_write on it.
 * The result has exactly the bits of orthrus_gemm(..., ORTHRUS_EPI_STORE, c = qkv) followed by
 * orthrus_rope_kv_write(..., qkv, ...).  Where the GEMM takes the k-split, the partials are
 * added, rotated and written row by row and `qkv` is not touched; otherwise the two calls run in
 * sequence through `qkv` (caller-owned [batch*block, (Hq + 2 Hkv) * D], contents undefined after).
 * Workspace as orthrus_gemm with ORTHRUS_EPI_STORE. */
int32_t orthrus_gemm_rope_kv_write(int32_t batch, int32_t block, int32_t q_heads, int32_t kv_heads,
                                   int32_t head_dim, int32_t page_size, int32_t max_pages,
                                   int32_t hidden, int32_t dtype, const void* a, const void* w,
                                   const float* rope_table, int32_t max_pos, const int32_t* ctx_len,
                                   const int32_t* page_table, void* qkv, void* q_out, void* k_dst,
                                   void* v_dst, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Split a QKV projection [batch*block, (Hq + 2 Hkv) * D] (q | k | v), apply rotate-half RoPE at
 * positions ctx_len[b] + s to q and k, write q_out [batch*block, Hq*D] and K/V either into the
 * paged cache at positions [ctx_len[b], ctx_len[b] + block) (page_table != NULL) or into
 * k_blk/v_blk [batch, block, Hkv, D] (page_table == NULL). */
int32_t orthrus_rope_kv_write(int32_t batch, int32_t block, int32_t q_heads, int32_t kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t max_pages, int32_t dtype,
                              const void* qkv, const float* rope_table, int32_t max_pos,
                              const int32_t* ctx_len, const int32_t* page_table, void* q_out,
                              void* k_dst, void* v_dst, void* stream);

/* x [batch*block, hidden] = embed[token(b, s)] where token(b, 0) = anchor[b] if anchor != NULL;
 * other slots read tokens[b * tok_stride + tok_offset + s - (anchor != NULL)] if tokens != NULL,
 * else mask_id. */
int32_t orthrus_embed_block(int32_t batch, int32_t block, int32_t hidden, int32_t dtype,
                            const void* embed, const int32_t* anchor, const int32_t* tokens,
                            int32_t tok_stride, int32_t tok_offset, int32_t mask_id, void* x,
                            void* stream);

/* ------------------------------------------------------------------------------------------
 * Two-step drafting (Orthrus paper summary, sec. 六: the ablation that borrows Fast-dLLM-v2's
 * two-pass completion; the diffusion view fills the block in two passes instead of one).
 *
 * orthrus_draft_fill, between the two diffusion passes:
 *   h [batch*block, hidden] (dtype): pass 1's final-normed hidden rows (the LM head's input);
 *   w [vocab, hidden] (dtype): the LM-head weight; lse [batch*block] fp32: logsumexp of pass 1's
 *   logits (orthrus_lmhead_argmax's lse_out at temperature 0); draft [batch, block]: pass 1's
 *   argmax, row j being the token for slot j+1.
 *   For each sequence, rows j < block-1 are scored by z[j, draft_j] - lse_j (the chosen token's
 *   log-probability; z recomputed in fp32 as one dot product; a NaN score counts as -inf) and
 *   the n_fill best (equal scores: lower j first) are filled:
 *     tokens2[b, j] = filled ? draft[b, j] : mask_id, filled[b, j] = 1 or 0, for j < block-1;
 *     tokens2[b, block-1] = mask_id, filled[b, block-1] = 0.
 *   tokens2 is the token list of pass 2's block after the anchor (orthrus_embed_block with
 *   tokens = tokens2, tok_stride = block, tok_offset = 0).
 *   Supported: 1 <= block <= 64, 0 <= n_fill <= block-1, dtype bf16 or fp32, hidden % 8 == 0.
 * orthrus_draft_merge, after pass 2's LM head:
 *   draft_out[i] = filled[i] ? tokens2[i] : draft2[i] over batch*block entries (a filled slot keeps
 *   its pass-1 token).  draft_out may alias draft2.
 * Both return ORTHRUS_ERR_INVALID_ARG for null pointers or sizes out of range before launching.
 * ------------------------------------------------------------------------------------------ */
int32_t orthrus_draft_fill(int32_t batch, int32_t block, int32_t hidden, int32_t vocab, int32_t dtype,
                           const void* h, const void* w, const float* lse, const int32_t* draft,
                           int32_t mask_id, int32_t n_fill, int32_t* tokens2, int32_t* filled,
                           void* stream);
int32_t orthrus_draft_merge(int32_t batch, int32_t block, const int32_t* filled,
                            const int32_t* tokens2, const int32_t* draft2, int32_t* draft_out,
                            void* stream);

/* Philox4x64-10 words for n counters (ctr [n, 4], out [n, 4] uint64), key (k0, k1). */
int32_t orthrus_philox4x64(int64_t n, const uint64_t* ctr, uint64_t k0, uint64_t k1,
                           uint64_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ORTHRUS_H_ */
