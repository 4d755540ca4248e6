// Intra-model consensus and commit (greedy), the rejection-sampling accept (temperature > 0)
// and a Philox4x64-10 word generator.
//
// Orthrus paper summary (cjcn.com.cn), sec. 四 step 3: compare left to right, accept while the
// draft equals the AR choice, emit the AR choice at the first disagreement, drop the rest and
// update the memory; at least one token per round.  With a temperature, strict rejection
// sampling (standard speculative sampling: accept with min(1, p/q), else draw from the
// normalised residual max(0, p - q)) keeps the AR distribution.
//
// The KV rollback is a length update only: slots at or beyond the new ctx_len are dead and the
// next verify pass overwrites them.
#include "common.hpp"

namespace orthrus {
namespace {

struct CommitState {
  int32_t* ctx_len;
  int32_t* anchor;
  int32_t* accept;
  int32_t* out_tokens;
  int32_t* out_len;
  int32_t* round;
  int32_t* done;
  int32_t max_out, max_ctx;
};

// Emit `count` tokens (token i provided by lane i) for sequence b; lanes < 32 participate.
__device__ __forceinline__ void commit_tokens(const CommitState& cs, int b, int K, int k, int count, int my_tok,
                                              int last_tok, int lane) {
  const int ol = cs.out_len[b];
  if (lane < count && ol + lane < cs.max_out) cs.out_tokens[(size_t)b * cs.max_out + ol + lane] = my_tok;
  if (lane == 0) {
    const int written = max(0, min(count, cs.max_out - ol));
    const int nol = ol + written;
    const int nctx = cs.ctx_len[b] + count;
    cs.out_len[b] = nol;
    cs.anchor[b] = last_tok;
    cs.ctx_len[b] = nctx;
    cs.accept[b] = k;
    cs.round[b] = cs.round[b] + 1;
    cs.done[b] = nol >= cs.max_out ? 1 : (nctx + K > cs.max_ctx ? -1 : 0);
  }
}

__global__ __launch_bounds__(64) void consensus_kernel(int K, const int32_t* __restrict__ draft,
                                                       const int32_t* __restrict__ target, CommitState cs) {
  const int b = blockIdx.x, lane = threadIdx.x;
  if (cs.done[b] != 0) {
    if (lane == 0) cs.accept[b] = -1;
    return;
  }
  int d = 0, t = 0;
  if (lane < K) {
    d = draft[(size_t)b * K + lane];
    t = target[(size_t)b * K + lane];
  }
  const uint64_t mism = __ballot(lane < K && d != t);
  const int k = mism ? __builtin_ctzll(mism) : K;   // accepted drafts
  const int count = min(k + 1, K);                   // tokens committed this round
  const int tk = __shfl(t, min(k, K - 1), 64);       // correction t_{k+1}
  const int my_tok = lane < k ? d : tk;
  const int last_tok = __shfl(my_tok, count - 1, 64);
  commit_tokens(cs, b, K, k, count, my_tok, last_tok, lane);
}

// The rejection accept runs in two launches.  The residual draw needs one Philox call per four
// vocabulary entries of the first rejected row, so it is spread over kRaceChunk-entry chunks
// (one workgroup each, grid chunks x batch); every chunk leaves the packed maximum of its race
// keys for the residual and for the fallback law p (grid batch x chunks, so the batch is not
// limited by the grid's second dimension).  A one-wavefront launch per sequence then
// takes the maximum over the chunks (exact and order-free, so the draw does not depend on the
// chunking) and commits.  Both launches recompute the accepted prefix k from the same inputs.
constexpr int kRaceThreads = 256;
constexpr int kRaceChunk = 2048;  // vocabulary entries per race workgroup

__host__ __device__ constexpr int race_chunks(int vocab) { return (vocab + kRaceChunk - 1) / kRaceChunk; }

// Leading accepted drafts of sequence b: slot i accepts iff u_i * q_i(d_i) < p_i(d_i).  Called by
// one full wavefront; every lane gets k.
__device__ __forceinline__ int accepted_prefix(int b, int K, int V, float inv_t, uint64_t seed, int rnd, int sid,
                                               const float* __restrict__ zd, const float* __restrict__ zt,
                                               const float* __restrict__ lse_d, const float* __restrict__ lse_t,
                                               const int32_t* __restrict__ draft, int lane) {
  bool acc = true;
  if (lane < K) {
    const int d = draft[(size_t)b * K + lane];
    const size_t row = (size_t)b * K + lane;
    if (d >= 0 && d < V) {
      const float q = expf(zd[row * V + d] * inv_t - lse_d[row]);
      const float p = expf(zt[row * V + d] * inv_t - lse_t[row]);
      const float u = philox_uniform(seed, ORTHRUS_STREAM_ACCEPT, lane, 0, rnd, sid);
      acc = u * q < p;
    } else {
      acc = false;  // an id outside the vocabulary is never accepted (and never read)
    }
  }
  const uint64_t rej = __ballot(lane < K && !acc);
  return rej ? __builtin_ctzll(rej) : K;
}

// Race keys over one chunk of the first rejected row: r(x) / E_x with E_x = -ln u_x, for the
// residual r = max(0, p - q) and for p itself.  part[b, chunk] = {residual max, p max} (0: no mass).
__global__ __launch_bounds__(kRaceThreads) void rejection_race_kernel(
    int K, int V, float inv_t, uint64_t seed, const int32_t* __restrict__ seq_id, const float* __restrict__ zd,
    const float* __restrict__ zt, const float* __restrict__ lse_d, const float* __restrict__ lse_t,
    const int32_t* __restrict__ draft, const int32_t* __restrict__ done, const int32_t* __restrict__ round,
    ulonglong2* __restrict__ part) {
  __shared__ int s_k;
  __shared__ uint64_t red[2][kRaceThreads / kWave];
  const int b = blockIdx.x, chunk = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (done[b] != 0) return;
  const int rnd = round[b], sid = seq_id[b];
  if (w == 0) {
    const int k = accepted_prefix(b, K, V, inv_t, seed, rnd, sid, zd, zt, lse_d, lse_t, draft, lane);
    if (lane == 0) s_k = k;
  }
  __syncthreads();
  const int k = s_k;
  if (k >= K) return;  // every draft accepted: nothing to draw
  const size_t row = (size_t)b * K + k;
  const float ld = lse_d[row], lt = lse_t[row];
  const float* zdr = zd + row * V;
  const float* ztr = zt + row * V;
  uint64_t best_r = 0, best_p = 0;
  const int x_end = min(V, (chunk + 1) * kRaceChunk);
  for (int x0 = chunk * kRaceChunk + tid * 4; x0 < x_end; x0 += kRaceThreads * 4) {
    const u64x4 wd = philox4x64_10((uint64_t)(x0 >> 2), 0, (uint64_t)rnd, (uint64_t)sid, seed, ORTHRUS_STREAM_RESID);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x = x0 + e;
      if (x >= x_end) break;
      const float p = expf(ztr[x] * inv_t - lt);
      const float rr = fmaxf(p - expf(zdr[x] * inv_t - ld), 0.0f);
      if (p > 0.0f) {
        const float E = -logf(word_to_uniform(wd.x[e]));
        best_p = umax64(best_p, pack_argmax(p / E, x));
        if (rr > 0.0f) best_r = umax64(best_r, pack_argmax(rr / E, x));
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    best_r = umax64(best_r, shfl_xor_u64(best_r, off));
    best_p = umax64(best_p, shfl_xor_u64(best_p, off));
  }
  if (lane == 0) { red[0][w] = best_r; red[1][w] = best_p; }
  __syncthreads();
  if (tid == 0) {
    uint64_t r = 0, q = 0;
#pragma unroll
    for (int i = 0; i < kRaceThreads / kWave; ++i) { r = umax64(r, red[0][i]); q = umax64(q, red[1][i]); }
    part[(size_t)b * gridDim.y + chunk] = make_ulonglong2(r, q);
  }
}

// One wavefront per sequence: the accepted prefix, the residual draw (maximum over the chunks'
// keys; the law p if the residual has no mass anywhere) and the commit.
__global__ __launch_bounds__(64) void rejection_commit_kernel(int K, int V, int nchunks, float inv_t, uint64_t seed,
                                                              const int32_t* __restrict__ seq_id,
                                                              const float* __restrict__ zd,
                                                              const float* __restrict__ zt,
                                                              const float* __restrict__ lse_d,
                                                              const float* __restrict__ lse_t,
                                                              const int32_t* __restrict__ draft,
                                                              const ulonglong2* __restrict__ part, CommitState cs) {
  const int b = blockIdx.x, lane = threadIdx.x;
  if (cs.done[b] != 0) {
    if (lane == 0) cs.accept[b] = -1;
    return;
  }
  const int rnd = cs.round[b], sid = seq_id[b];
  const int k = accepted_prefix(b, K, V, inv_t, seed, rnd, sid, zd, zt, lse_d, lse_t, draft, lane);
  int corr = 0;
  if (k < K) {
    uint64_t r = 0, q = 0;
    for (int c = lane; c < nchunks; c += 64) {
      const ulonglong2 v = part[(size_t)b * nchunks + c];
      r = umax64(r, v.x);
      q = umax64(q, v.y);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      r = umax64(r, shfl_xor_u64(r, off));
      q = umax64(q, shfl_xor_u64(q, off));
    }
    corr = unpack_idx(r != 0 ? r : q);
  }
  const int count = min(k + 1, K);
  const int d = lane < K ? draft[(size_t)b * K + lane] : 0;
  const int my_tok = lane < k ? d : corr;
  const int last_tok = __shfl(my_tok, count - 1, 64);
  commit_tokens(cs, b, K, k, count, my_tok, last_tok, lane);
}

__global__ void philox_kernel(int64_t n, const uint64_t* ctr, uint64_t k0, uint64_t k1, uint64_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const u64x4 w = philox4x64_10(ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3], k0, k1);
  for (int e = 0; e < 4; ++e) out[4 * i + e] = w.x[e];
}

int32_t check_state(int batch, int block, const int32_t* ctx_len, const int32_t* anchor, const int32_t* accept,
                    const int32_t* out_tokens, const int32_t* out_len, const int32_t* round, const int32_t* done,
                    int max_out, int max_ctx) {
  ORTHRUS_REQUIRE(batch >= 0 && block >= 1 && block <= 32, ORTHRUS_ERR_INVALID_ARG, "commit: batch %d / block %d",
                  batch, block);
  ORTHRUS_REQUIRE(max_out >= 0 && max_ctx >= block, ORTHRUS_ERR_INVALID_ARG, "commit: max_out / max_ctx");
  ORTHRUS_REQUIRE(ctx_len && anchor && accept && out_len && round && done && (out_tokens || max_out == 0),
                  ORTHRUS_ERR_INVALID_ARG, "commit: null state pointer");
  return ORTHRUS_OK;
}


// Two-step drafting (Orthrus paper summary, sec. 六: the Fast-dLLM-v2 style ablation in which the
// diffusion view completes a block in two passes).  After pass 1, row j's choice (the token for
// slot j+1) is scored by its log-probability z[j, d_j] - logsumexp(z[j]); the n_fill best of the
// K-1 masked slots (equal scores: lower slot first; NaN scores last) are written into their slots
// for pass 2, the others stay [MASK].  One workgroup per sequence: each wavefront recomputes the
// chosen logit of its rows as one dot product (16-byte loads, lane-strided, then a butterfly).
constexpr int kMaxFillBlock = 64;
constexpr float kNegInfF = -__builtin_huge_valf();

template <typename T>
__global__ __launch_bounds__(256) void draft_fill_kernel(int K, int hidden, int vocab, const T* __restrict__ h,
                                                         const T* __restrict__ w, const float* __restrict__ lse,
                                                         const int32_t* __restrict__ draft, int mask_id, int n_fill,
                                                         int32_t* tokens2, int32_t* filled) {
  constexpr int EPC = 16 / (int)sizeof(T);
  __shared__ float conf[kMaxFillBlock];
  const int b = blockIdx.x, tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  for (int j = wv; j < K - 1; j += 4) {
    const size_t row = (size_t)b * K + j;
    const int tok = draft[row];
    const bool ok = tok >= 0 && tok < vocab;
    float acc = 0.0f;
    if (ok) {
      const T* hr = h + row * hidden;
      const T* wr = w + (size_t)tok * hidden;
      for (int c = lane * EPC; c < hidden; c += 64 * EPC) {
        if constexpr (EPC == 8) {
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(hr + c);
          const bf16x8 y = *reinterpret_cast<const bf16x8*>(wr + c);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[e], (float)y[e], acc);
        } else {
          const f32x4 x = *reinterpret_cast<const f32x4*>(hr + c);
          const f32x4 y = *reinterpret_cast<const f32x4*>(wr + c);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(x[e], y[e], acc);
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      const float c = ok ? acc - lse[row] : kNegInfF;
      conf[j] = __builtin_isnan(c) ? kNegInfF : c;
    }
  }
  __syncthreads();
  if (tid < K) {
    int32_t t2 = mask_id, f = 0;
    if (tid < K - 1) {
      const float c = conf[tid];
      int rank = 0;
      for (int i = 0; i < K - 1; ++i) {
        const float ci = conf[i];
        rank += (ci > c || (ci == c && i < tid)) ? 1 : 0;
      }
      if (rank < n_fill) {
        t2 = draft[(size_t)b * K + tid];
        f = 1;
      }
    }
    tokens2[(size_t)b * K + tid] = t2;
    filled[(size_t)b * K + tid] = f;
  }
}

// The two-step draft: a filled slot keeps its pass-1 token, every other row takes pass 2's.
__global__ __launch_bounds__(256) void draft_merge_kernel(int n, const int32_t* __restrict__ filled,
                                                          const int32_t* __restrict__ tokens2, const int32_t* draft2,
                                                          int32_t* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = filled[i] ? tokens2[i] : draft2[i];
}

}  // namespace
}  // namespace orthrus

using namespace orthrus;

extern "C" int32_t orthrus_consensus_commit(int32_t batch, int32_t block, const int32_t* draft, const int32_t* target,
                                            int32_t* ctx_len, int32_t* anchor, int32_t* accept, int32_t* out_tokens,
                                            int32_t* out_len, int32_t* round, int32_t* done, int32_t max_out,
                                            int32_t max_ctx, void* stream) {
  if (int32_t s = check_state(batch, block, ctx_len, anchor, accept, out_tokens, out_len, round, done, max_out, max_ctx))
    return s;
  ORTHRUS_REQUIRE(draft && target, ORTHRUS_ERR_INVALID_ARG, "commit: null draft/target");
  if (batch == 0) return ORTHRUS_OK;
  CommitState cs{ctx_len, anchor, accept, out_tokens, out_len, round, done, max_out, max_ctx};
  hipLaunchKernelGGL(consensus_kernel, dim3(batch), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), block, draft,
                     target, cs);
  return check_launch("orthrus_consensus_commit");
}

extern "C" size_t orthrus_rejection_workspace_bytes(int32_t batch, int32_t vocab) {
  if (batch <= 0 || vocab <= 0) return 0;
  return (size_t)batch * race_chunks(vocab) * sizeof(ulonglong2);
}

extern "C" int32_t orthrus_rejection_accept(int32_t batch, int32_t block, int32_t vocab, float temperature,
                                            uint64_t seed, const int32_t* seq_id, const float* draft_logits,
                                            const float* target_logits, const float* draft_lse,
                                            const float* target_lse, const int32_t* draft, int32_t* ctx_len,
                                            int32_t* anchor, int32_t* accept, int32_t* out_tokens, int32_t* out_len,
                                            int32_t* round, int32_t* done, int32_t max_out, int32_t max_ctx,
                                            void* workspace, size_t workspace_bytes, void* stream) {
  if (int32_t s = check_state(batch, block, ctx_len, anchor, accept, out_tokens, out_len, round, done, max_out, max_ctx))
    return s;
  ORTHRUS_REQUIRE(vocab > 0 && temperature > 0.0f && std::isfinite(temperature), ORTHRUS_ERR_INVALID_ARG,
                  "rejection: vocab > 0 and finite temperature > 0 required");
  ORTHRUS_REQUIRE(seq_id && draft_logits && target_logits && draft_lse && target_lse && draft, ORTHRUS_ERR_INVALID_ARG,
                  "rejection: null pointer");
  if (batch == 0) return ORTHRUS_OK;
  const size_t need = orthrus_rejection_workspace_bytes(batch, vocab);
  ORTHRUS_REQUIRE(workspace && workspace_bytes >= need, ORTHRUS_ERR_WORKSPACE,
                  "rejection: workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  ORTHRUS_REQUIRE(((uintptr_t)workspace & 15) == 0, ORTHRUS_ERR_INVALID_ARG,
                  "rejection: workspace must be 16-byte aligned");
  const int nchunks = race_chunks(vocab);
  ORTHRUS_REQUIRE(nchunks <= 65535, ORTHRUS_ERR_UNSUPPORTED, "rejection: vocab %d above %d", vocab, 65535 * kRaceChunk);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  auto* part = static_cast<ulonglong2*>(workspace);
  const float inv_t = 1.0f / temperature;
  hipLaunchKernelGGL(rejection_race_kernel, dim3(batch, nchunks), dim3(kRaceThreads), 0, st, block, vocab, inv_t,
                     seed, seq_id, draft_logits, target_logits, draft_lse, target_lse, draft, done, round, part);
  if (int32_t s = check_launch("orthrus_rejection_accept (race)")) return s;
  CommitState cs{ctx_len, anchor, accept, out_tokens, out_len, round, done, max_out, max_ctx};
  hipLaunchKernelGGL(rejection_commit_kernel, dim3(batch), dim3(64), 0, st, block, vocab, nchunks, inv_t, seed, seq_id,
                     draft_logits, target_logits, draft_lse, target_lse, draft, part, cs);
  return check_launch("orthrus_rejection_accept");
}

extern "C" int32_t orthrus_philox4x64(int64_t n, const uint64_t* ctr, uint64_t k0, uint64_t k1, uint64_t* out,
                                      void* stream) {
  ORTHRUS_REQUIRE(n >= 0 && (n == 0 || (ctr && out)), ORTHRUS_ERR_INVALID_ARG, "philox: bad args");
  if (n == 0) return ORTHRUS_OK;
  hipLaunchKernelGGL(philox_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), n, ctr, k0, k1, out);
  return check_launch("orthrus_philox4x64");
}

extern "C" int32_t orthrus_draft_fill(int32_t batch, int32_t block, int32_t hidden, int32_t vocab, int32_t dtype,
                                      const void* h, const void* w, const float* lse, const int32_t* draft,
                                      int32_t mask_id, int32_t n_fill, int32_t* tokens2, int32_t* filled,
                                      void* stream) {
  ORTHRUS_REQUIRE(batch >= 0 && block >= 1 && block <= kMaxFillBlock && hidden > 0 && vocab > 0,
                  ORTHRUS_ERR_INVALID_ARG, "draft_fill: bad sizes (batch %d, block %d, hidden %d, vocab %d)", batch,
                  block, hidden, vocab);
  ORTHRUS_REQUIRE(n_fill >= 0 && n_fill <= block - 1, ORTHRUS_ERR_INVALID_ARG,
                  "draft_fill: n_fill %d outside [0, block - 1]", n_fill);
  ORTHRUS_REQUIRE(valid_dtype(dtype), ORTHRUS_ERR_UNSUPPORTED, "draft_fill: dtype %d", dtype);
  ORTHRUS_REQUIRE(hidden % 8 == 0, ORTHRUS_ERR_UNSUPPORTED, "draft_fill: hidden %% 8 != 0");
  ORTHRUS_REQUIRE(h && w && lse && draft && tokens2 && filled, ORTHRUS_ERR_INVALID_ARG, "draft_fill: null pointer");
  if (batch == 0) return ORTHRUS_OK;
  auto st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == ORTHRUS_BF16)
    hipLaunchKernelGGL(draft_fill_kernel<bf16>, dim3(batch), dim3(256), 0, st, block, hidden, vocab,
                       static_cast<const bf16*>(h), static_cast<const bf16*>(w), lse, draft, mask_id, n_fill, tokens2,
                       filled);
  else
    hipLaunchKernelGGL(draft_fill_kernel<float>, dim3(batch), dim3(256), 0, st, block, hidden, vocab,
                       static_cast<const float*>(h), static_cast<const float*>(w), lse, draft, mask_id, n_fill,
                       tokens2, filled);
  return check_launch("orthrus_draft_fill");
}

extern "C" int32_t orthrus_draft_merge(int32_t batch, int32_t block, const int32_t* filled, const int32_t* tokens2,
                                       const int32_t* draft2, int32_t* draft_out, void* stream) {
  ORTHRUS_REQUIRE(batch >= 0 && block >= 1, ORTHRUS_ERR_INVALID_ARG, "draft_merge: bad sizes");
  ORTHRUS_REQUIRE(filled && tokens2 && draft2 && draft_out, ORTHRUS_ERR_INVALID_ARG, "draft_merge: null pointer");
  const int64_t n = (int64_t)batch * block;
  ORTHRUS_REQUIRE(n < (1ll << 31), ORTHRUS_ERR_INVALID_ARG, "draft_merge: too many rows");
  if (n == 0) return ORTHRUS_OK;
  hipLaunchKernelGGL(draft_merge_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), (int)n, filled, tokens2, draft2, draft_out);
  return check_launch("orthrus_draft_merge");
}
