// LM head with fused token choice: z = h W_lm^T on MFMA, and in the same kernel the per-tile
// argmax (greedy) or Gumbel-max sample (temperature > 0), the per-tile logsumexp partials and
// optionally the fp32 logits.  A second small kernel merges the per-tile partials of each row
// in tile order (deterministic: no atomics, ties -> lowest id).
//
// Orthrus paper summary (cjcn.com.cn), sec. 四: each pass turns the block rows into one token
// per slot -- the diffusion view's candidates in step 1, the AR model's own choice in step 2.
#include "gemm_core.hpp"

namespace orthrus {
namespace {

struct LmArgs {
  const void* h;
  const void* w;
  const int32_t* seq_id;
  const int32_t* round;
  float* logits;
  uint64_t* part_best;  // [rows, ntiles]
  float* part_m;        // [rows, ntiles] max of z/T
  float* part_s;        // [rows, ntiles] sum exp(z/T - max)
  int32_t M, N, K, block, ntiles;
  int32_t tile0;        // first 128-column tile of this launch
  float inv_t;          // 1/T (1 when greedy)
  int32_t sample;       // temperature > 0
  uint64_t seed, stream_id;
};

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  s = s * expf(m - M) + s2 * expf(m2 - M);
  m = M;
}

constexpr int kLmBN = 128;

template <typename T, typename Cfg>
__global__ __launch_bounds__(Cfg::NT) ORTHRUS_GEMM_WAVES void lmhead_kernel(LmArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int mtiles = (a.M + Cfg::BM - 1) / Cfg::BM;
  int sp, mt, nt;
  xcd_tile_map(blockIdx.x, gridDim.x, 1, mtiles, sp, mt, nt);
  const int m0 = mt * Cfg::BM, n0 = a.tile0 * kLmBN + nt * Cfg::BN;
  constexpr int P = Cfg::BN / kLmBN, WPP = Cfg::WN / P;  // partial tiles per workgroup, waves per partial
  static_assert(P >= 1 && WPP >= 1 && P * kLmBN == Cfg::BN && WPP * P == Cfg::WN, "partials per 128 columns");
  f32x16 acc[Cfg::TM][Cfg::TN];
  gemm_mainloop<T, Cfg>(reinterpret_cast<const T*>(a.h), reinterpret_cast<const T*>(a.w), a.M, a.N, a.K, m0, n0, smem,
                        acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hh = lane >> 5, r = lane & 31;
  const int wm = w / Cfg::WN, wn = w % Cfg::WN;
  __syncthreads();  // LDS is reused below
  uint64_t* red_best = reinterpret_cast<uint64_t*>(smem);                 // [BM][WN]
  float* red_m = reinterpret_cast<float*>(red_best + Cfg::BM * Cfg::WN);  // [BM][WN]
  float* red_s = red_m + Cfg::BM * Cfg::WN;

#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int mrow = (wm * Cfg::TM + i) * 32 + acc_row(e, hh);
      const int m = m0 + mrow;
      const bool mok = m < a.M;
      int bseq = 0, slot = 0;
      if (a.sample && mok) { bseq = m / a.block; slot = m % a.block; }
      uint64_t best = 0;
      float lm = -__builtin_huge_valf(), ls = 0.0f;
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j) {
        const int n = n0 + (wn * Cfg::TN + j) * 32 + r;
        if (!mok || n >= a.N) continue;
        const float z = acc[i][j][e];
        if (a.logits) a.logits[(size_t)m * a.N + n] = z;
        const float zt = z * a.inv_t;
        float key = z;
        if (a.sample) {
          const float u = philox_uniform(a.seed, a.stream_id, slot, n, a.round[bseq], a.seq_id[bseq]);
          key = zt - logf(-logf(u));
        }
        best = umax64(best, pack_argmax(key, n));
        if (zt > lm) { ls = ls * expf(lm - zt) + 1.0f; lm = zt; }
        else ls += expf(zt - lm);
      }
      // reduce over the 32 columns held by this half-wave (same rows), fixed pattern
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        best = umax64(best, shfl_xor_u64(best, off));
        const float m2 = shfl_xor_f(lm, off), s2 = shfl_xor_f(ls, off);
        if (m2 != -__builtin_huge_valf()) {
          if (lm == -__builtin_huge_valf()) { lm = m2; ls = s2; }
          else lse_merge(lm, ls, m2, s2);
        }
      }
      if (r == 0) {
        red_best[mrow * Cfg::WN + wn] = best;
        red_m[mrow * Cfg::WN + wn] = lm;
        red_s[mrow * Cfg::WN + wn] = ls;
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < Cfg::BM * P; idx += Cfg::NT) {
    const int mrow = idx / P, pt = idx % P;
    const int m = m0 + mrow;
    const int tile = n0 / kLmBN + pt;
    if (m >= a.M || tile >= a.ntiles) continue;
    const int q0 = mrow * Cfg::WN + pt * WPP;
    uint64_t best = red_best[q0];
    float lm = red_m[q0], ls = red_s[q0];
    for (int q = 1; q < WPP; ++q) {
      best = umax64(best, red_best[q0 + q]);
      const float m2 = red_m[q0 + q];
      if (m2 != -__builtin_huge_valf()) {
        if (lm == -__builtin_huge_valf()) { lm = m2; ls = red_s[q0 + q]; }
        else lse_merge(lm, ls, m2, red_s[q0 + q]);
      }
    }
    const size_t o = (size_t)m * a.ntiles + tile;
    a.part_best[o] = best;
    a.part_m[o] = lm;
    a.part_s[o] = ls;
  }
}

// One wavefront per row: merge the row's tile partials (strided by lane, then a fixed xor tree).
__global__ __launch_bounds__(64) void lmhead_finalize(const uint64_t* part_best, const float* part_m, const float* part_s,
                                                      int ntiles, int32_t* token, float* lse) {
  const int row = blockIdx.x, lane = threadIdx.x;
  uint64_t best = 0;
  float lm = -__builtin_huge_valf(), ls = 0.0f;
  auto merge = [&](uint64_t b2, float m2, float s2) {
    best = umax64(best, b2);
    if (m2 != -__builtin_huge_valf()) {
      if (lm == -__builtin_huge_valf()) { lm = m2; ls = s2; }
      else lse_merge(lm, ls, m2, s2);
    }
  };
  // four of the lane's tiles are loaded before they are merged in tile order
  constexpr int U = 4;
  const size_t base = (size_t)row * ntiles;
  int t = lane;
  for (; t + 64 * (U - 1) < ntiles; t += 64 * U) {
    uint64_t b2[U];
    float m2[U], s2[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t o = base + t + 64 * u;
      b2[u] = part_best[o];
      m2[u] = part_m[o];
      s2[u] = part_s[o];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) merge(b2[u], m2[u], s2[u]);
  }
  for (; t < ntiles; t += 64) merge(part_best[base + t], part_m[base + t], part_s[base + t]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    best = umax64(best, shfl_xor_u64(best, off));
    const float m2 = shfl_xor_f(lm, off), s2 = shfl_xor_f(ls, off);
    if (m2 != -__builtin_huge_valf()) {
      if (lm == -__builtin_huge_valf()) { lm = m2; ls = s2; }
      else lse_merge(lm, ls, m2, s2);
    }
  }
  if (lane == 0) {
    token[row] = unpack_idx(best);
    if (lse) lse[row] = lm + logf(ls);
  }
}

template <typename T, typename Cfg>
int32_t launch(LmArgs& a, hipStream_t st, int tile0 = 0, int wg_tiles = -1) {
  const int mtiles = (a.M + Cfg::BM - 1) / Cfg::BM;
  const size_t lds = std::max(Cfg::RING, (size_t)Cfg::BM * Cfg::WN * 16);
  if (wg_tiles < 0) wg_tiles = (a.ntiles - tile0) / (Cfg::BN / kLmBN) + ((a.ntiles - tile0) % (Cfg::BN / kLmBN) != 0);
  if (wg_tiles == 0) return ORTHRUS_OK;
  a.tile0 = tile0;
  allow_lds(lmhead_kernel<T, Cfg>, lds);
  hipLaunchKernelGGL((lmhead_kernel<T, Cfg>), dim3(mtiles * wg_tiles), dim3(Cfg::NT), lds, st, a);
  return check_launch("orthrus_lmhead_argmax");
}

#ifndef ORTHRUS_LM_BIG_CFG
#define ORTHRUS_LM_BIG_CFG(T) GemmCfg<T, 128, kLmBN, 2, 2, 3, 2>
#endif
// above 128 rows: 256-row tiles of eight wavefronts (each weight tile streamed once per 256 rows)
#ifndef ORTHRUS_LM_HUGE_CFG
#define ORTHRUS_LM_HUGE_CFG(T) GemmCfg<T, 256, kLmBN, 4, 2, 2, 4>
#endif
// 256x256 pair tiles: eight 64x128 wavefronts, rings of two stages (128 KiB), main loop without the
// odd-stage tail (the host only takes this path when the stage count is even)
template <typename T> using LmPairCfg = GemmCfg<T, 256, 256, 4, 2, 2, 2, true>;

// Above 128 rows with an even number of k-stages: whole waves of 256x256 workgroups (eight 64x128
// wavefronts, each owning one 128-column partial tile), then the remaining tiles as 256x128
// workgroups in a second launch.  A 256x256 workgroup re-reads the 2 MiB activation tile from L2
// once per 256 columns instead of once per 128, which is what bounds the LM head; a grid of only
// 256x256 tiles would leave a last wave of 82 workgroups on 256 CUs at V = 151936, hence the mix.
// The partials stay per 128-column tile, so the finalize merge is the same whatever the split.
template <typename T>
int32_t launch_mixed(LmArgs& a, hipStream_t st) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  }
  const int mtiles = (a.M + 255) / 256;
  const int rounds = (a.ntiles * mtiles) / (2 * cus);
  int npairs = std::min(a.ntiles / 2, rounds * cus / mtiles);
  if (int32_t s = launch<T, LmPairCfg<T>>(a, st, 0, npairs)) return s;
  return launch<T, ORTHRUS_LM_HUGE_CFG(T)>(a, st, 2 * npairs);
}

}  // namespace
}  // namespace orthrus

using namespace orthrus;

extern "C" size_t orthrus_lmhead_workspace_bytes(const orthrus_lmhead_desc_t* d) {
  if (!d || d->rows < 0 || d->vocab <= 0) return 0;
  const size_t ntiles = (d->vocab + kLmBN - 1) / kLmBN;
  return (size_t)d->rows * ntiles * (sizeof(uint64_t) + 2 * sizeof(float));
}

extern "C" int32_t orthrus_lmhead_argmax(const orthrus_lmhead_desc_t* d, const void* h, const void* w,
                                         const int32_t* seq_id, const int32_t* round, int32_t* token_out,
                                         float* logits_out, float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  ORTHRUS_REQUIRE(d != nullptr, ORTHRUS_ERR_INVALID_ARG, "lmhead: null descriptor");
  ORTHRUS_REQUIRE(d->rows >= 0 && d->hidden > 0 && d->vocab > 0, ORTHRUS_ERR_INVALID_ARG, "lmhead: bad sizes");
  ORTHRUS_REQUIRE(d->hidden % 64 == 0, ORTHRUS_ERR_UNSUPPORTED, "lmhead: hidden %d not a multiple of 64", d->hidden);
  ORTHRUS_REQUIRE(valid_dtype(d->dtype), ORTHRUS_ERR_INVALID_ARG, "lmhead: bad dtype");
  ORTHRUS_REQUIRE(d->temperature >= 0.0f && std::isfinite(d->temperature), ORTHRUS_ERR_INVALID_ARG,
                  "lmhead: temperature must be finite and >= 0");
  ORTHRUS_REQUIRE(h && w && token_out, ORTHRUS_ERR_INVALID_ARG, "lmhead: null pointer");
  const bool sample = d->temperature > 0.0f;
  ORTHRUS_REQUIRE(!sample || (seq_id && round && d->block > 0 && d->rows % d->block == 0), ORTHRUS_ERR_INVALID_ARG,
                  "lmhead: sampling needs seq_id, round and rows %% block == 0");
  const size_t need = orthrus_lmhead_workspace_bytes(d);
  ORTHRUS_REQUIRE(ws && ws_bytes >= need, ORTHRUS_ERR_WORKSPACE, "lmhead: workspace %zu < %zu", ws_bytes, need);
  if (d->rows == 0) return ORTHRUS_OK;
  LmArgs a;
  a.tile0 = 0;
  a.h = h; a.w = w; a.seq_id = seq_id; a.round = round; a.logits = logits_out;
  a.M = d->rows; a.N = d->vocab; a.K = d->hidden; a.block = d->block > 0 ? d->block : 1;
  a.ntiles = (d->vocab + kLmBN - 1) / kLmBN;
  a.part_best = reinterpret_cast<uint64_t*>(ws);
  a.part_m = reinterpret_cast<float*>(a.part_best + (size_t)a.M * a.ntiles);
  a.part_s = a.part_m + (size_t)a.M * a.ntiles;
  a.inv_t = sample ? 1.0f / d->temperature : 1.0f;
  a.sample = sample;
  a.seed = d->seed;
  a.stream_id = (uint64_t)d->stream_id;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int32_t s;
  if (d->dtype == ORTHRUS_BF16) {
    if (a.M <= 32) s = launch<bf16, GemmCfg<bf16, 32, kLmBN, 1, 4, 4, 4>>(a, st);
    else if (a.M <= 64) s = launch<bf16, GemmCfg<bf16, 64, kLmBN, 2, 2, 3, 3>>(a, st);
    else if (a.M <= 128) s = launch<bf16, ORTHRUS_LM_BIG_CFG(bf16)>(a, st);
    else if (a.K % 128 == 0) s = launch_mixed<bf16>(a, st);
    else s = launch<bf16, ORTHRUS_LM_HUGE_CFG(bf16)>(a, st);
  } else {
    if (a.M <= 32) s = launch<float, GemmCfg<float, 32, kLmBN, 1, 4, 4, 4>>(a, st);
    else if (a.M <= 64) s = launch<float, GemmCfg<float, 64, kLmBN, 2, 2, 3, 3>>(a, st);
    else if (a.M <= 128) s = launch<float, ORTHRUS_LM_BIG_CFG(float)>(a, st);
    else s = launch<float, ORTHRUS_LM_HUGE_CFG(float)>(a, st);
  }
  if (s != ORTHRUS_OK) return s;
  hipLaunchKernelGGL(lmhead_finalize, dim3(a.M), dim3(64), 0, st, a.part_best, a.part_m, a.part_s, a.ntiles, token_out,
                     lse_out);
  return check_launch("orthrus_lmhead_argmax(finalize)");
}
