// LM head with fused token choice: z = h W_lm^T on MFMA, and in the same kernel the per-tile
// argmax or Gumbel-max sample, the per-32-column logsumexp partials when the caller asks for the
// logsumexp, and optionally the fp32 logits.  A second small kernel merges the partials of each
// row in a fixed order (deterministic: no atomics, ties -> lowest id).
//
// Orthrus paper summary (cjcn.com.cn), sec. 四: each pass turns the block rows into one token
// per slot -- the diffusion view's candidates in step 1, the AR model's own choice in step 2.
#include <mutex>

#include "gemm_core.hpp"

namespace orthrus {
namespace {

struct LmArgs {
  const void* h;
  const void* w;
  const int32_t* seq_id;
  const int32_t* round;
  float* logits;
  uint64_t* part_best;  // [rows, ntiles]  packed (key, id) maximum per 128-column tile
  float2* part_lse;     // [rows, ngroups] (max, sum exp(. - max)) of z/T per 32-column group
  int32_t M, N, K, block, ntiles, ngroups;
  int32_t tile0;        // first 128-column tile of this launch
  float inv_t;          // 1/T (1 when T == 0)
  uint64_t seed, stream_id;
};

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  s = s * expf(m - M) + s2 * expf(m2 - M);
  m = M;
}

// Merge (m2, s2) into (m, s) where either may be the empty partial (m = -inf).
__device__ __forceinline__ void lse_merge_opt(float& m, float& s, float m2, float s2) {
  if (m2 == -__builtin_huge_valf()) return;
  if (m == -__builtin_huge_valf()) { m = m2; s = s2; return; }
  lse_merge(m, s, m2, s2);
}

constexpr int kLmBN = 128;

// The epilogue per output element of a half-wave row:
//  * token choice: the packed maximum of (key, id), key = z (greedy) or z/T - ln(-ln u) (Gumbel-max
//    sample); reduced per 128-column tile, exact in any order;
//  * optionally the logsumexp of z/T, in an order that does not depend on the tiling: for each
//    32-column group (lane r holds column 32g + r in every tile layout) a 32-lane butterfly
//    takes the group maximum, then the sum of exp(z/T - max); the finalize merges the groups of a
//    row in an order fixed by the vocabulary size alone.  A row's logsumexp therefore has the same
//    bits whatever M, the tile shape or the launch split.
template <typename T, typename Cfg, bool kSample, bool kLse>
__global__ __launch_bounds__(Cfg::NT) ORTHRUS_GEMM_WAVES void lmhead_kernel(LmArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int mtiles = (a.M + Cfg::BM - 1) / Cfg::BM;
  int sp, mt, nt;
  xcd_tile_map(blockIdx.x, gridDim.x, 1, mtiles, sp, mt, nt);
  const int m0 = mt * Cfg::BM, n0 = a.tile0 * kLmBN + nt * Cfg::BN;
  constexpr int P = Cfg::BN / kLmBN, WPP = Cfg::WN / P;  // partial tiles per workgroup, waves per partial
  constexpr int NG = Cfg::BN / 32;                        // 32-column groups per workgroup tile
  static_assert(P >= 1 && WPP >= 1 && P * kLmBN == Cfg::BN && WPP * P == Cfg::WN, "partials per 128 columns");
  f32x16 acc[Cfg::TM][Cfg::TN];
  gemm_mainloop<T, Cfg>(reinterpret_cast<const T*>(a.h), reinterpret_cast<const T*>(a.w), a.M, a.N, a.K, m0, n0, smem,
                        acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hh = lane >> 5, r = lane & 31;
  const int wm = w / Cfg::WN, wn = w % Cfg::WN;
  __syncthreads();  // LDS is reused below
  uint64_t* red_best = reinterpret_cast<uint64_t*>(smem);                   // [BM][WN]
  float2* red_lse = reinterpret_cast<float2*>(red_best + Cfg::BM * Cfg::WN);  // [BM][NG]
  constexpr float kNegInf = -__builtin_huge_valf();

  // One output element (accumulator i, register e, column tile j) of a row: logits store, token
  // key, logsumexp group partial.  `u` is the element's uniform when sampling.
  auto element = [&](int i, int e, int j, int m, bool mok, float u, uint64_t& best) {
    const int mrow = (wm * Cfg::TM + i) * 32 + acc_row(e, hh);
    const int n = n0 + (wn * Cfg::TN + j) * 32 + r;
    const bool ok = mok && n < a.N;
    const float z = acc[i][j][e];
    if (ok && a.logits) a.logits[(size_t)m * a.N + n] = z;
    float key = z;
    if constexpr (kSample) key = z * a.inv_t - logf(-logf(u));
    if (ok) best = umax64(best, pack_argmax(key, n));
    if constexpr (kLse) {
      const float zt = ok ? z * a.inv_t : kNegInf;
      float gm = zt;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) gm = fmaxf(gm, shfl_xor_f(gm, off));
      float gs = ok ? expf(zt - gm) : 0.0f;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) gs += shfl_xor_f(gs, off);
      if (r == 0) red_lse[mrow * NG + wn * Cfg::TN + j] = make_float2(gm, gs);
    }
  };
  // reduce a row's choice over the 32 columns held by this half-wave
  auto finish_row = [&](int i, int e, uint64_t best) {
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) best = umax64(best, shfl_xor_u64(best, off));
    if (r == 0) red_best[((wm * Cfg::TM + i) * 32 + acc_row(e, hh)) * Cfg::WN + wn] = best;
  };

  if (kSample && a.block % 4 == 0) {
    // Registers 4q..4q+3 of a lane hold four consecutive rows, one aligned group of four block slots
    // of one sequence; the four words of the Philox call with counter (slot/4, n, round, seq) are
    // exactly their four uniforms, so one call serves the four rows.
    // compile-time loops: the accumulator registers must be indexed by constants
    static_for<Cfg::TM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      static_for<4>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        const int mb = m0 + (wm * Cfg::TM + i) * 32 + acc_row(4 * q, hh);  // first of the four rows
        uint64_t c0 = 0, c2 = 0, c3 = 0;
        if (mb < a.M) {
          const int bseq = mb / a.block;
          c0 = (uint64_t)((mb % a.block) >> 2);
          c2 = (uint64_t)a.round[bseq];
          c3 = (uint64_t)a.seq_id[bseq];
        }
        uint64_t best0 = 0, best1 = 0, best2 = 0, best3 = 0;
        static_for<Cfg::TN>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          const int n = n0 + (wn * Cfg::TN + j) * 32 + r;
          const u64x4 wd = philox4x64_10(c0, (uint64_t)n, c2, c3, a.seed, a.stream_id);
          element(i, 4 * q + 0, j, mb + 0, mb + 0 < a.M, word_to_uniform(wd.x[0]), best0);
          element(i, 4 * q + 1, j, mb + 1, mb + 1 < a.M, word_to_uniform(wd.x[1]), best1);
          element(i, 4 * q + 2, j, mb + 2, mb + 2 < a.M, word_to_uniform(wd.x[2]), best2);
          element(i, 4 * q + 3, j, mb + 3, mb + 3 < a.M, word_to_uniform(wd.x[3]), best3);
        });
        finish_row(i, 4 * q + 0, best0);
        finish_row(i, 4 * q + 1, best1);
        finish_row(i, 4 * q + 2, best2);
        finish_row(i, 4 * q + 3, best3);
      });
    });
  } else {
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + (wm * Cfg::TM + i) * 32 + acc_row(e, hh);
        const bool mok = m < a.M;
        int32_t rnd = 0, sid = 0, slot = 0;
        if (kSample && mok) {
          const int bseq = m / a.block;
          slot = m % a.block;
          rnd = a.round[bseq];
          sid = a.seq_id[bseq];
        }
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j) {
          float u = 0.0f;
          if constexpr (kSample) u = philox_uniform(a.seed, a.stream_id, slot, n0 + (wn * Cfg::TN + j) * 32 + r, rnd, sid);
          element(i, e, j, m, mok, u, best);
        }
        finish_row(i, e, best);
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
    for (int q = 1; q < WPP; ++q) best = umax64(best, red_best[q0 + q]);
    a.part_best[(size_t)m * a.ntiles + tile] = best;
  }
  if constexpr (kLse) {
    // the tile's group partials: consecutive threads take consecutive groups of a row
    const int g0 = n0 / 32;
    for (int idx = threadIdx.x; idx < Cfg::BM * NG; idx += Cfg::NT) {
      const int mrow = idx / NG, g = idx % NG;
      const int m = m0 + mrow;
      if (m >= a.M || g0 + g >= a.ngroups) continue;
      a.part_lse[(size_t)m * a.ngroups + g0 + g] = red_lse[idx];
    }
  }
}

// One wavefront per row: the packed maxima of the row's tiles (exact in any order) and, when asked
// for, the logsumexp of its 32-column groups merged lane-strided in group order, then by a fixed
// xor butterfly: an order set by the vocabulary size alone.
__global__ __launch_bounds__(64) void lmhead_finalize(const uint64_t* part_best, const float2* part_lse, int ntiles,
                                                      int ngroups, int32_t* token, float* lse) {
  const int row = blockIdx.x, lane = threadIdx.x;
  uint64_t best = 0;
  {
    constexpr int U = 4;  // four of the lane's tiles are loaded before they are merged
    const size_t base = (size_t)row * ntiles;
    int t = lane;
    for (; t + 64 * (U - 1) < ntiles; t += 64 * U) {
      uint64_t b2[U];
#pragma unroll
      for (int u = 0; u < U; ++u) b2[u] = part_best[base + t + 64 * u];
#pragma unroll
      for (int u = 0; u < U; ++u) best = umax64(best, b2[u]);
    }
    for (; t < ntiles; t += 64) best = umax64(best, part_best[base + t]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) best = umax64(best, shfl_xor_u64(best, off));
  }
  float lm = -__builtin_huge_valf(), ls = 0.0f;
  if (part_lse) {
    constexpr int U = 4;
    const size_t base = (size_t)row * ngroups;
    int g = lane;
    for (; g + 64 * (U - 1) < ngroups; g += 64 * U) {
      float2 p2[U];
#pragma unroll
      for (int u = 0; u < U; ++u) p2[u] = part_lse[base + g + 64 * u];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) lse_merge_opt(lm, ls, p2[u].x, p2[u].y);
    }
    for (; g < ngroups; g += 64) {
      const float2 p2 = part_lse[base + g];
      lse_merge_opt(lm, ls, p2.x, p2.y);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float m2 = shfl_xor_f(lm, off), s2 = shfl_xor_f(ls, off);
      lse_merge_opt(lm, ls, m2, s2);
    }
  }
  if (lane == 0) {
    token[row] = unpack_idx(best);
    if (lse) lse[row] = lm + logf(ls);
  }
}

template <typename T, typename Cfg, bool kSample, bool kLse>
int32_t launch_mode(const LmArgs& a, hipStream_t st, int grid, size_t lds) {
  allow_lds(lmhead_kernel<T, Cfg, kSample, kLse>, lds);
  hipLaunchKernelGGL((lmhead_kernel<T, Cfg, kSample, kLse>), dim3(grid), dim3(Cfg::NT), lds, st, a);
  return check_launch("orthrus_lmhead_argmax");
}

template <typename T, typename Cfg>
int32_t launch(LmArgs& a, bool sample, bool lse, hipStream_t st, int tile0 = 0, int wg_tiles = -1) {
  const int mtiles = (a.M + Cfg::BM - 1) / Cfg::BM;
  const size_t red = (size_t)Cfg::BM * Cfg::WN * sizeof(uint64_t) + (size_t)Cfg::BM * (Cfg::BN / 32) * sizeof(float2);
  const size_t lds = std::max(Cfg::RING, red);
  if (wg_tiles < 0) wg_tiles = (a.ntiles - tile0) / (Cfg::BN / kLmBN) + ((a.ntiles - tile0) % (Cfg::BN / kLmBN) != 0);
  if (wg_tiles == 0) return ORTHRUS_OK;
  a.tile0 = tile0;
  const int grid = mtiles * wg_tiles;
  if (sample) return lse ? launch_mode<T, Cfg, true, true>(a, st, grid, lds) : launch_mode<T, Cfg, true, false>(a, st, grid, lds);
  return lse ? launch_mode<T, Cfg, false, true>(a, st, grid, lds) : launch_mode<T, Cfg, false, false>(a, st, grid, lds);
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
// wavefronts, each owning one 128-column partial tile), then the remaining tiles as 128x128
// workgroups of four wavefronts in a second launch.  A 256x256 workgroup re-reads the 2 MiB
// activation tile from L2 once per 256 columns instead of once per 128, which is what bounds the LM
// head; a grid of only 256x256 tiles would leave a last wave of 82 workgroups on 256 CUs at
// V = 151936, hence the mix.  The rest (163 tiles at M = 256) runs as 326 row-halves rather than
// 163 workgroups of 256 rows, so more CUs share it (391-398 against 401-406 us per call); rows do
// not change an element's k order, so the bits are the same.
// The partials stay per 128-column tile, so the finalize merge is the same whatever the split.
template <typename T>
int32_t launch_mixed(LmArgs& a, bool sample, bool lse, hipStream_t st) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  }
  const int mtiles = (a.M + 255) / 256;
  const int rounds = (a.ntiles * mtiles) / (2 * cus);
  int npairs = std::min(a.ntiles / 2, rounds * cus / mtiles);
  if (int32_t s = launch<T, LmPairCfg<T>>(a, sample, lse, st, 0, npairs)) return s;
  return launch<T, ORTHRUS_LM_BIG_CFG(T)>(a, sample, lse, st, 2 * npairs);
}

}  // namespace
}  // namespace orthrus

using namespace orthrus;

// Workspace: the packed maxima of every (row, 128-column tile), then the logsumexp partials of
// every (row, 32-column group).
extern "C" size_t orthrus_lmhead_workspace_bytes(const orthrus_lmhead_desc_t* d) {
  if (!d || d->rows < 0 || d->vocab <= 0) return 0;
  const size_t ntiles = (d->vocab + kLmBN - 1) / kLmBN, ngroups = (d->vocab + 31) / 32;
  return (size_t)d->rows * (ntiles * sizeof(uint64_t) + ngroups * sizeof(float2));
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
  ORTHRUS_REQUIRE(d->sample == 0 || d->sample == 1, ORTHRUS_ERR_INVALID_ARG, "lmhead: sample must be 0 or 1");
  ORTHRUS_REQUIRE(h && w && token_out, ORTHRUS_ERR_INVALID_ARG, "lmhead: null pointer");
  const bool sample = d->sample != 0;
  ORTHRUS_REQUIRE(!sample || d->temperature > 0.0f, ORTHRUS_ERR_INVALID_ARG, "lmhead: sampling needs temperature > 0");
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
  a.ngroups = (d->vocab + 31) / 32;
  a.part_best = reinterpret_cast<uint64_t*>(ws);
  a.part_lse = reinterpret_cast<float2*>(a.part_best + (size_t)a.M * a.ntiles);
  a.inv_t = d->temperature > 0.0f ? 1.0f / d->temperature : 1.0f;
  a.seed = d->seed;
  a.stream_id = (uint64_t)d->stream_id;
  const bool lse = lse_out != nullptr;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int32_t s;
  if (d->dtype == ORTHRUS_BF16) {
    if (a.M <= 32) s = launch<bf16, GemmCfg<bf16, 32, kLmBN, 1, 4, 4, 4>>(a, sample, lse, st);
    else if (a.M <= 64) s = launch<bf16, GemmCfg<bf16, 64, kLmBN, 2, 2, 3, 3>>(a, sample, lse, st);
    else if (a.M <= 128) s = launch<bf16, ORTHRUS_LM_BIG_CFG(bf16)>(a, sample, lse, st);
    else if (a.K % 128 == 0) s = launch_mixed<bf16>(a, sample, lse, st);
    else s = launch<bf16, ORTHRUS_LM_HUGE_CFG(bf16)>(a, sample, lse, st);
  } else {
    if (a.M <= 32) s = launch<float, GemmCfg<float, 32, kLmBN, 1, 4, 4, 4>>(a, sample, lse, st);
    else if (a.M <= 64) s = launch<float, GemmCfg<float, 64, kLmBN, 2, 2, 3, 3>>(a, sample, lse, st);
    else if (a.M <= 128) s = launch<float, ORTHRUS_LM_BIG_CFG(float)>(a, sample, lse, st);
    else s = launch<float, ORTHRUS_LM_HUGE_CFG(float)>(a, sample, lse, st);
  }
  if (s != ORTHRUS_OK) return s;
  hipLaunchKernelGGL(lmhead_finalize, dim3(a.M), dim3(64), 0, st, a.part_best, lse ? a.part_lse : nullptr, a.ntiles,
                     a.ngroups, token_out, lse_out);
  return check_launch("orthrus_lmhead_argmax(finalize)");
}

// ------------------------------------------------------------------------------------------
// The same call with its partials in a static device array instead of a caller workspace, for
// callers that cannot allocate.  Each device holds its own copy of `scratch` from the module load
// until the process ends; its address on a device is taken once with hipGetSymbolAddress (with
// that device current) and kept per device, since the host-side name is not a device address.
// ------------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[ORTHRUS_LMHEAD_SCRATCH_BYTES];

namespace orthrus {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int32_t scratch_address(hipStream_t st, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(ORTHRUS_ERR_HIP, "lmhead_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  int dev = cur;
  if (st != nullptr) {
    e = hipStreamGetDevice(st, &dev);
    if (e != hipSuccess) return fail(ORTHRUS_ERR_HIP, "lmhead_noalloc: hipStreamGetDevice: %s", hipGetErrorString(e));
  }
  ORTHRUS_REQUIRE(dev >= 0 && dev < kMaxDevices, ORTHRUS_ERR_UNSUPPORTED, "lmhead_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(ORTHRUS_ERR_HIP, "lmhead_noalloc: hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr)
      return fail(ORTHRUS_ERR_HIP, "lmhead_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ORTHRUS_OK;
}

}  // namespace
}  // namespace orthrus

extern "C" int32_t orthrus_lmhead_argmax_noalloc(const orthrus_lmhead_desc_t* d, const void* h, const void* w,
                                                 const int32_t* seq_id, const int32_t* round, int32_t* token_out,
                                                 float* logits_out, float* lse_out, void* stream) {
  ORTHRUS_REQUIRE(d != nullptr, ORTHRUS_ERR_INVALID_ARG, "lmhead_noalloc: null descriptor");
  const size_t need = orthrus_lmhead_workspace_bytes(d);
  ORTHRUS_REQUIRE(need <= (size_t)ORTHRUS_LMHEAD_SCRATCH_BYTES, ORTHRUS_ERR_WORKSPACE,
                  "lmhead_noalloc: %d rows x vocab %d need %zu bytes of partials, above the static scratch of %zu",
                  d->rows, d->vocab, need, (size_t)ORTHRUS_LMHEAD_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int32_t s = scratch_address(reinterpret_cast<hipStream_t>(stream), &ws)) return s;
  return orthrus_lmhead_argmax(d, h, w, seq_id, round, token_out, logits_out, lse_out, ws,
                               (size_t)ORTHRUS_LMHEAD_SCRATCH_BYTES, stream);
}
