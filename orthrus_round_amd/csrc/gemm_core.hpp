// MFMA main loop for C = A W^T with A [M, K] and W [N, K] both K-contiguous (the layout of
// activations and of Linear weights), shared by the layer GEMMs and the LM head.
//
// A workgroup of 4 wavefronts computes a BM x BN tile over a k range; the waves form a WM x WN
// grid and each owns TM x TN 32x32 MFMA accumulators.  K is consumed in stages of 128 bytes per
// row.  Tiles move HBM -> LDS with gfx950's direct global_load_lds (16 bytes per lane, no
// register staging) into a ring of STAGES LDS buffers, so STAGES-1 stages are in flight while
// one is multiplied.  Rows are stored unpadded with their 16-byte chunks XOR-swizzled by
// (row / 2) mod 8, which makes the MFMA fragment reads (32 rows, same chunk) bank-conflict free.
// Every output element accumulates its k-steps in ascending order with the same instruction
// whatever BM/BN are, so a row's result never depends on how many rows share the launch.
#pragma once

#include "common.hpp"

namespace orthrus {

#ifndef ORTHRUS_GEMM_STAGES
#define ORTHRUS_GEMM_STAGES 3
#endif

template <typename T, int BM_, int BN_, int WM_, int WN_, int STAGES_ = ORTHRUS_GEMM_STAGES>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr bool KSPLIT = false;
  static constexpr int NT = 256;
  static_assert(WM * WN == 4, "4 wavefronts per workgroup");
  static constexpr int TM = BM / (32 * WM), TN = BN / (32 * WN);
  static_assert(TM >= 1 && TN >= 1 && TM * 32 * WM == BM && TN * 32 * WN == BN, "tile shape");
  static constexpr int EPC = 16 / sizeof(T);    // elements per 16-byte chunk
  static constexpr int BK = 8 * EPC;            // 128 bytes of k per stage
  static constexpr int ROWB = 128;              // bytes per tile row per stage
  static constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  static constexpr int NI = (BM + BN) / 32;     // load instructions per wave per stage
  static_assert(NI * 32 == BM + BN, "tile rows must split into 8-row wave loads");
  static constexpr size_t LDS_BYTES = (size_t)STAGES * STAGE_BYTES;
};

// Map the linear workgroup id to (split, m_tile, n_tile) so that the splits and m-tiles sharing
// a slice of W run back to back on the same XCD (workgroups are dealt round-robin to the 8 XCDs,
// each with its own L2): W then comes from HBM once and split partials stay in that L2.
// XCD x receives ids x, x+8, ...; with total = 8q + r the first r XCDs get q+1 of them, and XCD x
// takes the contiguous logical range starting at x*q + min(x, r), so the map is a bijection.
__device__ __forceinline__ int xcd_linear(int id, int total) {
  const int x = id & 7, slot = id >> 3, q = total >> 3, r = total & 7;
  return x * q + (x < r ? x : r) + slot;
}

__device__ __forceinline__ void xcd_tile_map(int id, int total, int splits, int mtiles, int& s, int& mt, int& nt) {
  int L = xcd_linear(id, total);
  s = L % splits;
  L /= splits;
  mt = L % mtiles;
  nt = L / mtiles;
}

__device__ __forceinline__ int lds_swizzle(int row) { return (row >> 1) & 7; }

template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS at dst + lane * 16 (dst wave-uniform).
__device__ __forceinline__ void load_to_lds16(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

template <typename T, typename Cfg, typename Acc>
__device__ __forceinline__ void gemm_mainloop(const T* __restrict__ A, const T* __restrict__ W, int M, int N, int K,
                                              int m0, int n0, int k_begin, int k_len, unsigned char* lds, Acc& acc) {
  using MF = Mfma<T>;
  constexpr int BM = Cfg::BM, BK = Cfg::BK, EPC = Cfg::EPC, ROWB = Cfg::ROWB;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, S = Cfg::STAGES, NI = Cfg::NI;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hh = lane >> 5, r = lane & 31;
  const int wm = w / Cfg::WN, wn = w % Cfg::WN;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  // Per-lane source pointers for the NI wave loads of a stage (k offset added per stage).  Load j
  // of wave w covers tile rows (j*4 + w)*8 .. +7 of the combined [A rows | W rows] space; lane l
  // lands in row +l/8, slot l%8, and fetches the chunk that slot holds under the swizzle.  Rows
  // past M or N read a clamped valid row: those outputs are never stored.
  const T* src[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int row = (j * 4 + w) * 8 + (lane >> 3);
    const bool is_a = row < BM;
    const int trow = is_a ? row : row - BM;
    const int chunk = (lane & 7) ^ lds_swizzle(trow);
    const T* base = is_a ? A + (size_t)min(m0 + trow, M - 1) * K : W + (size_t)min(n0 + trow, N - 1) * K;
    src[j] = base + k_begin + chunk * EPC;
  }
  auto issue = [&](int kt, int buf) {
    unsigned char* dst = lds + buf * Cfg::STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < NI; ++j)
      load_to_lds16(src[j] + (size_t)kt * BK, dst + (j * 4 + w) * 8 * ROWB);
  };
  auto frag = [&](const unsigned char* tile, int row, int kk) -> typename MF::frag {
    if constexpr (MF::KW == 8) {
      const int chunk = 2 * kk + hh;
      return *reinterpret_cast<const bf16x8*>(tile + row * ROWB + ((chunk ^ lds_swizzle(row)) << 4));
    } else {
      const int e = kk * MF::KSTEP + hh;  // element within the 32-element stage row
      return *reinterpret_cast<const float*>(tile + row * ROWB + (((e >> 2) ^ lds_swizzle(row)) << 4) + ((e & 3) << 2));
    }
  };
  // all of a stage's fragments are read from LDS before its MFMAs issue, so the LDS latency of
  // later k-steps hides behind the MFMAs of earlier ones
  auto compute = [&](int buf) {
    const unsigned char* ta = lds + buf * Cfg::STAGE_BYTES;
    const unsigned char* tb = ta + BM * ROWB;
    constexpr int KPS = BK / MF::KSTEP;
    typename MF::frag af[KPS][TM], bfr[KPS][TN];
#pragma unroll
    for (int kk = 0; kk < KPS; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i) af[kk][i] = frag(ta, (wm * TM + i) * 32 + r, kk);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[kk][j] = frag(tb, (wn * TN + j) * 32 + r, kk);
    }
#pragma unroll
    for (int kk = 0; kk < KPS; ++kk)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = MF::mma(af[kk][i], bfr[kk][j], acc[i][j]);
  };

  const int nk = k_len / BK;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once at most S-2 younger stages are still outstanding
    if (kt + S - 2 < nk) wait_vmcnt<(S - 2) * NI>();
    else wait_vmcnt<0>();
    // Every wave's share of stage kt is in LDS and stage kt-1 is fully consumed (its fragments
    // fed MFMAs already).  A bare s_barrier: __syncthreads() would add a fence that waits for
    // ALL outstanding loads, i.e. for the stages still in flight.
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + S - 1 < nk) issue(kt + S - 1, (kt + S - 1) % S);
    compute(kt % S);
  }
}

}  // namespace orthrus

namespace orthrus {

// Layer-GEMM main loop: a BM x BN tile per workgroup in which each of the 4 wavefronts owns the
// WHOLE tile for one quarter of the k-steps (wave w takes the k-steps s with s mod 4 == w), and
// the four partial tiles are summed in wave order through LDS.  Small tiles keep enough
// workgroups streaming weights for every decode shape without any cross-workgroup reduction,
// and the summation order is the same for every M.
template <typename T, int BM_, int BN_, int STAGES_ = 4>
struct KsCfg {
  static constexpr int BM = BM_, BN = BN_, STAGES = STAGES_;
  static constexpr bool KSPLIT = true;
  static constexpr int WM = 1, WN = 1;
  static constexpr int TM = BM / 32, TN = BN / 32;
  static constexpr int EPC = 16 / sizeof(T);
  static constexpr int BK = 8 * EPC;
  static constexpr int ROWB = 128;
  static constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  static constexpr int NI = (BM + BN) / 32;
  static_assert(NI * 32 == BM + BN, "tile rows must split into 8-row wave loads");
  static constexpr int PART_BYTES = 4 * TM * TN * 16 * 64 * 4;  // 4 waves' partial tiles
  static constexpr size_t LDS_BYTES =
      (size_t)STAGES * STAGE_BYTES > (size_t)PART_BYTES ? (size_t)STAGES * STAGE_BYTES : (size_t)PART_BYTES;
};

template <typename T, typename Cfg, typename Acc>
__device__ __forceinline__ void gemm_mainloop_ks4(const T* __restrict__ A, const T* __restrict__ W, int M, int N,
                                                  int K, int m0, int n0, unsigned char* lds, Acc& acc) {
  using MF = Mfma<T>;
  constexpr int BM = Cfg::BM, BK = Cfg::BK, EPC = Cfg::EPC, ROWB = Cfg::ROWB;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, S = Cfg::STAGES, NI = Cfg::NI;
  constexpr int KPS = BK / MF::KSTEP;  // k-steps per stage (4 for bf16, 16 for fp32)
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hh = lane >> 5, r = lane & 31;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const T* src[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int row = (j * 4 + w) * 8 + (lane >> 3);
    const bool is_a = row < BM;
    const int trow = is_a ? row : row - BM;
    const int chunk = (lane & 7) ^ lds_swizzle(trow);
    const T* base = is_a ? A + (size_t)min(m0 + trow, M - 1) * K : W + (size_t)min(n0 + trow, N - 1) * K;
    src[j] = base + chunk * EPC;
  }
  auto issue = [&](int kt, int buf) {
    unsigned char* dst = lds + buf * Cfg::STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < NI; ++j) load_to_lds16(src[j] + (size_t)kt * BK, dst + (j * 4 + w) * 8 * ROWB);
  };
  auto frag = [&](const unsigned char* tile, int row, int kk) -> typename MF::frag {
    if constexpr (MF::KW == 8) {
      const int chunk = 2 * kk + hh;
      return *reinterpret_cast<const bf16x8*>(tile + row * ROWB + ((chunk ^ lds_swizzle(row)) << 4));
    } else {
      const int e = kk * MF::KSTEP + hh;
      return *reinterpret_cast<const float*>(tile + row * ROWB + (((e >> 2) ^ lds_swizzle(row)) << 4) + ((e & 3) << 2));
    }
  };
  auto compute = [&](int buf) {
    const unsigned char* ta = lds + buf * Cfg::STAGE_BYTES;
    const unsigned char* tb = ta + BM * ROWB;
#pragma unroll
    for (int kk = w; kk < KPS; kk += 4) {
      typename MF::frag af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = frag(ta, i * 32 + r, kk);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = frag(tb, j * 32 + r, kk);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = MF::mma(af[i], bfr[j], acc[i][j]);
    }
  };

  const int nk = K / BK;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + S - 2 < nk) wait_vmcnt<(S - 2) * NI>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + S - 1 < nk) issue(kt + S - 1, (kt + S - 1) % S);
    compute(kt % S);
  }

  // every wave parks its partial tile in LDS (lane-major, 16-byte stores); ks4_sum() then adds the
  // four partials of one 32x32 block in wave order
  __syncthreads();
  f32x4* part = reinterpret_cast<f32x4*>(lds);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part[(((w * TM + i) * TN + j) * 4 + e) * 64 + lane] =
            f32x4{acc[i][j][4 * e], acc[i][j][4 * e + 1], acc[i][j][4 * e + 2], acc[i][j][4 * e + 3]};
  __syncthreads();
}

template <typename Cfg>
__device__ __forceinline__ f32x16 ks4_sum(const unsigned char* lds, int i, int j) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN;
  const int lane = threadIdx.x & 63;
  const f32x4* part = reinterpret_cast<const f32x4*>(lds);
  f32x16 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f32x4 v = part[(((0 * TM + i) * TN + j) * 4 + e) * 64 + lane];
#pragma unroll
    for (int q = 1; q < 4; ++q) v += part[(((q * TM + i) * TN + j) * 4 + e) * 64 + lane];
    out[4 * e] = v[0];
    out[4 * e + 1] = v[1];
    out[4 * e + 2] = v[2];
    out[4 * e + 3] = v[3];
  }
  return out;
}

}  // namespace orthrus
