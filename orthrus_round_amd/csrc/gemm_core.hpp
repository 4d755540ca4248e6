// MFMA main loop for C = A W^T with A [M, K] and W [N, K] both K-contiguous (the layout of
// activations and of Linear weights), shared by the layer GEMMs and the LM head.
//
// A workgroup of 4 wavefronts computes a BM x BN tile; the waves form a WM x WN grid and each
// owns TM x TN 32x32 MFMA accumulators.  K is consumed in LDS stages of 128 bytes per row,
// prefetched into registers one stage ahead; every output element accumulates its k-steps in
// ascending order with the same instruction whatever BM/BN are, so a row's result never
// depends on how many rows share the launch.
#pragma once

#include "common.hpp"

namespace orthrus {

template <typename T, int BM_, int BN_, int WM_, int WN_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NT = 256;
  static_assert(WM * WN == 4, "4 wavefronts per workgroup");
  static constexpr int TM = BM / (32 * WM), TN = BN / (32 * WN);
  static_assert(TM >= 1 && TN >= 1 && TM * 32 * WM == BM && TN * 32 * WN == BN, "tile shape");
  static constexpr int EPC = 16 / sizeof(T);    // elements per 16-byte chunk
  static constexpr int BK = 8 * EPC;            // 128 bytes of k per stage
  static constexpr int LDS_LD = BK + EPC;       // padded LDS row
  static constexpr int ACH = BM * 8 / NT;       // A chunks per thread per stage
  static constexpr int BCH = BN * 8 / NT;
  static_assert(ACH >= 1 && BCH >= 1, "tile too small for 256 threads");
  static constexpr size_t LDS_BYTES = (size_t)(BM + BN) * LDS_LD * sizeof(T);
};

// Map the linear workgroup id to (m_tile, n_tile) so that the m-tiles sharing a slice of W run
// back to back on the same XCD (workgroups are dealt round-robin to the 8 XCDs, each with its
// own L2): W then comes from HBM once.
__device__ __forceinline__ void xcd_tile_map(int id, int total, int mtiles, int& mt, int& nt) {
  int L = id;
  if (total % 8 == 0) L = (id % 8) * (total / 8) + id / 8;
  mt = L % mtiles;
  nt = L / mtiles;
}

template <typename T, typename Cfg>
__device__ __forceinline__ void gemm_mainloop(const T* __restrict__ A, const T* __restrict__ W, int M, int N, int K,
                                              int m0, int n0, T* lds, f32x16 (&acc)[Cfg::TM][Cfg::TN]) {
  using MF = Mfma<T>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, EPC = Cfg::EPC, LD = Cfg::LDS_LD;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, NT = Cfg::NT;
  T* lds_a = lds;
  T* lds_b = lds + BM * LD;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hh = lane >> 5, r = lane & 31;
  const int wm = w / Cfg::WN, wn = w % Cfg::WN;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  u32x4 areg[Cfg::ACH], breg[Cfg::BCH];
  auto load = [&](int kt) {
#pragma unroll
    for (int j = 0; j < Cfg::ACH; ++j) {
      const int ci = tid + j * NT, row = ci >> 3, part = ci & 7;
      const int gm = m0 + row;
      areg[j] = gm < M ? *reinterpret_cast<const u32x4*>(A + (size_t)gm * K + kt * BK + part * EPC) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < Cfg::BCH; ++j) {
      const int ci = tid + j * NT, row = ci >> 3, part = ci & 7;
      const int gn = n0 + row;
      breg[j] = gn < N ? *reinterpret_cast<const u32x4*>(W + (size_t)gn * K + kt * BK + part * EPC) : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < Cfg::ACH; ++j) {
      const int ci = tid + j * NT, row = ci >> 3, part = ci & 7;
      *reinterpret_cast<u32x4*>(&lds_a[row * LD + part * EPC]) = areg[j];
    }
#pragma unroll
    for (int j = 0; j < Cfg::BCH; ++j) {
      const int ci = tid + j * NT, row = ci >> 3, part = ci & 7;
      *reinterpret_cast<u32x4*>(&lds_b[row * LD + part * EPC]) = breg[j];
    }
  };

  const int nk = K / BK;
  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    store();
    __syncthreads();
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / MF::KSTEP; ++kk) {
      typename MF::frag af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const T* p = &lds_a[((wm * TM + i) * 32 + r) * LD + kk * MF::KSTEP + MF::KW * hh];
        if constexpr (MF::KW == 8) af[i] = *reinterpret_cast<const bf16x8*>(p);
        else af[i] = *p;
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const T* p = &lds_b[((wn * TN + j) * 32 + r) * LD + kk * MF::KSTEP + MF::KW * hh];
        if constexpr (MF::KW == 8) bfr[j] = *reinterpret_cast<const bf16x8*>(p);
        else bfr[j] = *p;
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = MF::mma(af[i], bfr[j], acc[i][j]);
    }
  }
}

}  // namespace orthrus
