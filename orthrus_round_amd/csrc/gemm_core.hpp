// MFMA main loops for C = A W^T with A [M, K] and W [N, K] both K-contiguous (the layout of
// activations and of Linear weights), shared by the layer GEMMs and the LM head.
//
// A workgroup of 4 wavefronts computes a BM x BN tile.  K is consumed in stages of 128 bytes per
// row.  Tiles move to LDS with gfx950's direct global_load_lds (16 bytes per lane, no register
// staging).  Rows are stored unpadded with their 16-byte chunks XOR-swizzled by (row / 2) mod 8,
// which makes the MFMA fragment reads (32 rows, same chunk) bank-conflict free.
//
// Loads are split by operand: waves 0-1 stream the A tile (activations, small and L2-resident)
// through a shallow ring of SA stages, waves 2-3 stream the W tile (weights, from HBM) through a
// deep ring of SW stages.  The vector-memory counter is per wave, so each role waits only for its
// own ring, and the slow weight stream keeps SW-1 stages in flight however fast A arrives.  One
// barrier per stage publishes both tiles and retires the stage consumed before it.
//
// Two compute layouts:
//  * plain (GemmCfg): the waves form a WM x WN grid over the tile and each runs every k-step;
//  * k-split (KsCfg): each wave owns the WHOLE tile for one quarter of the k-steps (wave w takes
//    k-step w of every 4-step stage), and the four partial tiles are summed in wave order
//    through LDS afterwards.
// In both, an output element's summation order depends on K only, never on BM/BN or M, so a row's
// result does not depend on how many rows share the launch.
#pragma once

#include "common.hpp"

// The rings take up to 80 KiB of LDS, so at most two workgroups (two waves per SIMD) share a CU:
// tell the compiler, so that it spends the registers that occupancy leaves free on keeping a
// stage's fragments in flight instead of minimising them.
// MFMAs per software-pipeline part of the plain layout (see gemm_mainloop)
#ifndef ORTHRUS_PART_MFMAS
#define ORTHRUS_PART_MFMAS 8
#endif

#ifndef ORTHRUS_GEMM_WAVES
#define ORTHRUS_GEMM_WAVES __attribute__((amdgpu_waves_per_eu(1, 2)))
#endif

namespace orthrus {

template <typename T, int BM_, int BN_, int SA_, int SW_, int NW_>
struct StageRings {
  static constexpr int BM = BM_, BN = BN_, SA = SA_, SW = SW_;
  static constexpr int NW = NW_, NT = 64 * NW_;  // wavefronts and threads per workgroup
  static constexpr int RW = NW_ / 2;             // wavefronts per load role (A or W)
  static constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  static constexpr int BK = 8 * EPC;          // 128 bytes of k per stage
  static constexpr int ROWB = 128;            // bytes per tile row per stage
  static constexpr int A_STAGE = BM * ROWB, W_STAGE = BN * ROWB;
  static constexpr int NLA = BM / (8 * RW);   // 1 KiB wave loads per A-wave per stage
  static constexpr int NLW = BN / (8 * RW);   // per W-wave per stage
  static_assert(NW == 4 || NW == 8, "four or eight wavefronts per workgroup");
  static_assert(NLA * 8 * RW == BM && NLW * 8 * RW == BN && NLA >= 1 && NLW >= 1,
                "tile rows must split over each role's waves");
  static_assert(SA >= 2 && SW >= 2, "rings need two stages");
  static_assert((SA - 2) * NLA < 64 && (SW - 2) * NLW < 64, "loads in flight must fit the vmcnt counter");
  static constexpr size_t RING_BYTES = (size_t)SA * A_STAGE + (size_t)SW * W_STAGE;
};

template <typename T, int BM_, int BN_, int WM_, int WN_, int SA_, int SW_, bool EVEN_ = false>
struct GemmCfg : StageRings<T, BM_, BN_, SA_, SW_, WM_ * WN_> {
  static constexpr int WM = WM_, WN = WN_;
  static constexpr bool KSPLIT = false;
  static constexpr bool EVEN_STAGES = EVEN_;
  static constexpr int TM = BM_ / (32 * WM), TN = BN_ / (32 * WN);
  static_assert(TM >= 1 && TN >= 1 && TM * 32 * WM == BM_ && TN * 32 * WN == BN_, "tile shape");
  static constexpr size_t TILE_BYTES = (size_t)BM_ * BN_ * 4;  // the fp32 tile parked for the epilogue
  static constexpr size_t RING = StageRings<T, BM_, BN_, SA_, SW_, WM_ * WN_>::RING_BYTES;
  static constexpr size_t LDS_BYTES = RING > TILE_BYTES ? RING : TILE_BYTES;
};

template <typename T, int BM_, int BN_, int SA_, int SW_>
struct KsCfg : StageRings<T, BM_, BN_, SA_, SW_, 4> {
  static constexpr int WM = 1, WN = 1;
  static constexpr bool KSPLIT = true;
  static constexpr bool EVEN_STAGES = false;
  static constexpr int TM = BM_ / 32, TN = BN_ / 32;
  static constexpr size_t PART_BYTES = (size_t)4 * TM * TN * 16 * 64 * 4;  // 4 waves' partial tiles
  static constexpr size_t RING = StageRings<T, BM_, BN_, SA_, SW_, 4>::RING_BYTES;
  static constexpr size_t LDS_BYTES = RING > PART_BYTES ? RING : PART_BYTES;
};

// Map the linear workgroup id to (split, m_tile, n_tile) so that the splits and m-tiles sharing
// a slice of W run back to back on the same XCD (workgroups are dealt round-robin to the 8 XCDs,
// each with its own L2): W then comes from HBM once.
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

// The k-split variant: the split index varies slowest, so each XCD works on one slice of K (or
// one of its halves' tiles) and fetches only that slice of the activation, instead of all of it
// on every XCD; within a slice the m-tiles sharing a slice of W still run back to back.  Only the
// placement changes: each (split, m_tile, n_tile) is computed exactly as before.
__device__ __forceinline__ void xcd_tile_map_ksplit(int id, int total, int splits, int mtiles, int& s, int& mt,
                                                    int& nt) {
  const int per_split = total / splits;  // total = splits * mtiles * ntiles
  int L = xcd_linear(id, total);
  s = L / per_split;
  L -= s * per_split;
  mt = L % mtiles;
  nt = L / mtiles;
}

__device__ __forceinline__ int lds_swizzle(int row) { return (row >> 1) & 7; }

template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `younger` stages of NL loads each are outstanding (0 <= younger <= S-2).
template <int S, int NL, int I = S - 2>
__device__ __forceinline__ void wait_stages(int younger) {
  if constexpr (I <= 0) {
    wait_vmcnt<0>();
  } else {
    if (younger >= I) wait_vmcnt<I * NL>();
    else wait_stages<S, NL, I - 1>(younger);
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS at dst + lane * 16 (dst wave-uniform).
__device__ __forceinline__ void load_to_lds16(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

// Stage kt of one role's ring: load j of wave wl (of RW role waves) fills tile rows
// (RW*j + wl)*8 .. +7 of slot kt % S.  Takes its state by value: lambdas capturing the per-lane
// pointers by reference were left in scratch memory by the compiler when the two rings differ in
// depth.
template <int S, int NL, int STAGE, int BK, int RW, typename T>
__device__ __forceinline__ void issue_stage(const T* src0, int row0, int lim, int K, unsigned char* ring, int kt,
                                            int wl) {
  unsigned char* dst = ring + (kt % S) * STAGE;
#pragma unroll
  for (int j = 0; j < NL; ++j)
    load_to_lds16(src0 + (size_t)min(row0 + 8 * RW * j, lim) * K + (size_t)kt * BK, dst + (RW * j + wl) * 8 * 128);
}

// Shared main loop.  On return acc holds this wave's accumulators: its WM x WN share of the tile
// (plain), or its k-quarter partial of the whole tile, already parked in LDS for ks4_sum (k-split).
// K is the row stride of A and W; kext (default K) is how many k of each row the loop consumes,
// starting at the given A and W pointers.
template <typename T, typename Cfg, typename Acc>
__device__ __forceinline__ void gemm_mainloop(const T* __restrict__ A, const T* __restrict__ W, int M, int N, int K,
                                              int m0, int n0, unsigned char* lds, Acc& acc, int kext = -1) {
  using MF = Mfma<T>;
  constexpr int BK = Cfg::BK, EPC = Cfg::EPC, ROWB = Cfg::ROWB;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, SA = Cfg::SA, SW = Cfg::SW;
  constexpr int NLA = Cfg::NLA, NLW = Cfg::NLW;
  constexpr int KPS = BK / MF::KSTEP;  // k-steps per stage (4 for bf16, 16 for fp32)
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, r = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform wave index
  constexpr int RW = Cfg::RW;
  const bool w_role = wu >= RW;                               // the upper half loads W, the lower A
  const int wl = wu % RW;                                     // wave within its role
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  unsigned char* const ring_a = lds;
  unsigned char* const ring_w = lds + (size_t)SA * Cfg::A_STAGE;

  // Per-lane source pointers of this wave's loads (k offset added per stage).  Load j of role wave
  // wl fills tile rows (RW*j + wl)*8 .. +7; lane l lands in row +l/8, slot l%8, and fetches the
  // chunk that slot holds under the swizzle.  Rows past M or N read a clamped valid row: those
  // outputs are never stored.
  // Row trow = 8RW*j + 8wl + l/8 has swizzle (trow/2) mod 8 = (4wl + l/16) mod 8 for every j
  // (4RW*j is a multiple of 8).
  // The row offset is recomputed per load: an array of per-load pointers ends up in scratch.
  const T* const mat = w_role ? W : A;
  const int lim = (w_role ? N : M) - 1;
  const int row0 = (w_role ? n0 : m0) + wl * 8 + (lane >> 3);
  const T* const src0 = mat + ((lane & 7) ^ lds_swizzle(wl * 8 + (lane >> 3))) * EPC;
  auto issue_a = [&](int kt) __attribute__((always_inline)) {
    issue_stage<SA, NLA, Cfg::A_STAGE, BK, RW>(src0, row0, lim, K, ring_a, kt, wl);
  };
  auto issue_w = [&](int kt) __attribute__((always_inline)) {
    issue_stage<SW, NLW, Cfg::W_STAGE, BK, RW>(src0, row0, lim, K, ring_w, kt, wl);
  };
  auto frag = [&](const unsigned char* tile, int row, int kk) __attribute__((always_inline)) -> typename MF::frag {
    if constexpr (MF::KW == 8) {
      const int chunk = 2 * kk + hh;
      return *reinterpret_cast<const bf16x8*>(tile + row * ROWB + ((chunk ^ lds_swizzle(row)) << 4));
    } else {
      const int e = kk * MF::KSTEP + hh;  // element within the 32-element stage row
      return *reinterpret_cast<const float*>(tile + row * ROWB + (((e >> 2) ^ lds_swizzle(row)) << 4) + ((e & 3) << 2));
    }
  };
  auto compute = [&](int kt) __attribute__((always_inline)) {
    const unsigned char* ta = ring_a + (kt % SA) * Cfg::A_STAGE;
    const unsigned char* tb = ring_w + (kt % SW) * Cfg::W_STAGE;
    if constexpr (Cfg::KSPLIT) {
      static_assert(KPS % 4 == 0, "k-steps per stage split four ways");
#pragma unroll
      for (int q = 0; q < KPS / 4; ++q) {
        const int kk = 4 * q + wu;
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
    }
  };
  // Plain layout, software-pipelined over parts of KPP k-steps: the fragment reads of part q are
  // issued before the MFMAs of part q-1, which do not depend on them, so those MFMAs cover the
  // LDS latency.  A part holds about 8 MFMAs; two register buffers alternate.
  constexpr int KPP_W = ORTHRUS_PART_MFMAS / (TM * TN) < 1 ? 1 : ORTHRUS_PART_MFMAS / (TM * TN);
  constexpr int KPP = Cfg::KSPLIT ? 1 : (KPP_W > KPS ? KPS : KPP_W);
  constexpr int NP = KPS / KPP;  // parts per stage
  static_assert(KPS % KPP == 0, "parts tile a stage");
  constexpr int FA = KPP * TM, FB = KPP * TN;
  using Frag = typename MF::frag;
  const int wm = wu / Cfg::WN, wn = wu % Cfg::WN;
  auto read_part = [&](int kt, int p, Frag (&af)[FA], Frag (&bfr)[FB]) __attribute__((always_inline)) {
    const unsigned char* ta = ring_a + (kt % SA) * Cfg::A_STAGE;
    const unsigned char* tb = ring_w + (kt % SW) * Cfg::W_STAGE;
#pragma unroll
    for (int k = 0; k < KPP; ++k) {
#pragma unroll
      for (int i = 0; i < TM; ++i) af[k * TM + i] = frag(ta, (wm * TM + i) * 32 + r, p * KPP + k);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[k * TN + j] = frag(tb, (wn * TN + j) * 32 + r, p * KPP + k);
    }
  };
  auto mma_part = [&](const Frag (&af)[FA], const Frag (&bfr)[FB]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KPP; ++k)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = MF::mma(af[k * TM + i], bfr[k * TN + j], acc[i][j]);
  };

  const int nk = (kext < 0 ? K : kext) / BK;
  if (w_role) {
    for (int s = 0; s < SW - 1 && s < nk; ++s) issue_w(s);
  } else {
    for (int s = 0; s < SA - 1 && s < nk; ++s) issue_a(s);
  }
  // Make stage kt visible to every wave and refill the ring slot of stage kt-1.
  auto sync_stage = [&](int kt) __attribute__((always_inline)) {
    // this wave's share of stage kt has landed once only its younger stages are outstanding
    if (w_role) wait_stages<SW, NLW>(min(SW - 2, nk - 1 - kt));
    else wait_stages<SA, NLA>(min(SA - 2, nk - 1 - kt));
    // This wave's LDS reads of stage kt-1 are complete, so after the barrier its slot may be
    // overwritten.  A bare s_barrier: __syncthreads() would add a fence that waits for every
    // outstanding load.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (w_role) {
      if (kt + SW - 1 < nk) issue_w(kt + SW - 1);
    } else {
      if (kt + SA - 1 < nk) issue_a(kt + SA - 1);
    }
  };
  if constexpr (Cfg::KSPLIT) {
    for (int kt = 0; kt < nk; ++kt) {
      sync_stage(kt);
      compute(kt);
    }
  } else {
    // Part q = NP*kt + p goes to buffer q % 2.  The loop runs two stages per trip so that the
    // buffer of every part is a compile-time choice whatever NP is.
    Frag fa[2][FA], fb[2][FB];
    auto run_stage = [&](int kt, int par) __attribute__((always_inline)) {
      sync_stage(kt);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int cur = (par * NP + p) & 1;
        read_part(kt, p, fa[cur], fb[cur]);
        // keep the scheduler from hoisting the independent MFMAs above the reads, which would
        // leave the next part's MFMAs waiting on them again
        __builtin_amdgcn_sched_barrier(0);
        if (p > 0 || kt > 0) mma_part(fa[cur ^ 1], fb[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      run_stage(kt, 0);
      run_stage(kt + 1, 1);
    }
    if constexpr (Cfg::EVEN_STAGES) {
      mma_part(fa[(2 * NP - 1) & 1], fb[(2 * NP - 1) & 1]);
    } else if (kt < nk) {
      run_stage(kt, 0);
      mma_part(fa[(NP - 1) & 1], fb[(NP - 1) & 1]);
    } else {
      mma_part(fa[(2 * NP - 1) & 1], fb[(2 * NP - 1) & 1]);
    }
  }

  if constexpr (Cfg::KSPLIT) {
    // every wave parks its partial tile in LDS (lane-major, 16-byte stores); ks4_sum() then adds
    // the four partials of one 32x32 block in wave order
    __syncthreads();
    f32x4* part = reinterpret_cast<f32x4*>(lds);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          part[(((wu * TM + i) * TN + j) * 4 + e) * 64 + lane] =
              f32x4{acc[i][j][4 * e], acc[i][j][4 * e + 1], acc[i][j][4 * e + 2], acc[i][j][4 * e + 3]};
    __syncthreads();
  }
}

// Plain layout: every wave parks its accumulator blocks in LDS (block-major, lane-major 16-byte
// stores), so that any wave can read any 32x32 block of the tile in the epilogue.
template <typename Cfg, typename Acc>
__device__ __forceinline__ void park_plain(unsigned char* lds, const Acc& acc) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN, NBJ = Cfg::BN / 32;
  const int lane = threadIdx.x & 63;
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wu / Cfg::WN, wn = wu % Cfg::WN;
  __syncthreads();  // the ring is free: every wave finished its last stage
  f32x4* part = reinterpret_cast<f32x4*>(lds);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part[(((wm * TM + i) * NBJ + wn * TN + j) * 4 + e) * 64 + lane] =
            f32x4{acc[i][j][4 * e], acc[i][j][4 * e + 1], acc[i][j][4 * e + 2], acc[i][j][4 * e + 3]};
  __syncthreads();
}

template <typename Cfg>
__device__ __forceinline__ f32x16 plain_block(const unsigned char* lds, int i, int j) {
  constexpr int NBJ = Cfg::BN / 32;
  const int lane = threadIdx.x & 63;
  const f32x4* part = reinterpret_cast<const f32x4*>(lds);
  f32x16 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x4 v = part[((i * NBJ + j) * 4 + e) * 64 + lane];
    out[4 * e] = v[0];
    out[4 * e + 1] = v[1];
    out[4 * e + 2] = v[2];
    out[4 * e + 3] = v[3];
  }
  return out;
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
