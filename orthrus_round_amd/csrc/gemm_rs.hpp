// Register-streamed MFMA main loop for C = A W^T at 128+ rows (bf16): the weights go from HBM
// straight into VGPRs in MFMA fragment order, and only the activations pass through LDS.
//
// The 256-row GEMMs of a round are bound by the operand bytes each CU pulls, not by the matrix
// cores: when both operands go global -> LDS -> VGPR, every stage costs a CU about 1.75x its MFMA
// time in LDS port cycles, and the weight stream waits on the per-stage barrier.  Here a
// wavefront owns ALL BM rows of its workgroup tile and TNW 32-column blocks:
//  * its weight fragments are private to it, so they need no LDS: each k-step's fragment of a
//    32-column block is one contiguous 1 KiB wave load from the packed weight layout (below), and
//    NB stages of them are kept in flight in registers (no barrier ever waits on the weights);
//  * the activation tile (BM rows x 128 bytes per stage, L2-resident) is shared through an LDS
//    ring of SA stages filled by direct global->LDS loads, one barrier per stage;
//  * LDS traffic per MFMA falls to BM*128 bytes read per wave and stage for BM*TNW*4/32 MFMAs.
// The k order of every output element is the plain chain over the k-steps, the same MFMA sequence
// as gemm_mainloop's one-loop family (N >= 16384), so results have the same bits as those kernels.
//
// Fragment-packed weight layout (orthrus_pack_gate_up_fragments): W [N, K] -> stage-major 4 KiB
// pieces: piece (ks, nb) at (ks * nblk + nb) * 4 KiB holds, for 32-row block nb, 128-byte stage
// ks (64 bf16 of k), k-step kk = 0..3 and lane l = 0..63, the 8 values
// W[32 nb + l % 32][64 ks + 16 kk + 8 (l / 32) + e], e = 0..7 (the B operand of
// v_mfma_f32_32x32x16_bf16 for that block and k-step).  Stage-major: at any moment the workgroups
// stream neighbouring pieces of one stage slab instead of pieces a power-of-two block stride apart,
// which would pile onto the same memory channels.
#pragma once

#include "gemm_core.hpp"

namespace orthrus {

// Element offset of W[n][k] (bf16) in the fragment-packed layout of an [N, K] matrix: 64 k per
// stage, four 16-k steps per stage, fragments of 8 consecutive k.
__host__ __device__ inline size_t packed_offset(int n, int k, int N, int K) {
  const int nblk = (N + 31) >> 5;
  const int nb = n >> 5, r = n & 31, ks = k / 64, kin = k % 64, kk = kin / 16, h = (kin % 16) / 8, e = kin % 8;
  (void)K;
  return ((((size_t)ks * nblk + nb) * 4 + kk) * 64 + (h * 32 + r)) * 8 + e;
}

// NW compute wavefronts own the tile's column blocks.  With NL = 0 they also load the activation
// stages; with NL > 0, NL more wavefronts do only that, so that a compute wave's vector-memory
// counter tracks its weight loads alone and its wait for an activation stage (the barrier) never
// drains weight loads still in flight.
template <int TMW_, int TNW_, int NW_, int SA_, int NB_, int NL_ = 0>
struct RsCfg {
  static constexpr int TMW = TMW_, TNW = TNW_, NW = NW_, SA = SA_, NB = NB_, NL = NL_;
  static constexpr int BM = 32 * TMW, BN = 32 * TNW * NW, NT = 64 * (NW + NL);
  static constexpr int A_STAGE = BM * 128;    // one stage of the activation tile in LDS
  // The activation stage is BM / 8 wave loads of 1 KiB, dealt round-robin to the AW loading waves:
  // loading wave i issues loads i, i + AW, ...; when AW does not divide them the first waves issue
  // one more.
  static constexpr int AW = NL > 0 ? NL : NW;
  static constexpr int ALOADS = BM / 8;
  static constexpr int NLA = (ALOADS + AW - 1) / AW;  // most activation loads of a wave per stage
  static constexpr int NLA_MIN = ALOADS / AW;         // fewest
  static constexpr int NLW = TNW * 4;         // weight fragment loads per wave per stage
  static constexpr size_t RING = (size_t)SA * A_STAGE;
  static_assert(NLA_MIN >= 1 && ALOADS * 8 == BM, "every wave issues activation loads");
  static_assert(AW % 2 == 0, "the activation swizzle assumes an even number of loading waves");
  static_assert(SA >= 2 && NB >= 1, "ring depths");
  // Loads issued after stage s's activation loads, when the stage count is NKS: the prologue
  // issues activation stages 0..SA-2 then weight stages 0..NB-1; stage t issues activation stage
  // t+SA-1 then weight stage t+NB, each only if it exists.  Waiting until at most that many loads
  // are outstanding guarantees stage s's activations (loads complete in issue order).  The count
  // takes NLA_MIN activation loads per stage: a wave that issues more waits a little longer.
  static constexpr int vm_after_a(int s, int NKS) {
    auto a_exists = [&](int st) { return st < NKS; };
    auto w_exists = [&](int st) { return st < NKS; };
    int n = 0;
    if (s <= SA - 2) {
      for (int st = s + 1; st <= SA - 2; ++st) n += a_exists(st) ? NLA_MIN : 0;
      for (int st = 0; st < NB; ++st) n += w_exists(st) ? NLW : 0;
      for (int t = 0; t < s; ++t) n += (a_exists(t + SA - 1) ? NLA_MIN : 0) + (w_exists(t + NB) ? NLW : 0);
    } else {
      const int t0 = s - SA + 1;  // the stage that issued stage s's activations
      n += w_exists(t0 + NB) ? NLW : 0;
      for (int t = t0 + 1; t < s; ++t) n += (a_exists(t + SA - 1) ? NLA_MIN : 0) + (w_exists(t + NB) ? NLW : 0);
    }
    return n < 63 ? n : 63;  // more than 63 outstanding cannot be expressed: wait a little longer
  }
  // The same for a loading wave of the NL > 0 layout, which issues activation loads only: stage
  // s's have landed once those of stages s+1 .. s+SA-2 alone are outstanding.
  static constexpr int vm_after_a_only(int s, int NKS) {
    int n = 0;
    for (int st = s + 1; st <= s + SA - 2; ++st) n += st < NKS ? NLA_MIN : 0;
    return n < 63 ? n : 63;
  }
};

// s_waitcnt vmcnt(N) as a builtin (expcnt and lgkmcnt left unconstrained), which the compiler's own
// wait insertion understands: after it the compiler knows that at most N loads are outstanding, so
// its waits for the weight registers count the loads still in flight instead of draining them all.
template <int N>
__device__ __forceinline__ void waitcnt_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The main loop over stages [ks0, ks0 + nks) of K (absolute 64-element stages).  acc[i][j] is this
// wave's 32x32 block (row block i of the tile, column block j of the wave's TNW blocks).
template <typename Cfg, int NKS>
__device__ __forceinline__ void rs_mainloop(const bf16* __restrict__ A, const bf16* __restrict__ Wp, int M, int N,
                                            int K, int m0, int n0, int ks0, unsigned char* lds,
                                            f32x16 (&acc)[Cfg::TMW][Cfg::TNW]) {
  constexpr int nks = NKS;
  using MF = Mfma<bf16>;
  constexpr int TMW = Cfg::TMW, TNW = Cfg::TNW, NW = Cfg::NW, SA = Cfg::SA, NB = Cfg::NB, NLA = Cfg::NLA;
  constexpr int BK = 64, EPC = 8;
  constexpr int NL = Cfg::NL, AW = Cfg::AW;
  const int lane = threadIdx.x & 63, hh = lane >> 5, r = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool loader = NL > 0 && wu >= NW;  // a wave that only loads activations
  const int ai = NL > 0 ? wu - NW : wu;     // this wave's index among the activation-loading waves
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j) acc[i][j] = f32x16{};

  // activation loads: load j of loading wave ai fills tile rows (AW*j + ai)*8 .. +7 (when AW*j + ai
  // < ALOADS); lane l lands in row +l/8, 16-byte slot l%8, and fetches the chunk that slot holds
  // under the swizzle (the swizzle of those rows is the same for every j since 4*AW*j is a multiple
  // of 8).  Rows past M re-read row M-1; those outputs are never stored.
  // addresses: a wave-uniform base plus a loop-invariant 32-bit per-lane byte offset
  uint32_t aoff[NLA];
#pragma unroll
  for (int j = 0; j < NLA; ++j) {
    const int row = min(m0 + ai * 8 + (lane >> 3) + 8 * AW * j, M - 1);
    aoff[j] = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)(((lane & 7) ^ lds_swizzle(ai * 8 + (lane >> 3))) * 16);
  }
  auto issue_a = [&](int s) __attribute__((always_inline)) {
    unsigned char* dst = lds + (s % SA) * Cfg::A_STAGE;
    const char* base = reinterpret_cast<const char*>(A + (size_t)(ks0 + s) * BK);
#pragma unroll
    for (int j = 0; j < NLA; ++j)
      if (NLA == Cfg::NLA_MIN || AW * j + ai < Cfg::ALOADS)  // wave-uniform
        load_to_lds16(base + aoff[j], dst + (AW * j + ai) * 8 * 128);
  };
  // weight fragments of this wave's TNW column blocks: one 1 KiB contiguous wave load per
  // (block, k-step); blocks past N re-read the last block (their columns are never stored)
  const int nblk = (N + 31) >> 5;
  const uint32_t woff = (uint32_t)lane * 16u;
  int wblk[TNW];
#pragma unroll
  for (int j = 0; j < TNW; ++j) wblk[j] = min((n0 >> 5) + wu * TNW + j, nblk - 1);
  typedef bf16x8 WFrag[TNW][4];
  auto issue_w = [&](int s, WFrag& buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TNW; ++j) {
      const char* base = reinterpret_cast<const char*>(Wp + ((size_t)(ks0 + s) * nblk + wblk[j]) * 2048);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) buf[j][kk] = *reinterpret_cast<const bf16x8*>(base + kk * 1024 + woff);
    }
  };
  auto afrag = [&](const unsigned char* tile, int row, int kk) __attribute__((always_inline)) -> bf16x8 {
    const int chunk = 2 * kk + hh;
    return *reinterpret_cast<const bf16x8*>(tile + row * 128 + ((chunk ^ lds_swizzle(row)) << 4));
  };
  auto compute = [&](int s, const WFrag& wb) __attribute__((always_inline)) {
    const unsigned char* ta = lds + (s % SA) * Cfg::A_STAGE;
    bf16x8 af[2][TMW];
#pragma unroll
    for (int i = 0; i < TMW; ++i) af[0][i] = afrag(ta, i * 32 + r, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) {
#pragma unroll
        for (int i = 0; i < TMW; ++i) af[(kk + 1) & 1][i] = afrag(ta, i * 32 + r, kk + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TMW; ++i)
#pragma unroll
        for (int j = 0; j < TNW; ++j) acc[i][j] = MF::mma(af[kk & 1][i], wb[j][kk], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The stage loop is unrolled completely (NKS is a compile-time count): a weight buffer loaded in
  // one stage and consumed NB stages later would be a loop-carried pending load, for which the
  // compiler's wait insertion falls back to draining every load at the loop head; in straight-line
  // code its wait before each stage's MFMAs counts exactly the loads issued after that buffer's.
  // Every wave executes the same NKS barriers, whichever role's loop it runs.
  if (loader) {
    static_for<SA - 1>([&](auto sc) {
      if constexpr (decltype(sc)::value < NKS) issue_a(decltype(sc)::value);
    });
    static_for<NKS>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      waitcnt_vm<Cfg::vm_after_a_only(s, NKS)>();  // stage s's activations have landed
      __builtin_amdgcn_s_barrier();
      if constexpr (s + SA - 1 < NKS) issue_a(s + SA - 1);  // into the slot of stage s-1
    });
  } else {
    WFrag wb[NB];
    if constexpr (NL == 0) {
      static_for<SA - 1>([&](auto sc) {
        if constexpr (decltype(sc)::value < NKS) issue_a(decltype(sc)::value);
      });
    }
    static_for<NB>([&](auto bc) {
      if constexpr (decltype(bc)::value < NKS) issue_w(decltype(bc)::value, wb[decltype(bc)::value]);
    });
    static_for<NKS>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      constexpr int b = s % NB;
      // stage s's activations have landed once only the loads issued after them are outstanding
      // (with loading waves, their wait before the barrier covers it)
      if constexpr (NL == 0) waitcnt_vm<Cfg::vm_after_a(s, NKS)>();
      // this wave's LDS reads of stage s-1 are complete before the barrier frees its slot
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
      __builtin_amdgcn_s_barrier();
      if constexpr (NL == 0 && s + SA - 1 < NKS) issue_a(s + SA - 1);  // into the slot of stage s-1
      __builtin_amdgcn_sched_barrier(0);
      compute(s, wb[b]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (s + NB < NKS) issue_w(s + NB, wb[b]);
    });
  }
  // LDS is reused by the caller's epilogue
  __syncthreads();
}

}  // namespace orthrus
