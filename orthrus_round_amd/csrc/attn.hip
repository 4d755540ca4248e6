// Dual-view block attention for the Orthrus round on gfx950 (draft mask and verify mask).
//
// Orthrus paper summary (cjcn.com.cn), sec. 二: the diffusion view's queries attend to the
// concatenation of the AR cache's keys/values and the parallel block's own keys/values;
// sec. 三: draft queries see the AR context before the block's anchor plus their whole block,
// the AR path keeps the causal mask.
//
// Work decomposition (one workgroup = one (sequence, kv head, key chunk); the existing items take
// the first slots of a grid sized for the longest context):
//  * the G query heads that share a kv head are G wavefronts; each wavefront owns one query
//    head's 32 block rows, so one K/V tile staged in LDS serves G*32 query rows (GQA reuse);
//  * keys are streamed in 32-key tiles at absolute positions 32t..32t+31, gathered from the
//    paged cache with direct 16-byte global->LDS loads into a ring of S tile stages (S-1 tiles
//    in flight while one is used); K and V rows are chunk-swizzled against bank conflicts, and
//    the loop is unrolled by S so every LDS address is a register plus an immediate;
//  * S^T = K Q^T and O^T += V^T P^T run on 32x32 MFMA (bf16 x16 or fp32 x2), so a lane owns one
//    query row of S and O and the online-softmax bookkeeping is lane-local; the reference
//    maximum is raised lazily (only when a tile exceeds it by 2^8), per row; in bf16 the
//    probabilities enter the PV product as a hi + lo pair of bf16 terms;
//  * fixed chunks of kv_chunk keys: a sequence with one chunk writes its output directly,
//    longer ones write (m, l, acc) partials that a combine kernel merges in chunk order.
// Every key tile, chunk and merge order is a function of absolute key positions only, so a
// query row's result is the same bits whatever the block size, batch or page order.
#include <type_traits>

#include "common.hpp"

namespace orthrus {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const void* q;
  const void* kp;
  const void* vp;
  const int32_t* page_table;
  const int32_t* ctx_len;
  const void* kb;
  const void* vb;
  void* out;
  float* part_acc;
  float* part_ml;
  int32_t Hq, Hkv, K, page, page_shift, max_pages, max_ctx, chunk, nchunk_max, batch;
  float scale_log2;
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr int kMaxChunkPages = 256;  // kv_chunk / page_size + 1 must not exceed this

template <bool DRAFT>
__device__ __forceinline__ int num_chunks(int n, int K, int C) {
  return DRAFT ? max(1, ceil_div(n, C)) : ceil_div(n + K, C);
}

__device__ __forceinline__ void load_to_lds16(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

__device__ __forceinline__ uint32_t lds_offset(const unsigned char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Eight gfx950 transposed LDS reads (ds_read_b64_tr_b16: 64 bits per lane, transposed within
// groups of 16 lanes) and the wait for them, in one asm block: the compiler cannot pair the
// builtin with the direct global->LDS tile loads and would drain every load in flight first.
// Outputs are early-clobber: a read may land before a later read has consumed its address.
// OFF is a compile-time byte offset added to every address (the instruction's immediate).
template <int OFF>
__device__ __forceinline__ void read_tr16_x8_at(const uint32_t (&addr)[8], u32x2 (&out)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%16\n"
      "ds_read_b64_tr_b16 %1, %9 offset:%16\n"
      "ds_read_b64_tr_b16 %2, %10 offset:%16\n"
      "ds_read_b64_tr_b16 %3, %11 offset:%16\n"
      "ds_read_b64_tr_b16 %4, %12 offset:%16\n"
      "ds_read_b64_tr_b16 %5, %13 offset:%16\n"
      "ds_read_b64_tr_b16 %6, %14 offset:%16\n"
      "ds_read_b64_tr_b16 %7, %15 offset:%16\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]), "=&v"(out[5]), "=&v"(out[6]),
        "=&v"(out[7])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
        "v"(addr[7]), "n"(OFF)
      : "memory");
}

#ifndef ORTHRUS_ATTN_STAGES
#define ORTHRUS_ATTN_STAGES 3
#endif

template <typename T, int D, int G>
struct AttnTile {
  static constexpr int NT = 64 * G;
  static constexpr int CPR = D * (int)sizeof(T) / 16;         // 16-byte chunks per key row
  static constexpr int ROWB = CPR * 16;
  static constexpr int RPL = 64 / CPR;                         // key rows per wave load
  static constexpr int TILE_BYTES = 32 * ROWB;                 // one 32-key tile of K (or V)
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;           // K tile then V tile
  static constexpr int NI = 32 * CPR / NT;                     // wave loads per thread per tile (K or V)
  // ring depth: loads allowed in flight must fit the 6-bit vmcnt, stage offsets the 16-bit
  // LDS immediate, and the ring the 160 KiB of LDS
  static constexpr int S_VM = 2 + 63 / (2 * NI);
  static constexpr int S_IMM = sizeof(T) == 2 ? (65535 - TILE_BYTES - 16 * ROWB) / STAGE_BYTES + 1 : 64;
  static constexpr int S_LDS = (160 * 1024 - 2048) / STAGE_BYTES;
  static constexpr int S_CAP = S_VM < S_IMM ? (S_VM < S_LDS ? S_VM : S_LDS) : (S_IMM < S_LDS ? S_IMM : S_LDS);
  static constexpr int STAGES = ORTHRUS_ATTN_STAGES < S_CAP ? ORTHRUS_ATTN_STAGES : S_CAP;
  static_assert(STAGES >= 2, "ring needs two stages");
  static_assert(NI >= 1 && NI * NT == 32 * CPR, "tile must split evenly over the workgroup");
  static constexpr size_t LDS_BYTES = (size_t)STAGES * STAGE_BYTES;
  // K and V rows are stored with their 16-byte chunks XOR-swizzled against LDS bank conflicts.
  // Two read patterns must be conflict-free: the K fragment reads (16 consecutive rows, the
  // same chunk) and the transposed V reads (4 consecutive keys 4e..4e+3 times chunks 4c..4c+3).
  // For 16-chunk rows the XOR mask is linear in the row's low four bits, bits 0..3 mapping to
  // masks 4, 10, 1, 2: a bijection on 16 rows (first pattern), and keys differing in bits 0-1
  // land in different groups of four chunks (second pattern).
  __host__ __device__ static constexpr int swz(int row) {
    return CPR >= 16 ? (((row & 1) << 2) ^ (((row >> 1) & 1) * 10) ^ ((row >> 2) & 3)) : ((row >> 1) & 7);
  }
};

// Softmax bookkeeping is in log2 units.  A row's reference maximum m is only raised when a tile
// brings a score more than kLazy above it; otherwise exp2(s - m) <= 2^kLazy and the running sums
// keep their old reference, which is exact because numerator and denominator share it.  The
// decision is per row, so a row's bits never depend on the other rows of the wavefront.
constexpr float kLazy = 8.0f;

template <typename T, typename OutT, int D, int G, bool DRAFT>
__global__ __launch_bounds__(64 * G) void attn_kernel(AttnArgs a) {
  using MF = Mfma<T>;
  using TL = AttnTile<T, D, G>;
  constexpr int NT = TL::NT, CPR = TL::CPR, ROWB = TL::ROWB, NI = TL::NI, S = TL::STAGES, RPL = TL::RPL;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int KSTEP = MF::KSTEP, KW = MF::KW;
  constexpr int NKK = D / KSTEP;
  constexpr int NDB = D / 32;
  constexpr bool BF = std::is_same<T, bf16>::value;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ int page_lds[kMaxChunkPages];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hh = lane >> 5, r = lane & 31;
  const int K = a.K, C = a.chunk;
  // The grid has nchunk_max x Hkv x batch slots, sized for the longest possible context.  The
  // (sequence, kv head, chunk) items that exist take the first slots, in the order chunk fastest,
  // then kv head, then sequence, and the remaining slots exit at once: a wave reads 64 sequences'
  // lengths at a time, scans their item counts and finds the sequence that holds this slot.  Only
  // the placement changes; each item is computed exactly as before.
  const int id = blockIdx.x;
  int seq = -1, first = 0, nch = 1;  // the slot's sequence, its first slot, its chunk count
  for (int b0 = 0, base = 0; b0 < a.batch; b0 += 64) {
    const int bi = b0 + lane;
    int items = 0, nc = 1;
    if (bi < a.batch) {
      const int nl = a.ctx_len[bi];
      nc = ((nl < 0) || (nl + K > a.max_ctx)) ? 1 : num_chunks<DRAFT>(nl, K, C);
      items = nc * a.Hkv;
    }
    int incl = items;  // inclusive scan over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    const int total = __shfl(incl, 63, 64);
    if (id < base + total) {
      const int L = __builtin_ctzll(__ballot(id < base + incl));
      seq = b0 + L;
      first = base + __shfl(incl, L, 64) - __shfl(items, L, 64);
      nch = __shfl(nc, L, 64);
      break;
    }
    base += total;
  }
  if (seq < 0) return;
  const int b = __builtin_amdgcn_readfirstlane(seq);
  const int nchunks = __builtin_amdgcn_readfirstlane(nch);
  const int item = id - __builtin_amdgcn_readfirstlane(first);
  const int hk = item / nchunks, c = item - hk * nchunks;
  const int n = a.ctx_len[b];
  const int hq = hk * G + w;
  const bool bad = (n < 0) || (n + K > a.max_ctx);
  OutT* out = reinterpret_cast<OutT*>(a.out);
  if (bad) {
    if (r < K) {
      for (int d = hh; d < D; d += 2)
        out[((size_t)(b * K + r) * a.Hq + hq) * D + d] = from_f32<OutT>(__builtin_nanf(""));
    }
    return;
  }

  // ---- this chunk's key tiles ----
  const int limit = DRAFT ? n : n + K;        // cache keys visible to some row
  const int kbeg = c * C;
  const int kend = min(limit, kbeg + C);
  const int ncache_tiles = kend > kbeg ? ceil_div(kend - kbeg, 32) : 0;
  const bool has_blk = DRAFT && (c == nchunks - 1);
  const int ntiles = ncache_tiles + (has_blk ? 1 : 0);

  // ---- query fragments (B operand of S^T = K Q^T): row r, k = kk*KSTEP + KW*hh + j ----
  const T* qbase = reinterpret_cast<const T*>(a.q) + ((size_t)(b * K + r) * a.Hq + hq) * D;
  typename MF::frag qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    if constexpr (BF) {
      if (r < K) qf[kk] = *reinterpret_cast<const bf16x8*>(qbase + kk * KSTEP + KW * hh);
      else qf[kk] = bf16x8{};
    } else {
      qf[kk] = (r < K) ? qbase[kk * KSTEP + hh] : 0.0f;
    }
  }

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;
  const float csc = a.scale_log2;

  // the chunk's physical pages, read once into LDS (keeps page lookups off the vector-memory
  // counter that tracks the tile loads in flight)
  {
    const int first = kbeg >> a.page_shift;
    const int np = kend > kbeg ? ((kend - 1) >> a.page_shift) - first + 1 : 0;
    for (int i = tid; i < np; i += NT) page_lds[i] = a.page_table[(size_t)b * a.max_pages + first + i];
    __syncthreads();
  }

  // Tile loads.  Wave load j of wave w fills LDS bytes [(j*G + w)*1024, +1024) of the tile: key
  // rows row0 = (j*G + w)*RPL .. row0 + RPL - 1, lane -> (row0 + lane / CPR, 16-byte slot
  // lane % CPR), whose global chunk is slot ^ swz(row).  The RPL rows of one wave load share a
  // page (page_size % RPL == 0, checked on the host), so its page id is one wave-uniform LDS read.
  // Rows past the chunk's last key (only in its last tile) re-read that key: their scores are
  // masked to -inf and weigh exactly 0.  Past the last tile the same loads re-read the last tile
  // (an L2 hit), so every iteration keeps the same number of loads in flight.
  const size_t head_stride_b = (size_t)a.page * D * sizeof(T);
  const size_t page_stride_b = (size_t)a.Hkv * head_stride_b;
  const unsigned char* kpb = reinterpret_cast<const unsigned char*>(a.kp) + (size_t)hk * head_stride_b;
  const unsigned char* vpb = reinterpret_cast<const unsigned char*>(a.vp) + (size_t)hk * head_stride_b;
  const size_t blk_row_b = (size_t)a.Hkv * D * sizeof(T);
  const unsigned char* kbb = reinterpret_cast<const unsigned char*>(a.kb) + (size_t)b * K * blk_row_b +
                             (size_t)hk * D * sizeof(T);
  const unsigned char* vbb = reinterpret_cast<const unsigned char*>(a.vb) + (size_t)b * K * blk_row_b +
                             (size_t)hk * D * sizeof(T);
  const int lr = lane / CPR, slot = lane % CPR;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int pmask = a.page - 1;
  const int pfirst = kbeg >> a.page_shift;  // logical page of page_lds[0]
  // byte offset of the lane's chunk inside its key row for wave load j
  auto lane_b = [&](int j) { return (uint32_t)((slot ^ TL::swz((j * G + wu) * RPL + lr)) << 4); };

  // Physical pages of tile t's wave loads, read from LDS one iteration before their loads are
  // issued, so that the LDS round trip is hidden behind a tile's compute instead of stalling the
  // issue (it cost 280-520 cycles per tile when read at issue time).  Block tiles need none.
  auto pages_of = [&](int t, int (&pg)[NI]) {
    t = min(t, ntiles - 1);
    const int base = kbeg + 32 * t;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int p0 = min(base + (j * G + wu) * RPL, kend - 1);
      pg[j] = t < ncache_tiles ? page_lds[(p0 >> a.page_shift) - pfirst] : 0;
    }
  };

  auto issue = [&](int t, unsigned char* kdst, const int (&pg)[NI]) {
    t = min(t, ntiles - 1);
    const int base = kbeg + 32 * t;
    const bool blk = has_blk && t == ncache_tiles;  // wave-uniform
    const bool tail = base + 32 > kend;             // wave-uniform
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int row0 = (j * G + wu) * RPL;  // wave-uniform
      const unsigned char *ksrc, *vsrc;     // wave-uniform bases
      uint32_t voff;                        // per-lane byte offset
      if (blk) {
        ksrc = kbb;
        vsrc = vbb;
        voff = (uint32_t)min(row0 + lr, K - 1) * (uint32_t)blk_row_b;
      } else {
        const int page = __builtin_amdgcn_readfirstlane(pg[j]);
        const size_t pofs = (size_t)page * page_stride_b;
        ksrc = kpb + pofs;
        vsrc = vpb + pofs;
        const int p = tail ? min(base + row0 + lr, kend - 1) : base + row0 + lr;  // same page as row0's
        voff = (uint32_t)(p & pmask) * ROWB;
      }
      voff += lane_b(j);
      const int lofs = (j * G + wu) * 1024;
      load_to_lds16(ksrc + voff, kdst + lofs);
      load_to_lds16(vsrc + voff, kdst + TL::TILE_BYTES + lofs);
    }
  };

  // Per-lane LDS byte offsets of the operand reads, relative to a tile.
  //  K (A operand of S^T): key row r, 16-byte chunk (kk*KSTEP + KW*hh) / EPC, swizzled.
  //  V^T (A operand of O^T, bf16): two transposed 64-bit reads per 32-column block db; in each
  //  16-lane group, source lane 4e+q points at (key e, columns 4q..4q+3 of the group's 16), and
  //  destination lane i receives (key e, column i) for e = 0..3.  Keys of half `hf` of step st
  //  are 16*st + 8*hf + 4*hh + e (the accumulator rows of P's lane-half hh); the swizzle of those
  //  rows does not depend on st, so step 1 is step 0 plus 16 rows.
  const uint32_t lds0 = lds_offset(lds);
  uint32_t vofs[8];
  if constexpr (BF) {
    const int e = (lane >> 2) & 3, q = lane & 3, dgrp = ((lane >> 4) & 1) * 16;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int key = 8 * hf + 4 * hh + e;
        const int d = (db % NDB) * 32 + dgrp + 4 * q;
        vofs[2 * db + hf] = lds0 + key * ROWB + (((d / EPC) ^ TL::swz(key)) << 4) + (d % EPC) * 2;
      }
  }

  auto compute = [&](int t, auto stage_c) {
    constexpr int ST = decltype(stage_c)::value;
    constexpr int KOFF = ST * TL::STAGE_BYTES;
    const unsigned char* kt = lds + KOFF;
    const unsigned char* vt = kt + TL::TILE_BYTES;
    const bool blk = has_blk && (t == ncache_tiles);
    const int base = kbeg + 32 * t;

    // S^T tile: rows = keys (lane's A row r), cols = query rows.
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      typename MF::frag af;
      if constexpr (BF) {
        const int chunk = (kk * KSTEP + KW * hh) / EPC;
        af = *reinterpret_cast<const bf16x8*>(kt + r * ROWB + ((chunk ^ TL::swz(r)) << 4));
      } else {
        const int e = kk * KSTEP + hh;
        af = *reinterpret_cast<const float*>(kt + r * ROWB + (((e / EPC) ^ TL::swz(r)) << 4) + (e % EPC) * 4);
      }
      sacc = MF::mma(af, qf[kk], sacc);
    }
    // Mask; lane holds query row r and keys acc_row(i, hh).  Tiles that end at or before the
    // context seen by every row skip the mask.
    float sv[16];
    float mt = kNegInf;
    const bool full = !blk && (base + 32 <= (DRAFT ? kend : min(kend, n + 1)));
    if (full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[i] = sacc[i];
        mt = fmaxf(mt, sv[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kl = acc_row(i, hh);
        const int p = base + kl;
        const bool ok = blk ? (kl < K) : ((p < kend) && (DRAFT || p <= n + r));
        sv[i] = ok ? sacc[i] : kNegInf;
        mt = fmaxf(mt, sv[i]);
      }
    }
    {
      // the row's tile maximum over both lane halves (a lane swap, not an LDS shuffle), in log2
      // units (scale > 0)
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * csc;
    }
    const bool raise = mt > m_run + kLazy;
    if (__any(raise)) {
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      m_run = raise ? mt : m_run;
    }
    const float m_use = (m_run == kNegInf) ? 0.0f : m_run;
    float p[16];
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], csc, -m_use));
      lsum += p[i];
    }
    l_run += lsum;

    // O^T += V^T P^T.  bf16: P enters as hi + lo bf16 terms (hi = P truncated to bf16, lo = the
    // exact remainder rounded to bf16), ~16 mantissa bits of P instead of 8.
    if constexpr (BF) {
      static_assert(NDB <= 4, "eight transposed reads cover four 32-column blocks");
      static_for<2>([&](auto stc) {
        constexpr int st = decltype(stc)::value;
        u32x4 hi4;
        bf16x8 pl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = p[8 * st + 2 * j], p1 = p[8 * st + 2 * j + 1];
          const uint32_t u0 = __float_as_uint(p0) & 0xffff0000u, u1 = __float_as_uint(p1) & 0xffff0000u;
          hi4[j] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
          pl[2 * j] = (bf16)(p0 - __uint_as_float(u0));
          pl[2 * j + 1] = (bf16)(p1 - __uint_as_float(u1));
        }
        const bf16x8 ph = __builtin_bit_cast(bf16x8, hi4);
        u32x2 vr[8];
        read_tr16_x8_at<KOFF + TL::TILE_BYTES + st * 16 * ROWB>(vofs, vr);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x4 lo4 = __builtin_bit_cast(bf16x4, vr[2 * db]);
          const bf16x4 hi4v = __builtin_bit_cast(bf16x4, vr[2 * db + 1]);
          const bf16x8 vf = {lo4[0], lo4[1], lo4[2], lo4[3], hi4v[0], hi4v[1], hi4v[2], hi4v[3]};
          o[db] = MF::mma(vf, ph, o[db]);
          o[db] = MF::mma(vf, pl, o[db]);
        }
      });
    } else {
      auto vaddr = [&](int key, int d) -> const unsigned char* {
        return vt + key * ROWB + (((d / EPC) ^ TL::swz(key)) << 4) + (d % EPC) * (int)sizeof(T);
      };
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const int key = acc_row(st, hh);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          o[db] = MF::mma(*reinterpret_cast<const float*>(vaddr(key, db * 32 + r)), p[st], o[db]);
      }
    }
  };

  // Ring of S stages, loop unrolled by S so that every LDS address is a per-lane register plus an
  // immediate.  Iteration t: tile t has landed once at most S-2 tiles' loads are outstanding; the
  // barrier also tells every wave that tile t-1 (whose stage the next issue overwrites) is done.
  int pg[NI];
#pragma unroll
  for (int st = 0; st < S - 1; ++st) {
    pages_of(st, pg);
    issue(st, lds + st * TL::STAGE_BYTES, pg);
  }
  pages_of(S - 1, pg);
  for (int t0 = 0; t0 < ntiles; t0 += S) {
    static_for<S>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      const int t = t0 + s;
      if (t < ntiles) {
        wait_vmcnt<(S - 2) * 2 * NI>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(t + S - 1, lds + ((s + S - 1) % S) * TL::STAGE_BYTES, pg);
        pages_of(t + S, pg);
        compute(t, sc);
      }
    });
  }

  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  if (nchunks == 1) {
    if (r < K) {
      OutT* orow = out + ((size_t)(b * K + r) * a.Hq + hq) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) orow[db * 32 + acc_row(i, hh)] = from_f32<OutT>(o[db][i] / l_tot);
    }
  } else {
    const size_t prow = (((size_t)(b * a.Hkv + hk) * a.nchunk_max + c) * G + w) * 32 + r;
    float* pa = a.part_acc + prow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        f32x4 v4 = {o[db][i], o[db][i + 1], o[db][i + 2], o[db][i + 3]};
        *reinterpret_cast<f32x4*>(pa + db * 32 + acc_row(i, hh)) = v4;
      }
    if (hh == 0) {
      a.part_ml[prow * 2] = m_run;
      a.part_ml[prow * 2 + 1] = l_tot;
    }
  }
}

// Merge per-chunk partials in chunk order: out = sum_c w_c acc_c / sum_c w_c l_c with
// w_c = 2^(m_c - max_c m_c).  One workgroup per (sequence, kv head, query head of the group).
template <typename OutT, int D, int G, bool DRAFT>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int b = blockIdx.z, hk = blockIdx.y, w = blockIdx.x;
  const int n = a.ctx_len[b];
  const int K = a.K;
  if (n < 0 || n + K > a.max_ctx) return;
  const int nchunks = num_chunks<DRAFT>(n, K, a.chunk);
  if (nchunks <= 1) return;
  constexpr int TPR = 8;  // threads per row
  const int r = threadIdx.x / TPR, part = threadIdx.x % TPR;
  if (r >= K) return;
  const size_t row0 = ((size_t)(b * a.Hkv + hk) * a.nchunk_max * G + w) * 32 + r;
  const size_t cstride = (size_t)G * 32;
  // several chunks' loads are kept in flight at once; the additions still run in chunk order
  float M = kNegInf;
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, a.part_ml[(row0 + c * cstride) * 2]);
  constexpr int NV = D / (4 * TPR);
  f32x4 acc[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) acc[j] = f32x4{0, 0, 0, 0};
  float lsum = 0.0f;
  auto add = [&](float m, float l, const f32x4 (&x)[NV]) {
    const float wc = exp2f(m - M);
    lsum += wc * l;
#pragma unroll
    for (int j = 0; j < NV; ++j) acc[j] += wc * x[j];
  };
  // four chunks' partials are loaded into separate registers before they are added in order
  constexpr int U = 4;
  int c = 0;
  for (; c + U <= nchunks; c += U) {
    float m[U], l[U];
    f32x4 x[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t row = row0 + (c + u) * cstride;
      m[u] = a.part_ml[row * 2];
      l[u] = a.part_ml[row * 2 + 1];
      const float* pa = a.part_acc + row * D;
#pragma unroll
      for (int j = 0; j < NV; ++j) x[u][j] = *reinterpret_cast<const f32x4*>(pa + (j * TPR + part) * 4);
    }
    // keep the scheduler from sinking each load next to its use, which would serialise them again
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) add(m[u], l[u], x[u]);
  }
  for (; c < nchunks; ++c) {
    const size_t row = row0 + c * cstride;
    const float* pa = a.part_acc + row * D;
    f32x4 x[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) x[j] = *reinterpret_cast<const f32x4*>(pa + (j * TPR + part) * 4);
    add(a.part_ml[row * 2], a.part_ml[row * 2 + 1], x);
  }
  OutT* orow = reinterpret_cast<OutT*>(a.out) + ((size_t)(b * K + r) * a.Hq + hk * G + w) * D;
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[(j * TPR + part) * 4 + e] = from_f32<OutT>(acc[j][e] / lsum);
}

int chunk_of(const orthrus_attn_desc_t* d) { return d->kv_chunk > 0 ? d->kv_chunk : 1024; }
int nchunk_max_of(const orthrus_attn_desc_t* d) {
  const int C = chunk_of(d);
  return std::max(1, (d->max_ctx + C - 1) / C);
}

int32_t validate(const orthrus_attn_desc_t* d) {
  ORTHRUS_REQUIRE(d != nullptr, ORTHRUS_ERR_INVALID_ARG, "attn: null descriptor");
  ORTHRUS_REQUIRE(d->batch >= 0 && d->q_heads > 0 && d->kv_heads > 0 && d->q_heads % d->kv_heads == 0,
                  ORTHRUS_ERR_INVALID_ARG, "attn: bad head counts (%d, %d)", d->q_heads, d->kv_heads);
  const int G = d->q_heads / d->kv_heads;
  ORTHRUS_REQUIRE(G == 2 || G == 4, ORTHRUS_ERR_UNSUPPORTED, "attn: group size %d not built (2, 4)", G);
  ORTHRUS_REQUIRE(d->head_dim == 64 || d->head_dim == 128, ORTHRUS_ERR_UNSUPPORTED, "attn: head_dim %d", d->head_dim);
  ORTHRUS_REQUIRE(d->block >= 1 && d->block <= 32, ORTHRUS_ERR_INVALID_ARG, "attn: block %d not in 1..32", d->block);
  ORTHRUS_REQUIRE(d->page_size >= 1 && d->max_pages >= 1, ORTHRUS_ERR_INVALID_ARG, "attn: bad paging");
  ORTHRUS_REQUIRE((d->page_size & (d->page_size - 1)) == 0, ORTHRUS_ERR_UNSUPPORTED,
                  "attn: page_size %d is not a power of two", d->page_size);
  {
    const int cpr = d->head_dim * (d->dtype == ORTHRUS_BF16 ? 2 : 4) / 16;  // 16-byte chunks per key row
    const int rows_per_load = 64 / cpr;
    ORTHRUS_REQUIRE(d->page_size % rows_per_load == 0, ORTHRUS_ERR_UNSUPPORTED,
                    "attn: page_size %d must be a multiple of %d for this head_dim/dtype", d->page_size,
                    rows_per_load);
  }
  ORTHRUS_REQUIRE(d->max_ctx >= d->block && (int64_t)d->max_ctx <= (int64_t)d->max_pages * d->page_size,
                  ORTHRUS_ERR_INVALID_ARG, "attn: max_ctx %d outside [block, max_pages*page_size]", d->max_ctx);
  const int C = chunk_of(d);
  ORTHRUS_REQUIRE(C % 32 == 0 && C > 0, ORTHRUS_ERR_INVALID_ARG, "attn: kv_chunk %d not a positive multiple of 32", C);
  ORTHRUS_REQUIRE(C / d->page_size + 1 <= kMaxChunkPages, ORTHRUS_ERR_UNSUPPORTED,
                  "attn: kv_chunk %d spans more than %d pages of %d keys", C, kMaxChunkPages - 1, d->page_size);
  ORTHRUS_REQUIRE(valid_dtype(d->dtype) && valid_dtype(d->out_dtype), ORTHRUS_ERR_INVALID_ARG, "attn: bad dtype");
  ORTHRUS_REQUIRE(!(d->dtype == ORTHRUS_F32 && d->out_dtype == ORTHRUS_BF16), ORTHRUS_ERR_UNSUPPORTED,
                  "attn: fp32 inputs with bf16 output not built");
  ORTHRUS_REQUIRE(std::isfinite(d->scale) && d->scale > 0.0f, ORTHRUS_ERR_INVALID_ARG,
                  "attn: scale must be finite and positive");
  return ORTHRUS_OK;
}

template <typename T, typename OutT, int D, int G, bool DRAFT>
int32_t launch_t(const orthrus_attn_desc_t* d, AttnArgs& a, hipStream_t st) {
  dim3 grid(a.nchunk_max * d->kv_heads * d->batch);  // slots past the existing items exit at once
  const size_t lds = AttnTile<T, D, G>::LDS_BYTES;
  allow_lds(attn_kernel<T, OutT, D, G, DRAFT>, lds);
  hipLaunchKernelGGL((attn_kernel<T, OutT, D, G, DRAFT>), grid, dim3(64 * G), lds, st, a);
  if (a.nchunk_max > 1) {
    dim3 g2(G, d->kv_heads, d->batch);
    hipLaunchKernelGGL((attn_combine_kernel<OutT, D, G, DRAFT>), g2, dim3(256), 0, st, a);
  }
  return check_launch(DRAFT ? "orthrus_draft_attn" : "orthrus_verify_attn");
}

template <bool DRAFT, int D, int G>
int32_t dispatch_dtype(const orthrus_attn_desc_t* d, AttnArgs& a, hipStream_t st) {
  if (d->dtype == ORTHRUS_BF16) {
    if (d->out_dtype == ORTHRUS_BF16) return launch_t<bf16, bf16, D, G, DRAFT>(d, a, st);
    return launch_t<bf16, float, D, G, DRAFT>(d, a, st);
  }
  return launch_t<float, float, D, G, DRAFT>(d, a, st);
}

template <bool DRAFT>
int32_t run(const orthrus_attn_desc_t* d, const void* q, const void* kp, const void* vp, const int32_t* pt,
            const int32_t* ctx, const void* kb, const void* vb, void* out, void* ws, size_t ws_bytes,
            void* stream) {
  if (int32_t s = validate(d)) return s;
  if (d->batch == 0) return ORTHRUS_OK;
  ORTHRUS_REQUIRE(q && kp && vp && pt && ctx && out, ORTHRUS_ERR_INVALID_ARG, "attn: null tensor pointer");
  ORTHRUS_REQUIRE(!DRAFT || (kb && vb), ORTHRUS_ERR_INVALID_ARG, "draft_attn: null block key/value pointer");
  const size_t need = orthrus_attn_workspace_bytes(d);
  ORTHRUS_REQUIRE(ws_bytes >= need && (need == 0 || ws), ORTHRUS_ERR_WORKSPACE,
                  "attn: workspace %zu bytes < required %zu", ws_bytes, need);
  AttnArgs a;
  a.q = q; a.kp = kp; a.vp = vp; a.page_table = pt; a.ctx_len = ctx; a.kb = kb; a.vb = vb; a.out = out;
  const int G = d->q_heads / d->kv_heads;
  a.nchunk_max = nchunk_max_of(d);
  const size_t acc_elems = (size_t)d->batch * d->kv_heads * a.nchunk_max * G * 32 * d->head_dim;
  a.part_acc = reinterpret_cast<float*>(ws);
  a.part_ml = a.nchunk_max > 1 ? a.part_acc + acc_elems : nullptr;
  a.Hq = d->q_heads; a.Hkv = d->kv_heads; a.K = d->block; a.page = d->page_size; a.max_pages = d->max_pages;
  a.page_shift = __builtin_ctz((unsigned)d->page_size);
  a.max_ctx = d->max_ctx; a.chunk = chunk_of(d); a.batch = d->batch; a.scale_log2 = d->scale * kLog2e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (d->head_dim == 128) {
    if (G == 4) return dispatch_dtype<DRAFT, 128, 4>(d, a, st);
    return dispatch_dtype<DRAFT, 128, 2>(d, a, st);
  }
  if (G == 4) return dispatch_dtype<DRAFT, 64, 4>(d, a, st);
  return dispatch_dtype<DRAFT, 64, 2>(d, a, st);
}

}  // namespace
}  // namespace orthrus

using namespace orthrus;

extern "C" size_t orthrus_attn_workspace_bytes(const orthrus_attn_desc_t* d) {
  if (!d || validate(d) != ORTHRUS_OK) return 0;
  const int ncm = nchunk_max_of(d);
  if (ncm <= 1) return 0;
  const size_t rows = (size_t)d->batch * d->kv_heads * ncm * (d->q_heads / d->kv_heads) * 32;
  return rows * (d->head_dim + 2) * sizeof(float);
}

extern "C" int32_t orthrus_draft_attn(const orthrus_attn_desc_t* d, const void* q, const void* kp, const void* vp,
                                      const int32_t* pt, const int32_t* ctx, const void* kb, const void* vb,
                                      void* out, void* ws, size_t ws_bytes, void* stream) {
  return run<true>(d, q, kp, vp, pt, ctx, kb, vb, out, ws, ws_bytes, stream);
}

extern "C" int32_t orthrus_verify_attn(const orthrus_attn_desc_t* d, const void* q, const void* kp, const void* vp,
                                       const int32_t* pt, const int32_t* ctx, void* out, void* ws, size_t ws_bytes,
                                       void* stream) {
  return run<false>(d, q, kp, vp, pt, ctx, nullptr, nullptr, out, ws, ws_bytes, stream);
}
