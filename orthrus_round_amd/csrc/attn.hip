// Dual-view block attention for the Orthrus round on gfx950 (draft mask and verify mask).
//
// Orthrus paper summary (cjcn.com.cn), sec. 二: the diffusion view's queries attend to the
// concatenation of the AR cache's keys/values and the parallel block's own keys/values;
// sec. 三: draft queries see the AR context before the block's anchor plus their whole block,
// the AR path keeps the causal mask.
//
// Work decomposition (one workgroup = one (sequence, kv head, key chunk)):
//  * the G query heads that share a kv head are G wavefronts; each wavefront owns one query
//    head's 32 block rows, so one K/V tile staged in LDS serves G*32 query rows (GQA reuse);
//  * keys are streamed in 32-key tiles at absolute positions 32t..32t+31, gathered from the
//    paged cache with direct 16-byte global->LDS loads into a ring of 4 tile stages (3 in
//    flight while one is used); K rows are chunk-swizzled against bank conflicts, V rows are
//    read in place;
//  * S^T = K Q^T and O^T += V^T P^T run on 32x32 MFMA (bf16 x16 or fp32 x2), so a lane owns one
//    query row of S and O and the online-softmax rescale is lane-local; in bf16 the
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
  int32_t Hq, Hkv, K, page, max_pages, max_ctx, chunk, nchunk_max;
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

// Eight gfx950 transposed LDS reads (ds_read_b64_tr_b16: 64 bits per lane, transposed within
// groups of 16 lanes) and the wait for them, in one asm block: the compiler cannot pair the
// builtin with the direct global->LDS tile loads and would drain every load in flight first.
// Outputs are early-clobber: a read may land before a later read has consumed its address.
__device__ __forceinline__ void read_tr16_x8(const uint32_t (&addr)[8], u32x2 (&out)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %9\n"
      "ds_read_b64_tr_b16 %2, %10\n"
      "ds_read_b64_tr_b16 %3, %11\n"
      "ds_read_b64_tr_b16 %4, %12\n"
      "ds_read_b64_tr_b16 %5, %13\n"
      "ds_read_b64_tr_b16 %6, %14\n"
      "ds_read_b64_tr_b16 %7, %15\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]), "=&v"(out[5]), "=&v"(out[6]),
        "=&v"(out[7])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
        "v"(addr[7])
      : "memory");
}

template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <typename T, int D, int G>
struct AttnTile {
  static constexpr int NT = 64 * G;
  static constexpr int CPR = D * (int)sizeof(T) / 16;         // 16-byte chunks per key row
  static constexpr int ROWB = CPR * 16;
  static constexpr int NI_ = 32 * CPR / NT;
  static constexpr int TILE_BYTES = 32 * ROWB;                 // one 32-key tile of K (or V)
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;           // K tile then V tile
#ifndef ORTHRUS_ATTN_STAGES
#define ORTHRUS_ATTN_STAGES 4
#endif
  static constexpr int NI = 32 * CPR / NT;                     // wave loads per thread per tile (K or V)
  // ring depth, capped so the loads allowed in flight fit the 6-bit vmcnt
  static constexpr int S_VM = 2 + 63 / (2 * NI);
  static constexpr int S_LDS = (160 * 1024 - 2048) / (2 * 32 * ROWB);
  static constexpr int STAGES = ORTHRUS_ATTN_STAGES < S_VM ? (ORTHRUS_ATTN_STAGES < S_LDS ? ORTHRUS_ATTN_STAGES : S_LDS)
                                                           : (S_VM < S_LDS ? S_VM : S_LDS);
  static_assert(NI >= 1 && NI * NT == 32 * CPR, "tile must split evenly over the workgroup");
  static constexpr size_t LDS_BYTES = (size_t)STAGES * STAGE_BYTES;
  // K rows are stored with their 16-byte chunks XOR-swizzled so that 32 lanes reading the same
  // chunk of 32 different rows hit distinct LDS banks.
  __device__ __forceinline__ static int swz(int row) { return CPR >= 16 ? (row & 15) : ((row >> 1) & 7); }
};

template <typename T, typename OutT, int D, int G, bool DRAFT>
__global__ __launch_bounds__(64 * G) void attn_kernel(AttnArgs a) {
  using MF = Mfma<T>;
  using TL = AttnTile<T, D, G>;
  constexpr int NT = TL::NT, CPR = TL::CPR, ROWB = TL::ROWB, NI = TL::NI, S = TL::STAGES;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int KSTEP = MF::KSTEP, KW = MF::KW;
  constexpr int NKK = D / KSTEP;
  constexpr int NDB = D / 32;
  constexpr bool BF = std::is_same<T, bf16>::value;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int b = blockIdx.z, hk = blockIdx.y, c = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hh = lane >> 5, r = lane & 31;
  const int K = a.K, C = a.chunk;
  const int n = a.ctx_len[b];
  const int hq = hk * G + w;
  const bool bad = (n < 0) || (n + K > a.max_ctx);
  const int nchunks = bad ? 1 : num_chunks<DRAFT>(n, K, C);
  if (c >= nchunks) return;
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

  const T* kpages = reinterpret_cast<const T*>(a.kp);
  const T* vpages = reinterpret_cast<const T*>(a.vp);
  const int32_t* ptab = a.page_table + (size_t)b * a.max_pages;

  // Tile t -> LDS stage buf with direct 16-byte global->LDS loads.  Wave load j of wave w covers
  // the tile's chunks [(j*G + w)*64, +64): rows row0 .. row0 + 64/CPR - 1, slot idx%CPR.  Rows past
  // the chunk's last key read a clamped valid key: their scores are masked to -inf, so they weigh
  // exactly 0.  The rows of one wave load share a page (page_size % (64/CPR) == 0, checked on the
  // host), so its physical page comes from one scalar page-table read.  Past the last tile the
  // same loads re-read the last tile (an L2 hit) so that every iteration has the same number of
  // loads in flight and the loop body stays branch-free.
  constexpr int RPL = 64 / CPR;  // key rows per wave load
  // the chunk's physical pages, read once into LDS (keeps page lookups off the vector-memory
  // counter that tracks the tile loads in flight)
  __shared__ int page_lds[kMaxChunkPages];
  {
    const int first = kbeg / a.page;
    const int np = kend > kbeg ? (kend - 1) / a.page - first + 1 : 0;
    for (int i = tid; i < np; i += NT) page_lds[i] = ptab[first + i];
    __syncthreads();
  }
  const size_t head_stride = (size_t)a.page * D;                        // elements
  const size_t page_stride = (size_t)a.Hkv * head_stride;
  const T* kblk = reinterpret_cast<const T*>(a.kb) + (size_t)b * K * a.Hkv * D + (size_t)hk * D;
  const T* vblk = reinterpret_cast<const T*>(a.vb) + (size_t)b * K * a.Hkv * D + (size_t)hk * D;
  auto issue = [&](int t, int buf) {
    t = min(t, ntiles - 1);
    const bool blk = has_blk && (t == ncache_tiles);
    const int base = kbeg + 32 * t;
    unsigned char* kdst = lds + buf * TL::STAGE_BYTES;
    unsigned char* vdst = kdst + TL::TILE_BYTES;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int idx = (j * G + w) * 64 + lane;
      const int row = idx / CPR, slot = idx % CPR;
      const int row0 = __builtin_amdgcn_readfirstlane((j * G + w) * RPL);
      const int kchunk = slot ^ TL::swz(row);
      size_t off;
      const T *ks, *vs;
      if (blk) {
        off = (size_t)min(row, K - 1) * a.Hkv * D;
        ks = kblk;
        vs = vblk;
      } else {
        const int p0 = min(base + row0, kend - 1);
        const int page = page_lds[(p0 - kbeg) / a.page];  // wave-uniform
        const int p = min(base + row, kend - 1);
        off = (size_t)page * page_stride + (size_t)hk * head_stride + (size_t)(p % a.page) * D;
        ks = kpages;
        vs = vpages;
      }
      const int lofs = (j * G + w) * 64 * 16;
      load_to_lds16(ks + off + kchunk * EPC, kdst + lofs);
      load_to_lds16(vs + off + kchunk * EPC, vdst + lofs);
    }
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(st, st);
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<(S - 2) * 2 * NI>();
    __builtin_amdgcn_s_barrier();  // tile t landed for every wave; tile t-1 fully consumed
    asm volatile("" ::: "memory");
    issue(t + S - 1, (t + S - 1) % S);
    const unsigned char* kt = lds + (t % S) * TL::STAGE_BYTES;
    const unsigned char* vt = kt + TL::TILE_BYTES;

    const bool blk = has_blk && (t == ncache_tiles);
    const int base = kbeg + 32 * t;
    // S^T tile: rows = keys (lane's A row r), cols = query rows.  Two accumulators over
    // alternating k-steps (summed once) halve the dependent MFMA chain.
    f32x16 s0 = f32x16{}, s1 = f32x16{};
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
      if (kk & 1) s1 = MF::mma(af, qf[kk], s1);
      else s0 = MF::mma(af, qf[kk], s0);
    }
    const f32x16 s = s0 + s1;
    // mask + scale; lane holds query row r, keys acc_row(i, hh).  Tiles that end at or before
    // the context (every key visible to every row) skip the mask.
    float sv[16];
    float mt = kNegInf;
    const bool full = !blk && (base + 32 <= (DRAFT ? kend : min(kend, n + 1)));
    if (full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[i] = s[i] * a.scale_log2;
        mt = fmaxf(mt, sv[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kl = acc_row(i, hh);
        const int p = base + kl;
        const bool ok = blk ? (kl < K) : ((p < kend) && (DRAFT || p <= n + r));
        sv[i] = ok ? s[i] * a.scale_log2 : kNegInf;
        mt = fmaxf(mt, sv[i]);
      }
    }
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float p[16];
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
      lsum += p[i];
    }
    l_run = l_run * alpha + lsum;
    // rescale only when some row's max moved (alpha == 1 exactly otherwise, and x * 1 == x)
    if (__any(m_new != m_run)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    m_run = m_new;

    // O^T += V^T P^T with V stored row = key (chunk-swizzled like K).  bf16 operands: P is split
    // into hi + lo bf16 terms (P - hi rounded again), so the product carries ~16 mantissa bits of
    // P instead of 8 and the attention output stays near fp32 accuracy.  The V^T fragment (lane:
    // column d = 32*db + r, 8 keys) comes from two transposed 64-bit LDS reads: in each 16-lane
    // group, source lane 4e+q points at (key e, columns 4q..4q+3 of the group's 16) and
    // destination lane i receives (key e, column i) for e = 0..3.
    auto vaddr = [&](int key, int d) -> const unsigned char* {
      return vt + key * ROWB + (((d / EPC) ^ TL::swz(key)) << 4) + (d % EPC) * (int)sizeof(T);
    };
    if constexpr (BF) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 ph, pl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pv = p[8 * st + j];
          const bf16 h = (bf16)pv;
          ph[j] = h;
          pl[j] = (bf16)(pv - (float)h);
        }
        (void)pl;
        const int e = (lane >> 2) & 3, q = lane & 3, dgrp = ((lane >> 4) & 1) * 16;
        static_assert(NDB <= 4, "eight transposed reads cover four 32-column blocks");
        uint32_t va[8];
        u32x2 vr[8];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = (db % NDB) * 32 + dgrp + 4 * q;
          va[2 * db] = lds_offset(vaddr(acc_row(8 * st + e, hh), d));
          va[2 * db + 1] = lds_offset(vaddr(acc_row(8 * st + 4 + e, hh), d));
        }
        read_tr16_x8(va, vr);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x4 lo4 = __builtin_bit_cast(bf16x4, vr[2 * db]);
          const bf16x4 hi4 = __builtin_bit_cast(bf16x4, vr[2 * db + 1]);
          const bf16x8 vf = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          o[db] = MF::mma(vf, ph, o[db]);
#ifndef ORTHRUS_ATTN_P_BF16_ONLY
          o[db] = MF::mma(vf, pl, o[db]);
#endif
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const int key = acc_row(st, hh);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          o[db] = MF::mma(*reinterpret_cast<const float*>(vaddr(key, db * 32 + r)), p[st], o[db]);
      }
    }
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
  float M = kNegInf;
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, a.part_ml[(row0 + c * cstride) * 2]);
  constexpr int NV = D / (4 * TPR);
  f32x4 acc[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) acc[j] = f32x4{0, 0, 0, 0};
  float lsum = 0.0f;
  for (int c = 0; c < nchunks; ++c) {
    const size_t row = row0 + c * cstride;
    const float wc = exp2f(a.part_ml[row * 2] - M);
    lsum += wc * a.part_ml[row * 2 + 1];
    const float* pa = a.part_acc + row * D;
#pragma unroll
    for (int j = 0; j < NV; ++j) acc[j] += wc * *reinterpret_cast<const f32x4*>(pa + (j * TPR + part) * 4);
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
  ORTHRUS_REQUIRE(std::isfinite(d->scale), ORTHRUS_ERR_INVALID_ARG, "attn: scale not finite");
  return ORTHRUS_OK;
}

template <typename T, typename OutT, int D, int G, bool DRAFT>
int32_t launch_t(const orthrus_attn_desc_t* d, AttnArgs& a, hipStream_t st) {
  dim3 grid(a.nchunk_max, d->kv_heads, d->batch);
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
  a.max_ctx = d->max_ctx; a.chunk = chunk_of(d); a.scale_log2 = d->scale * kLog2e;
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
