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
//    paged cache with 16-byte loads, prefetched into registers one tile ahead and staged in
//    LDS (K row-major, V transposed for the bf16 MFMA operand);
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

template <bool DRAFT>
__device__ __forceinline__ int num_chunks(int n, int K, int C) {
  return DRAFT ? max(1, ceil_div(n, C)) : ceil_div(n + K, C);
}

template <typename T, typename OutT, int D, int G, bool DRAFT>
__global__ __launch_bounds__(64 * G) void attn_kernel(AttnArgs a) {
  using MF = Mfma<T>;
  constexpr int NT = 64 * G;
  constexpr int KSTEP = MF::KSTEP, KW = MF::KW;
  constexpr int NKK = D / KSTEP;
  constexpr int NDB = D / 32;
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int CPR = D / EPC;                 // 16-byte chunks per key row
  constexpr int NCH = 32 * CPR / NT;           // chunks per thread per tile (each of K and V)
  static_assert(NCH >= 1 && NCH * NT == 32 * CPR, "tile must split evenly over threads");
  constexpr int KLD = D + EPC;                 // padded LDS row (elements)
  constexpr bool VT = std::is_same<T, bf16>::value;
  constexpr int VLD = VT ? 36 : KLD;
  __shared__ __attribute__((aligned(16))) T k_lds[32 * KLD];
  __shared__ __attribute__((aligned(16))) T v_lds[VT ? D * VLD : 32 * KLD];

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
    if constexpr (VT) {
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

  u32x4 kreg[NCH], vreg[NCH];
  auto load_tile = [&](int t) {
    const bool blk = has_blk && (t == ncache_tiles);
    const int base = kbeg + 32 * t;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ci = tid + j * NT;
      const int rk = ci / CPR, part = ci % CPR;
      u32x4 kv = u32x4{0, 0, 0, 0}, vv = u32x4{0, 0, 0, 0};
      if (blk) {
        if (rk < K) {
          const size_t off = ((size_t)(b * K + rk) * a.Hkv + hk) * D + part * EPC;
          kv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.kb) + off);
          vv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.vb) + off);
        }
      } else {
        const int p = base + rk;
        if (p < kend) {
          const int page = ptab[p / a.page];
          const size_t off = (((size_t)page * a.Hkv + hk) * a.page + (p % a.page)) * D + part * EPC;
          kv = *reinterpret_cast<const u32x4*>(kpages + off);
          vv = *reinterpret_cast<const u32x4*>(vpages + off);
        }
      }
      kreg[j] = kv;
      vreg[j] = vv;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ci = tid + j * NT;
      const int rk = ci / CPR, part = ci % CPR;
      *reinterpret_cast<u32x4*>(&k_lds[rk * KLD + part * EPC]) = kreg[j];
      if constexpr (VT) {
        const bf16x8 v8 = __builtin_bit_cast(bf16x8, vreg[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) v_lds[(part * 8 + e) * VLD + rk] = v8[e];
      } else {
        *reinterpret_cast<u32x4*>(&v_lds[rk * KLD + part * EPC]) = vreg[j];
      }
    }
  };

  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);  // prefetch overlaps this tile's math

    const bool blk = has_blk && (t == ncache_tiles);
    const int base = kbeg + 32 * t;
    // S^T tile: rows = keys (lane's A row r), cols = query rows.
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      typename MF::frag af;
      if constexpr (VT) af = *reinterpret_cast<const bf16x8*>(&k_lds[r * KLD + kk * KSTEP + KW * hh]);
      else af = k_lds[r * KLD + kk * KSTEP + hh];
      s = MF::mma(af, qf[kk], s);
    }
    // mask + scale; lane holds query row r, keys acc_row(i, hh)
    float sv[16];
    float mt = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kl = acc_row(i, hh);
      bool ok;
      if (blk) ok = kl < K;
      else {
        const int p = base + kl;
        ok = (p < kend) && (DRAFT || p <= n + r);
      }
      sv[i] = ok ? s[i] * a.scale_log2 : kNegInf;
      mt = fmaxf(mt, sv[i]);
    }
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float p[16];
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = exp2f(sv[i] - m_use);
      lsum += p[i];
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;

    // O^T += V^T P^T.  bf16 operands: P is split into hi + lo bf16 terms (P - hi rounded
    // again), so the product carries ~16 mantissa bits of P instead of 8 and the attention
    // output stays near fp32 accuracy; V is exact in bf16 already.
    if constexpr (VT) {
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
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16* vrow = &v_lds[(db * 32 + r) * VLD + 16 * st + 4 * hh];
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 8);
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[db] = MF::mma(vf, ph, o[db]);
          o[db] = MF::mma(vf, pl, o[db]);
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const int key = acc_row(st, hh);
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = MF::mma(v_lds[key * KLD + db * 32 + r], p[st], o[db]);
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
  ORTHRUS_REQUIRE(d->max_ctx >= d->block && (int64_t)d->max_ctx <= (int64_t)d->max_pages * d->page_size,
                  ORTHRUS_ERR_INVALID_ARG, "attn: max_ctx %d outside [block, max_pages*page_size]", d->max_ctx);
  const int C = chunk_of(d);
  ORTHRUS_REQUIRE(C % 32 == 0 && C > 0, ORTHRUS_ERR_INVALID_ARG, "attn: kv_chunk %d not a positive multiple of 32", C);
  ORTHRUS_REQUIRE(valid_dtype(d->dtype) && valid_dtype(d->out_dtype), ORTHRUS_ERR_INVALID_ARG, "attn: bad dtype");
  ORTHRUS_REQUIRE(!(d->dtype == ORTHRUS_F32 && d->out_dtype == ORTHRUS_BF16), ORTHRUS_ERR_UNSUPPORTED,
                  "attn: fp32 inputs with bf16 output not built");
  ORTHRUS_REQUIRE(std::isfinite(d->scale), ORTHRUS_ERR_INVALID_ARG, "attn: scale not finite");
  return ORTHRUS_OK;
}

template <typename T, typename OutT, int D, int G, bool DRAFT>
int32_t launch_t(const orthrus_attn_desc_t* d, AttnArgs& a, hipStream_t st) {
  dim3 grid(a.nchunk_max, d->kv_heads, d->batch);
  hipLaunchKernelGGL((attn_kernel<T, OutT, D, G, DRAFT>), grid, dim3(64 * G), 0, st, a);
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
