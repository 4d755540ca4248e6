// Layer GEMMs of both views: C = epilogue(A W^T) on MFMA with fused residual add or SwiGLU.
//
// Narrow outputs (N < 16384: the q/k/v, O and down projections) split K into S contiguous slices
// (S = 4, or 8 for the deep down projection), one workgroup per (tile, slice): each runs the plain
// MFMA chain over its slice and writes an fp32 partial tile, and a second kernel adds the S
// partials in slice order and applies the epilogue.  Splitting K across workgroups keeps 256+ workgroups busy with 128x128
// tiles, which stream half the operand bytes of 64x64 tiles through L2.  Wide outputs (gate/up)
// use plain tiles over the whole K.  Either way an output element's summation order depends on
// (N, K) only, so results are deterministic and a row's bits do not depend on the batch size.
#include "gemm_rs.hpp"
#include "gemm_core.hpp"

namespace orthrus {
namespace {

template <typename T, typename OutT, typename Cfg, int EPI>
__global__ __launch_bounds__(Cfg::NT) ORTHRUS_GEMM_WAVES void gemm_kernel(const T* __restrict__ A, const T* __restrict__ W,
                                                   const OutT* residual, OutT* C, int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int mtiles = (M + Cfg::BM - 1) / Cfg::BM;
  int sp, mt, nt;
  xcd_tile_map(blockIdx.x, gridDim.x, 1, mtiles, sp, mt, nt);
  const int m0 = mt * Cfg::BM, n0 = nt * Cfg::BN;
  f32x16 acc[Cfg::TM][Cfg::TN];
  const int lane = threadIdx.x & 63, hh = lane >> 5, r = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  gemm_mainloop<T, Cfg>(A, W, M, N, K, m0, n0, smem, acc);
  constexpr int NBI = Cfg::BM / 32, NBJ = Cfg::BN / 32;
  if constexpr (!Cfg::KSPLIT) park_plain<Cfg>(smem, acc);
  // the tile's 32x32 blocks are now in LDS (k-split: four partials each); wave q % NW stores block q
  auto block = [&](int i, int j) -> f32x16 {
    if constexpr (Cfg::KSPLIT) return ks4_sum<Cfg>(smem, i, j);
    else return plain_block<Cfg>(smem, i, j);
  };
  if constexpr (EPI == ORTHRUS_EPI_SWIGLU) {
    // columns come in (gate 32, up 32) pairs: block j even = gate, j+1 = its up block
    const int NO = N / 2;
#pragma unroll
    for (int i = 0; i < NBI; ++i)
#pragma unroll
      for (int j = 0; j < NBJ; j += 2) {
        if ((i * (NBJ / 2) + j / 2) % Cfg::NW != wu) continue;
        const int ng = n0 + j * 32;  // multiple of 64
        if (ng >= N) continue;
        const f32x16 g = block(i, j), u = block(i, j + 1);
        const int col = ng / 2 + r;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + i * 32 + acc_row(e, hh);
          if (m < M) {
            const float sg = g[e] / (1.0f + expf(-g[e]));
            C[(size_t)m * NO + col] = from_f32<OutT>(sg * u[e]);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < NBI; ++i)
#pragma unroll
      for (int j = 0; j < NBJ; ++j) {
        if ((i * NBJ + j) % Cfg::NW != wu) continue;
        const int n = n0 + j * 32 + r;
        if (n >= N) continue;
        const f32x16 v = block(i, j);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + i * 32 + acc_row(e, hh);
          if (m < M) {
            float x = v[e];
            if constexpr (EPI == ORTHRUS_EPI_RESIDUAL) x = to_f32(residual[(size_t)m * N + n]) + x;
            C[(size_t)m * N + n] = from_f32<OutT>(x);
          }
        }
      }
  }
}

// One k-slice of a BM x BN tile: the plain MFMA chain over k in [q K/S, (q+1) K/S), stored as an
// fp32 partial tile in P[q][M][N] straight from the accumulators (32 lanes write 32 consecutive
// columns of one row).
template <typename T, typename Cfg>
__global__ __launch_bounds__(Cfg::NT) ORTHRUS_GEMM_WAVES void gemm_quarter_kernel(const T* __restrict__ A,
                                                                                const T* __restrict__ W,
                                                                                float* __restrict__ P, int M, int N,
                                                                                int K, int S) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int mtiles = (M + Cfg::BM - 1) / Cfg::BM;
  int q, mt, nt;
  xcd_tile_map_ksplit(blockIdx.x, gridDim.x, S, mtiles, q, mt, nt);
  const int m0 = mt * Cfg::BM, n0 = nt * Cfg::BN, kq = K / S;
  f32x16 acc[Cfg::TM][Cfg::TN];
  gemm_mainloop<T, Cfg>(A + (size_t)q * kq, W + (size_t)q * kq, M, N, K, m0, n0, smem, acc, kq);
  const int lane = threadIdx.x & 63, hh = lane >> 5, r = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wu / Cfg::WN, wn = wu % Cfg::WN;
  float* Pq = P + (size_t)q * M * N;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int n = n0 + (wn * Cfg::TN + j) * 32 + r;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + (wm * Cfg::TM + i) * 32 + acc_row(e, hh);
        if (m < M) Pq[(size_t)m * N + n] = acc[i][j][e];
      }
    }
}

// c = epilogue(((P0 + P1) + P2) + ...), the S partials added in slice order.  V consecutive output
// columns per thread (V = 4 when the row length allows 16-byte partial loads).  SwiGLU columns come
// in (gate 32, up 32) groups, as in the plain epilogue.
template <typename OutT, int EPI, int V, int S>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ P, const OutT* residual, OutT* C,
                                                         int M, int N) {
  const size_t MN = (size_t)M * N;
  const int NO = EPI == ORTHRUS_EPI_SWIGLU ? N / 2 : N;
  const size_t idx = ((size_t)blockIdx.x * 256 + threadIdx.x) * V;  // first of V outputs
  if (idx >= (size_t)M * NO) return;
  const int m = (int)(idx / NO), c = (int)(idx % NO);
  auto sum = [&](int n, float (&s)[V]) {
    const size_t o = (size_t)m * N + n;
    if constexpr (V == 4) {
      f32x4 pp[S];
#pragma unroll
      for (int q = 0; q < S; ++q) pp[q] = *reinterpret_cast<const f32x4*>(P + o + q * MN);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        s[v] = pp[0][v];
#pragma unroll
        for (int q = 1; q < S; ++q) s[v] += pp[q][v];
      }
    } else {
      float pp[S];
#pragma unroll
      for (int q = 0; q < S; ++q) pp[q] = P[o + q * MN];
      s[0] = pp[0];
#pragma unroll
      for (int q = 1; q < S; ++q) s[0] += pp[q];
    }
  };
  float x[V];
  if constexpr (EPI == ORTHRUS_EPI_SWIGLU) {
    const int ng = (c / 32) * 64 + c % 32;  // V divides 32: the V gate columns share a group
    float g[V], u[V];
    sum(ng, g);
    sum(ng + 32, u);
#pragma unroll
    for (int v = 0; v < V; ++v) x[v] = g[v] / (1.0f + expf(-g[v])) * u[v];
  } else {
    sum(c, x);
    if constexpr (EPI == ORTHRUS_EPI_RESIDUAL) {
#pragma unroll
      for (int v = 0; v < V; ++v) x[v] = to_f32(residual[idx + v]) + x[v];
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v) C[idx + v] = from_f32<OutT>(x[v]);
}

// The residual k-slice reduce fused with the RMSNorm that follows every residual GEMM of a layer:
// x = x + (((P0 + P1) + P2) + ...) (stored), then y = rmsnorm(x) * g.  One workgroup per row with
// rmsnorm_kernel's shape: thread c owns 16-byte chunk c of the row, and issues its residual load and
// all S partial loads at once (one memory round trip); the sum of squares runs over the stored
// (rounded) x in rmsnorm_kernel's order (per thread in element order, a wave butterfly, then the
// waves in order), so the result has the bits of the residual GEMM followed by orthrus_rmsnorm.
template <typename T, int S>
__global__ __launch_bounds__(kNormMaxChunks) void gemm_reduce_rmsnorm_kernel(const float* __restrict__ P, T* x,
                                                                             const float* __restrict__ g, float eps,
                                                                             int M, int N, T* __restrict__ y) {
  constexpr int EPC = 16 / sizeof(T), NV = EPC / 4;  // elements and float4 partial loads per chunk
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  __shared__ float red[kNormMaxChunks / 64];
  const int m = blockIdx.x, c = threadIdx.x, nt = blockDim.x;
  const size_t MN = (size_t)M * N;
  T* xr = x + (size_t)m * N;
  T* yr = y + (size_t)m * N;
  const float* pr = P + (size_t)m * N;
  const bool own = c < N / EPC;
  u32x4_t buf = {0, 0, 0, 0};
  float ss = 0.0f;
  if (own) {
    const size_t o = (size_t)c * EPC;
    f32x4 pp[S][NV];
#pragma unroll
    for (int k = 0; k < S; ++k)
#pragma unroll
      for (int j = 0; j < NV; ++j) pp[k][j] = *reinterpret_cast<const f32x4*>(pr + o + 4 * j + k * MN);
    const u32x4_t rv = *reinterpret_cast<const u32x4_t*>(xr + o);
    const T* re = reinterpret_cast<const T*>(&rv);
    T* xe = reinterpret_cast<T*>(&buf);
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float sum = pp[0][j][v];
#pragma unroll
        for (int k = 1; k < S; ++k) sum += pp[k][j][v];
        xe[4 * j + v] = from_f32<T>(to_f32(re[4 * j + v]) + sum);
      }
    *reinterpret_cast<u32x4_t*>(xr + o) = buf;
#pragma unroll
    for (int i = 0; i < EPC; ++i) {
      const float v = to_f32(xe[i]);
      ss += v * v;
    }
  }
  ss = wave_sum(ss);
  if ((c & 63) == 0) red[c >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
  for (int w = 0; w < nt / 64; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)N + eps);
  if (own) {
    const T* e = reinterpret_cast<const T*>(&buf);
    u32x4_t o;
    T* oe = reinterpret_cast<T*>(&o);
#pragma unroll
    for (int i = 0; i < EPC; ++i) oe[i] = from_f32<T>(to_f32(e[i]) * inv * g[(size_t)c * EPC + i]);
    *reinterpret_cast<u32x4_t*>(yr + (size_t)c * EPC) = o;
  }
}

// The q/k/v k-slice reduce fused with RoPE and the K/V write (rope_kv_kernel's work): every q/k/v
// element is the sum of the S partials in slice order rounded to T, exactly the value the store
// epilogue would have written, and the rotation and the writes are rope_kv_kernel's, so the result has
// the bits of orthrus_gemm(STORE) followed by orthrus_rope_kv_write.  Workgroup (row m, head group y)
// handles 256 / (D/2) consecutive heads of the row's Hq + Hkv rotated heads and Hkv value heads, one
// rotation pair (or two copied value elements) per thread.
template <typename T, int S>
__global__ __launch_bounds__(256) void gemm_reduce_rope_kv_kernel(const float* __restrict__ P, int M,
                                                                  const float* __restrict__ table, int max_pos,
                                                                  const int32_t* __restrict__ ctx_len,
                                                                  const int32_t* __restrict__ page_table, int block,
                                                                  int Hq, int Hkv, int D, int page, int max_pages,
                                                                  T* __restrict__ q_out, T* __restrict__ k_dst,
                                                                  T* __restrict__ v_dst) {
  const int m = blockIdx.x, b = m / block, s = m % block;
  const int half = D / 2, hpw = 256 / half;  // heads per workgroup
  const int hd = blockIdx.y * hpw + (int)threadIdx.x / half, i = (int)threadIdx.x % half;
  if (hd >= Hq + 2 * Hkv) return;
  const int pos = ctx_len[b] + s;
  const int width = (Hq + 2 * Hkv) * D;
  const size_t MN = (size_t)M * width;
  const float* pr = P + (size_t)m * width;
  auto val = [&](int j) {
    float sum = pr[j];
#pragma unroll
    for (int k = 1; k < S; ++k) sum += pr[j + k * MN];
    return to_f32(from_f32<T>(sum));
  };
  const bool pos_ok = pos >= 0 && pos < max_pos;
  size_t kv_base = 0;
  bool kv_ok = pos_ok;
  if (page_table) {
    kv_ok = kv_ok && pos < max_pages * page;
    if (kv_ok) {
      const int pg = page_table[(size_t)b * max_pages + pos / page];
      kv_base = ((size_t)pg * Hkv * page + (pos % page)) * D;
    }
  } else {
    kv_base = (size_t)m * Hkv * D;
  }
  const size_t kv_head_stride = page_table ? (size_t)page * D : (size_t)D;
  if (hd < Hq + Hkv) {
    const float* cs = table + (size_t)(pos_ok ? pos : 0) * half * 2;
    const float c = cs[2 * i], sn = cs[2 * i + 1];
    const float x1 = val(hd * D + i), x2 = val(hd * D + i + half);
    const float y1 = pos_ok ? x1 * c - x2 * sn : __builtin_nanf("");
    const float y2 = pos_ok ? x2 * c + x1 * sn : __builtin_nanf("");
    if (hd < Hq) {
      T* qo = q_out + (size_t)m * Hq * D + hd * D;
      qo[i] = from_f32<T>(y1);
      qo[i + half] = from_f32<T>(y2);
    } else if (kv_ok) {
      T* ko = k_dst + kv_base + (hd - Hq) * kv_head_stride;
      ko[i] = from_f32<T>(y1);
      ko[i + half] = from_f32<T>(y2);
    }
  } else if (kv_ok) {
    const int hk = hd - Hq - Hkv;
    T* vo = v_dst + kv_base + hk * kv_head_stride;
    const int j0 = (Hq + Hkv) * D + hk * D;
    vo[i] = from_f32<T>(val(j0 + i));
    vo[i + half] = from_f32<T>(val(j0 + i + half));
  }
}

// Families chosen by (N, K) alone (so an output element's k order never depends on M):
//  * N < 16384 (QKV, O, down projections) with whole-stage quarters of K: plain tiles, one
//    workgroup per (tile, k-quarter), partials added by gemm_reduce_kernel;
//  * other N < 16384: KsCfg tiles, k-steps split four ways inside the workgroup;
//  * N >= 16384 (the gate/up projection): plain GemmCfg tiles, waves split the output tile.
// Within a family the tile height follows M only to avoid idle rows.
// Ring depths (A stages, W stages) keep each configuration at or under 80 KiB of LDS, so two
// workgroups share a CU, with the deeper ring on the weight stream.
#ifndef ORTHRUS_KSS_RINGS
#define ORTHRUS_KSS_RINGS 6, 6
#endif
#ifndef ORTHRUS_KSB_RINGS
#define ORTHRUS_KSB_RINGS 5, 5
#endif
#ifndef ORTHRUS_PB_RINGS
#define ORTHRUS_PB_RINGS 3, 2
#endif
template <typename T> using KsSmall = KsCfg<T, 32, 64, ORTHRUS_KSS_RINGS>;
template <typename T> using KsBig = KsCfg<T, 64, 64, ORTHRUS_KSB_RINGS>;
template <typename T> using PlainSmall = GemmCfg<T, 32, 128, 1, 4, 4, 4>;
template <typename T> using PlainMid = GemmCfg<T, 64, 128, 2, 2, 3, 3>;
template <typename T> using PlainBig = GemmCfg<T, 128, 128, 2, 2, ORTHRUS_PB_RINGS>;
// 128 x 192 tiles of eight 32 x 96 wavefronts, one workgroup per CU (128 KiB of LDS)
template <typename T> using Plain192 = GemmCfg<T, 128, 192, 4, 2, 2, 4>;
// 128 x 128 tiles of eight 32 x 64 wavefronts (80 KiB of rings) for the four-slice N = 4096 case (the
// O projection: 256 workgroups, one per CU): twice the wavefronts of PlainBig per tile to hide the
// short main loop's latency (27.6 -> 24.1 us per launch with its reduce at M = 256, same bits)
template <typename T> using Plain128w8 = GemmCfg<T, 128, 128, 4, 2, 2, 3>;
// Above 128 rows the wide family runs 128 x 192 tiles of eight 32 x 96 wavefronts (two per SIMD
// at one workgroup per CU).  At M = 256 the 24576-wide gate/up projection is then 2 x 128 = 256
// tiles, one per CU (256 x 128 tiles left 64 CUs idle), and each workgroup streams 2.5 MiB of
// operands instead of 3; xcd_tile_map keeps the two row tiles of a weight tile on one XCD, so
// the weights still come from HBM about once.  The weight ring is the deeper one: it streams
// from HBM, the activation ring from L2.  (192 columns are three 64-column gate/up pairs, so the
// SwiGLU epilogue never splits a pair.)
#ifndef ORTHRUS_WIDE_HUGE_CFG
#define ORTHRUS_WIDE_HUGE_CFG(T) Plain192<T>
#endif
constexpr int kWideN = 16384;

template <typename T, typename OutT, typename Cfg>
int32_t launch_cfg(int M, int N, int K, int epi, const void* a, const void* w, const void* res, void* c,
                   hipStream_t st) {
  const int mtiles = (M + Cfg::BM - 1) / Cfg::BM, ntiles = (N + Cfg::BN - 1) / Cfg::BN;
  dim3 grid(mtiles * ntiles);
  const size_t lds = Cfg::LDS_BYTES;
  const T* A = reinterpret_cast<const T*>(a);
  const T* Wt = reinterpret_cast<const T*>(w);
  const OutT* R = reinterpret_cast<const OutT*>(res);
  OutT* C = reinterpret_cast<OutT*>(c);
  switch (epi) {
    case ORTHRUS_EPI_STORE:
      allow_lds(gemm_kernel<T, OutT, Cfg, ORTHRUS_EPI_STORE>, lds);
      hipLaunchKernelGGL((gemm_kernel<T, OutT, Cfg, ORTHRUS_EPI_STORE>), grid, dim3(Cfg::NT), lds, st, A, Wt, R, C, M, N, K);
      break;
    case ORTHRUS_EPI_RESIDUAL:
      allow_lds(gemm_kernel<T, OutT, Cfg, ORTHRUS_EPI_RESIDUAL>, lds);
      hipLaunchKernelGGL((gemm_kernel<T, OutT, Cfg, ORTHRUS_EPI_RESIDUAL>), grid, dim3(Cfg::NT), lds, st, A, Wt, R, C, M,
                         N, K);
      break;
    default:
      allow_lds(gemm_kernel<T, OutT, Cfg, ORTHRUS_EPI_SWIGLU>, lds);
      hipLaunchKernelGGL((gemm_kernel<T, OutT, Cfg, ORTHRUS_EPI_SWIGLU>), grid, dim3(Cfg::NT), lds, st, A, Wt, R, C, M, N,
                         K);
      break;
  }
  return check_launch("orthrus_gemm");
}

// The k-split: S contiguous slices of K, each a whole number of 128-byte stages.  S = 8 for deep K
// (the down projection: 128x128 tiles x 8 slices put two workgroups on every CU, 49-50 us against
// 58-64 at M = 256), 4 otherwise (8 slices made q/k/v and O slower); 0 when K does not split or N
// is wide.  A function of (N, K) only, so a row's summation order never depends on M.
int k_splits(int N, int K, int dtype) {
  const int bk = dtype == ORTHRUS_BF16 ? 64 : 32;
  if (N >= kWideN) return 0;
  if (K >= 8192 && K % (8 * bk) == 0) return 8;
  return K % (4 * bk) == 0 ? 4 : 0;
}

template <typename T> constexpr int dtype_of() { return sizeof(T) == 2 ? ORTHRUS_BF16 : ORTHRUS_F32; }

// The S k-slice partial tiles of a [M, N] product into P; the tile height follows M only.
template <typename T, typename Cfg>
void launch_quarter_cfg(int M, int N, int K, int S, const void* a, const void* w, float* P, hipStream_t st) {
  const int mtiles = (M + Cfg::BM - 1) / Cfg::BM, ntiles = (N + Cfg::BN - 1) / Cfg::BN;
  allow_lds(gemm_quarter_kernel<T, Cfg>, Cfg::RING);
  hipLaunchKernelGGL((gemm_quarter_kernel<T, Cfg>), dim3(S * mtiles * ntiles), dim3(Cfg::NT), Cfg::RING, st,
                     reinterpret_cast<const T*>(a), reinterpret_cast<const T*>(w), P, M, N, K, S);
}

// Returns S, the number of partial tiles written.
template <typename T>
int launch_quarter_tiles(int M, int N, int K, const void* a, const void* w, float* P, hipStream_t st) {
  const int S = k_splits(N, K, dtype_of<T>());
  if (M <= 32) launch_quarter_cfg<T, PlainSmall<T>>(M, N, K, S, a, w, P, st);
  else if (M <= 64) launch_quarter_cfg<T, PlainMid<T>>(M, N, K, S, a, w, P, st);
  // q/k/v (N = 6144) at M = 256: 2 x 32 x 4 = 256 workgroups of 128 x 192 instead of 384 of 128 x 128
  // (31.7 -> 27.3-27.9 us back to back); O and down (N = 4096) keep 128 x 128 tiles, with eight
  // wavefronts when there are four slices (one workgroup per CU) and four when there are eight
  else if (N % 192 == 0) launch_quarter_cfg<T, Plain192<T>>(M, N, K, S, a, w, P, st);
  else if (S == 4) launch_quarter_cfg<T, Plain128w8<T>>(M, N, K, S, a, w, P, st);
  else launch_quarter_cfg<T, PlainBig<T>>(M, N, K, S, a, w, P, st);
  return S;
}

template <typename OutT, int S>
void launch_reduce(int M, int N, int epi, const float* P, const OutT* R, OutT* C, hipStream_t st) {
  const size_t outs = (size_t)M * (epi == ORTHRUS_EPI_SWIGLU ? N / 2 : N);
  // 16-byte partial loads need every row to start on a 4-column boundary (SwiGLU: N % 64 == 0)
  if (N % 4 == 0) {
    const dim3 rgrid((unsigned)((outs / 4 + 255) / 256));
    if (epi == ORTHRUS_EPI_STORE)
      hipLaunchKernelGGL((gemm_reduce_kernel<OutT, ORTHRUS_EPI_STORE, 4, S>), rgrid, dim3(256), 0, st, P, R, C, M, N);
    else if (epi == ORTHRUS_EPI_RESIDUAL)
      hipLaunchKernelGGL((gemm_reduce_kernel<OutT, ORTHRUS_EPI_RESIDUAL, 4, S>), rgrid, dim3(256), 0, st, P, R, C, M,
                         N);
    else
      hipLaunchKernelGGL((gemm_reduce_kernel<OutT, ORTHRUS_EPI_SWIGLU, 4, S>), rgrid, dim3(256), 0, st, P, R, C, M, N);
  } else {
    const dim3 rgrid((unsigned)((outs + 255) / 256));
    if (epi == ORTHRUS_EPI_STORE)
      hipLaunchKernelGGL((gemm_reduce_kernel<OutT, ORTHRUS_EPI_STORE, 1, S>), rgrid, dim3(256), 0, st, P, R, C, M, N);
    else
      hipLaunchKernelGGL((gemm_reduce_kernel<OutT, ORTHRUS_EPI_RESIDUAL, 1, S>), rgrid, dim3(256), 0, st, P, R, C, M,
                         N);
  }
}

template <typename T, typename OutT>
int32_t launch_quarters(int M, int N, int K, int epi, const void* a, const void* w, const void* res, void* c,
                        float* P, hipStream_t st) {
  const int S = launch_quarter_tiles<T>(M, N, K, a, w, P, st);
  const OutT* R = reinterpret_cast<const OutT*>(res);
  OutT* C = reinterpret_cast<OutT*>(c);
  if (S == 8) launch_reduce<OutT, 8>(M, N, epi, P, R, C, st);
  else launch_reduce<OutT, 4>(M, N, epi, P, R, C, st);
  return check_launch("orthrus_gemm");
}


// -------------------------------------------------------------------- fragment-packed gate/up
// The gate/up + SwiGLU GEMM on fragment-packed weights (gemm_rs.hpp): same k order as the one-loop
// family (N >= 16384), so the same bits as gemm_kernel with ORTHRUS_EPI_SWIGLU on the row-interleaved
// packing.  Workgroup tile 128 x 256 (four wavefronts of 128 x 64: two gate/up column-block pairs).
constexpr int kRsStages = 64;  // K = 64 * 64 = 4096, the instantiated width
using RsSwiglu = RsCfg<4, 2, 4, 2, 4>;
// 128x192 tiles of six 128x32 wavefronts: 256 workgroups at M = 256 and N = 24576 (every CU busy,
// against 192 with 128x256 tiles), 2.5 MiB of operands per workgroup instead of 3.  Two more
// wavefronts load the activation stages (a ring of four), so that the compute wavefronts' loads
// are their weight stages alone (four in flight).
#ifndef ORTHRUS_RS192_NB
#define ORTHRUS_RS192_NB 4
#endif
#ifndef ORTHRUS_RS192_SA
#define ORTHRUS_RS192_SA 4
#endif
#ifndef ORTHRUS_RS192_NL
#define ORTHRUS_RS192_NL 2
#endif
using RsSwiglu192 = RsCfg<4, 1, 6, ORTHRUS_RS192_SA, ORTHRUS_RS192_NB, ORTHRUS_RS192_NL>;

template <typename Cfg>
__global__ __launch_bounds__(Cfg::NT) void rs_swiglu_kernel(const bf16* __restrict__ A, const bf16* __restrict__ Wp,
                                                            bf16* __restrict__ C, int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int mtiles = (M + Cfg::BM - 1) / Cfg::BM;
  int sp, mt, nt;
  xcd_tile_map(blockIdx.x, gridDim.x, 1, mtiles, sp, mt, nt);
  const int m0 = mt * Cfg::BM, n0 = nt * Cfg::BN;
  f32x16 acc[Cfg::TMW][Cfg::TNW];
  rs_mainloop<Cfg, kRsStages>(A, Wp, M, N, K, m0, n0, 0, smem, acc);
  const int lane = threadIdx.x & 63, hh = lane >> 5, r = lane & 31, wu = threadIdx.x >> 6;
  const int NO = N / 2;
  if constexpr (Cfg::TNW == 1) {
    // one 32-column block per wave: gate blocks (even) and up blocks (odd) sit in neighbouring
    // waves, so each gate wave parks silu(g) in LDS (rows padded to 33 floats) for its up wave
    static_assert(Cfg::NW % 2 == 0, "gate/up wave pairs");
    constexpr int RS = 33;
    float* sg_lds = reinterpret_cast<float*>(smem) + (wu / 2) * Cfg::BM * RS;
    if (wu % 2 == 0 && wu < Cfg::NW) {  // (waves past NW load activations only)
#pragma unroll
      for (int i = 0; i < Cfg::TMW; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float g = acc[i][0][e];
          sg_lds[(i * 32 + acc_row(e, hh)) * RS + r] = g / (1.0f + expf(-g));
        }
    }
    __syncthreads();
    const int ng = n0 + (wu - 1) * 32;  // the pair's gate block
    if (wu % 2 == 1 && wu < Cfg::NW && ng < N) {
      const int col = ng / 2 + r;
#pragma unroll
      for (int i = 0; i < Cfg::TMW; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + i * 32 + acc_row(e, hh);
          if (m < M) C[(size_t)m * NO + col] = from_f32<bf16>(sg_lds[(i * 32 + acc_row(e, hh)) * RS + r] * acc[i][0][e]);
        }
    }
  } else {
    static_assert(Cfg::TNW % 2 == 0, "gate/up column-block pairs");
    if (wu >= Cfg::NW) return;  // a wave that loads activations only
#pragma unroll
    for (int jp = 0; jp < Cfg::TNW; jp += 2) {
      const int ng = n0 + (wu * Cfg::TNW + jp) * 32;  // the pair's gate block; the up block follows
      if (ng >= N) continue;
      const int col = ng / 2 + r;
#pragma unroll
      for (int i = 0; i < Cfg::TMW; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + i * 32 + acc_row(e, hh);
          if (m < M) {
            const float g = acc[i][jp][e], u = acc[i][jp + 1][e];
            const float sg = g / (1.0f + expf(-g));
            C[(size_t)m * NO + col] = from_f32<bf16>(sg * u);
          }
        }
    }
  }
}

// gate/up rows interleaved in 32-row groups (as pack_gate_up_kernel) and written in the
// fragment-packed layout, one 8-element chunk per thread
__global__ void pack_gate_up_fragments_kernel(const bf16* __restrict__ g, const bf16* __restrict__ u,
                                              bf16* __restrict__ p, int inter, int hidden) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int N = 2 * inter, K = hidden;
  if (t >= (size_t)N * (K / 8)) return;
  const int n = (int)(t / (K / 8)), k = (int)(t % (K / 8)) * 8;
  const int grp = n / 64, within = n % 64;
  const bf16* src = (within < 32 ? g : u) + (size_t)(grp * 32 + (within & 31)) * K + k;
  *reinterpret_cast<bf16x8*>(p + packed_offset(n, k, N, K)) = *reinterpret_cast<const bf16x8*>(src);
}

// 2 * inter in whole 128x192 tiles (six waves) or else whole 128x256 tiles (four waves)
bool rs_swiglu_ok(int inter, int hidden, int dtype) {
  return dtype == ORTHRUS_BF16 && hidden == 64 * kRsStages && 2 * inter >= kWideN &&
         ((2 * inter) % RsSwiglu192::BN == 0 || (2 * inter) % RsSwiglu::BN == 0);
}

template <typename Cfg>
int32_t launch_rs_swiglu(int M, int N, int K, const void* a, const void* w, void* c, hipStream_t st) {
  constexpr size_t epi = Cfg::TNW == 1 ? (size_t)(Cfg::NW / 2) * Cfg::BM * 33 * sizeof(float) : 0;
  constexpr size_t lds = Cfg::RING > epi ? Cfg::RING : epi;
  const int mtiles = (M + Cfg::BM - 1) / Cfg::BM, ntiles = N / Cfg::BN;
  allow_lds(rs_swiglu_kernel<Cfg>, lds);
  hipLaunchKernelGGL(rs_swiglu_kernel<Cfg>, dim3(mtiles * ntiles), dim3(Cfg::NT), lds, st,
                     reinterpret_cast<const bf16*>(a), reinterpret_cast<const bf16*>(w), reinterpret_cast<bf16*>(c),
                     M, N, K);
  return check_launch("orthrus_gemm_swiglu_fragments");
}

template <typename T, typename OutT>
int32_t launch(int M, int N, int K, int epi, const void* a, const void* w, const void* res, void* c, float* P,
               hipStream_t st) {
  if (N < kWideN) {
    if (k_splits(N, K, dtype_of<T>())) return launch_quarters<T, OutT>(M, N, K, epi, a, w, res, c, P, st);
    if (M <= 32) return launch_cfg<T, OutT, KsSmall<T>>(M, N, K, epi, a, w, res, c, st);
    return launch_cfg<T, OutT, KsBig<T>>(M, N, K, epi, a, w, res, c, st);
  }
  if (M <= 32) return launch_cfg<T, OutT, PlainSmall<T>>(M, N, K, epi, a, w, res, c, st);
  if (M <= 64) return launch_cfg<T, OutT, PlainMid<T>>(M, N, K, epi, a, w, res, c, st);
  if (M <= 128) return launch_cfg<T, OutT, PlainBig<T>>(M, N, K, epi, a, w, res, c, st);
  return launch_cfg<T, OutT, ORTHRUS_WIDE_HUGE_CFG(T)>(M, N, K, epi, a, w, res, c, st);
}

// The fused residual + RMSNorm pass applies when the GEMM takes the k-split and the row fits
// rmsnorm_kernel's register path (16-byte chunks, at most 1024 of them, 16-byte aligned rows).
template <typename T>
bool fused_norm_ok(int N, int K, int dtype, const void* x, const void* y) {
  constexpr int EPC = 16 / (int)sizeof(T);
  return k_splits(N, K, dtype) && N % EPC == 0 && N / EPC <= kNormMaxChunks &&
         ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15) == 0;
}

template <typename T>
int32_t launch_residual_rmsnorm(int M, int N, int K, const void* a, const void* w, void* x, const float* gain,
                                float eps, void* y, float* P, hipStream_t st) {
  const int S = launch_quarter_tiles<T>(M, N, K, a, w, P, st);
  const int nt = norm_threads(N, (int)sizeof(T));  // one thread per 16-byte chunk, as rmsnorm_kernel
  if (S == 8)
    hipLaunchKernelGGL((gemm_reduce_rmsnorm_kernel<T, 8>), dim3(M), dim3(nt), 0, st, P, reinterpret_cast<T*>(x), gain,
                       eps, M, N, reinterpret_cast<T*>(y));
  else
    hipLaunchKernelGGL((gemm_reduce_rmsnorm_kernel<T, 4>), dim3(M), dim3(nt), 0, st, P, reinterpret_cast<T*>(x), gain,
                       eps, M, N, reinterpret_cast<T*>(y));
  return check_launch("orthrus_gemm_residual_rmsnorm");
}

template <typename T>
__global__ void pack_gate_up_kernel(const T* g, const T* u, T* p, int inter, int hidden) {
  const int row = blockIdx.x;  // 0 .. 2*inter-1 of the packed matrix
  const int grp = row / 64, within = row % 64;
  const T* src = (within < 32 ? g : u) + (size_t)(grp * 32 + (within & 31)) * hidden;
  T* dst = p + (size_t)row * hidden;
  for (int i = threadIdx.x; i < hidden; i += blockDim.x) dst[i] = src[i];
}

int32_t validate(int32_t M, int32_t N, int32_t K, int32_t dtype, int32_t out_dtype, int32_t epilogue) {
  ORTHRUS_REQUIRE(M >= 0 && N > 0 && K > 0, ORTHRUS_ERR_INVALID_ARG, "gemm: bad sizes M=%d N=%d K=%d", M, N, K);
  ORTHRUS_REQUIRE(K % 64 == 0, ORTHRUS_ERR_UNSUPPORTED, "gemm: K=%d not a multiple of 64", K);
  ORTHRUS_REQUIRE(valid_dtype(dtype) && valid_dtype(out_dtype), ORTHRUS_ERR_INVALID_ARG, "gemm: bad dtype");
  ORTHRUS_REQUIRE(epilogue >= 0 && epilogue <= 2, ORTHRUS_ERR_INVALID_ARG, "gemm: bad epilogue %d", epilogue);
  ORTHRUS_REQUIRE(epilogue != ORTHRUS_EPI_SWIGLU || N % 64 == 0, ORTHRUS_ERR_INVALID_ARG,
                  "gemm: SwiGLU needs N %% 64 == 0 (got %d)", N);
  ORTHRUS_REQUIRE(!(dtype == ORTHRUS_F32 && out_dtype == ORTHRUS_BF16), ORTHRUS_ERR_UNSUPPORTED,
                  "gemm: fp32 inputs with bf16 output not built");
  return ORTHRUS_OK;
}

}  // namespace
}  // namespace orthrus

using namespace orthrus;

extern "C" size_t orthrus_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t dtype, int32_t epilogue) {
  (void)epilogue;
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return (size_t)k_splits(N, K, dtype) * M * N * sizeof(float);  // the S fp32 k-slice partials
}

extern "C" int32_t orthrus_gemm(int32_t M, int32_t N, int32_t K, int32_t dtype, int32_t out_dtype, int32_t epilogue,
                                const void* a, const void* w, const void* residual, void* c, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (int32_t s = validate(M, N, K, dtype, out_dtype, epilogue)) return s;
  ORTHRUS_REQUIRE(a && w && c, ORTHRUS_ERR_INVALID_ARG, "gemm: null pointer");
  ORTHRUS_REQUIRE(epilogue != ORTHRUS_EPI_RESIDUAL || residual, ORTHRUS_ERR_INVALID_ARG, "gemm: residual is null");
  if (M == 0) return ORTHRUS_OK;
  const size_t need = orthrus_gemm_workspace_bytes(M, N, K, dtype, epilogue);
  ORTHRUS_REQUIRE(need == 0 || (workspace && workspace_bytes >= need), ORTHRUS_ERR_WORKSPACE,
                  "gemm: workspace %zu < %zu bytes", workspace ? workspace_bytes : (size_t)0, need);
  ORTHRUS_REQUIRE(need == 0 || ((uintptr_t)workspace & 15) == 0, ORTHRUS_ERR_INVALID_ARG,
                  "gemm: workspace not 16-byte aligned");
  float* P = reinterpret_cast<float*>(workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == ORTHRUS_BF16) {
    if (out_dtype == ORTHRUS_BF16) return launch<bf16, bf16>(M, N, K, epilogue, a, w, residual, c, P, st);
    return launch<bf16, float>(M, N, K, epilogue, a, w, residual, c, P, st);
  }
  return launch<float, float>(M, N, K, epilogue, a, w, residual, c, P, st);
}

extern "C" int32_t orthrus_gemm_residual_rmsnorm(int32_t M, int32_t N, int32_t K, int32_t dtype, const void* a,
                                                 const void* w, void* x, const float* gain, float eps, void* y,
                                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (int32_t s = validate(M, N, K, dtype, dtype, ORTHRUS_EPI_RESIDUAL)) return s;
  ORTHRUS_REQUIRE(a && w && x && gain && y, ORTHRUS_ERR_INVALID_ARG, "gemm_residual_rmsnorm: null pointer");
  if (M == 0) return ORTHRUS_OK;
  const size_t need = orthrus_gemm_workspace_bytes(M, N, K, dtype, ORTHRUS_EPI_RESIDUAL);
  ORTHRUS_REQUIRE(need == 0 || (workspace && workspace_bytes >= need), ORTHRUS_ERR_WORKSPACE,
                  "gemm_residual_rmsnorm: workspace %zu < %zu bytes", workspace ? workspace_bytes : (size_t)0, need);
  ORTHRUS_REQUIRE(need == 0 || ((uintptr_t)workspace & 15) == 0, ORTHRUS_ERR_INVALID_ARG,
                  "gemm_residual_rmsnorm: workspace not 16-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float* P = reinterpret_cast<float*>(workspace);
  if (dtype == ORTHRUS_BF16 && fused_norm_ok<bf16>(N, K, dtype, x, y))
    return launch_residual_rmsnorm<bf16>(M, N, K, a, w, x, gain, eps, y, P, st);
  if (dtype == ORTHRUS_F32 && fused_norm_ok<float>(N, K, dtype, x, y))
    return launch_residual_rmsnorm<float>(M, N, K, a, w, x, gain, eps, y, P, st);
  // other shapes: the two calls in sequence (the fused pass has their bits)
  if (int32_t s = orthrus_gemm(M, N, K, dtype, dtype, ORTHRUS_EPI_RESIDUAL, a, w, x, x, workspace, workspace_bytes,
                               stream))
    return s;
  return orthrus_rmsnorm(M, N, dtype, x, gain, eps, y, stream);
}

extern "C" int32_t orthrus_gemm_rope_kv_write(int32_t batch, int32_t block, int32_t q_heads, int32_t kv_heads,
                                              int32_t head_dim, int32_t page_size, int32_t max_pages, int32_t hidden,
                                              int32_t dtype, const void* a, const void* w, const float* rope_table,
                                              int32_t max_pos, const int32_t* ctx_len, const int32_t* page_table,
                                              void* qkv, void* q_out, void* k_dst, void* v_dst, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  ORTHRUS_REQUIRE(batch >= 0 && block >= 1 && q_heads > 0 && kv_heads > 0 && head_dim > 0 && head_dim % 2 == 0,
                  ORTHRUS_ERR_INVALID_ARG, "gemm_rope_kv_write: bad sizes");
  const int M = batch * block, N = (q_heads + 2 * kv_heads) * head_dim, K = hidden;
  if (int32_t s = validate(M, N, K, dtype, dtype, ORTHRUS_EPI_STORE)) return s;
  ORTHRUS_REQUIRE(a && w && rope_table && ctx_len && qkv && q_out && k_dst && v_dst && max_pos > 0,
                  ORTHRUS_ERR_INVALID_ARG, "gemm_rope_kv_write: bad args");
  ORTHRUS_REQUIRE(!page_table || (page_size > 0 && max_pages > 0), ORTHRUS_ERR_INVALID_ARG,
                  "gemm_rope_kv_write: paging");
  if (batch == 0) return ORTHRUS_OK;
  const size_t need = orthrus_gemm_workspace_bytes(M, N, K, dtype, ORTHRUS_EPI_STORE);
  ORTHRUS_REQUIRE(need == 0 || (workspace && workspace_bytes >= need), ORTHRUS_ERR_WORKSPACE,
                  "gemm_rope_kv_write: workspace %zu < %zu bytes", workspace ? workspace_bytes : (size_t)0, need);
  ORTHRUS_REQUIRE(need == 0 || ((uintptr_t)workspace & 15) == 0, ORTHRUS_ERR_INVALID_ARG,
                  "gemm_rope_kv_write: workspace not 16-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!k_splits(N, K, dtype) || head_dim > 512 || 256 % (head_dim / 2) != 0) {
    // other shapes: the two calls in sequence through qkv (the fused pass has their bits)
    if (int32_t s = orthrus_gemm(M, N, K, dtype, dtype, ORTHRUS_EPI_STORE, a, w, nullptr, qkv, workspace,
                                 workspace_bytes, stream))
      return s;
    return orthrus_rope_kv_write(batch, block, q_heads, kv_heads, head_dim, page_size, max_pages, dtype, qkv,
                                 rope_table, max_pos, ctx_len, page_table, q_out, k_dst, v_dst, stream);
  }
  float* P = reinterpret_cast<float*>(workspace);
  auto quarters = [&](auto tag) {
    using T = decltype(tag);
    const int S = launch_quarter_tiles<T>(M, N, K, a, w, P, st);
    const int hpw = 256 / (head_dim / 2);
    const dim3 grid(M, (q_heads + 2 * kv_heads + hpw - 1) / hpw);
    if (S == 8)
      hipLaunchKernelGGL((gemm_reduce_rope_kv_kernel<T, 8>), grid, dim3(256), 0, st, P, M, rope_table, max_pos, ctx_len,
                         page_table, block, q_heads, kv_heads, head_dim, page_size, max_pages,
                         reinterpret_cast<T*>(q_out), reinterpret_cast<T*>(k_dst), reinterpret_cast<T*>(v_dst));
    else
      hipLaunchKernelGGL((gemm_reduce_rope_kv_kernel<T, 4>), grid, dim3(256), 0, st, P, M, rope_table, max_pos, ctx_len,
                         page_table, block, q_heads, kv_heads, head_dim, page_size, max_pages,
                         reinterpret_cast<T*>(q_out), reinterpret_cast<T*>(k_dst), reinterpret_cast<T*>(v_dst));
  };
  if (dtype == ORTHRUS_BF16) quarters(bf16{});
  else quarters(float{});
  return check_launch("orthrus_gemm_rope_kv_write");
}

extern "C" int32_t orthrus_pack_gate_up(int32_t inter, int32_t hidden, int32_t dtype, const void* gate,
                                        const void* up, void* packed, void* stream) {
  ORTHRUS_REQUIRE(inter > 0 && hidden > 0 && inter % 32 == 0, ORTHRUS_ERR_INVALID_ARG, "pack_gate_up: bad sizes");
  ORTHRUS_REQUIRE(valid_dtype(dtype) && gate && up && packed, ORTHRUS_ERR_INVALID_ARG, "pack_gate_up: bad args");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == ORTHRUS_BF16)
    hipLaunchKernelGGL(pack_gate_up_kernel<bf16>, dim3(2 * inter), dim3(256), 0, st, (const bf16*)gate, (const bf16*)up,
                       (bf16*)packed, inter, hidden);
  else
    hipLaunchKernelGGL(pack_gate_up_kernel<float>, dim3(2 * inter), dim3(256), 0, st, (const float*)gate,
                       (const float*)up, (float*)packed, inter, hidden);
  return check_launch("orthrus_pack_gate_up");
}

extern "C" int32_t orthrus_pack_gate_up_fragments(int32_t inter, int32_t hidden, int32_t dtype, const void* gate,
                                                  const void* up, void* packed, void* stream) {
  ORTHRUS_REQUIRE(inter > 0 && hidden > 0 && gate && up && packed, ORTHRUS_ERR_INVALID_ARG,
                  "pack_gate_up_fragments: bad args");
  ORTHRUS_REQUIRE(rs_swiglu_ok(inter, hidden, dtype), ORTHRUS_ERR_UNSUPPORTED,
                  "pack_gate_up_fragments: built for bf16, hidden %d and 2*inter a multiple of %d or %d, >= %d "
                  "(got dtype %d, hidden %d, inter %d)", 64 * kRsStages, RsSwiglu192::BN, RsSwiglu::BN, kWideN, dtype,
                  hidden, inter);
  ORTHRUS_REQUIRE(((reinterpret_cast<uintptr_t>(gate) | reinterpret_cast<uintptr_t>(up) |
                    reinterpret_cast<uintptr_t>(packed)) & 15) == 0, ORTHRUS_ERR_INVALID_ARG,
                  "pack_gate_up_fragments: pointers must be 16-byte aligned");
  const size_t n = (size_t)2 * inter * (hidden / 8);
  hipLaunchKernelGGL(pack_gate_up_fragments_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), (const bf16*)gate, (const bf16*)up, (bf16*)packed, inter,
                     hidden);
  return check_launch("orthrus_pack_gate_up_fragments");
}

extern "C" int32_t orthrus_gemm_swiglu_fragments(int32_t M, int32_t inter, int32_t hidden, int32_t dtype,
                                                 const void* a, const void* w_fragments, void* c, void* stream) {
  ORTHRUS_REQUIRE(M >= 0 && inter > 0 && hidden > 0, ORTHRUS_ERR_INVALID_ARG, "gemm_swiglu_fragments: bad sizes");
  ORTHRUS_REQUIRE(rs_swiglu_ok(inter, hidden, dtype), ORTHRUS_ERR_UNSUPPORTED,
                  "gemm_swiglu_fragments: built for bf16, hidden %d and 2*inter a multiple of %d or %d, >= %d",
                  64 * kRsStages, RsSwiglu192::BN, RsSwiglu::BN, kWideN);
  ORTHRUS_REQUIRE(a && w_fragments && c, ORTHRUS_ERR_INVALID_ARG, "gemm_swiglu_fragments: null pointer");
  ORTHRUS_REQUIRE(((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(w_fragments)) & 15) == 0,
                  ORTHRUS_ERR_INVALID_ARG, "gemm_swiglu_fragments: a and w must be 16-byte aligned");
  if (M == 0) return ORTHRUS_OK;
  const int N = 2 * inter;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (N % RsSwiglu192::BN == 0) return launch_rs_swiglu<RsSwiglu192>(M, N, hidden, a, w_fragments, c, st);
  return launch_rs_swiglu<RsSwiglu>(M, N, hidden, a, w_fragments, c, st);
}
