// Layer GEMMs of both views: C = epilogue(A W^T) on MFMA with fused residual add or SwiGLU.
#include "gemm_core.hpp"

namespace orthrus {
namespace {

template <typename T, typename OutT, typename Cfg, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const T* __restrict__ A, const T* __restrict__ W,
                                                   const OutT* residual, OutT* C, int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);
  const int mtiles = (M + Cfg::BM - 1) / Cfg::BM;
  int mt, nt;
  xcd_tile_map(blockIdx.x, gridDim.x, mtiles, mt, nt);
  const int m0 = mt * Cfg::BM, n0 = nt * Cfg::BN;
  f32x16 acc[Cfg::TM][Cfg::TN];
  gemm_mainloop<T, Cfg>(A, W, M, N, K, m0, n0, lds, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hh = lane >> 5, r = lane & 31;
  const int wm = w / Cfg::WN, wn = w % Cfg::WN;
  if constexpr (EPI == ORTHRUS_EPI_SWIGLU) {
    // columns come in (gate 32, up 32) pairs: tile j even = gate block, j+1 = its up block
    const int NO = N / 2;
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::TN; j += 2) {
        const int ng = n0 + (wn * Cfg::TN + j) * 32;  // multiple of 64
        const int col = ng / 2 + r;
        if (ng >= N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + (wm * Cfg::TM + i) * 32 + acc_row(e, hh);
          if (m < M) {
            const float g = acc[i][j][e], u = acc[i][j + 1][e];
            const float s = g / (1.0f + expf(-g));
            C[(size_t)m * NO + col] = from_f32<OutT>(s * u);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j) {
        const int n = n0 + (wn * Cfg::TN + j) * 32 + r;
        if (n >= N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + (wm * Cfg::TM + i) * 32 + acc_row(e, hh);
          if (m < M) {
            float v = acc[i][j][e];
            if constexpr (EPI == ORTHRUS_EPI_RESIDUAL) v = to_f32(residual[(size_t)m * N + n]) + v;
            C[(size_t)m * N + n] = from_f32<OutT>(v);
          }
        }
      }
  }
}

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
      hipLaunchKernelGGL((gemm_kernel<T, OutT, Cfg, ORTHRUS_EPI_STORE>), grid, dim3(256), lds, st, A, Wt, R, C, M, N, K);
      break;
    case ORTHRUS_EPI_RESIDUAL:
      hipLaunchKernelGGL((gemm_kernel<T, OutT, Cfg, ORTHRUS_EPI_RESIDUAL>), grid, dim3(256), lds, st, A, Wt, R, C, M, N, K);
      break;
    default:
      hipLaunchKernelGGL((gemm_kernel<T, OutT, Cfg, ORTHRUS_EPI_SWIGLU>), grid, dim3(256), lds, st, A, Wt, R, C, M, N, K);
      break;
  }
  return check_launch("orthrus_gemm");
}

template <typename T, typename OutT>
int32_t launch(int M, int N, int K, int epi, const void* a, const void* w, const void* res, void* c, hipStream_t st) {
  // Tile choice depends only on (M, N); the k order is the same for all of them.
  if (M <= 32 && epi != ORTHRUS_EPI_SWIGLU) return launch_cfg<T, OutT, GemmCfg<T, 32, 128, 1, 4>>(M, N, K, epi, a, w, res, c, st);
  if (M <= 64) return launch_cfg<T, OutT, GemmCfg<T, 64, 128, 2, 2>>(M, N, K, epi, a, w, res, c, st);
  return launch_cfg<T, OutT, GemmCfg<T, 128, 128, 2, 2>>(M, N, K, epi, a, w, res, c, st);
}

template <typename T>
__global__ void pack_gate_up_kernel(const T* g, const T* u, T* p, int inter, int hidden) {
  const int row = blockIdx.x;  // 0 .. 2*inter-1 of the packed matrix
  const int grp = row / 64, within = row % 64;
  const T* src = (within < 32 ? g : u) + (size_t)(grp * 32 + (within & 31)) * hidden;
  T* dst = p + (size_t)row * hidden;
  for (int i = threadIdx.x; i < hidden; i += blockDim.x) dst[i] = src[i];
}

}  // namespace
}  // namespace orthrus

using namespace orthrus;

extern "C" int32_t orthrus_gemm(int32_t M, int32_t N, int32_t K, int32_t dtype, int32_t out_dtype, int32_t epilogue,
                                const void* a, const void* w, const void* residual, void* c, void* stream) {
  ORTHRUS_REQUIRE(M >= 0 && N > 0 && K > 0, ORTHRUS_ERR_INVALID_ARG, "gemm: bad sizes M=%d N=%d K=%d", M, N, K);
  ORTHRUS_REQUIRE(K % 64 == 0, ORTHRUS_ERR_UNSUPPORTED, "gemm: K=%d not a multiple of 64", K);
  ORTHRUS_REQUIRE(valid_dtype(dtype) && valid_dtype(out_dtype), ORTHRUS_ERR_INVALID_ARG, "gemm: bad dtype");
  ORTHRUS_REQUIRE(epilogue >= 0 && epilogue <= 2, ORTHRUS_ERR_INVALID_ARG, "gemm: bad epilogue %d", epilogue);
  ORTHRUS_REQUIRE(epilogue != ORTHRUS_EPI_SWIGLU || N % 64 == 0, ORTHRUS_ERR_INVALID_ARG,
                  "gemm: SwiGLU needs N %% 64 == 0 (got %d)", N);
  ORTHRUS_REQUIRE(a && w && c, ORTHRUS_ERR_INVALID_ARG, "gemm: null pointer");
  ORTHRUS_REQUIRE(epilogue != ORTHRUS_EPI_RESIDUAL || residual, ORTHRUS_ERR_INVALID_ARG, "gemm: residual is null");
  ORTHRUS_REQUIRE(!(dtype == ORTHRUS_F32 && out_dtype == ORTHRUS_BF16), ORTHRUS_ERR_UNSUPPORTED,
                  "gemm: fp32 inputs with bf16 output not built");
  if (M == 0) return ORTHRUS_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == ORTHRUS_BF16) {
    if (out_dtype == ORTHRUS_BF16) return launch<bf16, bf16>(M, N, K, epilogue, a, w, residual, c, st);
    return launch<bf16, float>(M, N, K, epilogue, a, w, residual, c, st);
  }
  return launch<float, float>(M, N, K, epilogue, a, w, residual, c, st);
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
