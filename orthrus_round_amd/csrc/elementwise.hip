// Row-wise support kernels of the decoder layers: block embedding, RMSNorm, the RoPE table and
// the fused QKV split + RoPE + K/V write (paged cache for the AR view, block buffer for the
// diffusion view).
#include "common.hpp"

namespace orthrus {
namespace {

// ---------------------------------------------------------------------------------------- embed
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* __restrict__ embed, const int32_t* anchor,
                                                    const int32_t* tokens, int tok_stride, int tok_offset, int block,
                                                    int hidden, int mask_id, int vocab_guard, T* __restrict__ x) {
  const int m = blockIdx.x, b = m / block, s = m % block;
  int tok;
  if (anchor && s == 0) tok = anchor[b];
  else if (tokens) tok = tokens[(size_t)b * tok_stride + tok_offset + s - (anchor ? 1 : 0)];
  else tok = mask_id;
  if (tok < 0 || tok >= vocab_guard) tok = mask_id;  // out-of-range ids embed as [MASK]
  const T* src = embed + (size_t)tok * hidden;
  T* dst = x + (size_t)m * hidden;
  constexpr int EPC = 16 / sizeof(T);
  for (int i = threadIdx.x; i < hidden / EPC; i += 256)
    reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
}

// -------------------------------------------------------------------------------------- rmsnorm
// One workgroup per row.  Rows whose length is a multiple of 16 bytes and at most
// kNormMaxChunks 16-byte chunks take the register path: thread c owns chunk c (one 16-byte load,
// issued with every other load of the row at once), and the sum of squares is reduced in a fixed
// order: per thread in element order, a wave butterfly, then the waves in order.  The workgroup
// has one thread per chunk, rounded up to whole waves.  Other rows take a strided loop.
template <typename T>
__global__ __launch_bounds__(kNormMaxChunks) void rmsnorm_kernel(const T* __restrict__ x, const float* __restrict__ g,
                                                                 float eps, int hidden, T* __restrict__ y,
                                                                 int aligned16) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  __shared__ float red[kNormMaxChunks / 64];
  const int m = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const T* xr = x + (size_t)m * hidden;
  T* yr = y + (size_t)m * hidden;
  const int nch = hidden / EPC;
  const bool vec = aligned16 && hidden % EPC == 0 && nch <= nt;
  float ss = 0.0f;
  u32x4_t buf = {0, 0, 0, 0};
  if (vec) {
    if (tid < nch) {
      buf = *reinterpret_cast<const u32x4_t*>(xr + (size_t)tid * EPC);
      const T* e = reinterpret_cast<const T*>(&buf);
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        const float v = to_f32(e[i]);
        ss += v * v;
      }
    }
  } else {
    for (int i = tid; i < hidden; i += nt) {
      const float v = to_f32(xr[i]);
      ss += v * v;
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
  for (int w = 0; w < nt / 64; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)hidden + eps);
  if (vec) {
    if (tid < nch) {
      const T* e = reinterpret_cast<const T*>(&buf);
      u32x4_t o;
      T* oe = reinterpret_cast<T*>(&o);
#pragma unroll
      for (int i = 0; i < EPC; ++i) oe[i] = from_f32<T>(to_f32(e[i]) * inv * g[(size_t)tid * EPC + i]);
      *reinterpret_cast<u32x4_t*>(yr + (size_t)tid * EPC) = o;
    }
  } else {
    for (int i = tid; i < hidden; i += nt) yr[i] = from_f32<T>(to_f32(xr[i]) * inv * g[i]);
  }
}

// ----------------------------------------------------------------------------------------- rope
__global__ void rope_table_kernel(int max_pos, int half, double log_base, int head_dim, float* table) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)max_pos * half) return;
  const int pos = (int)(idx / half), i = (int)(idx % half);
  const double inv_freq = exp(-(2.0 * i / head_dim) * log_base);
  const double ang = (double)pos * inv_freq;
  table[idx * 2] = (float)cos(ang);
  table[idx * 2 + 1] = (float)sin(ang);
}

template <typename T>
__global__ __launch_bounds__(256) void rope_kv_kernel(const T* __restrict__ qkv, const float* __restrict__ table,
                                                      int max_pos, const int32_t* __restrict__ ctx_len,
                                                      const int32_t* __restrict__ page_table, int block, int Hq,
                                                      int Hkv, int D, int page, int max_pages, T* __restrict__ q_out,
                                                      T* __restrict__ k_dst, T* __restrict__ v_dst) {
  const int m = blockIdx.x, b = m / block, s = m % block;
  const int pos = ctx_len[b] + s;
  const int half = D / 2;
  const int width = (Hq + 2 * Hkv) * D;
  const T* row = qkv + (size_t)m * width;
  const bool pos_ok = pos >= 0 && pos < max_pos;
  size_t kv_base = 0;  // element offset of (kv head 0, d 0) for this row's key slot
  bool kv_ok = pos_ok;
  if (page_table) {
    kv_ok = kv_ok && pos < max_pages * page;
    if (kv_ok) {
      const int pg = page_table[(size_t)b * max_pages + pos / page];
      kv_base = ((size_t)pg * Hkv * page + (pos % page)) * D;  // + hk * page * D
    }
  } else {
    kv_base = (size_t)m * Hkv * D;  // + hk * D
  }
  const size_t kv_head_stride = page_table ? (size_t)page * D : (size_t)D;
  const float* cs = table + (size_t)(pos_ok ? pos : 0) * half * 2;
  // rotations of q heads and k heads: (Hq + Hkv) * half pairs
  const int nrot = (Hq + Hkv) * half;
  for (int t = threadIdx.x; t < nrot; t += 256) {
    const int hd = t / half, i = t % half;
    const float c = cs[2 * i], sn = cs[2 * i + 1];
    const float x1 = to_f32(row[hd * D + i]), x2 = to_f32(row[hd * D + i + half]);
    const float y1 = pos_ok ? x1 * c - x2 * sn : __builtin_nanf("");
    const float y2 = pos_ok ? x2 * c + x1 * sn : __builtin_nanf("");
    if (hd < Hq) {
      T* qo = q_out + (size_t)m * Hq * D + hd * D;
      qo[i] = from_f32<T>(y1);
      qo[i + half] = from_f32<T>(y2);
    } else if (kv_ok) {
      const int hk = hd - Hq;
      T* ko = k_dst + kv_base + hk * kv_head_stride;
      ko[i] = from_f32<T>(y1);
      ko[i + half] = from_f32<T>(y2);
    }
  }
  if (kv_ok) {
    const T* vsrc = row + (Hq + Hkv) * D;
    for (int t = threadIdx.x; t < Hkv * D; t += 256) {
      const int hk = t / D, d = t % D;
      v_dst[kv_base + hk * kv_head_stride + d] = vsrc[t];
    }
  }
}

}  // namespace
}  // namespace orthrus

using namespace orthrus;

extern "C" int32_t orthrus_embed_block(int32_t batch, int32_t block, int32_t hidden, int32_t dtype, const void* embed,
                                       const int32_t* anchor, const int32_t* tokens, int32_t tok_stride,
                                       int32_t tok_offset, int32_t mask_id, void* x, void* stream) {
  ORTHRUS_REQUIRE(batch >= 0 && block >= 1 && hidden > 0, ORTHRUS_ERR_INVALID_ARG, "embed: bad sizes");
  ORTHRUS_REQUIRE(valid_dtype(dtype) && embed && x, ORTHRUS_ERR_INVALID_ARG, "embed: bad args");
  ORTHRUS_REQUIRE(hidden % (16 / (int)dtype_size(dtype)) == 0, ORTHRUS_ERR_UNSUPPORTED, "embed: hidden alignment");
  ORTHRUS_REQUIRE(mask_id >= 0, ORTHRUS_ERR_INVALID_ARG, "embed: mask_id must be a valid id");
  if (batch == 0) return ORTHRUS_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int guard = mask_id + 1;  // ids above the reserved last id are invalid
  if (dtype == ORTHRUS_BF16)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(batch * block), dim3(256), 0, st, (const bf16*)embed, anchor, tokens,
                       tok_stride, tok_offset, block, hidden, mask_id, guard, (bf16*)x);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(batch * block), dim3(256), 0, st, (const float*)embed, anchor, tokens,
                       tok_stride, tok_offset, block, hidden, mask_id, guard, (float*)x);
  return check_launch("orthrus_embed_block");
}

extern "C" int32_t orthrus_rmsnorm(int32_t rows, int32_t hidden, int32_t dtype, const void* x, const float* gain,
                                   float eps, void* y, void* stream) {
  ORTHRUS_REQUIRE(rows >= 0 && hidden > 0 && valid_dtype(dtype) && x && gain && y, ORTHRUS_ERR_INVALID_ARG,
                  "rmsnorm: bad args");
  if (rows == 0) return ORTHRUS_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int aligned16 = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15) == 0;
  const int nt = norm_threads(hidden, dtype_size(dtype));
  if (dtype == ORTHRUS_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16>, dim3(rows), dim3(nt), 0, st, (const bf16*)x, gain, eps, hidden, (bf16*)y,
                       aligned16);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(rows), dim3(nt), 0, st, (const float*)x, gain, eps, hidden,
                       (float*)y, aligned16);
  return check_launch("orthrus_rmsnorm");
}

extern "C" int32_t orthrus_rope_table(int32_t max_pos, int32_t head_dim, double base, float* table, void* stream) {
  ORTHRUS_REQUIRE(max_pos > 0 && head_dim > 0 && head_dim % 2 == 0 && base > 1.0 && table, ORTHRUS_ERR_INVALID_ARG,
                  "rope_table: bad args");
  const size_t n = (size_t)max_pos * (head_dim / 2);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, max_pos, head_dim / 2,
                     std::log(base), head_dim, table);
  return check_launch("orthrus_rope_table");
}

extern "C" int32_t orthrus_rope_kv_write(int32_t batch, int32_t block, int32_t q_heads, int32_t kv_heads,
                                         int32_t head_dim, int32_t page_size, int32_t max_pages, int32_t dtype,
                                         const void* qkv, const float* rope_table, int32_t max_pos,
                                         const int32_t* ctx_len, const int32_t* page_table, void* q_out, void* k_dst,
                                         void* v_dst, void* stream) {
  ORTHRUS_REQUIRE(batch >= 0 && block >= 1 && q_heads > 0 && kv_heads > 0 && head_dim > 0 && head_dim % 2 == 0,
                  ORTHRUS_ERR_INVALID_ARG, "rope_kv_write: bad sizes");
  ORTHRUS_REQUIRE(valid_dtype(dtype) && qkv && rope_table && ctx_len && q_out && k_dst && v_dst && max_pos > 0,
                  ORTHRUS_ERR_INVALID_ARG, "rope_kv_write: bad args");
  ORTHRUS_REQUIRE(!page_table || (page_size > 0 && max_pages > 0), ORTHRUS_ERR_INVALID_ARG, "rope_kv_write: paging");
  if (batch == 0) return ORTHRUS_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == ORTHRUS_BF16)
    hipLaunchKernelGGL(rope_kv_kernel<bf16>, dim3(batch * block), dim3(256), 0, st, (const bf16*)qkv, rope_table,
                       max_pos, ctx_len, page_table, block, q_heads, kv_heads, head_dim, page_size, max_pages,
                       (bf16*)q_out, (bf16*)k_dst, (bf16*)v_dst);
  else
    hipLaunchKernelGGL(rope_kv_kernel<float>, dim3(batch * block), dim3(256), 0, st, (const float*)qkv, rope_table,
                       max_pos, ctx_len, page_table, block, q_heads, kv_heads, head_dim, page_size, max_pages,
                       (float*)q_out, (float*)k_dst, (float*)v_dst);
  return check_launch("orthrus_rope_kv_write");
}
