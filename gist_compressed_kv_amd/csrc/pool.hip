// Gist pool: caller-owned storage [L][N][2][H][k][d] holding, per item and
// layer, the k gist positions' K and V.  This is the stored object G of
// liam.page "把 item 压成 KV：gist 能不能用在相关性任务上", sections
// 论文做了什么 and 在线的一次 attention: 2·L·k·H·h elements per item, K
// kept rotated at the canonical positions 1..k.  An fp8 pool stores the same
// array as OCP E4M3 codes followed by one fp32 scale per (layer, item, K or
// V, head), [L][N][2][H].
#include <cstdlib>
#include <cstring>
#include <new>

#include "common.hpp"

namespace gist {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
gist_status fail(gist_status code, const std::string& msg) {
  g_last_error = msg;
  return code;
}
gist_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(GIST_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return GIST_OK;
}

// One thread per (item i, gist row j, head g, channel chunk c): chunk c holds
// channels [4c, 4c+4) and its RoPE partners [d/2 + 4c, d/2 + 4c + 4).
template <typename T>
__global__ void __launch_bounds__(256)
pool_write_kernel(T* __restrict__ pool, int64_t layer_off, int64_t N, int k, int H, int d,
                  const int32_t* __restrict__ ids, int64_t n, const T* __restrict__ ksrc,
                  const T* __restrict__ vsrc, int src_pos0, RopeFreqs freqs) {
  const int chunks = d / 8;  // chunk pairs per row
  const int64_t total = n * (int64_t)k * H * chunks;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= total) return;
  const int c = (int)(u % chunks);
  int64_t rest = u / chunks;
  const int g = (int)(rest % H);
  rest /= H;
  const int j = (int)(rest % k);
  const int64_t i = rest / k;
  const int32_t item = ids[i];
  if (item < 0 || item >= N) return;  // out-of-range destination: skipped

  const int64_t src = ((i * k + j) * H + g) * (int64_t)d;
  T* rec = pool + layer_off + (int64_t)item * 2 * H * k * d;
  const int64_t kdst = ((int64_t)g * k + j) * d;
  const int64_t vdst = ((int64_t)(H + g) * k + j) * d;
  const int half = d / 2;
  const double shift = 1.0 - (double)src_pos0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int lo = 4 * c + e, hi = half + 4 * c + e;
    float xl, xh;
    if constexpr (sizeof(T) == 2) {
      xl = bf16_bits_to_f32(ksrc[src + lo]);
      xh = bf16_bits_to_f32(ksrc[src + hi]);
    } else {
      xl = ksrc[src + lo];
      xh = ksrc[src + hi];
    }
    float cs = 1.f, sn = 0.f;
    if (src_pos0 != 1) rope_cos_sin(shift, freqs.rev[lo], cs, sn);
    const float yl = __builtin_fmaf(xl, cs, -(xh * sn));
    const float yh = __builtin_fmaf(xh, cs, xl * sn);
    if constexpr (sizeof(T) == 2) {
      const uint32_t p = pack2_bf16(yl, yh);
      rec[kdst + lo] = (T)(p & 0xffffu);
      rec[kdst + hi] = (T)(p >> 16);
      rec[vdst + lo] = vsrc[src + lo];
      rec[vdst + hi] = vsrc[src + hi];
    } else {
      rec[kdst + lo] = yl;
      rec[kdst + hi] = yh;
      rec[vdst + lo] = vsrc[src + lo];
      rec[vdst + hi] = vsrc[src + hi];
    }
  }
}

// Nearest OCP E4M3 code of y (ties to even mantissa), |y| clamped to 448,
// the largest finite value; the sign bit is kept, so -0 and small negative
// values that round to zero give 0x80.  y must not be NaN.
__device__ __forceinline__ uint32_t encode_e4m3(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    // below the smallest normal 2^-6 the values are m * 2^-9, m = 0..7; m = 8
    // is the smallest normal, whose code is 8 as well
    code = (uint32_t)rintf(a * 512.f);
  } else {
    const uint32_t b = __float_as_uint(a);
    const uint32_t e = (b >> 23) - 120u;  // exponent with bias 7 (1..15)
    const uint32_t m = b & 0x7fffffu;
    const uint32_t rem = m & 0xfffffu;    // the 20 mantissa bits dropped
    uint32_t m3 = m >> 20;
    m3 += (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ? 1u : 0u;
    code = (e << 3) + m3;  // a mantissa carry moves into the exponent
  }
  return sign | code;
}

// fp8 pool writer: one wave per (item i, K or V, head g) block of k*d values.
// The lane's units are (row j, chunk c): channels 4c..4c+3 and their RoPE
// partners d/2 + 4c..+3.  Pass 1 forms the values (K re-rotated in fp32) and
// their absolute maximum; pass 2 forms them again, divides by the block's
// scale and stores the codes, four per dword.
__global__ void __launch_bounds__(256)
pool_write_fp8_kernel(uint8_t* __restrict__ codes, float* __restrict__ scales, int64_t N, int k,
                      int H, int d, const int32_t* __restrict__ ids, int64_t n,
                      const bf16_t* __restrict__ ksrc, const bf16_t* __restrict__ vsrc,
                      int src_pos0, RopeFreqs freqs) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= n * 2 * H) return;
  const int g = (int)(w % H);
  const int kv = (int)((w / H) % 2);
  const int64_t i = w / (2 * H);
  const int32_t item = ids[i];
  if (item < 0 || item >= N) return;  // out-of-range destination: skipped
  const bf16_t* src = kv ? vsrc : ksrc;
  const bool rotate = kv == 0 && src_pos0 != 1;
  const int chunks = d / 8, half = d / 2;
  const int units = k * chunks;
  const double shift = 1.0 - (double)src_pos0;

  auto values = [&](int u, float* yl, float* yh) {
    const int j = u / chunks, c = u - (u / chunks) * chunks;
    const bf16_t* row = src + ((i * k + j) * H + g) * (int64_t)d;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int lo = 4 * c + e;
      const float xl = bf16_bits_to_f32(row[lo]), xh = bf16_bits_to_f32(row[half + lo]);
      if (rotate) {
        float cs, sn;
        rope_cos_sin(shift, freqs.rev[lo], cs, sn);
        yl[e] = __builtin_fmaf(xl, cs, -(xh * sn));
        yh[e] = __builtin_fmaf(xh, cs, xl * sn);
      } else {
        yl[e] = xl;
        yh[e] = xh;
      }
    }
  };

  float amax = 0.f;
  for (int u = lane; u < units; u += 64) {
    float yl[4], yh[4];
    values(u, yl, yh);
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(yl[e]), fabsf(yh[e])));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  // correctly rounded fp32 division (HIP's default for '/')
  const float scale = amax > 0.f ? amax / 448.f : 1.f;

  uint8_t* blk = codes + ((int64_t)item * 2 * H + (int64_t)kv * H + g) * k * d;
  for (int u = lane; u < units; u += 64) {
    float yl[4], yh[4];
    values(u, yl, yh);
    uint32_t pl = 0, ph = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pl |= encode_e4m3(yl[e] / scale) << (8 * e);
      ph |= encode_e4m3(yh[e] / scale) << (8 * e);
    }
    const int j = u / chunks, c = u - (u / chunks) * chunks;
    *(uint32_t*)(blk + j * d + 4 * c) = pl;
    *(uint32_t*)(blk + j * d + half + 4 * c) = ph;
  }
  if (lane == 0) scales[((int64_t)item * 2 + kv) * H + g] = scale;
}

}  // namespace gist

using namespace gist;

extern "C" size_t gist_pool_bytes(int L, int64_t N, int k, int H, int d, gist_dtype dtype) {
  if (L <= 0 || N <= 0 || k <= 0 || H <= 0 || d <= 0) return 0;
  if (dtype != GIST_BF16 && dtype != GIST_F32 && dtype != GIST_FP8_E4M3) return 0;
  if (dtype == GIST_FP8_E4M3)
    return (size_t)N * (size_t)L * (2 * (size_t)k * H * d + 2 * (size_t)H * sizeof(float));
  return (size_t)N * 2 * (size_t)L * k * H * d * elem_size(dtype);
}

extern "C" gist_status gist_pool_create(gist_pool** out, int L, int64_t N, int k, int H, int d,
                                        gist_dtype dtype, void* storage, size_t storage_bytes) {
  clear_error();
  if (!out) return fail(GIST_ERR_INVALID_ARG, "gist_pool_create: out is NULL");
  *out = nullptr;
  if (dtype != GIST_BF16 && dtype != GIST_F32 && dtype != GIST_FP8_E4M3)
    return fail(GIST_ERR_INVALID_ARG, "gist_pool_create: unknown dtype");
  if (L <= 0 || N <= 0 || k <= 0 || H <= 0 || d <= 0)
    return fail(GIST_ERR_INVALID_ARG, "gist_pool_create: L, N, k, H, d must be positive");
  if (d != 64 && d != 128)
    return fail(GIST_ERR_UNSUPPORTED, "gist_pool_create: head_dim must be 64 or 128");
  if (k > 64) return fail(GIST_ERR_UNSUPPORTED, "gist_pool_create: k must be <= 64");
  if (N > INT32_MAX) return fail(GIST_ERR_UNSUPPORTED, "gist_pool_create: N must fit int32 ids");
  if (!storage) return fail(GIST_ERR_INVALID_ARG, "gist_pool_create: storage is NULL");
  if (((uintptr_t)storage) % 16 != 0)
    return fail(GIST_ERR_INVALID_ARG, "gist_pool_create: storage must be 16-byte aligned");
  const size_t need = gist_pool_bytes(L, N, k, H, d, dtype);
  if (storage_bytes != need)
    return fail(GIST_ERR_INVALID_ARG, "gist_pool_create: storage_bytes " +
                                          std::to_string(storage_bytes) + " != required " +
                                          std::to_string(need));
  gist_pool* p = new (std::nothrow) gist_pool;
  if (!p) return fail(GIST_ERR_INVALID_ARG, "gist_pool_create: out of host memory");
  p->L = L;
  p->N = N;
  p->k = k;
  p->H = H;
  p->d = d;
  p->dtype = dtype;
  p->storage = storage;
  p->bytes = storage_bytes;
  *out = p;
  return GIST_OK;
}

extern "C" gist_status gist_pool_destroy(gist_pool* pool) {
  clear_error();
  delete pool;
  return GIST_OK;
}

extern "C" gist_status gist_pool_write(const gist_pool* pool, int layer, const int32_t* ids,
                                       int64_t n, const void* k_src, const void* v_src,
                                       int src_pos0, float rope_base, void* stream) {
  clear_error();
  if (!pool) return fail(GIST_ERR_INVALID_ARG, "gist_pool_write: pool is NULL");
  if (layer < 0 || layer >= pool->L)
    return fail(GIST_ERR_OUT_OF_RANGE, "gist_pool_write: layer out of range");
  if (n < 0) return fail(GIST_ERR_INVALID_ARG, "gist_pool_write: n < 0");
  if (n == 0) return GIST_OK;
  if (!ids || !k_src || !v_src)
    return fail(GIST_ERR_INVALID_ARG, "gist_pool_write: NULL ids/k_src/v_src");
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return fail(GIST_ERR_INVALID_ARG, "gist_pool_write: rope_base must be positive");
  RopeFreqs f;
  make_rope_freqs(f, pool->d, rope_base);
  const int64_t layer_off = (int64_t)layer * pool->N * record_elems(pool);
  const int64_t total = n * (int64_t)pool->k * pool->H * (pool->d / 8);
  const int64_t blocks = (total + 255) / 256;
  if (blocks > INT32_MAX) return fail(GIST_ERR_UNSUPPORTED, "gist_pool_write: n too large");
  hipStream_t s = (hipStream_t)stream;
  if (pool->dtype == GIST_FP8_E4M3) {
    const int64_t waves = n * 2 * pool->H;
    if ((waves + 3) / 4 > INT32_MAX)
      return fail(GIST_ERR_UNSUPPORTED, "gist_pool_write: n too large");
    uint8_t* codes = (uint8_t*)pool->storage + layer_off;
    float* scales = (float*)fp8_layer_scales(pool, layer);
    hipLaunchKernelGGL(pool_write_fp8_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s,
                       codes, scales, pool->N, pool->k, pool->H, pool->d, ids, n,
                       (const bf16_t*)k_src, (const bf16_t*)v_src, src_pos0, f);
    return check_launch("gist_pool_write(fp8)");
  }
  if (pool->dtype == GIST_BF16)
    hipLaunchKernelGGL(pool_write_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       (bf16_t*)pool->storage, layer_off, pool->N, pool->k, pool->H, pool->d, ids,
                       n, (const bf16_t*)k_src, (const bf16_t*)v_src, src_pos0, f);
  else
    hipLaunchKernelGGL(pool_write_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s,
                       (float*)pool->storage, layer_off, pool->N, pool->k, pool->H, pool->d, ids,
                       n, (const float*)k_src, (const float*)v_src, src_pos0, f);
  return check_launch("gist_pool_write");
}

extern "C" const char* gist_last_error(void) { return g_last_error.c_str(); }
