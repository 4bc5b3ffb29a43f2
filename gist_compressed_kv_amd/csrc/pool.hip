// Gist pool: caller-owned storage [L][N][2][H][k][d] holding, per item and
// layer, the k gist positions' K and V.  This is the stored object G of
// liam.page "把 item 压成 KV：gist 能不能用在相关性任务上", sections
// 论文做了什么 and 在线的一次 attention: 2·L·k·H·h elements per item, K
// kept rotated at the canonical positions 1..k.
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
  const double shift = (double)(1 - src_pos0);
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

}  // namespace gist

using namespace gist;

extern "C" size_t gist_pool_bytes(int L, int64_t N, int k, int H, int d, gist_dtype dtype) {
  if (L <= 0 || N <= 0 || k <= 0 || H <= 0 || d <= 0) return 0;
  if (dtype != GIST_BF16 && dtype != GIST_F32) return 0;
  return (size_t)N * 2 * (size_t)L * k * H * d * elem_size(dtype);
}

extern "C" gist_status gist_pool_create(gist_pool** out, int L, int64_t N, int k, int H, int d,
                                        gist_dtype dtype, void* storage, size_t storage_bytes) {
  clear_error();
  if (!out) return fail(GIST_ERR_INVALID_ARG, "gist_pool_create: out is NULL");
  *out = nullptr;
  if (dtype != GIST_BF16 && dtype != GIST_F32)
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
