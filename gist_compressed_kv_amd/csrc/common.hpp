// Shared device/host helpers of libgist_attn.so (HIP, gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>

#include "../../include/gist_attn.h"

namespace gist {

// ---------------------------------------------------------------------------
// Error state (thread-local message behind gist_last_error)
// ---------------------------------------------------------------------------
void set_error(const std::string& msg);
void clear_error();
gist_status fail(gist_status code, const std::string& msg);
gist_status check_launch(const char* what);

// ---------------------------------------------------------------------------
// Element types
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;  // bfloat16 bits in memory

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Unpack 8 bf16 held in a uint4 into floats.
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  f[0] = __uint_as_float(u.x << 16);
  f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16);
  f[3] = __uint_as_float(u.y & 0xffff0000u);
  f[4] = __uint_as_float(u.z << 16);
  f[5] = __uint_as_float(u.z & 0xffff0000u);
  f[6] = __uint_as_float(u.w << 16);
  f[7] = __uint_as_float(u.w & 0xffff0000u);
}

// Round two floats to bf16 (nearest-even, hardware v_cvt_pk_bf16_f32) and
// pack them low-first into one dword.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint4 pack8_bf16(const float* f) {
  return make_uint4(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]), pack2_bf16(f[4], f[5]),
                    pack2_bf16(f[6], f[7]));
}

// Four OCP FP8 E4M3 codes (one dword, lowest byte first) to floats.  gfx950's
// v_cvt_pk_f32_fp8 decodes exactly this format (bias 7, subnormals, 0x7F and
// 0xFF NaN).
// Two E4M3 codes (bytes 0-1 of w, or 2-3 with HI) as two bf16 values packed
// low first: gfx950's scaled conversion at scale 1, exact since every E4M3
// value is a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ void decode4_e4m3(uint32_t w, float* f) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo.x;
  f[1] = lo.y;
  f[2] = hi.x;
  f[3] = hi.y;
}

// ---------------------------------------------------------------------------
// RoPE angles.  The host computes theta_i / (2*pi) = base^(-2i/d) / (2*pi)
// (revolutions per position) in double.  The device forms pos * rev in double,
// keeps the fractional revolution (exact in double, |f| <= 1/2) and feeds it
// to the hardware v_sin_f32 / v_cos_f32, whose argument is in revolutions.
// The fp64 reduction keeps the angle exact for positions in the thousands;
// the hardware sine/cosine contribute an absolute error of a few 1e-7.
// ---------------------------------------------------------------------------
constexpr int kMaxHalfDim = 64;  // d <= 128

struct RopeFreqs {
  double rev[kMaxHalfDim];  // revolutions per position of channel pair i
};

inline void make_rope_freqs(RopeFreqs& f, int d, float base) {
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < kMaxHalfDim; ++i)
    f.rev[i] = (i < d / 2) ? std::pow((double)base, -2.0 * (double)i / (double)d) / two_pi : 0.0;
}

__device__ __forceinline__ void rope_cos_sin(double pos, double rev, float& c, float& s) {
  const double r = pos * rev;
  const float f = (float)(r - rint(r));
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

// ---------------------------------------------------------------------------
// LDS layout of row-major key rows (one row per key, D channels) whose V is
// read back as MFMA A fragments with the LDS transpose read
// (ds_read_b64_tr_b16).  One such read covers rows R0..R0+3 (R0 a multiple
// of 4) and the same 8-byte half of four 16-byte chunks per pass.  With a row
// stride of D + 4 elements (8 bytes of padding) and the chunks of row R
// rotated by 3*((R >> 1) & 1), those 16 pieces land on 32 distinct banks, as
// do the 16-byte row writes of the staging.
// ---------------------------------------------------------------------------
__device__ __forceinline__ constexpr int vrow_off(int R, int ch, int D) {
  return R * (D + 4) + ((((ch >> 3) + 3 * ((R >> 1) & 1)) & (D / 8 - 1)) << 3) + (ch & 7);
}

// Row of the Vᵀ tile that MFMA row r of d-tile dt stands for (16x16 tiles,
// sixteen channels per d-tile).  The mapping is chosen so that after the P·V
// product each lane holds, for every 32-channel step s, the eight consecutive
// channels 32s + 8*(lane/16) .. +8 of its token: the same layout the Q loads
// use, so output stores are 16-byte vectors.  A transpose read from
// vrow_off rows yields this mapping when the lane supplying a piece reads
// channels 32*(dt >> 1) + 4*(dt & 1) + 8*(lane & 3) .. +3.
__device__ __forceinline__ constexpr int vt_row(int dt, int r) {
  return 32 * (dt >> 1) + 8 * (r >> 2) + 4 * (dt & 1) + (r & 3);
}

// ---------------------------------------------------------------------------
// Host-side pool handle
// ---------------------------------------------------------------------------
}  // namespace gist

struct gist_pool {
  int L;
  int64_t N;
  int k;
  int H;
  int d;
  gist_dtype dtype;
  void* storage;
  size_t bytes;
};

namespace gist {
inline size_t elem_size(gist_dtype t) { return t == GIST_F32 ? 4 : (t == GIST_BF16 ? 2 : 1); }
// elements of one (layer, item) record: [2][H][k][d]
inline int64_t record_elems(const gist_pool* p) { return 2LL * p->H * p->k * p->d; }
// fp8 pools: byte offset of the scale array [L][N][2][H] behind the codes
inline int64_t fp8_scales_offset(const gist_pool* p) {
  return (int64_t)p->L * p->N * record_elems(p);
}
// fp8 pools: the scales of one layer, [N][2][H]
inline const float* fp8_layer_scales(const gist_pool* p, int layer) {
  return (const float*)((const char*)p->storage + fp8_scales_offset(p)) +
         (int64_t)layer * p->N * 2 * p->H;
}
}  // namespace gist
