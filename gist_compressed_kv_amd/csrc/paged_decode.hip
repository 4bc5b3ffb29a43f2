// paged_decode_attn: one decode step of R requests over a KV cache kept in
// fixed-size blocks scattered through a physical block pool.
//
// What is computed (mcfzz.com "为什么自回归推理缓存 KV，而不缓存历史 Q？",
// Reusable-state): the new token's rotated query attends, with softmax scale
// `scale`, over [the cached keys in logical order ; its own rotated key], and
// returns the matching weighted sum of [cached values ; its own value].  The
// logical -> physical block indirection is the block table of icman.com.cn
// news 64898 (section 6, problem 4; 256-token blocks in section 5).
//
// Two kernels (split-K, flash-decoding style):
//  * decode_split<T, D, MAXG>: one workgroup (4 wave64s) per (request, KV
//    head, 256-key split).  Each 16-lane row of a wave streams 16 consecutive
//    keys of one block (a row is 16 lanes x d/16 channels = one full K or V
//    row, so every load instruction reads whole contiguous rows), keeps an
//    online-softmax state (max, sum, weighted V) per query head of the GQA
//    group, and the states of the 16 rows of the workgroup are merged with
//    cross-lane shuffles and LDS.  The split's (o, m, l) goes to the fp32
//    workspace.
//  * decode_combine<T, D>: one wave64 per (request, query head) merges the
//    split states with the token's own key/value (log-sum-exp weights) and
//    writes the normalized output.
#include <type_traits>
#include <utility>

#include <mutex>
#include <string>

#include "common.hpp"

namespace gist {

constexpr int kSplitKeys = 256;  // keys per workgroup of the split kernel
constexpr int kWsPad = 4;        // workspace row = d channels + (m, l, 2 pad)
// A row's reference maximum moves only when a logit passes it by more than
// this many log2 units (weights up to 2^8 between moves).
constexpr float kLazyMax = 8.f;

struct DecodeArgs {
  const void* kc;
  const void* vc;
  int64_t nblk;
  int bs;
  const int32_t* table;
  int max_blk;
  const int32_t* ctx;
  int R;
  const void* q;
  const void* kn;
  const void* vn;
  const int32_t* positions;
  int Hq, H, G;
  float scale_log2;
  float* ws;
  int nsplit;
  void* out;
  // fp8 cache only: one fp32 scale per (physical block, KV head), [nblk][H]
  const float* ksc;
  const float* vsc;
  RopeFreqs freqs;
  // q^(2^b), b = 0..5, with q = base^(-2/d): rev_i = rev_0 * prod over the
  // set bits b of i (a lane's frequency from scalar arguments only)
  double rev_step[6];
};

// revolutions per position of channel pair i (lane-dependent i < 64) from
// scalar arguments: a lane-indexed read of the kernel-argument table would be
// a vector load, and its wait would drain the data loads issued before it
__device__ __forceinline__ double pair_rev(const DecodeArgs& a, int i) {
  double rev = a.freqs.rev[0];
#pragma unroll
  for (int b = 0; b < 6; ++b) rev *= ((i >> b) & 1) ? a.rev_step[b] : 1.0;
  return rev;
}

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1 in order.
template <class F, int... I>
__device__ __forceinline__ void for_each_const_d_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void for_each_const_d(F&& f) {
  for_each_const_d_impl(f, std::make_integer_sequence<int, N>{});
}

template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum_d(float x) {
  x += dpp_row<0xB1>(x);
  x += dpp_row<0x4E>(x);
  x += dpp_row<0x141>(x);
  x += dpp_row<0x140>(x);
  return x;
}

template <typename T, int N>
__device__ __forceinline__ void load_row_slice(const T* __restrict__ p, float* f) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (N == 8) {
      unpack8(*(const uint4*)p, f);
    } else {  // N == 4
      const uint2 v = *(const uint2*)p;
      f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
      f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 v = *(const float4*)(p + i);
      f[i] = v.x; f[i + 1] = v.y; f[i + 2] = v.z; f[i + 3] = v.w;
    }
  }
}

template <typename T>
__device__ __forceinline__ float elem_f(const T* p, int64_t i) {
  if constexpr (sizeof(T) == 2)
    return bf16_bits_to_f32(p[i]);
  else
    return p[i];
}

// Merge online-softmax state (m2, l2, o2) into (m, l, o).
template <int N>
__device__ __forceinline__ void merge_state(float& m, float& l, float* o, float m2, float l2,
                                            const float* o2) {
  const float mm = fmaxf(m, m2);
  float a1 = 0.f, a2 = 0.f;
  if (mm != -INFINITY) {
    a1 = exp2f(m - mm);
    a2 = exp2f(m2 - mm);
  }
#pragma unroll
  for (int e = 0; e < N; ++e) o[e] = o[e] * a1 + o2[e] * a2;
  l = l * a1 + l2 * a2;
  m = mm;
}

// 32-bit words of one lane's slice of a cache row, as a vector (one word: a
// plain scalar)
template <int N>
struct words {
  typedef unsigned int type __attribute__((ext_vector_type(N)));
  static __device__ __forceinline__ unsigned int at(const type& w, int i) { return w[i]; }
};
template <>
struct words<1> {
  typedef unsigned int type;
  static __device__ __forceinline__ unsigned int at(const type& w, int) { return w; }
};

// T: element type of q, k_new, v_new and out (and of the cache unless FP8).
// FP8: the cache holds OCP E4M3 codes (1 sign, 4 exponent bits with bias 7,
// 3 mantissa bits; gfx950's v_cvt_pk_f32_fp8 decodes exactly this format),
// element = decode(code) * scale[block][KV head].
template <typename T, int D, int MAXG, bool FP8 = false>
__global__ void __launch_bounds__(256)
decode_split(const DecodeArgs a) {
  constexpr int E = D / 16;  // channels per lane
  __shared__ float red[4][MAXG][D + 2];

  const int bid = blockIdx.x;
  const int s = bid % a.nsplit;
  const int rg = bid / a.nsplit;
  const int g = rg % a.H;
  const int r = rg / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int gi = lane >> 4, c = lane & 15;
  const int G = a.G;

  const int ctx = a.ctx[r];
  const int64_t cap = (int64_t)a.max_blk * a.bs;
  const bool ctx_bad = ctx < 0 || ctx > cap;
  const int kbeg = s * kSplitKeys + 64 * wv + 16 * gi;  // this row's 16 keys
  const int kend = ctx_bad ? 0 : min(kbeg + 16, ctx);

  // rotated query slice of every head of the group: channels [E*c, E*c+E)
  float qv[MAXG][E];
  {
    const double pos = (double)a.positions[r];
    const int ch0 = E * c;
    const bool low = ch0 < D / 2;
    const int partner = low ? ch0 + D / 2 : ch0 - D / 2;
    const int fi = low ? ch0 : partner;  // frequency index of the pair
    float cs[E], sn[E];
    double rev = pair_rev(a, fi);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      rope_cos_sin(pos, rev, cs[e], sn[e]);
      rev *= a.rev_step[0];
    }
#pragma unroll
    for (int hh = 0; hh < MAXG; ++hh) {
      if (hh < G) {
        const T* qr = (const T*)a.q + ((int64_t)r * a.Hq + (int64_t)g * G + hh) * D;
        float x[E], y[E];
        load_row_slice<T, E>(qr + ch0, x);
        load_row_slice<T, E>(qr + partner, y);
#pragma unroll
        for (int e = 0; e < E; ++e)
          qv[hh][e] = __builtin_fmaf(x[e], cs[e], low ? -(y[e] * sn[e]) : y[e] * sn[e]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) qv[hh][e] = 0.f;
      }
    }
  }

  float m[MAXG], l[MAXG], o[MAXG][E];
#pragma unroll
  for (int hh = 0; hh < MAXG; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[hh][e] = 0.f;
  }
  // ---- this row's 16 keys: unconditional loads (rows past the context, or
  // of a row with no keys, read a valid row and are masked), PD keys in
  // flight, fully unrolled so every wait covers exactly the loads it needs
  const int nkeys = kend > kbeg ? kend - kbeg : 0;
  int32_t phys = 0;
  if (nkeys > 0) phys = a.table[(int64_t)r * a.max_blk + kbeg / a.bs];
  const bool row_ok = nkeys > 0 && phys >= 0 && phys < a.nblk;
  const bool blk_bad = nkeys > 0 && !row_ok;
  // 16 keys of one row lie in one block (block_size is a multiple of 16)
  const int64_t base =
      row_ok ? (((int64_t)phys * a.H + g) * a.bs + (kbeg % a.bs)) * D + E * c : (int64_t)E * c;
  const int nvalid = row_ok ? nkeys : 0;
  const int klast = nvalid > 0 ? nvalid - 1 : 0;
  typedef std::conditional_t<FP8, uint8_t, T> C;  // cache element
  const C* kp = (const C*)a.kc + base;
  const C* vp = (const C*)a.vc + base;
  constexpr int NW = E * (int)sizeof(C) / 4;  // 32-bit words per lane and key
  typedef typename words<NW>::type rawv_t;
  // fp8: the row's block scales, folded into the logit and into the weight
  // that multiplies V (not into the softmax sum)
  float kmul = a.scale_log2, vmul = 1.f;
  if constexpr (FP8) {
    const int64_t si = row_ok ? (int64_t)phys * a.H + g : 0;
    kmul *= a.ksc[si];
    vmul = a.vsc[si];
  }
  // keys in flight per lane: 8, or 4 when the per-head state of a wide group
  // already takes most of the registers
  constexpr int PD = MAXG * E >= 32 ? 4 : 8;
  rawv_t kb[PD], vb[PD];
  auto issue = [&](auto tc) {
    constexpr int t = decltype(tc)::value;
    const int64_t off = (int64_t)(t < klast ? t : klast) * D;
    // the cache is streamed once per step, in whole rows: non-temporal loads
    kb[t % PD] = __builtin_nontemporal_load((const rawv_t*)(kp + off));
    vb[t % PD] = __builtin_nontemporal_load((const rawv_t*)(vp + off));
  };
  auto unpack = [](const rawv_t& w, float* f) {
    if constexpr (FP8) {
      typedef float f2_t __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)words<NW>::at(w, i), false);
        const f2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)words<NW>::at(w, i), true);
        f[4 * i] = lo.x;
        f[4 * i + 1] = lo.y;
        f[4 * i + 2] = hi.x;
        f[4 * i + 3] = hi.y;
      }
    } else if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        f[2 * i] = __uint_as_float(words<NW>::at(w, i) << 16);
        f[2 * i + 1] = __uint_as_float(words<NW>::at(w, i) & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) f[i] = __uint_as_float(words<NW>::at(w, i));
    }
  };
  for_each_const_d<PD>([&](auto tc) { issue(tc); });
  for_each_const_d<16>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    float kf[E], vf[E];
    unpack(kb[t % PD], kf);
    unpack(vb[t % PD], vf);
    if constexpr (t + PD < 16) issue(std::integral_constant<int, t + PD>{});
    const bool valid = t < nvalid;
    if constexpr (!FP8) {
      // running maximum updated at every key
#pragma unroll
      for (int hh = 0; hh < MAXG; ++hh) {
        if (hh == 0 || hh < G) {  // head 0 always exists: no branch around it
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) part = fmaf(qv[hh][e], kf[e], part);
          // the logit is formed for every key and masked by selects (no branch,
          // so the loads stay where they were issued)
          const float dot = row16_sum_d(part) * kmul;
          const float sc = valid ? dot : -INFINITY;
          const float mnew = fmaxf(m[hh], sc);
          // exponents never see -inf - -inf: an all-masked state keeps alpha = 1,
          // a masked key gets weight exp2(-inf) = 0
          const float alpha = __builtin_amdgcn_exp2f(mnew == -INFINITY ? 0.f : m[hh] - mnew);
          const float pw = __builtin_amdgcn_exp2f(valid ? sc - mnew : -INFINITY);
          m[hh] = mnew;
          l[hh] = l[hh] * alpha + pw;
          const float pv = pw * vmul;
#pragma unroll
          for (int e = 0; e < E; ++e) o[hh][e] = fmaf(pv, vf[e], o[hh][e] * alpha);
        }
      }
    } else {
      // the logit of this key for every head of the group (log2 units), formed
      // for every key and masked by selects
      float sc[MAXG];
      bool up = false;
#pragma unroll
      for (int hh = 0; hh < MAXG; ++hh) {
        if (hh == 0 || hh < G) {  // head 0 always exists: no branch around it
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) part = fmaf(qv[hh][e], kf[e], part);
          const float dot = row16_sum_d(part) * kmul;
          sc[hh] = valid ? dot : -INFINITY;
          up = up || sc[hh] > m[hh] + kLazyMax;
        }
      }
      // fp8 cache (its decode adds VALU work per key): the state (m, l, o) is
      // kept relative to a reference maximum m that moves only when a logit
      // passes it by more than kLazyMax (always at a row's first valid key), so
      // most keys cost no rescale of o and l; the weights stay below
      // 2^kLazyMax.  The branch is taken by the whole wave when any of its rows
      // needs it (alpha = 1 for the others).
      if (__builtin_expect(__any(up) != 0, 0)) {
#pragma unroll
        for (int hh = 0; hh < MAXG; ++hh) {
          if (hh == 0 || hh < G) {
            const float mnew = fmaxf(m[hh], sc[hh]);
            // an all-masked state keeps alpha = 1 (no -inf - -inf)
            const float alpha = __builtin_amdgcn_exp2f(mnew == -INFINITY ? 0.f : m[hh] - mnew);
            m[hh] = mnew;
            l[hh] *= alpha;
#pragma unroll
            for (int e = 0; e < E; ++e) o[hh][e] *= alpha;
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < MAXG; ++hh) {
        if (hh == 0 || hh < G) {
          // a masked key gets weight exp2(-inf) = 0; a valid key has a finite
          // reference maximum by now (its own logit at the latest)
          const float pw = __builtin_amdgcn_exp2f(valid ? sc[hh] - m[hh] : -INFINITY);
          l[hh] += pw;
          const float pv = pw * vmul;
#pragma unroll
          for (int e = 0; e < E; ++e) o[hh][e] = fmaf(pv, vf[e], o[hh][e]);
        }
      }
    }
  });

  // merge the four rows of the wave (lane ^ 16, lane ^ 32)
#pragma unroll
  for (int span = 16; span <= 32; span <<= 1) {
#pragma unroll
    for (int hh = 0; hh < MAXG; ++hh) {
      float o2[E];
#pragma unroll
      for (int e = 0; e < E; ++e) o2[e] = __shfl_xor(o[hh][e], span);
      const float m2 = __shfl_xor(m[hh], span);
      const float l2 = __shfl_xor(l[hh], span);
      merge_state<E>(m[hh], l[hh], o[hh], m2, l2, o2);
    }
  }
  // a bad block anywhere poisons the split
  const bool wave_bad = __any(blk_bad) != 0;

  // merge the four waves through LDS
  if (gi == 0) {
#pragma unroll
    for (int hh = 0; hh < MAXG; ++hh) {
#pragma unroll
      for (int e = 0; e < E; ++e) red[wv][hh][E * c + e] = o[hh][e];
      if (c == 0) {
        red[wv][hh][D] = m[hh];
        red[wv][hh][D + 1] = wave_bad ? __int_as_float(0x7fc00000) : l[hh];
      }
    }
  }
  __syncthreads();
  if (wv == 0 && gi == 0) {
#pragma unroll
    for (int hh = 0; hh < MAXG; ++hh) {
      if (hh >= G) continue;
      float mm = red[0][hh][D], ll = red[0][hh][D + 1];
      float oo[E];
#pragma unroll
      for (int e = 0; e < E; ++e) oo[e] = red[0][hh][E * c + e];
#pragma unroll
      for (int w2 = 1; w2 < 4; ++w2) {
        float o2[E];
#pragma unroll
        for (int e = 0; e < E; ++e) o2[e] = red[w2][hh][E * c + e];
        merge_state<E>(mm, ll, oo, red[w2][hh][D], red[w2][hh][D + 1], o2);
      }
      if (ctx_bad) ll = __int_as_float(0x7fc00000);
      float* dst = a.ws + (((int64_t)r * a.Hq + (int64_t)g * G + hh) * a.nsplit + s) * (D + kWsPad);
#pragma unroll
      for (int e = 0; e < E; ++e) dst[E * c + e] = oo[e];
      if (c == 0) {
        dst[D] = mm;
        dst[D + 1] = ll;
      }
    }
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(64)
decode_combine(const DecodeArgs a) {
  constexpr int EC = D / 64;  // channels per lane: d = lane + 64*e
  const int bid = blockIdx.x;
  const int h = bid % a.Hq;
  const int r = bid / a.Hq;
  const int g = h / a.G;
  const int lane = threadIdx.x;
  const double pos = (double)a.positions[r];
  const T* qr = (const T*)a.q + ((int64_t)r * a.Hq + h) * D;
  const T* kr = (const T*)a.kn + ((int64_t)r * a.H + g) * D;
  const T* vr = (const T*)a.vn + ((int64_t)r * a.H + g) * D;

  float part = 0.f;
  float vself[EC];
#pragma unroll
  for (int e = 0; e < EC; ++e) {
    const int d = lane + 64 * e;
    const bool low = d < D / 2;
    const int partner = low ? d + D / 2 : d - D / 2;
    float cs, sn;
    rope_cos_sin(pos, pair_rev(a, low ? d : partner), cs, sn);
    const float qd = elem_f(qr, d), qp = elem_f(qr, partner);
    const float kd = elem_f(kr, d), kpn = elem_f(kr, partner);
    const float qrot = __builtin_fmaf(qd, cs, low ? -(qp * sn) : qp * sn);
    const float krot = __builtin_fmaf(kd, cs, low ? -(kpn * sn) : kpn * sn);
    part = fmaf(qrot, krot, part);
    vself[e] = elem_f(vr, d);
  }
  part += __shfl_xor(part, 32);
  part += __shfl_xor(part, 16);
  const float sself = row16_sum_d(part) * a.scale_log2;

  const float* ws = a.ws + ((int64_t)r * a.Hq + h) * a.nsplit * (D + kWsPad);
  const int ns = a.nsplit;
  // split maxima: lane s covers splits s, s + 64, ... (independent loads),
  // then a wave reduction
  float mloc = sself;
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) mloc = fmaxf(mloc, ws[(int64_t)(s0 + lane) * (D + kWsPad) + D]);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, sh));
  const float mm = mloc;
  const float wself = __builtin_amdgcn_exp2f(sself - mm);
  float ll = wself;
  float acc[EC];
#pragma unroll
  for (int e = 0; e < EC; ++e) acc[e] = wself * vself[e];
  for (int s0 = 0; s0 < ns; s0 += 64) {
    // weight of split s0 + lane; a NaN l (bad block or context) poisons the sum
    float wl = 0.f, lterm = 0.f;
    if (s0 + lane < ns) {
      const float* row = ws + (int64_t)(s0 + lane) * (D + kWsPad);
      const float ms = row[D], ls = row[D + 1];
      wl = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - mm);
      lterm = ls * wl;  // NaN l stays NaN even where the weight is 0
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) lterm += __shfl_xor(lterm, sh);
    ll += lterm;
    // weighted split outputs, eight splits per round of independent loads
    const int n = ns - s0 < 64 ? ns - s0 : 64;
    for (int i0 = 0; i0 < n; i0 += 8) {
      float v[8][EC];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int si = s0 + (i0 + i < n ? i0 + i : n - 1);
#pragma unroll
        for (int e = 0; e < EC; ++e) v[i][e] = ws[(int64_t)si * (D + kWsPad) + lane + 64 * e];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float w = i0 + i < n ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i0 + i)) : 0.f;
#pragma unroll
        for (int e = 0; e < EC; ++e) acc[e] = fmaf(v[i][e], w, acc[e]);
      }
    }
  }
  const float inv = 1.f / ll;
  T* orow = (T*)a.out + ((int64_t)r * a.Hq + h) * D;
#pragma unroll
  for (int e = 0; e < EC; ++e) {
    const float y = acc[e] * inv;
    if constexpr (sizeof(T) == 2)
      orow[lane + 64 * e] = (T)(pack2_bf16(y, 0.f) & 0xffffu);
    else
      orow[lane + 64 * e] = y;
  }
}

}  // namespace gist

using namespace gist;

namespace {
int num_splits(int max_blocks, int block_size) {
  const int64_t keys = (int64_t)max_blocks * block_size;
  return (int)((keys + kSplitKeys - 1) / kSplitKeys);
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

template <typename T, int D, bool FP8 = false>
void launch_decode(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid1((unsigned)((int64_t)a.R * a.H * a.nsplit));
  if (a.G <= 1)
    hipLaunchKernelGGL((decode_split<T, D, 1, FP8>), grid1, dim3(256), 0, s, a);
  else if (a.G <= 2)
    hipLaunchKernelGGL((decode_split<T, D, 2, FP8>), grid1, dim3(256), 0, s, a);
  else if (a.G <= 4)
    hipLaunchKernelGGL((decode_split<T, D, 4, FP8>), grid1, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split<T, D, 8, FP8>), grid1, dim3(256), 0, s, a);
  hipLaunchKernelGGL((decode_combine<T, D>), dim3((unsigned)((int64_t)a.R * a.Hq)), dim3(64), 0,
                     s, a);
}
}  // namespace

extern "C" size_t paged_decode_workspace_bytes(int R, int Hq, int max_blocks, int block_size,
                                               int d) {
  if (R < 0 || Hq <= 0 || max_blocks <= 0 || block_size <= 0 || d <= 0) return 0;
  return (size_t)R * Hq * num_splits(max_blocks, block_size) * (d + kWsPad) * sizeof(float);
}

// ---------------------------------------------------------------------------
// Library-owned split-K scratch for paged_decode_attn_noalloc: one array per
// GPU, alive until the process ends.  Host code never passes the array's name
// to a kernel (in host code it is a host-side stand-in); it uses the device
// address hipGetSymbolAddress returns, looked up once per device with that
// device current.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (nullptr on failure,
// with the error recorded).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    set_error("paged_decode_attn_noalloc: no current HIP device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      set_error(std::string("paged_decode_attn_noalloc: hipGetSymbolAddress failed: ") +
                hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

namespace {
// Shared by the entry points: fp8 selects the E4M3 cache with per-(block,
// KV head) scales (activations in bf16); `fn` names the entry point in errors.
// use_scratch: the split-K partials go to the library's scratch array instead
// of the caller's workspace (which is then ignored); every argument is checked
// before the scratch address is looked up.
gist_status decode_call(const char* fn, bool fp8, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale, int64_t n_blocks,
                        int block_size, const int32_t* block_table, int max_blocks,
                        const int32_t* context_lens, int R, const void* q, const void* k_new,
                        const void* v_new, const int32_t* positions, int Hq, int H, int d,
                        gist_dtype dtype, float rope_base, float scale, void* out,
                        void* workspace, size_t workspace_bytes, void* stream,
                        bool use_scratch = false) {
  clear_error();
  const std::string name(fn);
  if (dtype != GIST_BF16 && dtype != GIST_F32)
    return fail(GIST_ERR_INVALID_ARG, name + ": unknown dtype");
  if (R < 0) return fail(GIST_ERR_INVALID_ARG, name + ": R < 0");
  if (H <= 0 || Hq < H || Hq % H != 0)
    return fail(GIST_ERR_INVALID_ARG, name + ": Hq must be a positive multiple of H");
  if (Hq / H > 8) return fail(GIST_ERR_UNSUPPORTED, name + ": Hq/H must be <= 8");
  if (d != 64 && d != 128)
    return fail(GIST_ERR_UNSUPPORTED, name + ": head_dim must be 64 or 128");
  if (block_size <= 0 || block_size % 16 != 0)
    return fail(GIST_ERR_UNSUPPORTED, name + ": block_size must be a multiple of 16");
  if (n_blocks <= 0 || max_blocks <= 0)
    return fail(GIST_ERR_INVALID_ARG, name + ": n_blocks and max_blocks must be > 0");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(GIST_ERR_INVALID_ARG, name + ": scale must be positive and finite");
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return fail(GIST_ERR_INVALID_ARG, name + ": rope_base must be positive");
  if (R == 0) return GIST_OK;
  if (!k_cache || !v_cache || !block_table || !context_lens || !q || !k_new || !v_new ||
      !positions || !out || (!use_scratch && !workspace) || (fp8 && (!k_scale || !v_scale)))
    return fail(GIST_ERR_INVALID_ARG, name + ": NULL pointer argument");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(k_new) ||
      !aligned16(v_new) || !aligned16(out) || (!use_scratch && !aligned16(workspace)))
    return fail(GIST_ERR_INVALID_ARG, name + ": tensors must be 16-byte aligned");
  if (fp8 && ((((uintptr_t)k_scale) & 3) != 0 || (((uintptr_t)v_scale) & 3) != 0))
    return fail(GIST_ERR_INVALID_ARG, name + ": scales must be 4-byte aligned");
  const size_t need = paged_decode_workspace_bytes(R, Hq, max_blocks, block_size, d);
  if (use_scratch && need > kScratchBytes)
    return fail(GIST_ERR_UNSUPPORTED, name + ": the call needs " + std::to_string(need) +
                                          " bytes of split-K scratch, more than the " +
                                          std::to_string(kScratchBytes) +
                                          " the library holds (use paged_decode_attn with a "
                                          "workspace)");
  if (!use_scratch && workspace_bytes < need)
    return fail(GIST_ERR_INVALID_ARG, name + ": workspace too small (" +
                                          std::to_string(workspace_bytes) + " < " +
                                          std::to_string(need) + ")");
  const int nsplit = num_splits(max_blocks, block_size);
  if ((int64_t)R * H * nsplit > INT32_MAX)
    return fail(GIST_ERR_UNSUPPORTED, name + ": too many splits for one launch");
  if (use_scratch) {
    workspace = scratch_address();
    if (!workspace) return GIST_ERR_HIP;
  }

  DecodeArgs a;
  a.kc = k_cache;
  a.vc = v_cache;
  a.nblk = n_blocks;
  a.bs = block_size;
  a.table = block_table;
  a.max_blk = max_blocks;
  a.ctx = context_lens;
  a.R = R;
  a.q = q;
  a.kn = k_new;
  a.vn = v_new;
  a.positions = positions;
  a.Hq = Hq;
  a.H = H;
  a.G = Hq / H;
  {
    double qs = std::pow((double)rope_base, -2.0 / (double)d);
    for (int b = 0; b < 6; ++b, qs *= qs) a.rev_step[b] = qs;
  }
  a.scale_log2 = scale * 1.4426950408889634f;
  a.ws = (float*)workspace;
  a.nsplit = nsplit;
  a.out = out;
  a.ksc = k_scale;
  a.vsc = v_scale;
  make_rope_freqs(a.freqs, d, rope_base);
  hipStream_t s = (hipStream_t)stream;
  if (fp8) {
    if (d == 64) launch_decode<bf16_t, 64, true>(a, s);
    else launch_decode<bf16_t, 128, true>(a, s);
  } else if (dtype == GIST_BF16) {
    if (d == 64) launch_decode<bf16_t, 64>(a, s);
    else launch_decode<bf16_t, 128>(a, s);
  } else {
    if (d == 64) launch_decode<float, 64>(a, s);
    else launch_decode<float, 128>(a, s);
  }
  return check_launch(fn);
}
}  // namespace

extern "C" gist_status paged_decode_attn(const void* k_cache, const void* v_cache,
                                         int64_t n_blocks, int block_size,
                                         const int32_t* block_table, int max_blocks,
                                         const int32_t* context_lens, int R, const void* q,
                                         const void* k_new, const void* v_new,
                                         const int32_t* positions, int Hq, int H, int d,
                                         gist_dtype dtype, float rope_base, float scale, void* out,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call("paged_decode_attn", false, k_cache, v_cache, nullptr, nullptr, n_blocks,
                     block_size, block_table, max_blocks, context_lens, R, q, k_new, v_new,
                     positions, Hq, H, d, dtype, rope_base, scale, out, workspace, workspace_bytes,
                     stream);
}

extern "C" gist_status paged_decode_attn_fp8(const void* k_cache, const void* v_cache,
                                             const float* k_scale, const float* v_scale,
                                             int64_t n_blocks, int block_size,
                                             const int32_t* block_table, int max_blocks,
                                             const int32_t* context_lens, int R, const void* q,
                                             const void* k_new, const void* v_new,
                                             const int32_t* positions, int Hq, int H, int d,
                                             float rope_base, float scale, void* out,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream) {
  return decode_call("paged_decode_attn_fp8", true, k_cache, v_cache, k_scale, v_scale,
                     n_blocks, block_size, block_table, max_blocks, context_lens, R, q, k_new,
                     v_new, positions, Hq, H, d, GIST_BF16, rope_base, scale, out, workspace,
                     workspace_bytes, stream);
}

extern "C" gist_status paged_decode_attn_noalloc(const void* k_cache, const void* v_cache,
                                                 int64_t n_blocks, int block_size,
                                                 const int32_t* block_table, int max_blocks,
                                                 const int32_t* context_lens, int R,
                                                 const void* q, const void* k_new,
                                                 const void* v_new, const int32_t* positions,
                                                 int Hq, int H, int d, gist_dtype dtype,
                                                 float rope_base, float scale, void* out,
                                                 void* stream) {
  return decode_call("paged_decode_attn_noalloc", false, k_cache, v_cache, nullptr, nullptr,
                     n_blocks, block_size, block_table, max_blocks, context_lens, R, q, k_new,
                     v_new, positions, Hq, H, d, dtype, rope_base, scale, out, nullptr, 0, stream,
                     true);
}
