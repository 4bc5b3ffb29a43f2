// gist_attn_forward: one layer of online gist attention for a batch of
// (item, query) pairs.
//
// What is computed (liam.page "把 item 压成 KV：gist 能不能用在相关性任务上",
// section 在线的一次 attention; query-gist variant in section 能不能再进一步):
// per pair p and query head h with KV head g = h / (Hq/H), the keys are
//   [item gist K (k rows, stored rotated at 1..k) ; query gist K (k' rows) ;
//    RoPE(K_new[t], pos0 + t) for t < ell]
// and the values the matching V rows.  Query token t, rotated at pos0 + t,
// sees every gist key and new keys 0..t, and gets softmax(scale·q·Kᵀ)·V
// (mcfzz.com "为什么自回归推理缓存 KV，而不缓存历史 Q？", Reusable-state).
//
// Two kernels:
//  * gist_fwd_mfma<D>  bf16, 2 <= ell <= 64, k+k'+ell <= 128.  One workgroup
//    (4 wave64s) per (pair, KV head).  All keys of the pair are staged once
//    in LDS (K row-major with RoPE applied on load, V transposed), and each
//    wave owns 16 query tokens and loops over the G query heads of the GQA
//    group, so every K/V tile in LDS serves all G heads.  Logits are
//    computed transposed, Sᵀ = K·Qᵀ, with v_mfma_f32_16x16x32_bf16, so each
//    lane ends up holding four keys of one token; that is exactly the B
//    operand layout of the P·V product (v_mfma_f32_16x16x16_bf16, Oᵀ = Vᵀ·Pᵀ)
//    and the softmax never leaves registers.  Softmax is online over 16-key
//    tiles (running max and sum in fp32, exp2 with log2(e) folded into the
//    scale); causally invisible tiles are skipped.
//  * gist_fwd_valu<T, D, MAXH>  any ell, any gist length, bf16 or fp32.  One
//    wave64 per (pair, KV head, token); four 16-lane rows split the heads of
//    the group (or, for G < 4, the keys), each lane holds d/16 channels
//    including both members of its RoPE pairs, dot products reduce across the
//    16-lane row with DPP.  This is the ell = 1 path (EOS over item gist +
//    query gist + itself) and the fp32 path.
#include <cfloat>

#include "common.hpp"

namespace gist {

struct FwdArgs {
  const void* pool;
  int64_t pool_layer_off;  // elements
  int64_t N;
  int k;
  const void* qpool;
  int64_t qpool_layer_off;
  int64_t qN;
  int kq;  // 0 when there is no query gist
  const int32_t* item_ids;
  const int32_t* q_ids;
  const void* q;
  const void* k_new;
  const void* v_new;
  void* out;
  int P, ell, Hq, H, G;
  int pos0;
  float scale_log2;  // softmax scale * log2(e)
  RopeFreqs freqs;
};

// ---------------------------------------------------------------------------
// Shared helpers
// ---------------------------------------------------------------------------

// DPP row (16-lane) butterflies: quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return x;
}

template <typename T>
__device__ __forceinline__ T nan_value() {
  if constexpr (sizeof(T) == 2)
    return (T)0x7fc0;
  else
    return __int_as_float(0x7fc00000);
}

// ---------------------------------------------------------------------------
// MFMA kernel (bf16)
// ---------------------------------------------------------------------------

// Row of the Vᵀ tile that MFMA row r of d-tile dt stands for.  The mapping is
// chosen so that after the P·V product each lane holds, for every 32-channel
// step s, the eight consecutive channels 32s + 8*(lane/16) .. +8 of its token:
// the same layout the Q loads use, so output stores are 16-byte vectors.
__device__ __forceinline__ int vt_row(int dt, int r) {
  return 32 * (dt >> 1) + 8 * (r >> 2) + 4 * (dt & 1) + (r & 3);
}

template <int D>
__global__ void __launch_bounds__(256)
gist_fwd_mfma(const FwdArgs a, int nk_pad, int vs) {
  extern __shared__ __align__(16) bf16_t smem[];
  constexpr int KS = D + 8;  // K row stride in LDS (elements): 16*odd bytes
  constexpr int NS = D / 32;  // 32-channel k-steps of the Q·Kᵀ product
  constexpr int NP = NS / 2;  // RoPE: step s pairs with step s + NP
  constexpr int NDT = D / 16; // 16-channel tiles of the output
  bf16_t* Ks = smem;               // [nk_pad][KS]
  bf16_t* Vt = smem + nk_pad * KS; // [D][vs]

  const int p = blockIdx.x / a.H;
  const int g = blockIdx.x - p * a.H;
  const int tid = threadIdx.x;
  const int kg = a.k + a.kq;
  const int nk = kg + a.ell;
  const int ell = a.ell;
  const int Hq = a.Hq, H = a.H, G = a.G;

  bf16_t* out = (bf16_t*)a.out;

  // ---- ids (bounds-checked; a bad id turns the pair's rows into NaN) ------
  const int32_t item = a.item_ids[p];
  int32_t qid = 0;
  bool bad = item < 0 || item >= a.N;
  if (a.kq) {
    qid = a.q_ids[p];
    bad = bad || qid < 0 || qid >= a.qN;
  }
  if (bad) {
    const int per_t = G * D;
    for (int u = tid; u < ell * per_t; u += 256) {
      const int t = u / per_t, r = u - t * per_t;
      out[((int64_t)p * ell + t) * Hq * D + (int64_t)g * G * D + r] = nan_value<bf16_t>();
    }
    return;
  }
  const bf16_t* pool = (const bf16_t*)a.pool;
  const int64_t rec_i = 2LL * H * a.k * D;
  const bf16_t* gK = pool + a.pool_layer_off + (int64_t)item * rec_i + (int64_t)g * a.k * D;
  const bf16_t* gV = gK + (int64_t)H * a.k * D;
  const bf16_t* qK = nullptr;
  const bf16_t* qV = nullptr;
  if (a.kq) {
    const int64_t rec_q = 2LL * H * a.kq * D;
    qK = (const bf16_t*)a.qpool + a.qpool_layer_off + (int64_t)qid * rec_q +
         (int64_t)g * a.kq * D;
    qV = qK + (int64_t)H * a.kq * D;
  }
  const bf16_t* knew = (const bf16_t*)a.k_new;
  const bf16_t* vnew = (const bf16_t*)a.v_new;

  // ---- stage K (rotating the new rows) ------------------------------------
  constexpr int CH = D / 16;  // chunk pairs (8 channels + their RoPE partners)
  for (int u = tid; u < nk_pad * CH; u += 256) {
    const int j = u / CH, c = u - j * CH;
    uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
    if (j < nk) {
      const bf16_t* src;
      if (j < a.k) {
        src = gK + (int64_t)j * D;
      } else if (j < kg) {
        src = qK + (int64_t)(j - a.k) * D;
      } else {
        src = knew + (((int64_t)p * ell + (j - kg)) * H + g) * D;
      }
      lo = *(const uint4*)(src + 8 * c);
      hi = *(const uint4*)(src + D / 2 + 8 * c);
      if (j >= kg) {
        float xl[8], xh[8], yl[8], yh[8];
        unpack8(lo, xl);
        unpack8(hi, xh);
        const double pos = (double)(a.pos0 + (j - kg));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float cs, sn;
          rope_cos_sin(pos, a.freqs.theta[8 * c + e], cs, sn);
          yl[e] = xl[e] * cs - xh[e] * sn;
          yh[e] = xh[e] * cs + xl[e] * sn;
        }
        lo = pack8_bf16(yl);
        hi = pack8_bf16(yh);
      }
    }
    *(uint4*)(Ks + j * KS + 8 * c) = lo;
    *(uint4*)(Ks + j * KS + D / 2 + 8 * c) = hi;
  }
  // ---- stage V transposed, two keys per thread ----------------------------
  {
    const int npairs = nk_pad / 2;
    constexpr int CV = D / 8;
    for (int u = tid; u < npairs * CV; u += 256) {
      const int c = u / npairs, jp = u - c * npairs;
      uint4 v[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int j = 2 * jp + m;
        v[m] = make_uint4(0, 0, 0, 0);
        if (j < nk) {
          const bf16_t* src;
          if (j < a.k)
            src = gV + (int64_t)j * D;
          else if (j < kg)
            src = qV + (int64_t)(j - a.k) * D;
          else
            src = vnew + (((int64_t)p * ell + (j - kg)) * H + g) * D;
          v[m] = *(const uint4*)(src + 8 * c);
        }
      }
      const uint32_t a0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
      const uint32_t a1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // channel 8c+2e: low halves; channel 8c+2e+1: high halves
        const uint32_t w0 = (a0[e] & 0xffffu) | (a1[e] << 16);
        const uint32_t w1 = (a0[e] >> 16) | (a1[e] & 0xffff0000u);
        *(uint32_t*)(Vt + (8 * c + 2 * e) * vs + 2 * jp) = w0;
        *(uint32_t*)(Vt + (8 * c + 2 * e + 1) * vs + 2 * jp) = w1;
      }
    }
  }
  __syncthreads();

  // ---- per wave: 16 query tokens, all G heads ------------------------------
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int t0 = 16 * wv;
  if (t0 >= ell) return;
  const int n = lane & 15, q4 = lane >> 4;
  const int t = t0 + n;
  const bool tvalid = t < ell;
  const int tlast = min(t0 + 15, ell - 1);
  const int nkt = (kg + tlast + 1 + 15) >> 4;
  const int vis_last = kg + t;  // key j visible to token t iff j <= kg + t

  float qc[NP][8], qsn[NP][8];
  {
    const double pos = (double)(a.pos0 + t);
#pragma unroll
    for (int s = 0; s < NP; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) rope_cos_sin(pos, a.freqs.theta[32 * s + 8 * q4 + e], qc[s][e], qsn[s][e]);
  }

  const bf16_t* qg = (const bf16_t*)a.q;
  const float sl2 = a.scale_log2;
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    const int64_t row = (((int64_t)p * ell + t) * Hq + h) * D;
    uint4 raw[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
      raw[s] = tvalid ? *(const uint4*)(qg + row + 32 * s + 8 * q4) : make_uint4(0, 0, 0, 0);
    bf16x8_t qf[NS];
#pragma unroll
    for (int s = 0; s < NP; ++s) {
      float xl[8], xh[8], yl[8], yh[8];
      unpack8(raw[s], xl);
      unpack8(raw[s + NP], xh);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        yl[e] = xl[e] * qc[s][e] - xh[e] * qsn[s][e];
        yh[e] = xh[e] * qc[s][e] + xl[e] * qsn[s][e];
      }
      qf[s] = __builtin_bit_cast(bf16x8_t, pack8_bf16(yl));
      qf[s + NP] = __builtin_bit_cast(bf16x8_t, pack8_bf16(yh));
    }

    float m = -INFINITY, lsum = 0.f;
    f32x4_t o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int kt = 0; kt < nkt; ++kt) {
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
      const bf16_t* krow = Ks + (16 * kt + n) * KS + 8 * q4;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8_t kf = *(const bf16x8_t*)(krow + 32 * s);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sacc, 0, 0, 0);
      }
      float sv[4];
      const int key0 = 16 * kt + 4 * q4;
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = (key0 + i <= vis_last) ? sacc[i] * sl2 : -INFINITY;
      float tmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(m, tmax);
      const float alpha = exp2f(m - mnew);
      m = mnew;
      bf16x4_t pf;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __bf16 pb = (__bf16)exp2f(sv[i] - mnew);
        pf[i] = pb;
        psum += (float)pb;  // the denominator sums the same rounded weights
      }
      lsum = lsum * alpha + psum;
      const bf16_t* vrow = Vt + 16 * kt + 4 * q4;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        o[dt] *= alpha;
        const bf16x4_t vf = *(const bf16x4_t*)(vrow + vt_row(dt, n) * vs);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pf, o[dt], 0, 0, 0);
      }
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const float inv = 1.f / lsum;
    if (tvalid) {
      bf16_t* orow = out + row;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = o[2 * s][i] * inv;
          v[4 + i] = o[2 * s + 1][i] * inv;
        }
        *(uint4*)(orow + 32 * s + 8 * q4) = pack8_bf16(v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// VALU kernel (any ell; bf16 or fp32)
// ---------------------------------------------------------------------------

template <typename T, int N>
__device__ __forceinline__ void load_n(const T* __restrict__ p, float* f) {
  if constexpr (sizeof(T) == 4) {
    if constexpr (N == 4) {
      const float4 v = *(const float4*)p;
      f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
    } else {
      const float2 v = *(const float2*)p;
      f[0] = v.x; f[1] = v.y;
    }
  } else {
    if constexpr (N == 4) {
      const uint2 v = *(const uint2*)p;
      f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
      f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    } else {
      const uint32_t v = *(const uint32_t*)p;
      f[0] = __uint_as_float(v << 16); f[1] = __uint_as_float(v & 0xffff0000u);
    }
  }
}

template <typename T, int N>
__device__ __forceinline__ void store_n(T* __restrict__ p, const float* f) {
  if constexpr (sizeof(T) == 4) {
    if constexpr (N == 4)
      *(float4*)p = make_float4(f[0], f[1], f[2], f[3]);
    else
      *(float2*)p = make_float2(f[0], f[1]);
  } else {
    if constexpr (N == 4)
      *(uint2*)p = make_uint2(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]));
    else
      *(uint32_t*)p = pack2_bf16(f[0], f[1]);
  }
}

template <typename T, int D, int MAXH>
__global__ void __launch_bounds__(64)
gist_fwd_valu(const FwdArgs a) {
  constexpr int E2 = D / 32;  // channels per lane in each half
  const int ell = a.ell, H = a.H, G = a.G, Hq = a.Hq;
  const int t = blockIdx.x % ell;
  const int pg = blockIdx.x / ell;
  const int g = pg % H;
  const int p = pg / H;
  const int lane = threadIdx.x;
  const int gi = lane >> 4, c = lane & 15;
  const int ngh = G < 4 ? G : 4;   // rows that take distinct heads
  const int ksplit = 4 / ngh;      // rows that split the keys of one head
  const int hs = gi % ngh, kp = gi / ngh;
  const bool active = kp < ksplit;
  const int hpg = (G + ngh - 1) / ngh;
  const int kg = a.k + a.kq;
  const int nk = kg + t + 1;
  T* out = (T*)a.out;

  const int32_t item = a.item_ids[p];
  int32_t qid = 0;
  bool bad = item < 0 || item >= a.N;
  if (a.kq) {
    qid = a.q_ids[p];
    bad = bad || qid < 0 || qid >= a.qN;
  }
  const int64_t orow0 = (((int64_t)p * ell + t) * Hq + (int64_t)g * G) * D;
  if (bad) {
    for (int u = lane; u < G * D; u += 64) out[orow0 + u] = nan_value<T>();
    return;
  }
  const T* pool = (const T*)a.pool;
  const T* gK = pool + a.pool_layer_off + (int64_t)item * 2 * H * a.k * D + (int64_t)g * a.k * D;
  const T* gV = gK + (int64_t)H * a.k * D;
  const T* qK = nullptr;
  const T* qV = nullptr;
  if (a.kq) {
    qK = (const T*)a.qpool + a.qpool_layer_off + (int64_t)qid * 2 * H * a.kq * D +
         (int64_t)g * a.kq * D;
    qV = qK + (int64_t)H * a.kq * D;
  }
  const int lo = E2 * c, hi = D / 2 + E2 * c;

  // query rotation at pos0 + t for this lane's channel pairs
  float qcs[E2], qsn[E2];
#pragma unroll
  for (int e = 0; e < E2; ++e) rope_cos_sin((double)(a.pos0 + t), a.freqs.theta[lo + e], qcs[e], qsn[e]);

  float qv[MAXH][2 * E2];
  float m[MAXH], l[MAXH], o[MAXH][2 * E2];
#pragma unroll
  for (int mh = 0; mh < MAXH; ++mh) {
    m[mh] = -INFINITY;
    l[mh] = 0.f;
#pragma unroll
    for (int e = 0; e < 2 * E2; ++e) o[mh][e] = 0.f, qv[mh][e] = 0.f;
    const int hh = hs + ngh * mh;
    if (mh < hpg && hh < G) {
      const T* qr = (const T*)a.q + (((int64_t)p * ell + t) * Hq + (int64_t)g * G + hh) * D;
      float xl[E2], xh[E2];
      load_n<T, E2>(qr + lo, xl);
      load_n<T, E2>(qr + hi, xh);
#pragma unroll
      for (int e = 0; e < E2; ++e) {
        qv[mh][e] = xl[e] * qcs[e] - xh[e] * qsn[e];
        qv[mh][E2 + e] = xh[e] * qcs[e] + xl[e] * qsn[e];
      }
    }
  }

  if (active) {
    const T* knew = (const T*)a.k_new;
    const T* vnew = (const T*)a.v_new;
    for (int j = kp; j < nk; j += ksplit) {
      const T* ks;
      const T* vsrc;
      if (j < a.k) {
        ks = gK + (int64_t)j * D;
        vsrc = gV + (int64_t)j * D;
      } else if (j < kg) {
        ks = qK + (int64_t)(j - a.k) * D;
        vsrc = qV + (int64_t)(j - a.k) * D;
      } else {
        const int64_t r = (((int64_t)p * ell + (j - kg)) * H + g) * D;
        ks = knew + r;
        vsrc = vnew + r;
      }
      float kv[2 * E2], vv[2 * E2];
      load_n<T, E2>(ks + lo, kv);
      load_n<T, E2>(ks + hi, kv + E2);
      load_n<T, E2>(vsrc + lo, vv);
      load_n<T, E2>(vsrc + hi, vv + E2);
      if (j >= kg) {
        const int tj = j - kg;
#pragma unroll
        for (int e = 0; e < E2; ++e) {
          float cs = qcs[e], sn = qsn[e];
          if (tj != t) rope_cos_sin((double)(a.pos0 + tj), a.freqs.theta[lo + e], cs, sn);
          const float xl = kv[e], xh = kv[E2 + e];
          kv[e] = xl * cs - xh * sn;
          kv[E2 + e] = xh * cs + xl * sn;
        }
      }
#pragma unroll
      for (int mh = 0; mh < MAXH; ++mh) {
        if (mh < hpg) {
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < 2 * E2; ++e) part = fmaf(qv[mh][e], kv[e], part);
          const float s = row16_sum(part) * a.scale_log2;
          const float mnew = fmaxf(m[mh], s);
          const float alpha = exp2f(m[mh] - mnew);
          const float pw = exp2f(s - mnew);
          m[mh] = mnew;
          l[mh] = l[mh] * alpha + pw;
#pragma unroll
          for (int e = 0; e < 2 * E2; ++e) o[mh][e] = fmaf(pw, vv[e], o[mh][e] * alpha);
        }
      }
    }
  }

  // merge the rows that split the keys of one head (ksplit = 2 or 4)
  for (int span = 16 * ngh; span < 16 * ngh * ksplit; span <<= 1) {
#pragma unroll
    for (int mh = 0; mh < MAXH; ++mh) {
      const float m2 = __shfl_xor(m[mh], span);
      const float l2 = __shfl_xor(l[mh], span);
      const float mm = fmaxf(m[mh], m2);
      float a1 = 0.f, a2 = 0.f;
      if (mm != -INFINITY) {
        a1 = exp2f(m[mh] - mm);
        a2 = exp2f(m2 - mm);
      }
#pragma unroll
      for (int e = 0; e < 2 * E2; ++e) {
        const float o2 = __shfl_xor(o[mh][e], span);
        o[mh][e] = o[mh][e] * a1 + o2 * a2;
      }
      l[mh] = l[mh] * a1 + l2 * a2;
      m[mh] = mm;
    }
  }

  if (active && kp == 0) {
#pragma unroll
    for (int mh = 0; mh < MAXH; ++mh) {
      const int hh = hs + ngh * mh;
      if (mh < hpg && hh < G) {
        const float inv = 1.f / l[mh];
        float y[2 * E2];
#pragma unroll
        for (int e = 0; e < 2 * E2; ++e) y[e] = o[mh][e] * inv;
        T* orow = out + orow0 + (int64_t)hh * D;
        store_n<T, E2>(orow + lo, y);
        store_n<T, E2>(orow + hi, y + E2);
      }
    }
  }
}

}  // namespace gist

using namespace gist;

namespace {

size_t mfma_lds_bytes(int d, int nk_pad, int vs) {
  return ((size_t)nk_pad * (d + 8) + (size_t)d * vs) * sizeof(bf16_t);
}

template <typename T, int D>
void launch_valu(const FwdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.P * a.H * a.ell));
  const int ngh = a.G < 4 ? a.G : 4;
  const int hpg = (a.G + ngh - 1) / ngh;
  if (hpg <= 1)
    hipLaunchKernelGGL((gist_fwd_valu<T, D, 1>), grid, dim3(64), 0, s, a);
  else if (hpg <= 2)
    hipLaunchKernelGGL((gist_fwd_valu<T, D, 2>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((gist_fwd_valu<T, D, 8>), grid, dim3(64), 0, s, a);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" gist_status gist_attn_forward(const gist_pool* pool, int layer, const int32_t* item_ids,
                                         int P, int ell, int Hq, const void* q, const void* k_new,
                                         const void* v_new, int pos0, float rope_base, float scale,
                                         const gist_pool* qpool, const int32_t* q_ids, void* out,
                                         void* stream) {
  clear_error();
  if (!pool) return fail(GIST_ERR_INVALID_ARG, "gist_attn_forward: pool is NULL");
  if (layer < 0 || layer >= pool->L)
    return fail(GIST_ERR_OUT_OF_RANGE, "gist_attn_forward: layer out of range");
  if (P < 0) return fail(GIST_ERR_INVALID_ARG, "gist_attn_forward: P < 0");
  if (ell < 1 || ell > 1024)
    return fail(GIST_ERR_UNSUPPORTED, "gist_attn_forward: ell must be in [1, 1024]");
  const int H = pool->H, d = pool->d;
  if (Hq < H || Hq % H != 0)
    return fail(GIST_ERR_INVALID_ARG, "gist_attn_forward: Hq must be a positive multiple of H");
  if (Hq / H > 32) return fail(GIST_ERR_UNSUPPORTED, "gist_attn_forward: Hq/H must be <= 32");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(GIST_ERR_INVALID_ARG, "gist_attn_forward: scale must be positive and finite");
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return fail(GIST_ERR_INVALID_ARG, "gist_attn_forward: rope_base must be positive");
  if (qpool) {
    if (qpool->H != H || qpool->d != d || qpool->dtype != pool->dtype || qpool->L != pool->L)
      return fail(GIST_ERR_INVALID_ARG,
                  "gist_attn_forward: qpool must match pool in L, H, d and dtype");
    if (!q_ids) return fail(GIST_ERR_INVALID_ARG, "gist_attn_forward: q_ids is NULL");
  }
  if (P == 0) return GIST_OK;
  if (!item_ids || !q || !k_new || !v_new || !out)
    return fail(GIST_ERR_INVALID_ARG, "gist_attn_forward: NULL tensor argument");
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
    return fail(GIST_ERR_INVALID_ARG, "gist_attn_forward: tensors must be 16-byte aligned");
  if ((int64_t)P * H * ell > INT32_MAX)
    return fail(GIST_ERR_UNSUPPORTED, "gist_attn_forward: P*H*ell too large for one launch");

  FwdArgs a;
  a.pool = pool->storage;
  a.pool_layer_off = (int64_t)layer * pool->N * record_elems(pool);
  a.N = pool->N;
  a.k = pool->k;
  a.qpool = qpool ? qpool->storage : nullptr;
  a.qpool_layer_off = qpool ? (int64_t)layer * qpool->N * record_elems(qpool) : 0;
  a.qN = qpool ? qpool->N : 0;
  a.kq = qpool ? qpool->k : 0;
  a.item_ids = item_ids;
  a.q_ids = qpool ? q_ids : nullptr;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.out = out;
  a.P = P;
  a.ell = ell;
  a.Hq = Hq;
  a.H = H;
  a.G = Hq / H;
  a.pos0 = pos0;
  a.scale_log2 = scale * 1.4426950408889634f;
  make_rope_freqs(a.freqs, d, rope_base);
  hipStream_t s = (hipStream_t)stream;

  const int kg = a.k + a.kq;
  const int nk_pad = ((kg + ell + 15) / 16) * 16;
  const int vs = nk_pad + 8;
  const size_t lds = mfma_lds_bytes(d, nk_pad, vs);
  if (pool->dtype == GIST_BF16 && ell >= 2 && ell <= 64 && kg + ell <= 128 && lds <= 65536) {
    const dim3 grid((unsigned)((int64_t)P * H));
    if (d == 64)
      hipLaunchKernelGGL(gist_fwd_mfma<64>, grid, dim3(256), lds, s, a, nk_pad, vs);
    else
      hipLaunchKernelGGL(gist_fwd_mfma<128>, grid, dim3(256), lds, s, a, nk_pad, vs);
    return check_launch("gist_attn_forward(mfma)");
  }
  if (pool->dtype == GIST_BF16) {
    if (d == 64) launch_valu<bf16_t, 64>(a, s);
    else launch_valu<bf16_t, 128>(a, s);
  } else {
    if (d == 64) launch_valu<float, 64>(a, s);
    else launch_valu<float, 128>(a, s);
  }
  return check_launch("gist_attn_forward(valu)");
}
