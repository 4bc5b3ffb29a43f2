// Offline gist extraction, one layer: causal self-attention of packed
// sequences [item tokens ; k gist tokens], with the gist positions' K/V
// written to a gist pool.  liam.page "把 item 压成 KV：gist 能不能用在相关性任务上",
// sections 论文做了什么 (the item is run with its gist tokens appended and
// the gist positions' K/V in every layer are what is kept) and 在线的一次
// attention (the stored K sits at the canonical positions 1..k, so the query
// meets it at distance k as in training).  Over [item ; gist] alone the gist
// mask of training is the plain causal mask: it only removes item keys from
// tokens after the gist, and none are present.
//
// Two launches per call:
//   prefill_prep   rotates every K row at its own position (a bf16 pair hi +
//                  lo, into the caller's workspace) and, for the last k rows
//                  of each sequence, writes K rotated at 1..k and V into the
//                  pool;
//   prefill_attn   causal attention (MFMA), Q rotated on load.
// Precision: the rotated Q (times the softmax scale and log2 e) and the
// rotated K are each carried as bf16 pairs hi + lo, and the logits take
// K_hi·Q_hi + K_hi·Q_lo + K_lo·Q_hi, which holds the fp32 rotation to about
// 2^-16 of |q||k|; P is rounded to bf16 for the P·V product.
// K is rotated once in the first launch: every query block and every query
// head of the group reads it again, and rotating it there would repeat the
// rotation Hq/H times per query block.
#include "common.hpp"

namespace gist {

namespace {

struct PrefillArgs {
  const bf16_t* q;      // [T][Hq][d]
  const bf16_t* k;      // [T][H][d], not rotated
  const bf16_t* v;      // [T][H][d]
  const int32_t* seq_start;  // [B + 1]
  bf16_t* k_rot;        // workspace [2][T][H][d]: rotated K, hi then lo
  bf16_t* out;          // [T][Hq][d]
  int64_t T;
  int B, max_len, Hq, H, G;
  float scale_log2;     // softmax scale * log2(e)
  // optional gist pool (bf16): this layer's records, item ids, k
  bf16_t* pool;
  int64_t N;
  int kk;
  const int32_t* item_ids;
  RopeFreqs freqs;
};

// Bounds of sequence b, or false when seq_start is inconsistent there (the
// sequence is then skipped).
__device__ __forceinline__ bool seq_bounds(const PrefillArgs& a, int b, int64_t& s0, int& len) {
  const int64_t lo = a.seq_start[b], hi = a.seq_start[b + 1];
  if (lo < 0 || hi < lo || hi > a.T || hi - lo > a.max_len) return false;
  s0 = lo;
  len = (int)(hi - lo);
  return true;
}

// Split fp32 values into a bf16 pair hi + lo: hi the nearest bf16 of x, lo
// the nearest bf16 of x - hi (exact in fp32).
__device__ __forceinline__ void split8(const float* y, uint4& hi, uint4& lo) {
  hi = pack8_bf16(y);
  float h[8], r[8];
  unpack8(hi, h);
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = y[e] - h[e];
  lo = pack8_bf16(r);
}

// One thread per (sequence b, token t, KV head g, chunk pair c): channels
// 8c..8c+7 and their RoPE partners d/2 + 8c..  K is rotated at position t+1
// and stored as a bf16 pair hi + lo; a gist row i (the last k of the
// sequence) is also rotated at its canonical position 1+i and stored, rounded
// to bf16, with its V in the pool record of item_ids[b].
template <int D>
__global__ void __launch_bounds__(256) prefill_prep(const PrefillArgs a) {
  constexpr int CP = D / 16;  // chunk pairs per row
  const int b = blockIdx.y;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t s0;
  int len;
  if (!seq_bounds(a, b, s0, len)) return;
  const int c = (int)(u % CP);
  const int64_t rest = u / CP;
  const int g = (int)(rest % a.H);
  const int64_t t = rest / a.H;
  if (t >= len) return;
  const int64_t row = ((s0 + t) * a.H + g) * D;
  float xl[8], xh[8];
  unpack8(*(const uint4*)(a.k + row + 8 * c), xl);
  unpack8(*(const uint4*)(a.k + row + D / 2 + 8 * c), xh);
  // lo_dst: where the bf16 remainders go (nullptr: rounded to bf16 only)
  auto rotate_store = [&](double pos, bf16_t* dst, bf16_t* lo_dst) {
    float yl[8], yh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float cs, sn;
      rope_cos_sin(pos, a.freqs.rev[8 * c + e], cs, sn);
      yl[e] = __builtin_fmaf(xl[e], cs, -(xh[e] * sn));
      yh[e] = __builtin_fmaf(xh[e], cs, xl[e] * sn);
    }
    uint4 hl, ll, hh, lh;
    split8(yl, hl, ll);
    split8(yh, hh, lh);
    *(uint4*)(dst + 8 * c) = hl;
    *(uint4*)(dst + D / 2 + 8 * c) = hh;
    if (lo_dst) {
      *(uint4*)(lo_dst + 8 * c) = ll;
      *(uint4*)(lo_dst + D / 2 + 8 * c) = lh;
    }
  };
  rotate_store((double)(t + 1), a.k_rot + row, a.k_rot + a.T * a.H * D + row);
  if (a.pool != nullptr && len >= a.kk && t >= len - a.kk) {
    const int32_t item = a.item_ids[b];
    if (item < 0 || item >= a.N) return;  // out-of-range destination: skipped
    const int i = (int)(t - (len - a.kk));
    bf16_t* rec = a.pool + (int64_t)item * 2 * a.H * a.kk * D;
    rotate_store((double)(1 + i), rec + ((int64_t)g * a.kk + i) * D, nullptr);
    bf16_t* vdst = rec + ((int64_t)(a.H + g) * a.kk + i) * D;
    *(uint4*)(vdst + 8 * c) = *(const uint4*)(a.v + row + 8 * c);
    *(uint4*)(vdst + D / 2 + 8 * c) = *(const uint4*)(a.v + row + D / 2 + 8 * c);
  }
}

// max of x and of x in the lane 32 (resp. 16) apart, with the gfx950 lane
// swaps: each of the two results of a swap holds the partner's value in one
// half of the wave and the lane's own value in the other
__device__ __forceinline__ float xmax32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, __uint_as_float(r[0])),
                                       __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, __uint_as_float(r[0])),
                                       __uint_as_float(r[1]));
}

// Causal attention, flash style.  Workgroup = 128 query tokens of one
// sequence and one query head; wave w holds tokens q0 + 32w .. +31 as two
// 16-token MFMA column tiles.  Key blocks of 32 tokens are staged in LDS (K
// rotated, hi and lo, from the workspace; V) with the next block's loads in
// flight while the current one is computed.  Per key block and column tile:
//   Sᵀ = K·Qᵀ       two 16-key tiles, three v_mfma_f32_16x16x32_bf16 per
//                   32 channels (K_hi·Q_hi + K_hi·Q_lo + K_lo·Q_hi; keys are
//                   MFMA rows, so a lane's logits belong to its own query and
//                   the softmax weights are the B operand of the P·V product)
//   l += Pᵀ·1, Oᵀ += Vᵀ·Pᵀ   v_mfma_f32_16x16x32_bf16 over all 32 keys: K-index
//                   8*q4 + e stands for key 4*q4 + e (e < 4) of the first tile
//                   and 4*q4 + e - 4 of the second, which is what a lane's
//                   weights of the two tiles are and what two LDS transpose
//                   reads (one per tile) give the Vᵀ operand
// A diagonal block (keys up to the wave's own tokens) is the only one that
// needs the causal mask; the branch to it is marked unlikely so that the
// other blocks carry no mask selects.
// The running maximum is only moved (and O, l rescaled) when a block's
// maximum exceeds it by more than 8 in log2 units, so most blocks skip the
// rescale; the weights exp2(s - m) then stay below 2^8.
template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
prefill_attn(const PrefillArgs a) {
  constexpr int NS = D / 32;  // 32-channel steps of the Q·Kᵀ product
  constexpr int NP = NS / 2;  // RoPE: step s pairs with step s + NP
  constexpr int NDT = D / 16;
  // K and V rows are D + 16 elements apart (160 B at d = 64, 288 B at 128):
  // with that stride the 16-row b128 reads of K and the transposed b64 reads
  // of V run at the LDS's full rate; a stride of D + 8 costs 1.9x and 1.5x.
  constexpr int KS = D + 16;
  constexpr int BN = 32;      // keys per block
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int SU = BN * CPR / 256;  // staging chunks per thread per tensor
  static_assert(SU >= 1 && BN * CPR % 256 == 0, "staging layout");
  __shared__ __align__(16) bf16_t Ks[BN * KS];
  __shared__ __align__(16) bf16_t Kl[BN * KS];
  // V row r holds channel ch at vpos(ch): the four channels that a lane of
  // the transposed read takes for output tile dt sit at 16 dt + 4 (lane & 3),
  // so the four lanes of a row read 32 contiguous bytes
  __shared__ __align__(16) bf16_t Vs[BN * KS];
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4v;
  typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

  const int b = blockIdx.z, h = blockIdx.y;
  const int qb = gridDim.x - 1 - blockIdx.x;  // the longest blocks first
  int64_t s0;
  int len;
  if (!seq_bounds(a, b, s0, len)) return;
  const int q0 = 128 * qb;
  if (q0 >= len) return;
  const int g = h / a.G;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15, q4 = lane >> 4;
  const int qw = q0 + 32 * w;                  // this wave's first token
  const int last = min(q0 + 127, len - 1);
  const int nkb = last / BN + 1;               // key blocks of the workgroup
  const int kb_diag = qw / BN;                 // this wave's diagonal block
  const bool wave_active = qw < len;

  // ---- Q of the wave's two column tiles, rotated at t+1 and multiplied by
  // scale * log2(e) (the logits then come out in log2 units), as bf16 pairs
  // hi + lo in the MFMA B layout --------------------------------------------
  const float sl2 = a.scale_log2;
  bf16x8_t qf[2][NS], qfl[2][NS];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int t = min(qw + 16 * ct + n, len - 1);
    const bf16_t* qrow = a.q + ((s0 + t) * a.Hq + h) * D;
    u32x4_t raw[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) raw[s] = *(const u32x4_t*)(qrow + 32 * s + 8 * q4);
#pragma unroll
    for (int s = 0; s < NP; ++s) {
      float xl[8], xh[8], yl[8], yh[8];
      unpack8(make_uint4(raw[s].x, raw[s].y, raw[s].z, raw[s].w), xl);
      unpack8(make_uint4(raw[s + NP].x, raw[s + NP].y, raw[s + NP].z, raw[s + NP].w), xh);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float cs, sn;
        rope_cos_sin((double)(t + 1), a.freqs.rev[32 * s + 8 * q4 + e], cs, sn);
        yl[e] = __builtin_fmaf(xl[e], cs, -(xh[e] * sn)) * sl2;
        yh[e] = __builtin_fmaf(xh[e], cs, xl[e] * sn) * sl2;
      }
      uint4 hl, ll, hh, lh;
      split8(yl, hl, ll);
      split8(yh, hh, lh);
      qf[ct][s] = __builtin_bit_cast(bf16x8_t, hl);
      qfl[ct][s] = __builtin_bit_cast(bf16x8_t, ll);
      qf[ct][s + NP] = __builtin_bit_cast(bf16x8_t, hh);
      qfl[ct][s + NP] = __builtin_bit_cast(bf16x8_t, lh);
    }
  }

  // ---- staging: chunk u = tid + 256*i covers row u / CPR, chunk u % CPR;
  // rows past the sequence read its last row (masked: they follow every
  // query of the workgroup) -------------------------------------------------
  const bf16_t* kseq = a.k_rot + (s0 * a.H + g) * D;
  const bf16_t* klseq = kseq + a.T * a.H * D;
  const bf16_t* vseq = a.v + (s0 * a.H + g) * D;
  // element offsets inside the sequence fit 32 bits (len * H * d < 2^31 is
  // checked on the host) and rows times the row stride fit a 24-bit product
  const unsigned rstride = (unsigned)(a.H * D);
  u32x4_t kst[SU], klst[SU], vst[SU];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = tid + 256 * i;
      const unsigned r = (unsigned)min(BN * kb + u / CPR, len - 1), c = u % CPR;
      const unsigned e = __umul24(r, rstride) + 8 * c;
      kst[i] = *(const u32x4_t*)(kseq + e);
      klst[i] = *(const u32x4_t*)(klseq + e);
      vst[i] = *(const u32x4_t*)(vseq + e);
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = tid + 256 * i;
      const int r = u / CPR, c = u % CPR;
      *(u32x4_t*)(Ks + r * KS + 8 * c) = kst[i];
      *(u32x4_t*)(Kl + r * KS + 8 * c) = klst[i];
      // channels 8c..8c+3 go to vpos(8c) = 32 (c >> 2) + 4 (c & 3), and
      // 8c+4..8c+7 sixteen elements further
      bf16_t* vrow = Vs + r * KS + 32 * (c >> 2) + 4 * (c & 3);
      *(uint2*)vrow = make_uint2(vst[i].x, vst[i].y);
      *(uint2*)(vrow + 16) = make_uint2(vst[i].z, vst[i].w);
    }
  };

  bf16x8_t ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.f;
  f32x4_t o[2][NDT], lacc[2];
  // minus the running maximum of the logits (log2 units) per column tile, in
  // all four entries: the logit accumulators start from it, so they hold the
  // logit minus the maximum.  0 before the first block, where the maximum is
  // always taken.
  f32x4_t negm[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    negm[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lacc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[ct][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  load_block(0);
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();  // every wave is done with the previous block
    store_block();
    __syncthreads();
    if (kb + 1 < nkb) load_block(kb + 1);
    if (!wave_active || kb > kb_diag) continue;
    const bool diag = kb == kb_diag;

    // logits Sᵀ[key][token] for the two key tiles and two column tiles
    f32x4_t sacc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      bf16x8_t kf[NS], kfl[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        kf[s] = *(const bf16x8_t*)(Ks + (16 * kt + n) * KS + 32 * s + 8 * q4);
        kfl[s] = *(const bf16x8_t*)(Kl + (16 * kt + n) * KS + 32 * s + 8 * q4);
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4_t acc = negm[ct];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[ct][s], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qfl[ct][s], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[s], qf[ct][s], acc, 0, 0, 0);
        }
        sacc[ct][kt] = acc;
      }
    }
    // V operands of the weighted sum, read now so that the LDS latency is
    // covered by the softmax: channels 32 (dt >> 1) + 4 (dt & 1) + 8 (lane & 3)
    // .. +3 of key rows 16 kt + (lane >> 2)
    bf16x8_t vf[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      s16x4 vv[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        vv[kt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(
            Vs + (16 * kt + (lane >> 2)) * KS + 16 * dt + 4 * (lane & 3)));
      vf[dt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(vv[0], vv[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
    if (diag) [[unlikely]] {
      // key 32kb + 16kt + 4q4 + r against token qw + 16ct + n
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kt + 4 * q4 + r > 16 * ct + n) sacc[ct][kt][r] = -INFINITY;
    }

    // online softmax with a lazily moved maximum.  The accumulators hold the
    // logits minus the running maximum, so the weights are their exponentials
    // as they stand, formed alongside the lane-local maxima.  If no lane holds
    // a value above 8 (log2 units), no column maximum exceeds the running one
    // by more than 8, nothing moves, and the cross-lane reduction is skipped.
    // Otherwise, and always on the first block, the columns whose maximum
    // moved rescale O and l and form their weights again.
    float w[2][8];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) w[ct][4 * kt + r] = __builtin_amdgcn_exp2f(sacc[ct][kt][r]);
    auto mx3 = [](float x, float y, float z) {
      return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z);
    };
    float ml[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float m = mx3(sacc[ct][0][0], sacc[ct][0][1], sacc[ct][0][2]);
      m = mx3(m, sacc[ct][0][3], sacc[ct][1][0]);
      m = mx3(m, sacc[ct][1][1], sacc[ct][1][2]);
      ml[ct] = __builtin_elementwise_maximum(m, sacc[ct][1][3]);
    }
    const bool first = kb == 0;
    if (first || __builtin_amdgcn_ballot_w64(ml[0] > 8.f || ml[1] > 8.f)) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        // the column maximum relative to the running one; on the first block
        // O and l are still zero and the maximum is taken as it is
        const float mb = xmax16(xmax32(ml[ct]));
        const float dm = (first || mb > 8.f) ? mb : 0.f;
        const float nm = negm[ct][0] - dm;
        negm[ct] = f32x4_t{nm, nm, nm, nm};
        if (!first) {
          const float alpha = __builtin_amdgcn_exp2f(-dm);
#pragma unroll
          for (int r = 0; r < 4; ++r) lacc[ct][r] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[ct][dt][r] *= alpha;
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) w[ct][4 * kt + r] = __builtin_amdgcn_exp2f(sacc[ct][kt][r] - dm);
      }
    }
    bf16x8_t pf[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      pf[ct] = __builtin_bit_cast(bf16x8_t, pack8_bf16(w[ct]));
      lacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[ct], lacc[ct], 0, 0, 0);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        o[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf[ct], o[ct][dt], 0, 0, 0);
  }

  // ---- normalize and store: lane holds channels 32s + 8q4 .. +7 ----------
  if (!wave_active) return;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int t = qw + 16 * ct + n;
    if (t < len) {
      const float inv = __builtin_amdgcn_rcpf(lacc[ct][0]);
      bf16_t* orow = a.out + ((s0 + t) * a.Hq + h) * D + 8 * q4;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = o[ct][2 * s][r] * inv;
          v[4 + r] = o[ct][2 * s + 1][r] * inv;
        }
        *(uint4*)(orow + 32 * s) = pack8_bf16(v);
      }
    }
  }
}

}  // namespace

}  // namespace gist

using namespace gist;

extern "C" size_t gist_prefill_workspace_bytes(int64_t n_tokens, int H, int d) {
  if (n_tokens < 0 || H <= 0 || d <= 0) return 0;
  return 2 * (size_t)n_tokens * H * d * sizeof(bf16_t);
}

extern "C" gist_status gist_prefill_attn(const void* q, const void* k, const void* v,
                                         const int32_t* seq_start, int B, int64_t n_tokens,
                                         int max_len, int Hq, int H, int d, float rope_base,
                                         float scale, void* out, void* workspace,
                                         size_t workspace_bytes, const gist_pool* pool, int layer,
                                         const int32_t* item_ids, void* stream) {
  clear_error();
  if (B < 0 || n_tokens < 0) return fail(GIST_ERR_INVALID_ARG, "gist_prefill_attn: B, n_tokens < 0");
  if (max_len < 1) return fail(GIST_ERR_INVALID_ARG, "gist_prefill_attn: max_len must be >= 1");
  if (H < 1 || Hq < H || Hq % H != 0)
    return fail(GIST_ERR_INVALID_ARG, "gist_prefill_attn: Hq must be a positive multiple of H");
  if (d != 64 && d != 128) return fail(GIST_ERR_UNSUPPORTED, "gist_prefill_attn: d must be 64 or 128");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(GIST_ERR_INVALID_ARG, "gist_prefill_attn: scale must be positive and finite");
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return fail(GIST_ERR_INVALID_ARG, "gist_prefill_attn: rope_base must be positive");
  if (pool) {
    if (pool->dtype != GIST_BF16)
      return fail(GIST_ERR_UNSUPPORTED, "gist_prefill_attn: the pool must be bf16");
    if (pool->H != H || pool->d != d)
      return fail(GIST_ERR_INVALID_ARG, "gist_prefill_attn: pool H and d must match");
    if (layer < 0 || layer >= pool->L)
      return fail(GIST_ERR_OUT_OF_RANGE, "gist_prefill_attn: layer out of range");
    if (!item_ids && B > 0) return fail(GIST_ERR_INVALID_ARG, "gist_prefill_attn: item_ids is NULL");
  }
  if (B == 0 || n_tokens == 0) return GIST_OK;
  if (!q || !k || !v || !seq_start || !out || !workspace)
    return fail(GIST_ERR_INVALID_ARG, "gist_prefill_attn: NULL tensor argument");
  for (const void* p : {q, k, v, (const void*)out, (const void*)workspace})
    if (((uintptr_t)p & 15) != 0)
      return fail(GIST_ERR_INVALID_ARG, "gist_prefill_attn: tensors must be 16-byte aligned");
  if (workspace_bytes < gist_prefill_workspace_bytes(n_tokens, H, d))
    return fail(GIST_ERR_INVALID_ARG, "gist_prefill_attn: workspace too small");
  const int64_t prep_blocks = ((int64_t)max_len * H * (d / 16) + 255) / 256;
  const int64_t qblocks = (max_len + 127) / 128;
  if (prep_blocks > INT32_MAX || B > 65535 || Hq > 65535 || (int64_t)max_len * H * d >= (1LL << 31))
    return fail(GIST_ERR_UNSUPPORTED, "gist_prefill_attn: shape too large for one launch");

  PrefillArgs a;
  a.q = (const bf16_t*)q;
  a.k = (const bf16_t*)k;
  a.v = (const bf16_t*)v;
  a.seq_start = seq_start;
  a.k_rot = (bf16_t*)workspace;
  a.out = (bf16_t*)out;
  a.T = n_tokens;
  a.B = B;
  a.max_len = max_len;
  a.Hq = Hq;
  a.H = H;
  a.G = Hq / H;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.pool = pool ? (bf16_t*)pool->storage + (int64_t)layer * pool->N * record_elems(pool) : nullptr;
  a.N = pool ? pool->N : 0;
  a.kk = pool ? pool->k : 0;
  a.item_ids = pool ? item_ids : nullptr;
  make_rope_freqs(a.freqs, d, rope_base);
  hipStream_t s = (hipStream_t)stream;
  const dim3 pgrid((unsigned)prep_blocks, (unsigned)B);
  const dim3 agrid((unsigned)qblocks, (unsigned)Hq, (unsigned)B);
  if (d == 64) {
    hipLaunchKernelGGL(prefill_prep<64>, pgrid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(prefill_attn<64>, agrid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(prefill_prep<128>, pgrid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(prefill_attn<128>, agrid, dim3(256), 0, s, a);
  }
  return check_launch("gist_prefill_attn");
}
