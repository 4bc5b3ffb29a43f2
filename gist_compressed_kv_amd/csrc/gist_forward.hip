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
// Three kernels:
//  * gist_fwd_mfma  bf16 activations, 2 <= ell <= 64, k+k'+ell <= 128, bf16
//    or fp8 gist pools.  One workgroup (4 wave64s) per (pair, KV head).  All
//    keys of the pair are staged once in LDS (K row-major with RoPE applied on
//    load, V transposed), and each wave owns 16 query tokens and loops over
//    the G query heads of the GQA group, so every K/V tile in LDS serves all
//    G heads.  Logits are computed transposed, Sᵀ = K·Qᵀ, with
//    v_mfma_f32_16x16x32_bf16, so each lane ends up holding four keys of one
//    token: exactly the B operand layout of the P·V product (Oᵀ = Vᵀ·Pᵀ,
//    v_mfma_f32_16x16x32_bf16 over pairs of key tiles, 16x16x16 for an
//    unpaired last one), and the softmax never leaves
//    registers.  All keys of a token are in registers at once, so the row
//    maximum is exact before the exponentials; causally invisible tiles are
//    skipped.
//  * gist_fwd_eos  ell = 1 (the EOS token over item gist + query gist +
//    itself), bf16 activations, bf16 or fp8 gist pools, G <= 16, k+k' <= 32.
//    One wave per (pair, KV head); the G query heads are the MFMA columns.
//  * gist_fwd_valu<T, D, MAXH>  every other shape (bf16 with ell > 64 or
//    long gists, and fp32).  One wave64 per (pair, KV head, token); four
//    16-lane rows split the heads of the group (or, for G < 4, the keys), each
//    lane holds d/16 channels including both members of its RoPE pairs, dot
//    products reduce across the 16-lane row with DPP.
#include <atomic>
#include <cfloat>
#include <type_traits>
#include <utility>

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
  // q^(2^b), b = 0..5, with q = base^(-2/d): rev_i = rev_0 * prod over the
  // set bits b of i, for kernels that form a lane's frequency from scalars
  double rev_step[6];
  // fp8 pools: this layer's scales [N][2][H] (and [qN][2][H]); pool offsets
  // are then in bytes
  const float* pool_scales;
  const float* qpool_scales;
  // the VALU kernel produces only the last token's rows (q, out: one row per pair)
  int last_only;
  // paged gists (EOS and l >= 2 kernels): item_ids and q_ids are block indices of a paged
  // cache [N][H][block_size][d] (N blocks; qN = N); the item gist is rows
  // 0..k-1 of its block, the query gist rows q_row0..q_row0+k'-1 of its block
  int paged;
  const void* paged_k;
  const void* paged_v;
  int block_size;
  int q_row0;
  // fp8 paged gist: one scale per (block, KV head) for K and one for V
  const float* paged_kscales;
  const float* paged_vscales;
};

// (cos, sin) of channel pair i at position pos0, evaluated on the host in
// double: the EOS kernel's single token of every pair sits at pos0
struct CsPos0 {
  float v[kMaxHalfDim][2];
};

// What one workgroup of the l >= 2 kernel reads and writes: its call's
// activations, outputs, ids and pool layer, and its (pair, KV head)
struct Slice {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* out;
  const int32_t* item_ids;
  const int32_t* q_ids;
  int64_t pool_off, qpool_off;  // first element (fp8: byte) of the layer
  const float* pool_scales;     // fp8: the layer's scales
  const float* qpool_scales;
  int p, g;                     // pair within the call, KV head
  int bid;                      // workgroup index of the launch
};

// Groups of one grouped launch (gist_attn_forward_grouped), passed by value
constexpr int kMaxGroups = 32;
struct GroupEntry {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* out;
  const int32_t* item_ids;
  const int32_t* q_ids;
  int64_t layer;
};
struct GroupTable {
  // running count of (pair, KV head) units after group i (INT_MAX past the
  // last): the l >= 2 kernel's workgroups, the EOS kernel's waves
  int wg_end[kMaxGroups];
  int units;  // all groups' units
  GroupEntry e[kMaxGroups];
  int64_t pool_layer_stride, qpool_layer_stride;    // elements (fp8: bytes) per layer
  int64_t scale_layer_stride, qscale_layer_stride;  // fp8 scales per layer
};
// the grouped EOS launch passes all three by value
static_assert(sizeof(FwdArgs) + sizeof(CsPos0) + sizeof(GroupTable) <= 4096,
              "kernel arguments within 4 KiB");

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

// max of three floats: IEEE-754-2019 maximum (NaN-propagating), which gfx950
// executes as one v_maximum3_f32 with no NaN canonicalization of its inputs
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// max of x over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four rows of an
// MFMA 16x16 accumulator column) with the gfx950 lane swaps: after a swap of
// x with itself, one result holds the partner's value in one half of the
// wave and the lane's own value in the other, the second result the
// reverse, so the maximum of x and both is the pair's maximum.  The values
// stay in VALU registers (no LDS round trip, unlike ds_bpermute).
__device__ __forceinline__ float col4_max(float x) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax3(x, __uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax3(x, __uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Orders the LDS accesses of one wave around an exchange between its lanes
// (one lane writes what another reads).  A wave's LDS accesses already
// complete in program order, so this emits no instruction; it keeps the
// compiler from moving or reusing a lane's LDS loads across the point as if
// no other lane wrote there.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1 in order.
template <class F, int... I>
__device__ __forceinline__ void for_each_const_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void for_each_const(F&& f) {
  for_each_const_impl(f, std::make_integer_sequence<int, N>{});
}


// Source row of key j (K or V part selected by `v`) of pair p, KV head g.
__device__ __forceinline__ const bf16_t* key_row(const FwdArgs& a, const bf16_t* gK,
                                                 const bf16_t* qK, int p, int g, int j, int kg,
                                                 int D, bool v) {
  if (j < a.k) return gK + (int64_t)((v ? a.H * a.k : 0) + j) * D;
  if (j < kg) return qK + (int64_t)((v ? a.H * a.kq : 0) + (j - a.k)) * D;
  const bf16_t* base = (const bf16_t*)(v ? a.v_new : a.k_new);
  return base + (((int64_t)p * a.ell + (j - kg)) * a.H + g) * D;
}

// Vᵀ element (channel row r, key column c) sits at r*VS + 4*(r >> 3) + c,
// with VS = 16 or 48 (mod 64) elements.  LDS serves 128 bytes per clock from
// 32 four-byte banks, so the sixteen lanes of one 8-byte read phase (MFMA
// rows n = 0..15 of one key group, same column) must cover all 32 banks.
// Those lanes read rows r = R + 8b + a (a, b < 4; R a per-d-tile constant,
// see vt_row): the row stride (8 or 24 dwords mod 32) puts a on banks
// 0/8/16/24 and the 4-element pad per 8-row block puts b on 0/2/4/6.
__device__ __forceinline__ constexpr int vt_off(int r, int c, int vs) {
  return r * vs + 4 * (r >> 3) + c;
}
__device__ __host__ constexpr int vt_stride(int keys) {
  return (keys % 64 == 16 || keys % 64 == 48) ? keys : keys + 16;
}

template <int D, int NKT>
struct MfmaLds {
  static constexpr int VS = vt_stride(16 * NKT);  // Vᵀ row stride (elements)
  // K rows hold D channels, no padding: the 16-byte chunks of row r are
  // XOR-swizzled by r & 7 (kchunk), so sixteen consecutive rows read at one
  // chunk position hit distinct banks.  Two arrays: the bf16 value of each
  // key (hi) and the bf16 rounding of what hi leaves out (lo).
  static constexpr size_t k_bytes(int nk_pad) { return (size_t)nk_pad * D * sizeof(bf16_t); }
  static constexpr size_t vt_bytes = ((size_t)D * VS + 4 * (D / 8)) * sizeof(bf16_t);
  static constexpr size_t kv_bytes(int nk_pad) { return 2 * k_bytes(nk_pad) + vt_bytes; }
  // four per-wave transpose buffers of 16 rows x 2*D bytes
  static constexpr size_t xpose_bytes = 4 * 16 * 2 * D;
  static constexpr size_t bytes(int nk_pad) { return kv_bytes(nk_pad) + xpose_bytes; }
};

// element offset of 16-byte chunk c of K row r
template <int D>
__device__ __forceinline__ int kchunk(int r, int c) {
  return r * D + ((c ^ (r & 7)) << 3);
}

// Split fp32 values into a bf16 pair hi + lo: hi is the nearest bf16 of x,
// lo the nearest bf16 of x - hi (exact in fp32), so hi + lo carries 16
// significant bits.  The product q·k of two such pairs, taken as
// qhi·khi + qlo·khi + qhi·klo on the matrix cores, has a relative error of
// about 2^-16, against 2^-8 for the product of the rounded values.
// Per pair of values: one conversion for hi, one v_dot2_f32_bf16 per value
// for the remainder and one conversion for lo.  The remainder x - hi is read
// straight off the packed pair: dot2(hi pair, (-1, 0), x0) = x0 - hi0 and
// dot2(hi pair, (0, -1), x1) = x1 - hi1.  Both products are exact and the
// difference is an fp32 number, so the result is exact whatever the
// instruction's internal rounding.
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2v;
struct SplitOnes {
  bf16x2v lo, hi;  // bf16 pairs (-1, 0) and (0, -1), low half first
};
// The two pairs live in registers: as an instruction constant, the
// compiler encodes (-1, 0) as the inline constant -1.0, which a packed-bf16
// operand does not read as that pair.  (The asm is not volatile: a volatile
// one counts as a possible memory write, which turns later uniform loads
// into vector loads.)
__device__ __forceinline__ SplitOnes split_ones() {
  uint32_t m_lo = 0x0000bf80u, m_hi = 0xbf800000u;
  asm("" : "+s"(m_lo), "+s"(m_hi));
  return SplitOnes{__builtin_bit_cast(bf16x2v, m_lo), __builtin_bit_cast(bf16x2v, m_hi)};
}
__device__ __forceinline__ void split8_bf16(const float* y, uint4& hi, uint4& lo, const SplitOnes& m) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = pack2_bf16(y[2 * i], y[2 * i + 1]);
    const bf16x2v wv = __builtin_bit_cast(bf16x2v, w);
    h[i] = w;
    l[i] = pack2_bf16(__builtin_amdgcn_fdot2_f32_bf16(wv, m.lo, y[2 * i], false),
                      __builtin_amdgcn_fdot2_f32_bf16(wv, m.hi, y[2 * i + 1], false));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// D: head_dim.  NKT: maximum number of 16-key tiles (keys <= 16*NKT).
// QPF: Q ring depth: once head h has taken its Q out of the ring, the
// loads of heads h+1 .. h+QPF are in flight.  The instances with QPF = 1 and
// a compile-time group size serve single-generation launches: they load one
// head before the staging and keep three in flight after it.
// GT: the GQA group size when known at compile time (0 = taken from the
// arguments).  With GT > 0 the head loop is fully unrolled, so the compiler
// knows exactly which loads each wait has to cover and never drains the
// output stores (which share the vector-memory counter) before a Q load.
//
// LDS holds the pair's keys in reverse order: key κ (0 = first gist row) is
// row nk_pad-1-κ of Khi/Klo and column nk_pad-1-κ of Vᵀ.  A wave visits its
// key tiles from the causal edge backwards (j = 0 is the tile with the last
// visible key), so tile j sits at a compile-time offset from one per-wave
// base address, and only tiles j = 0 and j = 1 can hold keys that some token
// of the wave may not see.
// Precision: the rotated Q and the rotated new keys are carried as bf16
// pairs hi + lo (split8_bf16) and the logits take three products per tile,
// K_hi·Q_hi + K_hi·Q_lo + K_lo·Q_hi, so they hold the fp32 rotation to about
// 2^-16; the stored gist K is bf16 already (its lo rows are zero).  P is
// rounded to bf16 for the P·V product.
// RoPE: wave w rotates the new keys of token block w and, in the same lanes,
// the query rows of that block (lane (n, q4): token 16w + n, channel pairs
// 32s + 8*q4 + e), so each lane evaluates the angles of its own token once
// and uses them for both; no angle table and one barrier.
// LAST: only the last token's rows are produced (q and out hold one token
// per pair).  The keys are staged as for every token; every wave takes the
// 16-token block that holds the last token and the group's heads are spread
// over the four waves (head h on wave h mod 4), each storing that token alone.
// FP8: the gist pools hold E4M3 codes.  Each staged gist element is the
// decoded code times its block's scale in fp32, staged as a bf16 pair like
// the new keys (V: rounded to bf16 once); the rest of the kernel is the bf16
// one.
// Waves per SIMD: four workgroups per CU fit the LDS at d = 64 with up to
// 80 keys (so up to 128 VGPRs); otherwise two (up to 256 VGPRs).
template <int D, int NKT, int QPF, int GT, bool LAST, bool FP8>
__device__ __forceinline__ void mfma_body(const FwdArgs& a, const Slice& sl, int nk_pad) {
  extern __shared__ __align__(16) bf16_t smem[];
  constexpr int VS = MfmaLds<D, NKT>::VS;
  constexpr int NS = D / 32;   // 32-channel k-steps of the Q·Kᵀ product
  constexpr int NP = NS / 2;   // RoPE: step s pairs with step s + NP
  constexpr int NDT = D / 16;  // 16-channel tiles of the output
  constexpr int CV = D / 8;    // V staging units per key pair (8 channels)
  constexpr int IT = D / 32;   // V staging units per thread (nk_pad <= 128)
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int RPI = 64 / CPR; // token rows per coalesced instruction
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  bf16_t* Khi = smem;                   // [nk_pad][D], reversed key order
  bf16_t* Klo = smem + nk_pad * D;      // [nk_pad][D]
  bf16_t* Vt = smem + 2 * nk_pad * D;   // [D][VS], reversed key order
  char* xbuf = (char*)smem + MfmaLds<D, NKT>::kv_bytes(nk_pad);

  const int p = sl.p;
  const int g = sl.g;
  const int tid = threadIdx.x;
  const int kg = a.k + a.kq;
  const int ell = a.ell;
  const int nk = kg + ell;
  const int Hq = a.Hq, G = GT > 0 ? GT : a.G;
  bf16_t* out = (bf16_t*)sl.out;
  const SplitOnes so = split_ones();
  // Single-generation launches (the instances with a one-head Q ring and a
  // compile-time group size are used only when every workgroup of the grid
  // is resident at once): the SIMD's issue arbiter favours the oldest wave,
  // so the waves dispatched last fell behind and finished alone.  Instead
  // each wave's priority follows its remaining work (see the head loop),
  // and every wave stages its keys at the top priority.
  constexpr bool LPT = QPF == 1 && GT > 0 && !LAST;

  // ---- issue the first QPF heads' Q loads of this wave first: they do not
  // depend on the item id, so HBM traffic starts while the id is in flight --
  // (wave index read through readfirstlane so every per-wave quantity below
  // is a scalar and the tile loops branch on SGPRs)
  // The token block of a wave rotates with the workgroup index: later blocks
  // see more keys, and the rotation spreads that extra work over the SIMDs.
  const int wv = __builtin_amdgcn_readfirstlane(((tid >> 6) + sl.bid) & 3);
  const int lane = tid & 63;
  const int n = lane & 15, q4 = lane >> 4;
  const int t0 = LAST ? 16 * ((ell - 1) >> 4) : 16 * wv;
  const int t = t0 + n;
  const bool wave_active = LAST ? wv < G : t0 < ell;
  const bool tvalid = t < ell;
  // rows past ell read the last valid token (finite values, never stored)
  const int tl = tvalid ? t : ell - 1;
  // the new keys this wave rotates and stages: token block wv
  const int tk = 16 * wv + n;
  const int tkl = tk < ell ? tk : ell - 1;
  // Q and O move between HBM and registers in a coalesced layout: lane l
  // covers chunk l % CPR (8 channels, 16 bytes) of token row l / CPR, so
  // every 128-byte line of a (token, head) row is read or written whole by
  // one instruction.  A per-wave LDS buffer converts to and from the MFMA
  // operand layout.  Addresses are a wave-uniform base plus 32-bit lane
  // offsets (scalar-base addressing form).
  // Q is read once, in whole lines: its loads are non-temporal, as are the
  // bf16 V staging loads (whole rows); the K staging loads touch parts of
  // lines that other loads then reuse and are ordinary
  const int cl = lane % CPR, rl = lane / CPR;
  const int64_t pair_off = (int64_t)p * (LAST ? 1 : ell) * Hq * D;
  const char* qpair = (const char*)((const bf16_t*)sl.q + pair_off);
  char* opair = (char*)(out + pair_off);
  uint32_t qlane[NS], olane[NS];
  bool ovalid[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int tc = t0 + rl + RPI * s;
    // LAST: every token row reads the one Q row given, and only the last
    // token is stored, at the pair's one output row
    const int tq = LAST ? 0 : (tc < ell ? tc : ell - 1);
    ovalid[s] = LAST ? tc == ell - 1 : tc < ell;
    qlane[s] = (uint32_t)(((tq * Hq + g * G) * D + 8 * cl) * 2);
    olane[s] = (uint32_t)((((LAST ? 0 : tc) * Hq + g * G) * D + 8 * cl) * 2);
  }
  // Q ring held in native vectors (not the HIP uint4 struct) so it always
  // stays in registers.  QPF heads are loaded before the staging; after it
  // the ring holds DEP heads in flight (three in single-generation launches)
  constexpr int DEP = LPT ? 3 : QPF;
  constexpr int RQ = DEP > QPF ? DEP : QPF;
  u32x4_t raw[RQ][NS];
  auto load_q = [&](auto slot, const int hq) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      raw[decltype(slot)::value][s] =
          __builtin_nontemporal_load((const u32x4_t*)(qpair + qlane[s] + (uint32_t)(hq * D) * 2));
  };
#pragma unroll
  for (int i = 0; i < QPF; ++i) {
    // LAST: slot 0 holds this wave's first head
    const int hq = LAST ? (wv < G ? wv : G - 1) : (i < G ? i : G - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s)
      raw[i][s] = __builtin_nontemporal_load((const u32x4_t*)(qpair + qlane[s] + (uint32_t)(hq * D) * 2));
  }

  __builtin_amdgcn_sched_barrier(0);

  // ---- ids (bounds-checked; a bad id turns the pair's rows into NaN) ------
  const int32_t item = sl.item_ids[p];
  int32_t qid = 0;
  bool bad = item < 0 || item >= a.N;
  if (a.kq) {
    qid = sl.q_ids[p];
    bad = bad || qid < 0 || qid >= a.qN;
  }
  if (bad) {
    const int per_t = G * D, nt = LAST ? 1 : ell;
    for (int u = tid; u < nt * per_t; u += 256) {
      const int t = u / per_t, r = u - t * per_t;
      out[((int64_t)p * nt + t) * Hq * D + (int64_t)g * G * D + r] = nan_value<bf16_t>();
    }
    return;
  }
  typedef std::conditional_t<FP8, uint8_t, bf16_t> C;  // gist element
  // first K and V rows of the item gist and of the query gist: a pool record
  // (K of every head, then V of every head), or rows of the item's and the
  // query's blocks in a paged cache [N][H][block_size][d]
  const C *gK, *gV, *qK = nullptr, *qV = nullptr;
  if (a.paged) {
    const int64_t ib = ((int64_t)item * a.H + g) * a.block_size * D;
    gK = (const C*)a.paged_k + ib;
    gV = (const C*)a.paged_v + ib;
    if (a.kq) {
      const int64_t qb = (((int64_t)qid * a.H + g) * a.block_size + a.q_row0) * D;
      qK = (const C*)a.paged_k + qb;
      qV = (const C*)a.paged_v + qb;
    }
  } else {
    gK = (const C*)a.pool + sl.pool_off + (int64_t)item * 2 * a.H * a.k * D +
         (int64_t)g * a.k * D;
    gV = gK + (int64_t)a.H * a.k * D;
    if (a.kq) {
      qK = (const C*)a.qpool + sl.qpool_off + (int64_t)qid * 2 * a.H * a.kq * D +
           (int64_t)g * a.kq * D;
      qV = qK + (int64_t)a.H * a.kq * D;
    }
  }
  // fp8: K and V scales of the item gist and of the query gist (scalars)
  float ski = 1.f, svi = 1.f, skq = 1.f, svq = 1.f;
  if constexpr (FP8) {
    if (a.paged) {
      ski = a.paged_kscales[(int64_t)item * a.H + g];
      svi = a.paged_vscales[(int64_t)item * a.H + g];
      if (a.kq) {
        skq = a.paged_kscales[(int64_t)qid * a.H + g];
        svq = a.paged_vscales[(int64_t)qid * a.H + g];
      }
    } else {
      const float* si = sl.pool_scales + (int64_t)item * 2 * a.H;
      ski = si[g];
      svi = si[a.H + g];
      if (a.kq) {
        const float* sq = sl.qpool_scales + (int64_t)qid * 2 * a.H;
        skq = sq[g];
        svq = sq[a.H + g];
      }
    }
  }
  // (set after the id and scale loads: the compiler takes s_setprio for a
  // possible memory write and would otherwise turn those scalar loads into
  // vector loads that wait for the Q prefetch)
  if constexpr (LPT) __builtin_amdgcn_s_setprio(3);
  // Eight gist elements (channels ch.., K or V of gist key j < kg) as fp32.
  // fp8 gist rows are decoded and multiplied by their block's scale.  Every
  // lane issues one 16-byte load (fp8: the aligned 16 codes that hold its 8).
  auto gist_row = [&](int j, bool v) -> const C* {
    return j < a.k ? (v ? gV : gK) + (int64_t)j * D : (v ? qV : qK) + (int64_t)(j - a.k) * D;
  };
  auto gist_raw = [&](int j, bool v, int ch) -> u32x4_t {
    if constexpr (FP8) return *(const u32x4_t*)(gist_row(j, v) + (ch & ~15));
    else return *(const u32x4_t*)(gist_row(j, v) + ch);
  };
  auto gist_f32 = [&](const u32x4_t& raw, int j, bool v, int ch, float* f) {
    if constexpr (FP8) {
      const float sc = j < a.k ? (v ? svi : ski) : (v ? svq : skq);
      decode4_e4m3((ch & 8) ? raw.z : raw.x, f);
      decode4_e4m3((ch & 8) ? raw.w : raw.y, f + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= sc;
    } else {
      unpack8(make_uint4(raw.x, raw.y, raw.z, raw.w), f);
    }
  };
  // V of key j (< nk) as eight bf16: gist rows through gist_f32 (fp8:
  // rounded to bf16 once), new rows as loaded
  auto v_load = [&](int j, int ch) -> u32x4_t {
    const bf16_t* nrow = (const bf16_t*)sl.v_new + (((int64_t)p * ell + (j < kg ? 0 : j - kg)) * a.H + g) * D;
    if constexpr (FP8) {
      // one unconditional load per lane: its gist row or its new row
      const bool gist = j < kg;
      return *(const u32x4_t*)(gist ? (const void*)(gist_row(j, true) + (ch & ~15))
                                    : (const void*)(nrow + ch));
    } else {
      // whole rows, read once: non-temporal
      return __builtin_nontemporal_load((const u32x4_t*)(j < kg ? gist_row(j, true) + ch : nrow + ch));
    }
  };
  auto v_bf16 = [&](const u32x4_t& raw, int j, int ch) -> uint4 {
    if constexpr (FP8) {
      if (j < kg) {
        float f[8];
        gist_f32(raw, j, true, ch, f);
        return pack8_bf16(f);
      }
    }
    return make_uint4(raw.x, raw.y, raw.z, raw.w);
  };

  // ---- issue every staging load of this thread ----------------------------
  // Every load below is unconditional (out-of-range units read a valid row
  // and are dropped or zeroed afterwards), so the compiler can count the
  // loads in flight exactly and later waits never have to drain the Q
  // prefetch.
  // new keys of token block wv, in the MFMA-operand channel layout of this
  // lane's own query token: step s holds channels 32s + 8*q4 .. +7
  u32x4_t kn[NS];
  {
    const bf16_t* krow = (const bf16_t*)sl.k_new + (((int64_t)p * ell + tkl) * a.H + g) * D + 8 * q4;
#pragma unroll
    for (int s = 0; s < NS; ++s) kn[s] = *(const u32x4_t*)(krow + 32 * s);
  }
  // first gist K unit of this thread (the rest, if kg*CPR > 256, below)
  const int gu_row = tid / CPR, gu_c = tid % CPR;
  const u32x4_t graw = gist_raw(gu_row < kg ? gu_row : 0, false, 8 * gu_c);
  // V unit (key pair jp, 8-channel chunk cv), chunks fastest: the lanes of
  // one instruction read whole rows of eight keys (pairs past nk read row 0)
  u32x4_t v0[IT], v1[IT];
  const int npairs = nk_pad >> 1;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int u = tid + 256 * it;
    const int jp = u / CV, cv = u - jp * CV;
    v0[it] = v_load(2 * jp < nk ? 2 * jp : 0, 8 * cv);
    v1[it] = v_load(2 * jp + 1 < nk ? 2 * jp + 1 : 0, 8 * cv);
  }

  // keep the staging loads together (the Q prefetch above was issued first
  // and has returned by the time the LDS stores wait for them)
  __builtin_amdgcn_sched_barrier(0);

  // ---- RoPE angles of this lane's token(s) while the loads are in flight:
  // channel pairs i = 32s + 8*q4 + e (s < NP), position pos0 + token --------
  // The frequency of pair i is rev_i = rev_0 * r^i with r = base^(-2/d);
  // this lane's pairs are rev_{32s+e} (scalars) times r^(8*q4), formed from
  // the scalar powers r^8 and r^16, so no lane-indexed table is read.
  float qc[NP][8], qsn[NP][8];
  const double rq = ((q4 & 1) ? a.rev_step[3] : 1.0) * ((q4 & 2) ? a.rev_step[4] : 1.0);
  auto angles = [&](int tok, float (*c)[8], float (*sn)[8]) {
    const double pos = (double)a.pos0 + tok;  // no int32 overflow near INT_MAX
#pragma unroll
    for (int s = 0; s < NP; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        rope_cos_sin(pos, a.freqs.rev[32 * s + e] * rq, c[s][e], sn[s][e]);
  };
  angles(tl, qc, qsn);

  // ---- new keys: rotate (fp32), split into bf16 hi + lo, store reversed ----
  if (16 * wv < ell) {
    float kcs[NP][8], ksn[NP][8];
    if constexpr (LAST) angles(tkl, kcs, ksn);
    const float(*c)[8] = LAST ? kcs : qc;
    const float(*sn)[8] = LAST ? ksn : qsn;
    if (tk < ell) {
      const int R = nk_pad - 1 - (kg + tk);
#pragma unroll
      for (int s = 0; s < NP; ++s) {
        float xl[8], xh[8], yl[8], yh[8];
        unpack8(make_uint4(kn[s].x, kn[s].y, kn[s].z, kn[s].w), xl);
        unpack8(make_uint4(kn[s + NP].x, kn[s + NP].y, kn[s + NP].z, kn[s + NP].w), xh);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          yl[e] = __builtin_fmaf(xl[e], c[s][e], -(xh[e] * sn[s][e]));
          yh[e] = __builtin_fmaf(xh[e], c[s][e], xl[e] * sn[s][e]);
        }
        uint4 hl, ll, hh, lh;
        split8_bf16(yl, hl, ll, so);
        split8_bf16(yh, hh, lh, so);
        const int ol = kchunk<D>(R, 4 * s + q4), oh = kchunk<D>(R, 4 * (s + NP) + q4);
        *(uint4*)(Khi + ol) = hl;
        *(uint4*)(Klo + ol) = ll;
        *(uint4*)(Khi + oh) = hh;
        *(uint4*)(Klo + oh) = lh;
      }
    }
  }
  // ---- gist K rows (hi: the stored value; fp8: decoded times scale, lo its
  // remainder) and zero padding rows past nk ------------------------------
  auto put_gist = [&](const u32x4_t& raw, int j, int c) {
    const int R = nk_pad - 1 - j;
    uint4 hi, lo;
    if constexpr (FP8) {
      float f[8];
      gist_f32(raw, j, false, 8 * c, f);
      split8_bf16(f, hi, lo, so);
    } else {
      hi = make_uint4(raw.x, raw.y, raw.z, raw.w);
      lo = make_uint4(0, 0, 0, 0);
    }
    *(uint4*)(Khi + kchunk<D>(R, c)) = hi;
    *(uint4*)(Klo + kchunk<D>(R, c)) = lo;
  };
  if (gu_row < kg) put_gist(graw, gu_row, gu_c);
  for (int u = tid + 256; u < kg * CPR; u += 256) {  // long gists only
    const int j = u / CPR, c = u % CPR;
    put_gist(gist_raw(j, false, 8 * c), j, c);
  }
  for (int u = tid; u < (nk_pad - nk) * CPR; u += 256) {
    const int R = nk_pad - 1 - (nk + u / CPR), c = u % CPR;
    *(uint4*)(Khi + kchunk<D>(R, c)) = make_uint4(0, 0, 0, 0);
    *(uint4*)(Klo + kchunk<D>(R, c)) = make_uint4(0, 0, 0, 0);
  }
  // ---- V: transpose, store (reversed) ---------------------------------------
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int u = tid + 256 * it;
    const int jp = u / CV, cv = u - jp * CV;
    if (jp < npairs) {
      // keys 2jp, 2jp+1 land in reversed columns nk_pad-2-2jp (key 2jp+1)
      // and nk_pad-1-2jp (key 2jp): one dword, high key in the low half
      const uint4 zero = make_uint4(0, 0, 0, 0);
      const uint4 w0 = 2 * jp < nk ? v_bf16(v0[it], 2 * jp, 8 * cv) : zero;
      const uint4 w1 = 2 * jp + 1 < nk ? v_bf16(v1[it], 2 * jp + 1, 8 * cv) : zero;
      const uint32_t a0[4] = {w0.x, w0.y, w0.z, w0.w};
      const uint32_t a1[4] = {w1.x, w1.y, w1.z, w1.w};
      const int col = nk_pad - 2 - 2 * jp;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // channel 8cv+2e: low halves; channel 8cv+2e+1: high halves
        const int r = 8 * cv + 2 * e;
        *(uint32_t*)(Vt + vt_off(r, col, VS)) = (a1[e] & 0xffffu) | (a0[e] << 16);
        *(uint32_t*)(Vt + vt_off(r + 1, col, VS)) = (a1[e] >> 16) | (a0[e] & 0xffff0000u);
      }
    }
  }

  // per-wave transpose buffer: 16 rows of 2*D bytes, chunk c of row r stored
  // at chunk c ^ r.  A 16-byte access is served eight lanes per clock; the
  // coalesced side has those lanes on one row (distinct chunks), the MFMA
  // side has them on rows 0..7 of one chunk, which the XOR sends to eight
  // distinct chunks: both sides are free of bank conflicts.
  char* xb = xbuf + (tid >> 6) * (16 * 2 * D);
  auto xpos = [](int r, int c) -> uint32_t {
    return (uint32_t)(r * 2 * D + ((c ^ r) & (CPR - 1)) * 16);
  };
  uint32_t xw[NS], xr[NS];  // coalesced-layout and MFMA-layout slots
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    xw[s] = xpos(rl + RPI * s, cl);
    xr[s] = xpos(n, 4 * s + q4);
  }

  // Q of the head in ring slot i: to the MFMA layout through the wave's
  // buffer, rotated in fp32 and split into bf16 hi + lo
  auto prep_q = [&](auto slot, bf16x8_t* qh, bf16x8_t* ql) {
    constexpr int i = decltype(slot)::value;
    uint4 qm[NS];
    wave_lds_sync();  // the previous reads of the buffer are done
#pragma unroll
    for (int s = 0; s < NS; ++s) *(u32x4_t*)(xb + xw[s]) = raw[i][s];
    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4_t m = *(const u32x4_t*)(xb + xr[s]);
      qm[s] = make_uint4(m.x, m.y, m.z, m.w);
    }
#pragma unroll
    for (int s = 0; s < NP; ++s) {
      float xl[8], xh[8], yl[8], yh[8];
      unpack8(qm[s], xl);
      unpack8(qm[s + NP], xh);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        yl[e] = __builtin_fmaf(xl[e], qc[s][e], -(xh[e] * qsn[s][e]));
        yh[e] = __builtin_fmaf(xh[e], qc[s][e], xl[e] * qsn[s][e]);
      }
      uint4 h0, l0, h1, l1;
      split8_bf16(yl, h0, l0, so);
      split8_bf16(yh, h1, l1, so);
      qh[s] = __builtin_bit_cast(bf16x8_t, h0);
      ql[s] = __builtin_bit_cast(bf16x8_t, l0);
      qh[s + NP] = __builtin_bit_cast(bf16x8_t, h1);
      ql[s + NP] = __builtin_bit_cast(bf16x8_t, l1);
    }
  };
  // the wave's first head, before the barrier (its buffer is its own)
  bf16x8_t qh[NS], ql[NS];
  if (wave_active) prep_q(std::integral_constant<int, 0>{}, qh, ql);
  __syncthreads();
  if (!wave_active) return;

  const int tlast = min(t0 + 15, ell - 1);
  const int nkt = (kg + tlast + 1 + 15) >> 4;  // tiles holding any visible key
  // reversed-order base rows of tile j = 0 (key tile nkt-1); row0 is a
  // multiple of 16, so lane n reads rows with (row & 7) == (n & 7) in every
  // tile and its swizzled chunk offsets are fixed
  const int row0 = nk_pad - 16 * nkt;
  int koff[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) koff[s] = kchunk<D>(row0 + n, 4 * s + q4);
  // (the block pad of vt_off is the same for every d-tile: vt_row(dt, n) >> 3
  // differs from vt_row(0, n) >> 3 by 4*(dt >> 1), folded into the offsets)
  const bf16_t* vbase = Vt + vt_off(vt_row(0, n), row0 + 4 * q4, VS);
  // MFMA row m of tile j holds key 16*(nkt-1-j) + 15 - m; the S output slot
  // r of lane group q4 is row m = 4*q4 + r.  Visibility: key <= kg + t.
  const int lim = kg + t - (16 * (nkt - 1) + 15 - 4 * q4);  // key <= kg+t  <=>  -r - 16j <= lim
  // the causal bias of tiles j = 0 and 1 (0 or -inf per logit), the same for
  // every head: computed once and used as the accumulators' initial value
  f32x4_t bias0, bias1;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    bias0[r] = -r <= lim ? 0.f : -INFINITY;
    bias1[r] = -r - 16 <= lim ? 0.f : -INFINITY;
  }
  // (opaque, so the compiler keeps them in registers rather than rebuilding
  // them for every head)
  asm volatile("" : "+v"(bias0), "+v"(bias1));
  const float sl2 = a.scale_log2;
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4v;
  u32x4_t ones_w = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};  // eight bf16 1.0
  asm volatile("" : "+v"(ones_w));
  const bf16x8_t ones8 = __builtin_bit_cast(bf16x8_t, ones_w);
  const bf16x4v ones = __builtin_shufflevector(ones8, ones8, 0, 1, 2, 3);

  // Attention of one query head (Q in qh/ql), output rows of head hh.
  auto attend = [&](const int hh) {
    // logits Sᵀ = K·Qᵀ (unscaled; scale*log2 e is applied in the exponent)
    f32x4_t sacc[NKT];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NKT; ++j) {
      if (j == 0 || j < nkt) {  // an active wave has at least one tile
        f32x4_t acc = j == 0 ? bias0 : j == 1 ? bias1 : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8_t kh = *(const bf16x8_t*)(Khi + koff[s] + 16 * D * j);
          const bf16x8_t kl = *(const bf16x8_t*)(Klo + koff[s] + 16 * D * j);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[s], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[s], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[s], acc, 0, 0, 0);
        }
        sacc[j] = acc;
        mx = vmax3(mx, acc[0], acc[1]);
        mx = vmax3(mx, acc[2], acc[3]);
      }
    }
    // row max across the four lanes that share a token
    mx = col4_max(mx);

    // P = exp2((s - max) * scale*log2 e) in bf16, the product as one fma;
    // O = P·V and the row sum (P against a ones tile) both on the matrix
    // cores.  Key tiles go in pairs through v_mfma_f32_16x16x32_bf16:
    // contraction index 8*q4 + e stands for key row 4*q4 + e of tile j0
    // (e < 4) and 4*q4 + e - 4 of tile j0 + 1, which is what a lane's weights
    // of the two tiles are and what two 8-byte reads of Vᵀ give the A
    // operand.  An unpaired last tile takes the 16x16x16 form.
    const float nmx = -mx * sl2;
    f32x4_t o[NDT], lacc;
    auto weights = [&](int j) {
      float w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][r], sl2, nmx));
      return make_uint2(pack2_bf16(w[0], w[1]), pack2_bf16(w[2], w[3]));
    };
    auto vfrag = [&](int dt, int j) {
      return *(const bf16x4_t*)(vbase + (vt_off(vt_row(dt, 0), 0, VS) - vt_off(vt_row(0, 0), 0, VS)) + 16 * j);
    };
    // tiles j, j + 1 through one 16x16x32 product; first: the accumulators
    // start from zero (an inline constant, so nothing is zeroed beforehand)
    auto pair = [&](int j, bool first) {
      const uint2 p0 = weights(j), p1 = weights(j + 1);
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(p0.x, p0.y, p1.x, p1.y));
      lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pf, first ? f32x4_t{0.f, 0.f, 0.f, 0.f} : lacc, 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x8_t vf = __builtin_shufflevector(vfrag(dt, j), vfrag(dt, j + 1), 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, first ? f32x4_t{0.f, 0.f, 0.f, 0.f} : o[dt], 0, 0, 0);
      }
    };
    auto single = [&](int j, bool first) {
      const bf16x4v pf = __builtin_bit_cast(bf16x4v, weights(j));
      lacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, pf, first ? f32x4_t{0.f, 0.f, 0.f, 0.f} : lacc, 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vfrag(dt, j), pf, first ? f32x4_t{0.f, 0.f, 0.f, 0.f} : o[dt], 0, 0, 0);
    };
    // tiles 0 (and 1) first, then the later pairs, then an unpaired last tile;
    // the blocks after the first accumulate in place
    if (nkt >= 2) pair(0, true);
    else single(0, true);
#pragma unroll
    for (int j0 = 2; j0 + 1 < NKT; j0 += 2)
      if (j0 + 1 < nkt) pair(j0, false);
    if ((nkt & 1) && nkt >= 3) {
#pragma unroll
      for (int j = 2; j < NKT; j += 2)
        if (j == nkt - 1) single(j, false);
    }
    // O tile back to the coalesced layout through the same buffer, then
    // whole-line non-temporal stores (the output is not read again here)
    const float inv = __builtin_amdgcn_rcpf(lacc[0]);
    wave_lds_sync();  // the Q reads of the buffer are done
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = o[2 * s][r] * inv;
        v[4 + r] = o[2 * s + 1][r] * inv;
      }
      *(uint4*)(xb + xr[s]) = pack8_bf16(v);
    }
    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4_t x = *(const u32x4_t*)(xb + xw[s]);
      if (ovalid[s])
        __builtin_nontemporal_store(x, (u32x4_t*)(opair + olane[s] + (uint32_t)(hh * D) * 2));
    }
  };

  if constexpr (LAST) {
    // heads wv, wv + 4, ...: the first from the prefetch, the next loaded here
    using S0 = std::integral_constant<int, 0>;
    for (int hh = wv; hh < G; hh += 4) {
      if (hh != wv) {
        load_q(S0{}, hh);
        prep_q(S0{}, qh, ql);
      }
      attend(hh);
    }
  } else if constexpr (GT > 0) {
    // compile-time group size: the whole head sequence unrolls, so the ring
    // slot of every head and every wait count is known to the compiler.
    // Head h's Q was prepared before this point; its slot is refilled with
    // head h + QPF (heads past the group are not loaded, so the waits stay
    // exact), then head h attends and head h + 1's Q is prepared.
    // Heads QPF .. DEP-1 (a deeper ring than before the staging) are
    // issued first.
    for_each_const<DEP - QPF>([&](auto ic) {
      constexpr int j = QPF + decltype(ic)::value;
      if constexpr (j < GT) load_q(std::integral_constant<int, j % RQ>{}, j);
    });
    for_each_const<GT>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      if constexpr (LPT) {
        // remaining key tiles of this wave (this head's included), in
        // quarters of the most any wave starts with: the wave with the most
        // work left on a SIMD issues first (longest remaining job first).
        // Capped at 2, below the staging priority, so a wave still staging
        // its keys issues ahead of every wave in its heads.
        const int q = min(2, (4 * (GT - h) * nkt - 1) / (GT * NKT));
        if (q == 2) __builtin_amdgcn_s_setprio(2);
        else if (q == 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
      if constexpr (h + DEP < GT) load_q(std::integral_constant<int, (h + DEP) % RQ>{}, h + DEP);
      attend(h);
      if constexpr (h + 1 < GT) prep_q(std::integral_constant<int, (h + 1) % RQ>{}, qh, ql);
    });
  } else {
    // the ring is refilled with the head QPF further on (clamped: always a
    // valid row, so the load is unconditional; the last QPF heads thus read
    // head G-1 again, which is why the common group sizes have instances
    // with the group size fixed at compile time)
    for (int hb = 0; hb < G; hb += QPF) {
      for_each_const<QPF>([&](auto slot) {
        constexpr int i = decltype(slot)::value;
        const int hh = hb + i;
        if (hh < G) {
          if (hh > 0) prep_q(slot, qh, ql);
          load_q(slot, hh + QPF < G ? hh + QPF : G - 1);
          attend(hh);
        }
      });
    }
  }
}


template <int D, int NKT, int QPF, int GT, bool LAST, bool FP8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 && NKT <= 5 ? 4 : 2)))
gist_fwd_mfma(const FwdArgs a, int nk_pad) {
  Slice sl;
  sl.bid = blockIdx.x;
  sl.p = blockIdx.x / a.H;
  sl.g = blockIdx.x - sl.p * a.H;
  sl.q = a.q;
  sl.k_new = a.k_new;
  sl.v_new = a.v_new;
  sl.out = a.out;
  sl.item_ids = a.item_ids;
  sl.q_ids = a.q_ids;
  sl.pool_off = a.pool_layer_off;
  sl.qpool_off = a.qpool_layer_off;
  sl.pool_scales = a.pool_scales;
  sl.qpool_scales = a.qpool_scales;
  mfma_body<D, NKT, QPF, GT, LAST, FP8>(a, sl, nk_pad);
}

// Several independent calls of one shape (each with its own layer, pairs,
// activations and outputs) in one launch: the workgroups of group i follow
// those of group i - 1 in launch order, so one group's last workgroups run
// beside the next group's first.  Each workgroup finds its group from the
// table's running workgroup counts.
template <int D, int NKT, int QPF, int GT, bool FP8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 && NKT <= 5 ? 4 : 2)))
gist_fwd_mfma_grouped(const FwdArgs a, const GroupTable t, int nk_pad) {
  const int bid = blockIdx.x;
  int gi = 0;
#pragma unroll
  for (int i = 0; i < kMaxGroups - 1; ++i) gi += bid >= t.wg_end[i] ? 1 : 0;
  const GroupEntry& e = t.e[gi];
  const int local = bid - (gi == 0 ? 0 : t.wg_end[gi - 1]);
  Slice sl;
  sl.bid = bid;
  sl.p = local / a.H;
  sl.g = local - sl.p * a.H;
  sl.q = e.q;
  sl.k_new = e.k_new;
  sl.v_new = e.v_new;
  sl.out = e.out;
  sl.item_ids = e.item_ids;
  sl.q_ids = e.q_ids;
  sl.pool_off = (int64_t)e.layer * t.pool_layer_stride;
  sl.qpool_off = (int64_t)e.layer * t.qpool_layer_stride;
  sl.pool_scales = FP8 ? a.pool_scales + (int64_t)e.layer * t.scale_layer_stride : nullptr;
  sl.qpool_scales = FP8 && a.kq ? a.qpool_scales + (int64_t)e.layer * t.qscale_layer_stride : nullptr;
  mfma_body<D, NKT, QPF, GT, false, FP8>(a, sl, nk_pad);
}

// ---------------------------------------------------------------------------
// EOS kernel (bf16, ell = 1): one query token per pair, the GQA group's G
// query heads are the MFMA columns
// ---------------------------------------------------------------------------

// One wave per (pair, KV head) and per workgroup: no workgroup barrier, and
// a finished wave frees its slot at once (four independent waves per
// workgroup held each slot until the slowest of them ended).
//   keys, in order: gist tiles 0..ngt-1 hold the item gist then the query
//   gist (kg = k + k' rows, padded with copies of row 0 that the mask
//   removes), then the token's own key, at pos0 like the query.
//   The rotated Q is carried as a bf16 pair hi + lo (split8_bf16) and a gist
//   tile takes K·Q_hi + K·Q_lo on the matrix cores (the stored gist K is
//   exact in bf16).  The token's own logit is a single key per head: its
//   query and key share a position, so RoPE cancels and the logit is q·k of
//   the unrotated rows on the VALU (v_dot2, exact bf16 products, fp32 sums);
//   its V row enters the output by fp32 multiplies.  The softmax scale is
//   applied to the fp32 logits in the exponent.
// NGT: maximum number of gist tiles (kg <= 16*NGT).
// FP8: the gist pools hold E4M3 codes.  Every E4M3 value is also a bf16
// value, so the codes are decoded exactly into the bf16 MFMA operands; the K
// scale of a gist key multiplies its fp32 logit, and the V scale its softmax
// weight before that weight is rounded for the P·V product (the row sum takes
// the unscaled weight).
// QU: Q staging units per lane, G*D/16 units over 64 lanes (1 or 2).
template <int D, int NGT, bool FP8, int QU>
__device__ __forceinline__ void eos_body(const FwdArgs& a, const CsPos0& cs, const Slice& sl) {
  constexpr int NS = D / 32;
  constexpr int NDT = D / 16;
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int ROWS = 16 * NGT;
  // gist V rows are read in 16-byte units: 8 bf16 values or 16 fp8 codes
  constexpr int VCH = FP8 ? 2 : 1;   // 8-element chunks per unit
  constexpr int VPR = CPR / VCH;     // units per row
  constexpr int RITG = 16 * NGT * VPR / 64;  // gist V units per lane
  static_assert(16 * NGT * VPR % 64 == 0 && 2 * CPR <= 64 && NS % 2 == 0, "staging layout");
  // the workgroup is this one wave
  __shared__ __align__(16) bf16_t rows_lds[ROWS * (D + 4)];
  __shared__ __align__(16) float vself_lds[D];  // V_new of the token, fp32
  __shared__ __align__(16) float2 cs_lds[D / 2];  // (cos, sin) at pos0
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4v;
  typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
  typedef std::conditional_t<FP8, uint8_t, bf16_t> C;  // gist element
  typedef std::conditional_t<FP8, uint2, u32x4_t> CV;   // 8 gist elements

  const int lane = threadIdx.x & 63;
  const int n = lane & 15, q4 = lane >> 4;
  const int p = sl.p, g = sl.g;
  const int G = a.G, Hq = a.Hq;
  const int kg = a.k + a.kq;  // >= 1
  const int ngt = (kg + 15) >> 4;
  bf16_t* out = (bf16_t*)sl.out;
  const int64_t orow0 = ((int64_t)p * Hq + (int64_t)g * G) * D;
  // (cos, sin) at pos0 of channel pair `lane` (a lane-indexed read of the
  // arguments, hence a vector load: issued first, so that waiting for it
  // waits for nothing else)
  const float cs_c = cs.v[lane & (D / 2 - 1)][0], cs_s = cs.v[lane & (D / 2 - 1)][1];
  __builtin_amdgcn_sched_barrier(0);
  // the ids first: the gist loads wait for them, and issued ahead of the
  // token's row traffic they do not queue behind it (both loads are in
  // flight before either is waited on)
  const int32_t item = sl.item_ids[p];
  const int32_t qid = *(a.kq ? sl.q_ids + p : sl.item_ids + p);
  __builtin_amdgcn_sched_barrier(0);

  // ---- the token's own rows: they do not depend on the ids, so their HBM
  // traffic starts while the ids are in flight ------------------------------
  // Q, coalesced: unit u = lane + 64*i covers head u / (D/16) and its chunk
  // pair (channels 8c..8c+7 and their RoPE partners D/2 + 8c..), so each
  // head's row is read whole and once; units past the group read its last
  // head's first pair.  The same chunk pair of K_new goes with it (the
  // group's lanes share the one 128- or 256-byte row).
  constexpr int QCH = D / 16;  // chunk pairs per head
  const bf16_t* qgrp = (const bf16_t*)sl.q + ((int64_t)p * Hq + (int64_t)g * G) * D;
  const bf16_t* knew = (const bf16_t*)sl.k_new + ((int64_t)p * a.H + g) * D;
  const bf16_t* vnew = (const bf16_t*)sl.v_new + ((int64_t)p * a.H + g) * D;
  u32x4_t qlo[QU], qhi[QU], klo[QU], khi[QU];
#pragma unroll
  for (int i = 0; i < QU; ++i) {
    const int u = lane + 64 * i;
    const int uc = u < G * QCH ? u : (G - 1) * QCH;
    const bf16_t* src = qgrp + (uc / QCH) * D + 8 * (uc % QCH);
    qlo[i] = *(const u32x4_t*)src;
    qhi[i] = *(const u32x4_t*)(src + D / 2);
    klo[i] = *(const u32x4_t*)(knew + 8 * (uc % QCH));
    khi[i] = *(const u32x4_t*)(knew + D / 2 + 8 * (uc % QCH));
  }
  // V_new as a whole row: lane l covers chunk l % CPR (lanes past the row
  // read it again)
  const int sc = lane % CPR;
  const u32x4_t rself = *(const u32x4_t*)(vnew + 8 * sc);
  __builtin_amdgcn_sched_barrier(0);

  // the arguments that the gist addresses need, read in one batch here: left
  // to the branches below, they were fetched one dependent scalar round trip
  // at a time after the ids arrived.  The empty asm makes them (and the ids)
  // arrive at this point.
  const int paged = a.paged, ak = a.k, akq = a.kq, bsz = a.block_size, qrow0 = a.q_row0;
  const int64_t aN = a.N, aqN = a.qN, plo = sl.pool_off, qplo = sl.qpool_off;
  const C *pool_c = (const C*)a.pool, *qpool_c = (const C*)a.qpool;
  const C *pk_c = (const C*)a.paged_k, *pv_c = (const C*)a.paged_v;
  asm volatile("" ::"s"(paged), "s"(ak), "s"(akq), "s"(bsz), "s"(qrow0), "s"(aN), "s"(aqN), "s"(plo),
               "s"(qplo), "s"(pool_c), "s"(qpool_c), "s"(pk_c), "s"(pv_c), "s"(item), "s"(qid));

  // ---- ids (bounds-checked; a bad id turns the pair's rows into NaN) ------
  bool bad = item < 0 || item >= aN;
  if (akq) bad = bad || qid < 0 || qid >= aqN;
  if (bad) {
    for (int u = lane; u < G * D; u += 64) out[orow0 + u] = nan_value<bf16_t>();
    return;
  }
  // first K and V rows of the item gist and of the query gist
  const C *gK, *gV, *qK, *qV;
  if (paged) {
    const int64_t ib = ((int64_t)item * a.H + g) * bsz * D;
    const int64_t qb = (((int64_t)qid * a.H + g) * bsz + qrow0) * D;
    gK = pk_c + ib;
    gV = pv_c + ib;
    qK = pk_c + qb;
    qV = pv_c + qb;
  } else {
    // pool record: K of every head, then V of every head
    gK = pool_c + plo + (int64_t)item * 2 * a.H * ak * D + (int64_t)g * ak * D;
    gV = gK + (int64_t)a.H * ak * D;
    qK = gK;
    if (akq) qK = qpool_c + qplo + (int64_t)qid * 2 * a.H * akq * D + (int64_t)g * akq * D;
    qV = qK + (int64_t)a.H * akq * D;
  }
  // gist key j (< kg): its K row, or V row
  auto gist_row = [&](int j, bool v) -> const C* {
    if (j < ak) return (v ? gV : gK) + (int64_t)j * D;
    return (v ? qV : qK) + (int64_t)(j - ak) * D;
  };

  // ---- gist loads, all unconditional (clamped rows) ------------------------
  // K: MFMA A layout straight from HBM (lane n = key, 8 channels per step).
  // The contraction takes the 8-channel chunks in the order kc(s, q4): in
  // steps 2t and 2t + 1 lane q4 holds chunks 2q4 and 2q4 + 1 of channels
  // 64t..64t+63, so with fp8 codes one 16-byte load feeds both steps.  Q's B
  // fragments are read in the same order.
  auto kc = [](int s, int qq) { return 8 * (s >> 1) + 2 * qq + (s & 1); };
  CV kraw[NGT][NS];
#pragma unroll
  for (int kt = 0; kt < NGT; ++kt) {
    const int j = 16 * kt + n;
    const C* row = gist_row(j < kg ? j : 0, false);
    if constexpr (FP8) {
#pragma unroll
      for (int t = 0; t < NS / 2; ++t) {
        const uint4 w = *(const uint4*)(row + 64 * t + 16 * q4);
        kraw[kt][2 * t] = make_uint2(w.x, w.y);
        kraw[kt][2 * t + 1] = make_uint2(w.z, w.w);
      }
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) kraw[kt][s] = *(const CV*)(row + 8 * kc(s, q4));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // V rows, coalesced (lane covers unit u % VPR of row u / VPR); issued
  // last, so the logits of the gist tiles only wait for K and Q
  u32x4_t graw[RITG];
#pragma unroll
  for (int it = 0; it < RITG; ++it) {
    const int u = lane + 64 * it;
    const int r = u / VPR, c = u - (u / VPR) * VPR;
    graw[it] = *(const u32x4_t*)(gist_row(r < kg ? r : 0, true) + 8 * VCH * c);
  }
  __builtin_amdgcn_sched_barrier(0);
  // fp8: scales of the item and query gist (K, V); wave-uniform scalars.
  // (Vector loads, which would keep them off the counter the LDS waits below
  // share, cost a wave of occupancy and ran slower.)
  float ski = 1.f, svi = 1.f, skq = 1.f, svq = 1.f;
  if constexpr (FP8) {
    if (paged) {
      // paged cache: the scales of the gists' blocks
      ski = a.paged_kscales[(int64_t)item * a.H + g];
      svi = a.paged_vscales[(int64_t)item * a.H + g];
      if (akq) {
        skq = a.paged_kscales[(int64_t)qid * a.H + g];
        svq = a.paged_vscales[(int64_t)qid * a.H + g];
      }
    } else {
      const float* si = sl.pool_scales + (int64_t)item * 2 * a.H;
      ski = si[g];
      svi = si[a.H + g];
      if (akq) {
        const float* sq = sl.qpool_scales + (int64_t)qid * 2 * a.H;
        skq = sq[g];
        svq = sq[a.H + g];
      }
    }
  }
  // eight gist elements -> eight bf16 (exact for E4M3 codes: every E4M3
  // value is a bf16 value), two codes per conversion at unit scale
  auto to_bf16x8 = [](const CV& w) -> u32x4_t {
    if constexpr (FP8) {
      return u32x4_t{fp8x2_to_bf16x2<false>(w.x), fp8x2_to_bf16x2<true>(w.x),
                     fp8x2_to_bf16x2<false>(w.y), fp8x2_to_bf16x2<true>(w.y)};
    } else {
      return w;
    }
  };

  // ---- cos/sin at pos0 into the wave's table (lane i < D/2: pair i) -----
  float2* cst = cs_lds;
  if (lane < D / 2) cst[lane] = make_float2(cs_c, cs_s);
  wave_lds_sync();

  // ---- rotate Q at pos0 in the coalesced layout, split it into bf16 hi +
  // lo, then turn each into the MFMA B layout (lane n = query head, 8
  // channels of step s) through this wave's row buffer: hi first, then lo in
  // the same place (a wave's LDS accesses complete in order).  The buffer's
  // rows are written with keys only after the B fragments are read.  Row h
  // holds head h; chunk c sits at chunk c ^ h, so the eight lanes of a
  // 16-byte access phase hit distinct banks on both sides.
  bf16_t* Rl = rows_lds;
  static_assert(16 * D <= ROWS * (D + 4), "Q staging fits the row buffer");
  uint4 qlo_st[QU][2];
  float sdot[QU];  // this lane's part of the token's own logit q·k
  auto qpos = [](int h, int c) { return h * D + (((c ^ h) & (CPR - 1)) << 3); };
  // The token's own logit: its query and its key sit at the same position,
  // and a rotation keeps dot products, so q·k of the rotated rows is q·k of
  // the rows as given.  It is summed from the bf16 pairs as loaded (v_dot2:
  // the products of two bf16 values are exact in fp32); K_new is never
  // rotated or unpacked here.
  const SplitOnes so = split_ones();
  auto dot2 = [](uint32_t x, uint32_t y, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, x), __builtin_bit_cast(bf16x2v, y),
                                           acc, false);
  };
#pragma unroll
  for (int i = 0; i < QU; ++i) {
    const int u = lane + 64 * i;
    const int h = u / QCH, c = u - (u / QCH) * QCH;
    float dot = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dot = dot2(qlo[i][w], klo[i][w], dot);
      dot = dot2(qhi[i][w], khi[i][w], dot);
    }
    float xl[8], xh[8], yl[8], yh[8];
    unpack8(make_uint4(qlo[i].x, qlo[i].y, qlo[i].z, qlo[i].w), xl);
    unpack8(make_uint4(qhi[i].x, qhi[i].y, qhi[i].z, qhi[i].w), xh);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 cs = cst[8 * c + e];
      yl[e] = __builtin_fmaf(xl[e], cs.x, -(xh[e] * cs.y));
      yh[e] = __builtin_fmaf(xh[e], cs.x, xl[e] * cs.y);
    }
    // sum over the QCH lanes of head h (aligned groups of 4 or 8 lanes)
    dot += dpp_f<0xB1>(dot);
    dot += dpp_f<0x4E>(dot);
    if constexpr (QCH == 8) dot += dpp_f<0x141>(dot);
    sdot[i] = dot;
    uint4 hl, hh;
    split8_bf16(yl, hl, qlo_st[i][0], so);
    split8_bf16(yh, hh, qlo_st[i][1], so);
    if (u < G * QCH) {
      *(uint4*)(Rl + qpos(h, c)) = hl;
      *(uint4*)(Rl + qpos(h, c + QCH)) = hh;
    }
  }
  bf16x8_t qh[NS], ql[NS];
  // columns past the group read its last head (finite, never stored)
  const int hcol = n < G ? n : G - 1;
  // the token's own logit of column n: head hcol's sum, held by its units
  float sself;
  {
    const int su = hcol * QCH;
    sself = __int_as_float(__builtin_amdgcn_ds_bpermute((su & 63) << 2, __float_as_int(sdot[0])));
    if constexpr (QU == 2) {
      const float s1 = __int_as_float(__builtin_amdgcn_ds_bpermute((su & 63) << 2, __float_as_int(sdot[1])));
      sself = su >= 64 ? s1 : sself;
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int s = 0; s < NS; ++s) qh[s] = *(const bf16x8_t*)(Rl + qpos(hcol, kc(s, q4)));
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < QU; ++i) {
    const int u = lane + 64 * i;
    const int h = u / QCH, c = u - (u / QCH) * QCH;
    if (u < G * QCH) {
      *(uint4*)(Rl + qpos(h, c)) = qlo_st[i][0];
      *(uint4*)(Rl + qpos(h, c + QCH)) = qlo_st[i][1];
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int s = 0; s < NS; ++s) ql[s] = *(const bf16x8_t*)(Rl + qpos(hcol, kc(s, q4)));
  wave_lds_sync();  // the rows below overwrite the Q buffer

  // ---- logits Sᵀ[key][head] of the gist tiles (unscaled: scale*log2 e is
  // applied in the exponent); the stored gist K is exact in bf16 ------------
  f32x4_t sacc[NGT];
  float mx = sself;
#pragma unroll
  for (int kt = 0; kt < NGT; ++kt) {
    if (kt == 0 || kt < ngt) {
      f32x4_t acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = (FP8 || 16 * kt + 4 * q4 + r < kg) ? 0.f : -INFINITY;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, to_bf16x8(kraw[kt][s]));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qh[s], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, ql[s], acc, 0, 0, 0);
      }
      if constexpr (FP8) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * kt + 4 * q4 + r;
          acc[r] = row < kg ? acc[r] * (row < a.k ? ski : skq) : -INFINITY;
        }
      }
      sacc[kt] = acc;
      mx = vmax3(mx, acc[0], acc[1]);
      mx = vmax3(mx, acc[2], acc[3]);
    }
  }

  // ---- rows to LDS: the gist V rows, then V_new ------------------------------
  auto put = [&](int r, int c, const u32x4_t& w) {
    // rows are 8-byte aligned: two 8-byte stores
    uint2* dst = (uint2*)(Rl + vrow_off(r, 8 * c, D));
    dst[0] = make_uint2(w.x, w.y);
    dst[1] = make_uint2(w.z, w.w);
  };
#pragma unroll
  for (int it = 0; it < RITG; ++it) {
    const int u = lane + 64 * it;
    const int r = u / VPR, c = u - (u / VPR) * VPR;
    if constexpr (FP8) {
      put(r, 2 * c, to_bf16x8(make_uint2(graw[it].x, graw[it].y)));
      put(r, 2 * c + 1, to_bf16x8(make_uint2(graw[it].z, graw[it].w)));
    } else {
      put(r, c, graw[it]);
    }
  }
  // the token's V row in fp32, unpacked once (lanes past the row repeat it)
  float* vs = vself_lds;
  {
    float f[8];
    unpack8(make_uint4(rself.x, rself.y, rself.z, rself.w), f);
    if (lane < CPR) {
      *(float4*)(vs + 8 * sc) = make_float4(f[0], f[1], f[2], f[3]);
      *(float4*)(vs + 8 * sc + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
  }
  wave_lds_sync();
  mx = col4_max(mx);

  // ---- P = exp2((s - max) * scale*log2 e); O = P·V and row sums on the
  // matrix cores; V fragment (d-tile dt, key tile kt) by transpose read: the
  // lane supplying a piece reads key (lane >> 2) of the tile, channels
  // 32*(dt >> 1) + 4*(dt & 1) + 8*(lane & 3) .. +3, so MFMA row r of the tile
  // is channel vt_row(dt, r) and key k of the tile is MFMA column k
  // The weights are normalized before the P·V product: the row sums come
  // first (gist tiles on the matrix cores, against a ones tile, plus the
  // token's own weight), then each lane scales its four weights by 1/l of
  // its column, so the products land normalized.
  const bf16x4v ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
  const float sl2 = a.scale_log2, nmx = -mx * sl2;
  const float wself = __builtin_amdgcn_exp2f(__builtin_fmaf(sself, sl2, nmx));
  float w[NGT][4];
  f32x4_t lacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < NGT; ++kt) {
    if (kt == 0 || kt < ngt) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        w[kt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], sl2, nmx));
      const bf16x4v pf = __builtin_bit_cast(
          bf16x4v, make_uint2(pack2_bf16(w[kt][0], w[kt][1]), pack2_bf16(w[kt][2], w[kt][3])));
      lacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, pf, lacc, 0, 0, 0);
    }
  }
  const float inv = __builtin_amdgcn_rcpf(lacc[0] + wself);
  const float invi = FP8 ? inv * svi : inv, invq = FP8 ? inv * svq : inv;
  // the token's own value row, by fp32 FMAs: lane (n, q4) holds output
  // channels 32s + 8*q4 .. +7 of column n (see the stores below)
  f32x4_t o[NDT];
  {
    const float ws = wself * inv;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float4 v0 = *(const float4*)(vs + 32 * s + 8 * q4);
      const float4 v1 = *(const float4*)(vs + 32 * s + 8 * q4 + 4);
      o[2 * s] = f32x4_t{ws * v0.x, ws * v0.y, ws * v0.z, ws * v0.w};
      o[2 * s + 1] = f32x4_t{ws * v1.x, ws * v1.y, ws * v1.z, ws * v1.w};
    }
  }
#pragma unroll
  for (int kt = 0; kt < NGT; ++kt) {
    if (kt == 0 || kt < ngt) {
      float wn[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        wn[r] = w[kt][r] * (16 * kt + 4 * q4 + r < a.k ? invi : invq);
      const bf16x4v pv =
          __builtin_bit_cast(bf16x4v, make_uint2(pack2_bf16(wn[0], wn[1]), pack2_bf16(wn[2], wn[3])));
      const int R = 16 * kt + (lane >> 2);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int ch = 32 * (dt >> 1) + 4 * (dt & 1) + 8 * (lane & 3);
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(Rl + vrow_off(R, ch, D)));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, v), pv, o[dt],
                                                          0, 0, 0);
      }
    }
  }
  // The group's G output rows are one contiguous G*D block.  Lane (n, q4)
  // holds 16-byte chunks 4s + q4 of row n; they go through the row buffer
  // (chunk c of row n at chunk c ^ n: conflict-free on both sides, and every
  // P·V read of the buffer has completed, since o depends on it) so that the
  // stores write whole lines, non-temporal (read nowhere here).
  wave_lds_sync();
  if (n < G) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = o[2 * s][r];
        v[4 + r] = o[2 * s + 1][r];
      }
      *(uint4*)(Rl + qpos(n, 4 * s + q4)) = pack8_bf16(v);
    }
  }
  wave_lds_sync();
  static_assert(16 * D <= ROWS * (D + 4), "output staging fits the row buffer");
  for (int u = lane; u < G * CPR; u += 64) {
    const int h = u / CPR, c = u - (u / CPR) * CPR;
    const u32x4_t w = *(const u32x4_t*)(Rl + qpos(h, c));
    __builtin_nontemporal_store(w, (u32x4_t*)(out + orow0 + 8 * (int64_t)u));
  }
}

template <int D, int NGT, bool FP8, int QU>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(D == 128 && NGT == 2 ? 2 : 4)))
gist_fwd_eos(const FwdArgs a, const CsPos0 cs) {
  const int unit = blockIdx.x;
  if (unit >= a.P * a.H) return;
  Slice sl;
  sl.bid = blockIdx.x;
  sl.p = unit / a.H;
  sl.g = unit - sl.p * a.H;
  sl.q = a.q;
  sl.k_new = a.k_new;
  sl.v_new = a.v_new;
  sl.out = a.out;
  sl.item_ids = a.item_ids;
  sl.q_ids = a.q_ids;
  sl.pool_off = a.pool_layer_off;
  sl.qpool_off = a.qpool_layer_off;
  sl.pool_scales = a.pool_scales;
  sl.qpool_scales = a.qpool_scales;
  eos_body<D, NGT, FP8, QU>(a, cs, sl);
}

// The EOS kernel over the groups of a grouped launch: wave u of the launch
// takes (pair, KV head) unit u of the concatenated groups.
template <int D, int NGT, bool FP8, int QU>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(D == 128 && NGT == 2 ? 2 : 4)))
gist_fwd_eos_grouped(const FwdArgs a, const CsPos0 cs, const GroupTable t) {
  const int unit = blockIdx.x;
  if (unit >= t.units) return;
  int gi = 0;
#pragma unroll
  for (int i = 0; i < kMaxGroups - 1; ++i) gi += unit >= t.wg_end[i] ? 1 : 0;
  const GroupEntry& e = t.e[gi];
  const int local = unit - (gi == 0 ? 0 : t.wg_end[gi - 1]);
  Slice sl;
  sl.bid = blockIdx.x;
  sl.p = local / a.H;
  sl.g = local - sl.p * a.H;
  sl.q = e.q;
  sl.k_new = e.k_new;
  sl.v_new = e.v_new;
  sl.out = e.out;
  sl.item_ids = e.item_ids;
  sl.q_ids = e.q_ids;
  sl.pool_off = (int64_t)e.layer * t.pool_layer_stride;
  sl.qpool_off = (int64_t)e.layer * t.qpool_layer_stride;
  sl.pool_scales = FP8 ? a.pool_scales + (int64_t)e.layer * t.scale_layer_stride : nullptr;
  sl.qpool_scales = FP8 && a.kq ? a.qpool_scales + (int64_t)e.layer * t.qscale_layer_stride : nullptr;
  eos_body<D, NGT, FP8, QU>(a, cs, sl);
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
  // last_only: one block per (pair, KV head), for the last token, whose q and
  // out rows are the pair's only rows
  const int t = a.last_only ? ell - 1 : blockIdx.x % ell;
  const int pg = a.last_only ? blockIdx.x : blockIdx.x / ell;
  const int trow = a.last_only ? 0 : t;  // row of q and out within the pair
  const int nrow = a.last_only ? 1 : ell;
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
  const int64_t orow0 = (((int64_t)p * nrow + trow) * Hq + (int64_t)g * G) * D;
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
  for (int e = 0; e < E2; ++e) rope_cos_sin((double)a.pos0 + t, a.freqs.rev[lo + e], qcs[e], qsn[e]);

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
      const T* qr = (const T*)a.q + (((int64_t)p * nrow + trow) * Hq + (int64_t)g * G + hh) * D;
      float xl[E2], xh[E2];
      load_n<T, E2>(qr + lo, xl);
      load_n<T, E2>(qr + hi, xh);
#pragma unroll
      for (int e = 0; e < E2; ++e) {
        qv[mh][e] = __builtin_fmaf(xl[e], qcs[e], -(xh[e] * qsn[e]));
        qv[mh][E2 + e] = __builtin_fmaf(xh[e], qcs[e], xl[e] * qsn[e]);
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
          if (tj != t) rope_cos_sin((double)a.pos0 + tj, a.freqs.rev[lo + e], cs, sn);
          const float xl = kv[e], xh = kv[E2 + e];
          kv[e] = __builtin_fmaf(xl, cs, -(xh * sn));
          kv[E2 + e] = __builtin_fmaf(xh, cs, xl * sn);
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


template <typename T, int D>
void launch_valu(const FwdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.P * a.H * (a.last_only ? 1 : a.ell)));
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

// Compute units of the current device, queried once per device (a lookup
// that fails counts as 256, the MI355X figure).  Calls from several host
// threads may fill an entry at the same time; they store the same value.
int device_cu_count() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The l >= 2 kernel for a call's shape: head size, key tiles, gist element
// type, group size (compile-time instances for the common ones) and Q
// prefetch depth.
// The l >= 2 kernel instance for a call's shape; with a group table, the
// grouped kernel over all of its groups (wgs workgroups)
template <bool L, bool F8>
void launch_mfma_t(const FwdArgs& a, const GroupTable* t, int64_t wgs, int d, int nk_pad,
                   hipStream_t s) {
  const dim3 grid((unsigned)wgs);
  const int nkt = nk_pad / 16;
  const int G = a.G;
  // When the whole grid is resident at once (four workgroups per CU), every
  // workgroup issues its staging loads at the same moment and a deeper Q
  // prefetch only delays them: prefetch one head ahead.  With several
  // generations of workgroups, two heads ahead.  A compile-time group size
  // loads no Q row past the group (the generic instance's clamped ring
  // refills re-read the last head).
  const bool one_gen = wgs <= 4 * (int64_t)device_cu_count();
  auto go = [&](auto dc, auto nc, auto qc, auto gc) {
    constexpr int DD = decltype(dc)::value, NK = decltype(nc)::value;
    constexpr int QP = decltype(qc)::value, GG = decltype(gc)::value;
    const size_t lds = MfmaLds<DD, NK>::bytes(nk_pad);
    if (t) {
      if constexpr (!L)
        hipLaunchKernelGGL((gist_fwd_mfma_grouped<DD, NK, QP, GG, F8>), grid, dim3(256), lds, s, a, *t,
                           nk_pad);
    } else {
      hipLaunchKernelGGL((gist_fwd_mfma<DD, NK, QP, GG, L, F8>), grid, dim3(256), lds, s, a, nk_pad);
    }
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I0 = std::integral_constant<int, 0>;
  using I5 = std::integral_constant<int, 5>;
  using I7 = std::integral_constant<int, 7>;
  using I8 = std::integral_constant<int, 8>;
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (d == 64 && nkt <= 5) {
    if (G == 7 && one_gen) go(D64{}, I5{}, I1{}, I7{});
    else if (G == 7) go(D64{}, I5{}, I2{}, I7{});
    else if (G == 8 && one_gen) go(D64{}, I5{}, I1{}, I8{});
    else if (G == 8) go(D64{}, I5{}, I2{}, I8{});
    else go(D64{}, I5{}, I1{}, I0{});
  } else if (d == 64) {
    go(D64{}, I8{}, I1{}, I0{});
  } else if (nkt <= 5) {
    if (G == 8) go(D128{}, I5{}, I2{}, I8{});
    else go(D128{}, I5{}, I2{}, I0{});
  } else {
    go(D128{}, I8{}, I2{}, I0{});
  }
}

void launch_mfma(const FwdArgs& a, int d, int nk_pad, bool fp8, bool last, hipStream_t s) {
  const int64_t wgs = (int64_t)a.P * a.H;
  if (last && fp8) launch_mfma_t<true, true>(a, nullptr, wgs, d, nk_pad, s);
  else if (last) launch_mfma_t<true, false>(a, nullptr, wgs, d, nk_pad, s);
  else if (fp8) launch_mfma_t<false, true>(a, nullptr, wgs, d, nk_pad, s);
  else launch_mfma_t<false, false>(a, nullptr, wgs, d, nk_pad, s);
}

// The l = 1 (EOS) kernel for a call's shape.
void launch_eos(const FwdArgs& a, const GroupTable* t, int64_t units, int d, int kg, bool fp8,
                hipStream_t s) {
  const dim3 grid((unsigned)units);  // one wave per unit and per workgroup
  // (cos, sin) at pos0: the revolutions are reduced to a fraction in double
  // before the angle is formed, as the other kernels do on the device
  CsPos0 cs;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < kMaxHalfDim; ++i) {
    const double r = (double)a.pos0 * a.freqs.rev[i];
    const double f = r - std::rint(r);
    cs.v[i][0] = (float)std::cos(two_pi * f);
    cs.v[i][1] = (float)std::sin(two_pi * f);
  }
  // Q staging units per lane: G heads x d/16 chunk pairs over 64 lanes
  const bool qu2 = a.G * (d / 16) > 64;
  auto go = [&](auto d_c, auto ngt_c) {
    constexpr int DD = decltype(d_c)::value, NG = decltype(ngt_c)::value;
    auto launch = [&](auto f8_c, auto qu_c) {
      constexpr bool F8 = decltype(f8_c)::value;
      constexpr int QU = decltype(qu_c)::value;
      if (t)
        hipLaunchKernelGGL((gist_fwd_eos_grouped<DD, NG, F8, QU>), grid, dim3(64), 0, s, a, cs, *t);
      else
        hipLaunchKernelGGL((gist_fwd_eos<DD, NG, F8, QU>), grid, dim3(64), 0, s, a, cs);
    };
    using Q1 = std::integral_constant<int, 1>;
    using Q2 = std::integral_constant<int, 2>;
    if (fp8 && qu2) launch(std::true_type{}, Q2{});
    else if (fp8) launch(std::true_type{}, Q1{});
    else if (qu2) launch(std::false_type{}, Q2{});
    else launch(std::false_type{}, Q1{});
  };
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (d == 64) {
    if (kg <= 16) go(I64{}, I1{});
    else go(I64{}, I2{});
  } else {
    if (kg <= 16) go(I128{}, I1{});
    else go(I128{}, I2{});
  }
}

// RoPE tables of a call: revolutions per position of every channel pair and
// the scalar steps q^(2^b)
void set_rope(FwdArgs& a, int d, float rope_base) {
  make_rope_freqs(a.freqs, d, rope_base);
  double q = std::pow((double)rope_base, -2.0 / (double)d);
  for (int b = 0; b < 6; ++b, q *= q) a.rev_step[b] = q;
}

// The arguments shared by every workgroup of a pooled call at one layer
// (per-call pointers, P and last_only are left for the caller to set)
void fill_args(FwdArgs& a, const gist_pool* pool, const gist_pool* qpool, int layer, int ell,
               int Hq, int pos0, float rope_base, float scale) {
  const bool fp8 = pool->dtype == GIST_FP8_E4M3;
  const int H = pool->H, d = pool->d;
  a.pool = pool->storage;
  a.pool_layer_off = (int64_t)layer * pool->N * record_elems(pool);
  a.N = pool->N;
  a.k = pool->k;
  a.qpool = qpool ? qpool->storage : nullptr;
  a.qpool_layer_off = qpool ? (int64_t)layer * qpool->N * record_elems(qpool) : 0;
  a.qN = qpool ? qpool->N : 0;
  a.kq = qpool ? qpool->k : 0;
  a.pool_scales = fp8 ? fp8_layer_scales(pool, layer) : nullptr;
  a.qpool_scales = fp8 && qpool ? fp8_layer_scales(qpool, layer) : nullptr;
  a.item_ids = a.q_ids = nullptr;
  a.q = a.k_new = a.v_new = nullptr;
  a.out = nullptr;
  a.P = 0;
  a.ell = ell;
  a.Hq = Hq;
  a.H = H;
  a.G = Hq / H;
  a.pos0 = pos0;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.last_only = 0;
  a.paged = 0;
  a.paged_k = a.paged_v = nullptr;
  a.block_size = 0;
  a.q_row0 = 0;
  a.paged_kscales = a.paged_vscales = nullptr;
  set_rope(a, d, rope_base);
}

// gist_attn_forward and gist_attn_forward_last (last: q and out hold only the
// last token of each pair)
gist_status attn_forward(const gist_pool* pool, int layer, const int32_t* item_ids, int P, int ell,
                         int Hq, const void* q, const void* k_new, const void* v_new, int pos0,
                         float rope_base, float scale, const gist_pool* qpool,
                         const int32_t* q_ids, void* out, void* stream, bool last) {
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
  const bool fp8 = pool->dtype == GIST_FP8_E4M3;
  {
    // fp8 pools run on the MFMA and EOS kernels only
    const int kgv = pool->k + (qpool ? qpool->k : 0);
    const bool mfma_shape = ell >= 2 && ell <= 64 && (kgv + ell + 15) / 16 * 16 <= 128;
    const bool eos_shape = ell == 1 && Hq / H <= 16 && kgv <= 32;
    if (fp8 && !mfma_shape && !eos_shape)
      return fail(GIST_ERR_UNSUPPORTED,
                  "gist_attn_forward: fp8 pools support 2 <= ell <= 64 with k + k' + ell <= 128, "
                  "or ell == 1 with Hq/H <= 16 and k + k' <= 32");
  }
  if (P == 0) return GIST_OK;
  if (!item_ids || !q || !k_new || !v_new || !out)
    return fail(GIST_ERR_INVALID_ARG, "gist_attn_forward: NULL tensor argument");
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
    return fail(GIST_ERR_INVALID_ARG, "gist_attn_forward: tensors must be 16-byte aligned");
  if ((int64_t)P * H * ell > INT32_MAX)
    return fail(GIST_ERR_UNSUPPORTED, "gist_attn_forward: P*H*ell too large for one launch");

  FwdArgs a;
  fill_args(a, pool, qpool, layer, ell, Hq, pos0, rope_base, scale);
  a.item_ids = item_ids;
  a.q_ids = qpool ? q_ids : nullptr;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.out = out;
  a.P = P;
  a.last_only = last ? 1 : 0;
  hipStream_t s = (hipStream_t)stream;

  const int kg = a.k + a.kq;
  const int nk_pad = ((kg + ell + 15) / 16) * 16;
  if ((pool->dtype == GIST_BF16 || fp8) && ell >= 2 && ell <= 64 && nk_pad <= 128) {  // LDS <= 116 KiB per workgroup
    launch_mfma(a, d, nk_pad, fp8, last, s);
    return check_launch("gist_attn_forward(mfma)");
  }
  if ((pool->dtype == GIST_BF16 || fp8) && ell == 1 && a.G <= 16 && kg <= 32) {
    launch_eos(a, nullptr, (int64_t)a.P * a.H, d, kg, fp8, s);
    return check_launch("gist_attn_forward(eos)");
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

}  // namespace

extern "C" gist_status gist_attn_forward(const gist_pool* pool, int layer, const int32_t* item_ids,
                                         int P, int ell, int Hq, const void* q, const void* k_new,
                                         const void* v_new, int pos0, float rope_base, float scale,
                                         const gist_pool* qpool, const int32_t* q_ids, void* out,
                                         void* stream) {
  return attn_forward(pool, layer, item_ids, P, ell, Hq, q, k_new, v_new, pos0, rope_base, scale,
                      qpool, q_ids, out, stream, false);
}

extern "C" gist_status gist_attn_forward_grouped(const gist_pool* pool, const gist_pool* qpool,
                                                 const gist_group* groups, int n_groups, int ell,
                                                 int Hq, int pos0, float rope_base, float scale,
                                                 void* stream) {
  clear_error();
  const char* fn = "gist_attn_forward_grouped";
  auto err = [&](gist_status c, const char* m) { return fail(c, std::string(fn) + ": " + m); };
  if (!pool) return err(GIST_ERR_INVALID_ARG, "pool is NULL");
  if (n_groups < 0) return err(GIST_ERR_INVALID_ARG, "n_groups < 0");
  if (n_groups > kMaxGroups) return err(GIST_ERR_UNSUPPORTED, "n_groups must be <= 32");
  if (n_groups > 0 && !groups) return err(GIST_ERR_INVALID_ARG, "groups is NULL");
  const int H = pool->H, d = pool->d;
  if (Hq < H || Hq % H != 0) return err(GIST_ERR_INVALID_ARG, "Hq must be a positive multiple of H");
  if (Hq / H > 32) return err(GIST_ERR_UNSUPPORTED, "Hq/H must be <= 32");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return err(GIST_ERR_INVALID_ARG, "scale must be positive and finite");
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return err(GIST_ERR_INVALID_ARG, "rope_base must be positive");
  if (qpool && (qpool->H != H || qpool->d != d || qpool->dtype != pool->dtype || qpool->L != pool->L))
    return err(GIST_ERR_INVALID_ARG, "qpool must match pool in L, H, d and dtype");
  const int kg = pool->k + (qpool ? qpool->k : 0);
  const int nk_pad = ((kg + ell + 15) / 16) * 16;
  const bool eos = ell == 1 && Hq / H <= 16 && kg <= 32;
  const bool mfma = ell >= 2 && ell <= 64 && nk_pad <= 128;
  if (pool->dtype == GIST_F32 || !(eos || mfma))
    return err(GIST_ERR_UNSUPPORTED,
               "groups run the EOS kernel (ell == 1, Hq/H <= 16, k + k' <= 32) or the l >= 2 "
               "kernel (2 <= ell <= 64, k + k' + ell <= 128) over bf16 or fp8 pools");
  GroupTable t;
  int m = 0;
  int64_t wgs = 0;
  for (int i = 0; i < n_groups; ++i) {
    const gist_group& gr = groups[i];
    if (gr.layer < 0 || gr.layer >= pool->L) return err(GIST_ERR_OUT_OF_RANGE, "layer out of range");
    if (gr.P < 0) return err(GIST_ERR_INVALID_ARG, "P < 0");
    if (gr.P == 0) continue;
    if (!gr.item_ids || !gr.q || !gr.k_new || !gr.v_new || !gr.out || (qpool && !gr.q_ids))
      return err(GIST_ERR_INVALID_ARG, "NULL tensor argument");
    if (!aligned16(gr.q) || !aligned16(gr.k_new) || !aligned16(gr.v_new) || !aligned16(gr.out))
      return err(GIST_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if ((int64_t)gr.P * H * ell > INT32_MAX) return err(GIST_ERR_UNSUPPORTED, "P*H*ell too large");
    wgs += (int64_t)gr.P * H;
    if (wgs > INT32_MAX) return err(GIST_ERR_UNSUPPORTED, "too many workgroups for one launch");
    GroupEntry& e = t.e[m];
    e.q = gr.q;
    e.k_new = gr.k_new;
    e.v_new = gr.v_new;
    e.out = gr.out;
    e.item_ids = gr.item_ids;
    e.q_ids = qpool ? gr.q_ids : nullptr;
    e.layer = gr.layer;
    t.wg_end[m] = (int)wgs;
    ++m;
  }
  if (m == 0) return GIST_OK;
  for (int i = m; i < kMaxGroups; ++i) {
    t.wg_end[i] = INT32_MAX;
    t.e[i] = t.e[m - 1];
  }
  t.units = (int)wgs;
  const bool fp8 = pool->dtype == GIST_FP8_E4M3;
  FwdArgs a;
  fill_args(a, pool, qpool, 0, ell, Hq, pos0, rope_base, scale);
  t.pool_layer_stride = pool->N * record_elems(pool);
  t.qpool_layer_stride = qpool ? qpool->N * record_elems(qpool) : 0;
  t.scale_layer_stride = fp8 ? pool->N * 2 * H : 0;
  t.qscale_layer_stride = fp8 && qpool ? qpool->N * 2 * H : 0;
  hipStream_t s = (hipStream_t)stream;
  if (eos) launch_eos(a, &t, wgs, d, kg, fp8, s);
  else if (fp8) launch_mfma_t<false, true>(a, &t, wgs, d, nk_pad, s);
  else launch_mfma_t<false, false>(a, &t, wgs, d, nk_pad, s);
  return check_launch(fn);
}

namespace {
// gist_attn_forward_paged (k_scale == v_scale == NULL: bf16 cache) and
// gist_attn_forward_paged_fp8: ell = 1 runs the EOS kernel, 2 <= ell <= 64
// the l >= 2 kernel, both reading the gists through block indices
gist_status attn_forward_paged(const void* k_cache, const void* v_cache, const float* k_scale,
                               const float* v_scale, bool fp8, int64_t n_blocks, int block_size,
                               const int32_t* item_blocks, int k, const int32_t* query_blocks,
                               int kq, int q_row0, int P, int ell, int Hq, int H, int d,
                               const void* q, const void* k_new, const void* v_new, int pos0,
                               float rope_base, float scale, void* out, void* stream) {
  clear_error();
  const char* fn = fp8 ? "gist_attn_forward_paged_fp8" : "gist_attn_forward_paged";
  auto err = [&](gist_status c, const char* m) { return fail(c, std::string(fn) + ": " + m); };
  if (P < 0) return err(GIST_ERR_INVALID_ARG, "P < 0");
  if (n_blocks < 1 || n_blocks > INT32_MAX || block_size < 1)
    return err(GIST_ERR_INVALID_ARG, "bad n_blocks or block_size");
  if (d != 64 && d != 128) return err(GIST_ERR_UNSUPPORTED, "d must be 64 or 128");
  if (H < 1 || Hq < H || Hq % H != 0)
    return err(GIST_ERR_INVALID_ARG, "Hq must be a positive multiple of H");
  if (k < 1 || kq < 0 || q_row0 < 0 || k > block_size || q_row0 + kq > block_size)
    return err(GIST_ERR_INVALID_ARG, "gist rows must lie within one block (k >= 1)");
  if (ell < 1 || ell > 64) return err(GIST_ERR_UNSUPPORTED, "ell must be in [1, 64]");
  if (ell == 1) {
    if (Hq / H > 16) return err(GIST_ERR_UNSUPPORTED, "Hq/H must be <= 16 for ell = 1");
    if (k + kq > 32) return err(GIST_ERR_UNSUPPORTED, "k + k' must be <= 32 for ell = 1");
  } else {
    if (Hq / H > 32) return err(GIST_ERR_UNSUPPORTED, "Hq/H must be <= 32");
    if ((k + kq + ell + 15) / 16 * 16 > 128)
      return err(GIST_ERR_UNSUPPORTED, "k + k' + ell must fit 128 keys (16-key tiles)");
  }
  if (!(scale > 0.f) || !std::isfinite(scale))
    return err(GIST_ERR_INVALID_ARG, "scale must be positive and finite");
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return err(GIST_ERR_INVALID_ARG, "rope_base must be positive");
  if (kq > 0 && !query_blocks) return err(GIST_ERR_INVALID_ARG, "query_blocks is NULL");
  if (P == 0) return GIST_OK;
  if (!k_cache || !v_cache || !item_blocks || !q || !k_new || !v_new || !out ||
      (fp8 && (!k_scale || !v_scale)))
    return err(GIST_ERR_INVALID_ARG, "NULL tensor argument");
  if (fp8 && ((((uintptr_t)k_scale) | ((uintptr_t)v_scale)) & 3) != 0)
    return err(GIST_ERR_INVALID_ARG, "scales must be 4-byte aligned");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(k_new) ||
      !aligned16(v_new) || !aligned16(out))
    return err(GIST_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if ((int64_t)P * H * ell > INT32_MAX) return err(GIST_ERR_UNSUPPORTED, "P*H*ell too large for one launch");

  FwdArgs a = {};
  a.N = n_blocks;
  a.k = k;
  a.qN = n_blocks;
  a.kq = kq;
  a.item_ids = item_blocks;
  a.q_ids = kq ? query_blocks : nullptr;
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
  set_rope(a, d, rope_base);
  a.paged = 1;
  a.paged_k = k_cache;
  a.paged_v = v_cache;
  a.block_size = block_size;
  a.q_row0 = q_row0;
  a.paged_kscales = fp8 ? k_scale : nullptr;
  a.paged_vscales = fp8 ? v_scale : nullptr;
  hipStream_t s = (hipStream_t)stream;
  if (ell == 1) launch_eos(a, nullptr, (int64_t)P * H, d, k + kq, fp8, s);
  else launch_mfma(a, d, (k + kq + ell + 15) / 16 * 16, fp8, false, s);
  return check_launch(fn);
}
}  // namespace

extern "C" gist_status gist_attn_forward_paged(const void* k_cache, const void* v_cache,
                                               int64_t n_blocks, int block_size,
                                               const int32_t* item_blocks, int k,
                                               const int32_t* query_blocks, int kq, int q_row0,
                                               int P, int ell, int Hq, int H, int d,
                                               const void* q, const void* k_new,
                                               const void* v_new, int pos0, float rope_base,
                                               float scale, void* out, void* stream) {
  return attn_forward_paged(k_cache, v_cache, nullptr, nullptr, false, n_blocks, block_size,
                            item_blocks, k, query_blocks, kq, q_row0, P, ell, Hq, H, d, q, k_new,
                            v_new, pos0, rope_base, scale, out, stream);
}

extern "C" gist_status gist_attn_forward_paged_fp8(const void* k_cache, const void* v_cache,
                                                   const float* k_scale, const float* v_scale,
                                                   int64_t n_blocks, int block_size,
                                                   const int32_t* item_blocks, int k,
                                                   const int32_t* query_blocks, int kq, int q_row0,
                                                   int P, int ell, int Hq, int H, int d,
                                                   const void* q, const void* k_new,
                                                   const void* v_new, int pos0, float rope_base,
                                                   float scale, void* out, void* stream) {
  return attn_forward_paged(k_cache, v_cache, k_scale, v_scale, true, n_blocks, block_size,
                            item_blocks, k, query_blocks, kq, q_row0, P, ell, Hq, H, d, q, k_new,
                            v_new, pos0, rope_base, scale, out, stream);
}

extern "C" gist_status gist_attn_forward_last(const gist_pool* pool, int layer,
                                              const int32_t* item_ids, int P, int ell, int Hq,
                                              const void* q_last, const void* k_new,
                                              const void* v_new, int pos0, float rope_base,
                                              float scale, const gist_pool* qpool,
                                              const int32_t* q_ids, void* out, void* stream) {
  return attn_forward(pool, layer, item_ids, P, ell, Hq, q_last, k_new, v_new, pos0, rope_base,
                      scale, qpool, q_ids, out, stream, true);
}
