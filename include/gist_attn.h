/*
 * gist_attn.h — C ABI of libgist_attn.so: gist-compressed KV attention and
 * paged single-token decode on AMD MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [GIST] liam.page, "把 item 压成 KV：gist 能不能用在相关性任务上"
 *   [KVC]  mcfzz.com, "为什么自回归推理缓存 KV，而不缓存历史 Q？"
 *   [SFX]  icman.com.cn/news/64898 (suffix-cache article)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor argument is a plain device pointer owned by the caller.  The
 *   library never allocates device memory and never frees caller memory.
 * - Layouts are dense, row-major, with the last dimension contiguous.
 * - Element type: GIST_BF16 (bfloat16 bits) or GIST_F32.  All arithmetic
 *   inside the kernels is fp32; bf16 outputs are rounded to nearest-even.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  The
 *   calls enqueue work and return; results are visible after the stream syncs.
 * - Arguments are validated on the host before any HIP call.  On invalid
 *   arguments the call returns a negative gist_status, enqueues nothing and
 *   records a message readable with gist_last_error().  A launch failure
 *   reported by the HIP runtime returns GIST_ERR_HIP.
 * - Index arrays (item ids, block tables) are read on the device and are
 *   bounds-checked there: an out-of-range index never causes an access
 *   outside the pool; the rows that depend on it are written as NaN.
 * - Calls that write memory another call reads must be ordered by the
 *   caller's streams.
 * - RoPE: channel pair (i, i + d/2) turns by pos * base^(-2i/d) ("rotate
 *   half"); positions are 1-based.  Only position differences matter
 *   ([GIST] 在线的一次 attention), so any origin works if it is consistent.
 * - GQA: query head h reads KV head h / (Hq / H).
 */
#ifndef GIST_ATTN_H
#define GIST_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GIST_OK = 0,
  GIST_ERR_INVALID_ARG = -1,  /* null pointer, negative size, inconsistent shapes */
  GIST_ERR_UNSUPPORTED = -2,  /* valid request outside what the kernels implement */
  GIST_ERR_OUT_OF_RANGE = -3, /* a host-visible index (layer) is out of range */
  GIST_ERR_HIP = -4           /* the HIP runtime reported an error */
} gist_status;

/*
 * Element types.  GIST_FP8_E4M3 is a pool-only storage type: OCP FP8 E4M3
 * codes (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; largest
 * finite value 448; codes 0x7F and 0xFF are NaN) with one fp32 scale per
 * (layer, item, K or V, KV head).  The pages name KV quantization as a lever
 * without fixing a scheme ([GIST] 收益有多大：存储; [KVC] Memory: the
 * per-element byte count b = 1); the activations of calls on such a pool
 * are bf16.
 */
typedef enum { GIST_F32 = 0, GIST_BF16 = 1, GIST_FP8_E4M3 = 2 } gist_dtype;

/* Opaque handle describing a caller-owned gist pool (host metadata only). */
typedef struct gist_pool gist_pool;

/*
 * gist_pool_bytes — bytes of a pool holding N items, each with k gist
 * positions in each of L layers: N * 2*L*k*H*d * sizeof(dtype), the per-item
 * size 2·L·k·H·h·b of [GIST] 在线的一次 attention / 收益有多大：存储.  For
 * GIST_FP8_E4M3: N * L * (2*k*H*d + 2*H*4) (one byte per element plus the
 * fp32 scales).  Returns 0 for invalid shapes.
 */
size_t gist_pool_bytes(int L, int64_t N, int k, int H, int d, gist_dtype dtype);

/*
 * gist_pool_create — wrap caller-owned device storage as a gist pool.
 *   storage       device buffer of exactly gist_pool_bytes(...) bytes,
 *                 16-byte aligned, layout [L][N][2][H][k][d]; index 0 of the
 *                 "2" axis holds K, index 1 holds V.  For every (layer, item)
 *                 the K and V rows of all H heads form one contiguous record.
 *   K rows are stored already rotated at the canonical gist positions
 *   1..k ([GIST] 在线的一次 attention: the query sits k positions after the
 *   gist, as in training).  The handle is immutable and may be shared by
 *   concurrent streams.  Requires d in {64, 128}, 1 <= k <= 64, H >= 1.
 *   Writes the new handle to *out (host memory, freed by gist_pool_destroy).
 */
/*
 * GIST_FP8_E4M3 storage: the codes [L][N][2][H][k][d] (uint8, same order as
 * above) followed by the scales [L][N][2][H] (fp32; index 0 of the "2" axis
 * scales K, index 1 scales V).  Element value = decode(code) * scale of its
 * (layer, item, K/V, head).
 */
gist_status gist_pool_create(gist_pool** out, int L, int64_t N, int k, int H, int d,
                             gist_dtype dtype, void* storage, size_t storage_bytes);

/* gist_pool_destroy — free the handle (never the storage).  NULL is a no-op. */
gist_status gist_pool_destroy(gist_pool* pool);

/*
 * gist_pool_write — store n items' gist K/V for one layer (the offline
 * extraction output of [GIST] 论文做了什么 / 在线的一次 attention).
 *   ids      device int32 [n], destination item rows (each < N; out-of-range
 *            ids are skipped on the device)
 *   k_src    device [n][k][H][d], pool dtype; row i rotated at position
 *            src_pos0 + i.  It is re-rotated to the canonical position 1 + i
 *            (a rotation by 1 - src_pos0, formed in double, so any int
 *            src_pos0 is valid; a plain copy when src_pos0 == 1).
 *   v_src    device [n][k][H][d], pool dtype, copied unchanged.
 *   rope_base RoPE base used for the re-rotation.
 * Duplicate ids in one call race (one of the writes wins).  n == 0 is a no-op.
 * GIST_FP8_E4M3 pools take bf16 k_src/v_src and quantize each (item, K or V,
 * head) block of k*d values x (K after the re-rotation, in fp32): amax =
 * max |x|, scale = amax / 448 in fp32 (1 when amax is 0), code = x / scale
 * (fp32 quotient) rounded to the nearest E4M3 value, ties to even mantissa,
 * clamped to +-448.  Inputs must be finite.
 */
gist_status gist_pool_write(const gist_pool* pool, int layer, const int32_t* ids, int64_t n,
                            const void* k_src, const void* v_src, int src_pos0,
                            float rope_base, void* stream);

/*
 * gist_attn_forward — one layer of online gist attention for P (item, query)
 * pairs ([GIST] 在线的一次 attention; query-gist variant: 能不能再进一步).
 * For pair p and query head h (KV head g = h / (Hq/H)) the keys are
 *   [ item gist of item_ids[p] (k rows, from pool)
 *   ; query gist of q_ids[p] (k' rows, from qpool; only if qpool != NULL)
 *   ; RoPE(k_new[p][t][g], pos0 + t) for t < ell ]
 * and the values are the same sequence of V rows.  Query token t (rotated at
 * pos0 + t) sees every gist key and new keys 0..t (itself included); the
 * output is softmax(scale * q·K^T) V over those keys ([KVC] Reusable-state).
 *   pool      item gist pool; dtype, H and d of the call come from it
 *   item_ids  device int32 [P]
 *   q         device [P][ell][Hq][d]
 *   k_new     device [P][ell][H][d]   (not yet rotated)
 *   v_new     device [P][ell][H][d]
 *   pos0      position of the first new token: k + 1 (k + k' + 1 with a
 *             query gist), so the query-to-gist distance matches training.
 *             Any int: positions pos0 + t are formed in double, so they may
 *             run past 2^31 - 1.
 *   scale     softmax scale, normally 1/sqrt(d)
 *   qpool     optional query-gist pool (same L, H, d, dtype); NULL for none
 *   q_ids     device int32 [P] rows of qpool (ignored when qpool is NULL)
 *   out       device [P][ell][Hq][d], pool dtype; must not alias the inputs
 * Limits: 1 <= ell <= 1024, Hq % H == 0, Hq / H <= 32.  P == 0 is a no-op.
 * bf16 with 2 <= ell <= 64 and k + k' + ell <= 128 runs the MFMA kernel;
 * bf16 with ell == 1, Hq / H <= 16 and k + k' <= 32 the EOS kernel; every
 * other case runs the VALU kernel.
 * GIST_FP8_E4M3 pools: q, k_new, v_new and out are bf16 and qpool must be
 * fp8 too.  The MFMA shapes (2 <= ell <= 64, k + k' + ell <= 128) and the
 * EOS shapes (ell == 1, Hq / H <= 16, k + k' <= 32) are implemented; other
 * shapes return GIST_ERR_UNSUPPORTED.  Every E4M3 value is a bf16 value.
 * With ell == 1 the codes enter the matrix products exactly, a key's K scale
 * multiplies its fp32 logit and its V scale its softmax weight in the product
 * with V (the softmax denominator takes the unscaled weight).  With ell >= 2
 * each gist K element, decode(code) * scale in fp32, is staged as a bf16
 * pair (see Precision) and each gist V element is rounded to bf16 once.
 * Precision (bf16 MFMA and EOS kernels): the rotated Q and the rotated
 * K_new are carried as bf16 pairs hi + lo, hi the nearest bf16 value and lo
 * the nearest bf16 value of the remainder, and each logit takes
 * K_hi·Q_hi + K_hi·Q_lo + K_lo·Q_hi on the matrix cores with fp32
 * accumulation, about 2^-16 of |q||k|.  The softmax weights are rounded to
 * bf16 for the product with V.  The VALU kernel computes in fp32.
 */
gist_status gist_attn_forward(const gist_pool* pool, int layer, const int32_t* item_ids, int P,
                              int ell, int Hq, const void* q, const void* k_new,
                              const void* v_new, int pos0, float rope_base, float scale,
                              const gist_pool* qpool, const int32_t* q_ids, void* out,
                              void* stream);

/*
 * gist_attn_forward_paged — gist attention with the gists read from a paged
 * KV cache in the layout paged decode uses, so gist rows and decode sequences
 * can live in one block pool ([GIST] 能不能再进一步: align the gist rows to the
 * serving engine's block size).  With 16-token blocks, k + k' = 8 + 8 fills
 * one block exactly (the alignment the same section recommends): pass
 * query_blocks = item_blocks and q_row0 = k.  ell = 1 is the query-gist EOS
 * step (one token over the item gist, the query gist and itself); 2 <= ell
 * <= 64 is the item-only or query-gist online pass of gist_attn_forward with
 * the gist rows taken from blocks instead of pool records.
 *   k_cache, v_cache  device bf16 [n_blocks][H][block_size][d]; gist K rows
 *                     already rotated at their canonical positions (item
 *                     gist 1..k, query gist k+1..k+k')
 *   item_blocks       device int32 [P]: the item gist of pair p is rows
 *                     0..k-1 of block item_blocks[p]
 *   query_blocks      device int32 [P] (NULL when k' = 0): the query gist is
 *                     rows q_row0 .. q_row0+k'-1 of block query_blocks[p]
 *   q, k_new, v_new, out  as gist_attn_forward: q, out [P][ell][Hq][d];
 *                     k_new, v_new [P][ell][H][d]
 *   pos0              position of the first new token: k + k' + 1
 * Limits: d in {64, 128}; Hq % H == 0; 1 <= k; both gists within a block;
 * ell = 1: Hq/H <= 16 and k + k' <= 32; 2 <= ell <= 64: Hq/H <= 32 and
 * k + k' + ell <= 128 rounded up to 16 (else GIST_ERR_UNSUPPORTED).  Block
 * indices are bounds-checked on the device (out-of-range: the pair's rows are
 * NaN).  The results equal gist_attn_forward's over pools holding the same
 * rows, bit for bit.  P == 0 is a no-op.
 */
gist_status gist_attn_forward_paged(const void* k_cache, const void* v_cache, int64_t n_blocks,
                                    int block_size, const int32_t* item_blocks, int k,
                                    const int32_t* query_blocks, int kq, int q_row0, int P,
                                    int ell, int Hq, int H, int d, const void* q,
                                    const void* k_new, const void* v_new, int pos0,
                                    float rope_base, float scale, void* out, void* stream);

/*
 * gist_attn_forward_paged_fp8 — gist_attn_forward_paged over a paged cache of
 * fp8 codes (OCP FP8 E4M3, as paged_decode_attn_fp8) with one fp32 scale per
 * (block, KV head) for K and one for V: the fp8 pool of [GIST] 收益有多大：存储
 * in the block layout of [GIST] 能不能再进一步.  A block holding both gists
 * gives them one scale per head.
 *   k_cache, v_cache  device uint8 codes [n_blocks][H][block_size][d], 16-byte
 *                     aligned; element = decode(code) * k_scale[block][head]
 *                     (resp. v_scale)
 *   k_scale, v_scale  device fp32 [n_blocks][H], 4-byte aligned
 * q, k_new, v_new and out are bf16; every other argument, limit and error
 * behaviour is that of gist_attn_forward_paged.  With ell = 1 a key's K
 * scale multiplies its fp32 logit and its V scale its softmax weight; with
 * ell >= 2 each gist element, decode(code) * scale, is staged as for an fp8
 * pool (see gist_attn_forward).
 */
gist_status gist_attn_forward_paged_fp8(const void* k_cache, const void* v_cache,
                                        const float* k_scale, const float* v_scale,
                                        int64_t n_blocks, int block_size,
                                        const int32_t* item_blocks, int k,
                                        const int32_t* query_blocks, int kq, int q_row0, int P,
                                        int ell, int Hq, int H, int d, const void* q,
                                        const void* k_new, const void* v_new, int pos0,
                                        float rope_base, float scale, void* out, void* stream);

/*
 * gist_attn_forward_last — gist_attn_forward for the last query token of
 * each pair only.  At the final layer the relevance score reads only the
 * last position ([GIST] 在线的一次 attention: the score head is applied to
 * the EOS token's hidden state), so that layer needs one output row per pair.
 *   q_last   device [P][Hq][d]: Q of token ell-1 only (position pos0+ell-1)
 *   k_new, v_new  device [P][ell][H][d], every new token (all are keys of
 *            the last token)
 *   out      device [P][Hq][d]
 * Every other argument, limit and error behaviour is that of
 * gist_attn_forward; the result equals row ell-1 of gist_attn_forward's
 * output (bit for bit: the same kernel code computes it).
 */
gist_status gist_attn_forward_last(const gist_pool* pool, int layer, const int32_t* item_ids, int P,
                                   int ell, int Hq, const void* q_last, const void* k_new,
                                   const void* v_new, int pos0, float rope_base, float scale,
                                   const gist_pool* qpool, const int32_t* q_ids, void* out,
                                   void* stream);

/*
 * gist_attn_forward_grouped — several independent gist_attn_forward calls of
 * one shape in one launch.  Each group is one call of the online pass of
 * [GIST] 在线的一次 attention, or of its EOS step at ell = 1 ([GIST]
 * 能不能再进一步) (its own layer, pairs, ids, activations and outputs);
 * groups share the pools, ell, Hq, pos0, rope_base and scale.  A
 * caller that holds several such calls at once (micro-batches at different
 * layers of a pipelined schedule, or several query batches at one layer)
 * pays one launch instead of one per call, and the last workgroups of one
 * group run beside the first of the next instead of idling the GPU.
 *   groups    host array of n_groups descriptors, read during the call only
 *             (its device pointers are as in gist_attn_forward: q, out
 *             [P][ell][Hq][d]; k_new, v_new [P][ell][H][d]; item_ids [P];
 *             q_ids [P] when qpool != NULL)
 *   n_groups  0 .. 32 (more: GIST_ERR_UNSUPPORTED); groups with P == 0 are
 *             skipped, and a call with no pairs is a no-op
 * Limits: bf16 or fp8 pools, and either ell == 1 with Hq/H <= 16 and k + k'
 * <= 32 (the EOS kernel) or 2 <= ell <= 64 with k + k' + ell <= 128 rounded
 * up to 16 and Hq/H <= 32 (the l >= 2 kernel), else GIST_ERR_UNSUPPORTED; a
 * layer out of range is GIST_ERR_OUT_OF_RANGE.  Validation of every group
 * precedes the launch.  Each group's output equals gist_attn_forward's for
 * that group bit for bit (the same kernel code computes every row).  Groups
 * whose outputs overlap each other or any group's inputs race.
 */
typedef struct gist_group {
  int layer;                /* pool layer of this group's pass */
  int P;                    /* pairs */
  const int32_t* item_ids;  /* device [P] */
  const int32_t* q_ids;     /* device [P], or NULL without a query-gist pool */
  const void* q;            /* device bf16 [P][ell][Hq][d] */
  const void* k_new;        /* device bf16 [P][ell][H][d] */
  const void* v_new;        /* device bf16 [P][ell][H][d] */
  void* out;                /* device bf16 [P][ell][Hq][d] */
} gist_group;

gist_status gist_attn_forward_grouped(const gist_pool* pool, const gist_pool* qpool,
                                      const gist_group* groups, int n_groups, int ell, int Hq,
                                      int pos0, float rope_base, float scale, void* stream);

/*
 * gist_prefill_workspace_bytes — bytes of the workspace gist_prefill_attn
 * needs for n_tokens packed tokens, H KV heads and head size d: every K row
 * rotated, as a pair of bf16 arrays (the nearest bf16 values and the bf16
 * roundings of their remainders), 2 * n_tokens * H * d * 2 bytes.  Returns 0
 * for invalid shapes.
 */
size_t gist_prefill_workspace_bytes(int64_t n_tokens, int H, int d);

/*
 * gist_prefill_attn — offline gist extraction, one layer ([GIST] 论文做了什么:
 * the item runs with its k gist tokens appended, and every layer's K/V at the
 * gist positions are what is kept; 在线的一次 attention: they are stored at
 * the canonical positions 1..k).  Causal self-attention of B packed bf16
 * sequences [item tokens ; gist tokens] (over these alone the gist mask of
 * training is the causal mask) and, when pool != NULL, the store of each
 * sequence's last pool->k tokens as its gist.
 *   q          device [n_tokens][Hq][d]; k, v device [n_tokens][H][d]; Q and
 *              K not yet rotated
 *   seq_start  device int32 [B+1]: non-decreasing, seq_start[0] = 0,
 *              seq_start[B] = n_tokens, every length <= max_len.  Sequence b
 *              is tokens seq_start[b] .. seq_start[b+1]-1 at positions
 *              1..len.  A sequence whose bounds break these rules is skipped
 *              on the device (its output rows are not written).
 *   out        device [n_tokens][Hq][d]: token t of a sequence gets
 *              softmax(scale * q_t·K^T) V over its keys 0..t
 *   workspace  device buffer of >= gist_prefill_workspace_bytes(n_tokens, H,
 *              d) bytes, 16-byte aligned; receives every K row rotated at
 *              its position, as a bf16 pair (the K the attention reads)
 *   pool, layer, item_ids  optional bf16 gist pool with the call's H and d:
 *              the K of the last pool->k tokens of sequence b, rotated at
 *              1..k, and their V are stored at item item_ids[b] (device int32
 *              [B]).  Out-of-range ids and sequences shorter than k are
 *              skipped.  NULL pool: nothing is stored.
 * bf16 only; d in {64, 128}; Hq a multiple of H; B <= 65535;
 * max_len * H * d < 2^31 (else GIST_ERR_UNSUPPORTED).  B == 0 or
 * n_tokens == 0 is a no-op.  Two kernels run on the stream, K rotation (and
 * the gist store) first.
 */
gist_status gist_prefill_attn(const void* q, const void* k, const void* v, const int32_t* seq_start,
                              int B, int64_t n_tokens, int max_len, int Hq, int H, int d,
                              float rope_base, float scale, void* out, void* workspace,
                              size_t workspace_bytes, const gist_pool* pool, int layer,
                              const int32_t* item_ids, void* stream);

/*
 * paged_decode_workspace_bytes — fp32 workspace that paged_decode_attn needs
 * for R requests, Hq query heads, block tables of max_blocks entries of
 * block_size tokens and head size d.  Returns 0 for invalid shapes.
 */
size_t paged_decode_workspace_bytes(int R, int Hq, int max_blocks, int block_size, int d);

/*
 * paged_decode_attn — one decode step of R requests over a paged KV cache
 * ([KVC] Reusable-state: K_{<=t} = [K_{<t}; k_t], o_t = softmax(q_t K^T
 * /sqrt(d_k)) V; [SFX] section 6 problem 4: attention finds each logical
 * block through a logical->physical table; [SFX] section 5: 256-token blocks).
 *   k_cache, v_cache  device [n_blocks][H][block_size][d]; cached K is
 *                     already rotated at its own position
 *   block_table       device int32 [R][max_blocks]; logical token j of
 *                     request r is row j % block_size of physical block
 *                     block_table[r][j / block_size]
 *   context_lens      device int32 [R], cached tokens per request
 *                     (0 <= len <= max_blocks * block_size)
 *   q                 device [R][Hq][d]; k_new, v_new device [R][H][d]
 *   positions         device int32 [R], position of the new token
 *   out               device [R][Hq][d]
 *   workspace         device buffer of >= paged_decode_workspace_bytes(...)
 *                     bytes, 16-byte aligned; contents are scratch
 * The new token attends to the whole cache and to itself; k_new/v_new are
 * not written back.  Limits: d in {64, 128}, Hq % H == 0, Hq / H <= 8,
 * block_size a multiple of 16.  R == 0 is a no-op.
 */
gist_status paged_decode_attn(const void* k_cache, const void* v_cache, int64_t n_blocks,
                              int block_size, const int32_t* block_table, int max_blocks,
                              const int32_t* context_lens, int R, const void* q,
                              const void* k_new, const void* v_new, const int32_t* positions,
                              int Hq, int H, int d, gist_dtype dtype, float rope_base,
                              float scale, void* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * paged_decode_attn_fp8 — paged_decode_attn over a KV cache stored as fp8
 * codes (OCP FP8 E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; largest finite value 448; codes 0x7F and 0xFF are NaN) with one fp32
 * scale per (physical block, KV head) for K and one for V.  The pages fix no
 * quantized format; this one halves the cache bytes the decode step streams
 * ([KVC] Memory: M_KV = 2*B*L*T*h_kv*d_h*b with b = 1).
 *   k_cache, v_cache  device uint8 codes [n_blocks][H][block_size][d];
 *                     element = decode(code) * k_scale[block][head] (resp. v)
 *   k_scale, v_scale  device fp32 [n_blocks][H], 4-byte aligned
 *   q, k_new, v_new, out  bf16, as in paged_decode_attn (the new token's own
 *                     key and value are not quantized)
 * Every other argument, the workspace size and the error behaviour are those
 * of paged_decode_attn.
 */
gist_status paged_decode_attn_fp8(const void* k_cache, const void* v_cache, const float* k_scale,
                                  const float* v_scale, int64_t n_blocks, int block_size,
                                  const int32_t* block_table, int max_blocks,
                                  const int32_t* context_lens, int R, const void* q,
                                  const void* k_new, const void* v_new, const int32_t* positions,
                                  int Hq, int H, int d, float rope_base, float scale, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_decode_attn_noalloc — paged_decode_attn for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  It allocates
 * nothing: the split-K partials go to a scratch array of 16 MiB that the
 * library holds on each GPU it runs on until the process ends (its address is
 * looked up once per device, on the first call with that device current).
 *   Arguments, layouts, results and limits are those of paged_decode_attn
 *   without the workspace; the results are identical to it.
 *   A call whose partials need more than 16 MiB
 *   (paged_decode_workspace_bytes(R, Hq, max_blocks, block_size, d) >
 *   16 * 2^20) returns GIST_ERR_UNSUPPORTED before any HIP call; the 32
 *   requests x 4096 tokens x 32 heads decode step needs 8.65 MB.
 *   GIST_ERR_HIP if the scratch address cannot be obtained.
 * Concurrency: every call on one GPU uses that GPU's one scratch array, so
 * calls that may overlap on one GPU (other streams, other host threads) race
 * and give wrong results; order them on one stream.  Nothing in the scratch
 * needs clearing between calls: each call writes every partial it reads.
 */
gist_status paged_decode_attn_noalloc(const void* k_cache, const void* v_cache, int64_t n_blocks,
                                      int block_size, const int32_t* block_table, int max_blocks,
                                      const int32_t* context_lens, int R, const void* q,
                                      const void* k_new, const void* v_new,
                                      const int32_t* positions, int Hq, int H, int d,
                                      gist_dtype dtype, float rope_base, float scale, void* out,
                                      void* stream);

/* gist_last_error — message of the last failed call on this thread ("" if none). */
const char* gist_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GIST_ATTN_H */
