/*
 * kvq — group-wise KV-cache quantization and fused-dequant decode attention
 * for AMD Instinct MI355X (gfx950).  Plain C ABI: host integers, floats and
 * device pointers only.
 *
 * Pages the operations follow (titles as published):
 *  [Oaken]      "大模型KV缓存量化技术：原理、优化与实践" (jsqmd.com)
 *  [KVQ-Eng]    "大模型推理加速之KV Cache量化压缩原理与工程实现" (yunthe.com)
 *  [Cocktail]   Cocktail chunk-adaptive mixed-precision KV-cache page (peacm.com)
 *  [TurboQuant] TurboQuant KV-cache page (bhfrc.com)
 *  [KVO-LLM]    "长上下文LLM推理中的KV Cache优化技术解析" (intelliparadigm.com)
 *
 * Conventions shared by every entry point
 *  - Layout of K and V follows the cache-size formula of [KVQ-Eng]
 *    ("KV Cache的显存瓶颈" section): [batch][kv_heads][seq][head_dim], fp16,
 *    row-major, head_dim == 128.
 *  - Ownership: the caller allocates and frees every buffer (sizes from
 *    kvq_cache_bytes / kvq_decode_workspace_bytes).  The library never
 *    allocates, frees or synchronizes, and keeps no state beyond the fixed
 *    per-device array of kvq_decode_attn_noalloc; all work is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream) and buffers must
 *    stay alive until that work has completed.  Pre-allocating the cache is
 *    the practice [Cocktail] §5.2 recommends.
 *  - Errors: arguments visible to the host are checked before any HIP call;
 *    a negative kvq_status is returned and nothing is enqueued.  A failed
 *    launch returns KVQ_ERR_HIP.  Conditions only the device can see set bits
 *    in the cache's `status` word (KVQ_FLAG_*), which the caller reads after
 *    synchronizing; the library never clears it.
 *  - Pointers: device pointers must be 16-byte aligned, except `status`
 *    (4-byte) and the byte arrays `zero`/`zero2`/`chunk_bits` (1-byte).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_HEAD_DIM 128

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent field */
  KVQ_ERR_UNSUPPORTED = -2, /* valid but not implemented (head_dim != 128, ...) */
  KVQ_ERR_CAPACITY = -3,    /* t_new or max_len larger than the cache holds */
  KVQ_ERR_ALIGNMENT = -4,   /* a device pointer is not aligned as required, or an OAKEN
                               sparse_cap is not a multiple of 4 */
  KVQ_ERR_WORKSPACE = -5,   /* decode workspace missing or too small */
  KVQ_ERR_HIP = -6          /* a HIP launch failed */
} kvq_status;

/* Cache organisation. */
enum {
  KVQ_MODE_UNIFORM = 0,     /* one bit-width per tensor */
  KVQ_MODE_CHUNK_MIXED = 1, /* Cocktail: FP16 / INT4 / INT2 per 32-token chunk, reordered */
  KVQ_MODE_OAKEN = 2,       /* Oaken: dense INT4 body + sparse shifted outer values */
  KVQ_MODE_DSQ = 3          /* KVO-LLM DSQ: significant tokens INT8, the others INT2 */
};

/* Grouping axis of a tensor. */
enum {
  KVQ_AXIS_TOKEN = 0,  /* groups of `group` consecutive channels of one token */
  KVQ_AXIS_CHANNEL = 1 /* groups of `group` consecutive tokens of one channel (K only) */
};

/* Code format of a tensor. */
enum {
  KVQ_FMT_INT = 0, /* integer codes as described below */
  KVQ_FMT_E4M3 = 1, /* FP8 E4M3 codes ([KVQ-Eng] §"主流KV Cache量化方案对比", FP8 item);
                       UNIFORM mode, bits 8, TOKEN axis, symmetric 0, K and V alike */
  KVQ_FMT_E5M2 = 2   /* FP8 E5M2 codes (the same item's other format); same constraints */
};

/* Device status bits (OR-ed into *status by kernels). */
#define KVQ_FLAG_POS_RANGE 1u       /* pos[b] + t_new > max_seq, or pos[b] < 0: rows skipped */
#define KVQ_FLAG_SPARSE_FULL 2u     /* Oaken sparse list full: outer entries dropped */
#define KVQ_FLAG_LEN_RANGE 4u       /* decode seq_len[b] outside [0, max_len]: clamped */
#define KVQ_FLAG_BAD_CHUNK_BITS 8u  /* chunk bit-width not in {16, 4, 2}: used as 2 */
#define KVQ_FLAG_PAGE_RANGE 16u     /* paged cache: block-table entry outside [0, num_pages):
                                       append rows skipped, decode reads page 0 instead */

/*
 * One quantized tensor (K or V) of the cache.
 *
 * Quantizer ([Oaken] §2.1 scale formula, [Cocktail] §3.2.2 code formula),
 * per group of fp16 values x, in IEEE binary32 with round-half-to-even:
 *   asymmetric: lo = min(0, min x), hi = max(0, max x), s = (hi - lo) / (2^bits - 1),
 *               z = clamp(rne(-lo / s), 0, 2^bits - 1),
 *               q = clamp(rne(x / s) + z, 0, 2^bits - 1),  x_hat = (q - z) * s;
 *               an all-zero group has s = 0, z = 0, q = 0.
 *   symmetric (bits 8, [KVQ-Eng] INT8 listing): s = max|x| / 127,
 *               q = clamp(rne(x / s), -128, 127), x_hat = q * s.
 *   E4M3 (format KVQ_FMT_E4M3): s = max|x| / 448, q = the OCP E4M3 value
 *               (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 *               infinities, largest finite 448) nearest to x / s, ties to
 *               the even mantissa, saturating at 448, sign bit of x / s;
 *               x_hat = value(q) * s.  Stored like symmetric INT8 (one
 *               byte per code, no zero buffer).
 *   E5M2 (format KVQ_FMT_E5M2): s = max|x| / 57344, q = the OCP E5M2 value
 *               (1 sign, 5 exponent bits with bias 15, 2 mantissa bits)
 *               nearest to x / s, ties to the even mantissa, saturating at
 *               57344 (no infinity is stored), sign bit of x / s; stored as
 *               E4M3 is.
 *
 * Buffers by mode (B = batch, H = kv_heads, S = max_seq, D = 128,
 * RB = D * bits / 8 bytes per token row, NG = D / group):
 *  UNIFORM, TOKEN axis:
 *    codes  [B][H][S][RB]  one packed row per token (row layouts below)
 *    scale  [B][H][S][NG]  float
 *    zero   [B][H][S][NG]  uint8 (unused and may be NULL when symmetric)
 *  UNIFORM, CHANNEL axis (K only, group == 64 tokens; asymmetric):
 *    codes  [B][H][S][RB]  token rows as above, for complete 64-token blocks
 *    scale  [B][H][S/64][D] float, zero [B][H][S/64][D] uint8
 *    codes16 [B][H][64][D] fp16 residual tail: the tokens of the block not
 *                          yet complete, row t - 64 floor(t / 64) for token
 *                          t, in the fp16 K row layout of the CHUNK_MIXED
 *                          FP16 pool (below)
 *  OAKEN (bits 4, TOKEN axis, group 32 or 64; [Oaken] §3.1-3.2):
 *    codes, scale, zero    the dense body as UNIFORM/TOKEN over the
 *                          non-outer values; outer positions hold code z
 *    oscale [B][H][S][NG]  float outer scale max|delta| / 31 per group
 *    rowptr [B][H][S+1]    uint32: entries of token t are
 *                          sparse[rowptr[t] .. rowptr[t+1]) of that (b, h)
 *    sparse [B][H][sparse_cap] uint16 entries
 *                          idx | side << 7 | mag << 8 | tag << 13:
 *                          idx the channel, side 1 above T_hi_outer,
 *                          x_hat = T_hi_outer + mag * oscale (side 1) or
 *                          T_lo_outer - mag * oscale (side 0); tag the
 *                          entry's token index mod 8 (a row tag for
 *                          decode, redundant with rowptr)
 *  CHUNK_MIXED ([Cocktail] §3.1.2; C = S / chunk_tokens chunk slots, each
 *  class pool holds up to C chunks per (b, h) in reordered slot order):
 *    codes16 [B][H][C][chunk_tokens][D] fp16, the FP16 chunks, plus 64
 *                          spare rows at the end; chunk C - 1 of a (b, h)
 *                          holds the waiting tokens of kvq_append_chunks
 *                          until the sequence's final chunk
 *    codes/scale/zero   INT4 pool, TOKEN-axis layout with C*chunk_tokens rows
 *    codes2/scale2/zero2 INT2 pool, same layout
 *  DSQ ([KVO-LLM] §3.1; Q = S / 64 token groups per (b, h), n = dsq_sig
 *  significant tokens per group, group = 32 for both tensors, bits and
 *  symmetric ignored):
 *    codes  [B][H][Q][16][D]  int8 rows of the significant tokens, slot i =
 *                          the group's i-th significant token in token order;
 *                          code = clamp(rne(x / s_d), -128, 127) with the
 *                          channel scale s_d = max|x| / 127 over the group's
 *                          significant tokens; slots n .. 15 hold zeros
 *    scale  [B][H][Q][D]   float channel scales s_d
 *    codes2 [B][H][Q][64][D/4] INT2 rows of the other tokens, slot j = the
 *                          group's j-th other token in token order; slots
 *                          64 - n .. 63 hold zeros.  K rows as usual; V rows
 *                          blocked: the 2-byte column word n (V word order)
 *                          of slot j sits at byte ((j / 8) * 16 + n) * 16 +
 *                          (j % 8) * 2 of the group's 2048 bytes, so the
 *                          words of 8 consecutive slots of one column are
 *                          one 16-byte run
 *    scale2, zero2 [B][H][Q][64][D/32] float / uint8, asymmetric groups of
 *                          32 channels (quantizer above, bits 2).  V rows
 *                          quantize v; K rows quantize the difference
 *                          delta = fl(k - base_d) from the group's base row
 *                          base_d = fl(fl(sum_i fl(s_d * c_id)) / n), the mean
 *                          of its dequantized significant K rows summed in
 *                          slot order, so k_hat = base + (c - z) * s
 *    codes16 [B][H][64][D] fp16 tail: the tokens of the group not yet
 *                          complete, row t - 64 floor(t / 64) for token t, K
 *                          rows in the K row layout and V rows in the V row
 *                          layout of the CHUNK_MIXED FP16 pool
 *    oscale (K only) [B][H][64] float: the scores of the tail's tokens
 *    dsq_mask (cache) [B][H][Q] uint64, bit t set when token t of the group
 *                          is significant
 *
 * Packed rows.  A row holds the 128 codes of one token in 16 words of 8
 * codes (a word is 8 * bits / 8 bytes; inside a word, code e sits at bits
 * e*bits .. e*bits + bits - 1 counted from the least significant bit of the
 * little-endian word; 8-bit symmetric codes are two's complement).  The
 * channel order differs between K and V so that the decode kernel can feed
 * rows straight into the matrix cores:
 *    K rows: word 4 q + s holds channels 32 s + 8 q + e    (q, s in 0..3)
 *    V rows: word n holds channels n + 16 e                (n in 0..15)
 * fp16 rows of the CHUNK_MIXED FP16 pool use the same word positions (16-byte
 * words); inside a K word the 8 halves hold channel offsets
 * 0, 4, 1, 5, 2, 6, 3, 7, inside a V word channels n + 16 e in order e.
 */
typedef struct kvq_tensor {
  int32_t bits;       /* UNIFORM: 8, 4 or 2.  OAKEN: 4.  CHUNK_MIXED: ignored */
  int32_t symmetric;  /* 1: symmetric INT8 (bits 8, TOKEN axis) */
  int32_t axis;       /* KVQ_AXIS_TOKEN or KVQ_AXIS_CHANNEL */
  int32_t group;      /* TOKEN: 32, 64 or 128 channels.  CHANNEL: 64 tokens */
  int32_t format;     /* KVQ_FMT_INT or KVQ_FMT_E4M3 */
  float thr[4];       /* OAKEN: T_lo_outer, T_lo_inner, T_hi_inner, T_hi_outer (inner ones
                         are informational; [Oaken] §3.2.1) */
  int64_t sparse_cap; /* OAKEN: capacity of `sparse` per (b, h), in entries, at most
                         2^31 - 4 (else KVQ_ERR_INVALID_ARG); a multiple of 4, so that
                         every (b, h) list starts 8-byte aligned (decode reads four
                         entries per load); else KVQ_ERR_ALIGNMENT */
  void* codes;
  float* scale;
  uint8_t* zero;
  float* oscale;
  uint32_t* rowptr;
  uint16_t* sparse;
  void* codes16;
  void* codes2;
  float* scale2;
  uint8_t* zero2;
} kvq_tensor;

typedef struct kvq_cache {
  int32_t batch;
  int32_t kv_heads;
  int32_t max_seq;      /* token capacity per (b, h); CHUNK_MIXED: multiple of chunk_tokens */
  int32_t head_dim;     /* must be 128 */
  int32_t mode;         /* KVQ_MODE_* */
  int32_t chunk_tokens; /* CHUNK_MIXED: tokens per chunk (16, 32 or 64) */
  kvq_tensor k;
  kvq_tensor v;
  int32_t* perm;        /* CHUNK_MIXED: [B][C] original chunk id at each slot */
  int32_t* seg;         /* CHUNK_MIXED: [B][4] {n_fp16, n_int4, n_int2, n_chunks} */
  uint32_t* status;     /* device word for KVQ_FLAG_* bits (required) */
  /* Paged layout (every mode; page_tokens 0 = contiguous).  Every per-token
   * buffer (codes, scale, zero, and Oaken's oscale) is then a pool of
   * num_pages pages [num_pages][H][page_tokens][row], and token t of
   * sequence b lives in page block_table[b][t / page_tokens], row
   * t % page_tokens of its head.
   *  - UNIFORM with a CHANNEL-axis K: K's per-block scale and zero are pools
   *    [num_pages][H][page_tokens / 64][128] (a 64-token block never
   *    straddles a page); the fp16 tail (codes16) stays per sequence.
   *  - OAKEN: the sparse lists (rowptr, sparse) stay per (sequence, head) as
   *    without pages: a dense page table plus per-sequence sparse lists,
   *    after the dual dense / sparse page management of [Oaken] §3.2.3.
   *  - CHUNK_MIXED: each class pool (FP16: codes16; INT4: codes, scale,
   *    zero; INT2: codes2, scale2, zero2) is a pool of num_pages pages, and
   *    block_table holds one table per class, int32
   *    [3][batch][max_seq / page_tokens] (FP16, INT4, INT2): class-local row
   *    r of sequence b (class-local chunk k holds rows k * chunk_tokens ..)
   *    lives in page block_table[cls][b][r / page_tokens].  The waiting
   *    chunk of streaming appends is the FP16 class's last chunk, so the
   *    last entry of each sequence's FP16 table must be mapped when
   *    kvq_append_chunks is used.
   *  - DSQ: pages hold page_tokens / 64 whole groups: every per-group buffer
   *    (codes, scale, codes2, scale2, zero2 and dsq_mask) is a pool
   *    [num_pages][H][page_tokens / 64][...] and group g of sequence b is
   *    group g % (page_tokens / 64) of page block_table[b][g * 64 /
   *    page_tokens]; the fp16 tails stay per sequence.
   * Pages are owned by the caller, who may map any page to any (b, logical
   * page); a page shared by two sequences is written by both.  An append
   * row or chunk whose table entry lies outside [0, num_pages) is skipped
   * and raises KVQ_FLAG_PAGE_RANGE. */
  int32_t page_tokens;          /* 0, 64, 128 or 256; max_seq a multiple of it */
  int32_t num_pages;            /* pages in each pool (paged: >= 1) */
  const int32_t* block_table;   /* paged: device int32 [batch][max_seq / page_tokens]
                                   (CHUNK_MIXED: [3][batch][max_seq / page_tokens]) */
  /* DSQ mode ([KVO-LLM] §3.1): significant tokens per 64-token group (1 .. 16;
   * the page's top 20 % of 64 is 12.8, so 13) and the significance mask. */
  int32_t dsq_sig;
  uint64_t* dsq_mask;           /* device [batch][kv_heads][max_seq / 64], 8-byte aligned */
} kvq_cache;

/* Byte sizes of every buffer of one tensor; 0 = buffer not used. */
typedef struct kvq_tensor_bytes {
  size_t codes, scale, zero, oscale, rowptr, sparse, codes16, codes2, scale2, zero2;
} kvq_tensor_bytes;

typedef struct kvq_cache_bytes_t {
  kvq_tensor_bytes k, v;
  size_t perm, seg, status;
  size_t dsq_mask;
} kvq_cache_bytes_t;

/*
 * Sizes of all buffers the cache described by `c` needs (pointer fields of
 * `c` are ignored).  Host only, no HIP call.  Returns INVALID_ARG /
 * UNSUPPORTED for a configuration the other entry points would reject.
 */
kvq_status kvq_cache_bytes(const kvq_cache* c, kvq_cache_bytes_t* out);

/*
 * Quantize t_new new tokens per sequence and write them into the cache
 * ([Oaken] §3.1 online stage; [Cocktail] §3.2.2 group quantization).
 *  k_new, v_new: device fp16 [batch][kv_heads][t_new][128].
 *  pos:          device int32 [batch]; token t of sequence b goes to cache
 *                position pos[b] + t.
 *  batch * kv_heads * t_new must be below 2^31 (UNSUPPORTED otherwise).
 *  UNIFORM/TOKEN: any pos, t_new >= 1.
 *  UNIFORM/CHANNEL: any t_new >= 1, appended as a stream: pos[b] must be
 *                the sequence's current length.  K blocks of 64 tokens that
 *                are complete after the call are quantized (their earlier
 *                tokens read from the fp16 tail); the new tokens of a block
 *                left incomplete are stored in the tail.  V rows are
 *                quantized per token as for the TOKEN axis.
 *  OAKEN:        rowptr[b][h][pos[b]] must already hold the entry count of
 *                the earlier tokens (0 at pos 0; this call writes
 *                rowptr[pos[b] + 1 .. pos[b] + t_new]); entries past
 *                sparse_cap are dropped with KVQ_FLAG_SPARSE_FULL.
 *  CHUNK_MIXED:  whole-sequence prefill: t_new == max_seq and pos[b] == 0;
 *                perm/seg from kvq_reorder_chunks select, for every slot,
 *                the source chunk and its class (FP16 chunks are copied).
 *  DSQ:          not accepted (INVALID_ARG): use kvq_dsq_append, which
 *                takes the token scores the selection needs.
 */
kvq_status kvq_quant_append(const kvq_cache* c, const void* k_new, const void* v_new,
                            int32_t t_new, const int32_t* pos, void* stream);

/*
 * [Cocktail] §3.1.2 reorder: for every sequence, place the chunks in class
 * order FP16, INT4, INT2, stable within a class, writing c->perm (slot ->
 * original chunk id) and c->seg ({n_fp16, n_int4, n_int2, n_chunks}).
 *  chunk_bits: device uint8 [batch][n_chunks], each 16, 4 or 2 (the
 *              per-chunk precision from the query-chunk similarity search,
 *              [Cocktail] §3.1.1); other values count as 2 and set
 *              KVQ_FLAG_BAD_CHUNK_BITS.
 *  n_chunks:   must equal max_seq / chunk_tokens.  CHUNK_MIXED mode only.
 */
kvq_status kvq_reorder_chunks(const kvq_cache* c, const uint8_t* chunk_bits, int32_t n_chunks,
                              void* stream);

/*
 * Cocktail streaming append ([Cocktail] §3.1.2: chunks kept contiguous by
 * class; §3.2.2 group quantization): t_new new tokens per sequence continue
 * it at pos[b], its current length, which must satisfy pos[b] /
 * chunk_tokens == seg[b][3] (the chunks complete so far; a new cache has
 * zeroed seg).  Tokens of the chunk not yet complete wait as fp16 in the
 * last chunk of the FP16 pool (chunk max_seq / chunk_tokens - 1, free until
 * the sequence's final chunk).  The i-th chunk this call completes in
 * sequence b takes the bit-width new_bits[b * n_new + i] (16, 4 or 2; other
 * values count as 2 and set KVQ_FLAG_BAD_CHUNK_BITS) and is copied (16) or
 * quantized (groups of `group` channels) into the next chunk of its class
 * pool; perm and seg are updated so that they, and the pools, equal what
 * kvq_reorder_chunks and a whole-sequence append would give for the
 * complete chunks.
 *  k_new, v_new: device fp16 [batch][kv_heads][t_new][128].
 *  new_bits:     device uint8 [batch][n_new]; n_new at least
 *                (t_new + chunk_tokens - 1) / chunk_tokens.
 *  A sequence whose pos[b] does not match seg, or which would pass max_seq,
 *  is skipped and sets KVQ_FLAG_POS_RANGE.  CHUNK_MIXED mode only.
 *  Decode attends the complete chunks and, when seq_len is given, the
 *  waiting tokens seg[b][3] * chunk_tokens .. seq_len[b] - 1.
 */
kvq_status kvq_append_chunks(const kvq_cache* c, const void* k_new, const void* v_new, int32_t t_new,
                             const int32_t* pos, const uint8_t* new_bits, int32_t n_new, void* stream);

/*
 * [KVO-LLM] §3.1 differential significant-token quantization of t_new new
 * tokens per sequence (DSQ mode only; layout and arithmetic in the DSQ
 * buffer description above), appended as a stream: pos[b] must be the
 * sequence's current length.  Every 64-token group that is complete after
 * the call is quantized (its tokens below pos[b] read from the tails); the
 * new tokens of the group left incomplete are stored in the tails with
 * their scores.  In each group the dsq_sig tokens with the largest scores
 * are significant: scores are ordered by their binary32 bit patterns as a
 * total order (-0 below +0, NaNs at the ends by sign), ties to the lower
 * token index, so exactly dsq_sig tokens are chosen.
 *  k_new, v_new: device fp16 [batch][kv_heads][t_new][128].
 *  score:        device float [batch][kv_heads][t_new], the per-token
 *                attention statistic of the page (e.g. attention mass over a
 *                recent window), 4-byte aligned.
 *  t_new:        >= 0 (0: nothing is enqueued).
 *  pos:          device int32 [batch]; a sequence whose pos[b] is negative
 *                or past max_seq - t_new is skipped and sets
 *                KVQ_FLAG_POS_RANGE.
 * Decode (kvq_decode_attn) attends the complete groups below seq_len[b] and
 * reads the tokens from 64 floor(seq_len[b] / 64) on from the tails, so
 * seq_len[b] is the appended length or a multiple of 64 not above it.
 */
kvq_status kvq_dsq_append(const kvq_cache* c, const void* k_new, const void* v_new, const float* score,
                          int32_t t_new, const int32_t* pos, void* stream);

/*
 * Workspace needed by kvq_decode_attn for the same (c, q_heads, max_len,
 * num_splits).  Host only.  The workspace holds the split partials (m, l,
 * unnormalized output per batch, query head and split; none when the chosen
 * split count is 1) and, for OAKEN, each token's share of the scores from
 * the K outer values ([batch][q_heads][max_len] binary32, from a 256-byte
 * aligned offset), formed by a first kernel of the same call.  Other modes
 * with one split need 0 bytes.  One workspace serves one call at a time.
 */
kvq_status kvq_decode_workspace_bytes(const kvq_cache* c, int32_t q_heads, int32_t max_len,
                                      int32_t num_splits, size_t* bytes);

/*
 * One decode step of softmax attention over the quantized cache, with the
 * dequantization fused into the q.K and p.V loops ([TurboQuant] §2.3, end:
 * dequantization inside the attention product, no separate pass).  The
 * sequence is split across workgroups and the partial results are merged
 * with the log-sum-exp rule ([Cocktail] §3.2.3: per-block attention whose
 * merge equals ordinary attention) by a second, small kernel.
 *  q:        device fp16 [batch][q_heads][128]; q_heads a multiple of
 *            kv_heads; query head h reads KV head h / (q_heads / kv_heads).
 *  seq_len:  device int32 [batch], tokens 0 .. seq_len[b]-1 are attended
 *            (UNIFORM/OAKEN; values outside [0, max_len] are clamped and set
 *            KVQ_FLAG_LEN_RANGE).  UNIFORM/CHANNEL reads K of the tokens
 *            from 64 floor(seq_len[b] / 64) on from the fp16 tail, so
 *            seq_len[b] is the appended length or a multiple of 64 not above
 *            it.  CHUNK_MIXED attends all chunks counted in seg, and with
 *            seq_len the tokens from seg[b][3] * chunk_tokens up to seq_len[b]
 *            waiting in the FP16 pool's last chunk (kvq_append_chunks; at
 *            most chunk_tokens - 1 of them); seq_len may be NULL.
 *  max_len:  host bound on seq_len (CHUNK_MIXED: max_seq), sizes the grid.
 *  sm_scale: score scale, usually 1/sqrt(128).
 *  out:      device fp32 [batch][q_heads][128]; a sequence with no tokens
 *            gets zeros.
 *  num_splits: sequence splits per (b, kv head); 0 picks one from the shape.
 *            Pieces are rounded up to whole 64-token steps (chunk-mixed:
 *            whole chunks), so a split count that does not divide the
 *            length evenly may come out lower; kvq_decode_workspace_bytes
 *            applies the same rule.  The result does not depend on the
 *            split count beyond binary32 rounding, and two calls with the
 *            same arguments give the same bits.
 */
kvq_status kvq_decode_attn(const kvq_cache* c, const void* q, int32_t q_heads,
                           const int32_t* seq_len, int32_t max_len, float sm_scale, float* out,
                           void* workspace, size_t workspace_bytes, int32_t num_splits,
                           void* stream);

/*
 * kvq_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops that forbid hipMalloc): the same
 * arguments without the workspace, and the same kernels; what the workspace
 * would hold (split partials, OAKEN's score shares) goes to a fixed array of
 * KVQ_STATIC_SCRATCH_BYTES in the library's device image, one per device,
 * held until the process ends.  The array's device
 * address is looked up on the first call on each device (the current
 * device), after which no call allocates or frees anything.
 *  Returns KVQ_ERR_WORKSPACE, before any launch, when the call needs more
 *  than KVQ_STATIC_SCRATCH_BYTES (kvq_decode_workspace_bytes gives the
 *  need), else as kvq_decode_attn.
 *  Every call on a device shares that device's array: calls that overlap on
 *  one device (two streams, two threads) race and must be ordered by the
 *  caller.  Each call writes every value of the array that enters its
 *  result before reading it, so the array needs no clearing between calls.
 */
#define KVQ_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
kvq_status kvq_decode_attn_noalloc(const kvq_cache* c, const void* q, int32_t q_heads,
                                   const int32_t* seq_len, int32_t max_len, float sm_scale, float* out,
                                   int32_t num_splits, void* stream);

/*
 * [Cocktail] §3.1.1 chunk precision search: for every sequence b, the
 * cosine similarity sim_i = q.c_i / (|q| |c_i|) of its query embedding with
 * each chunk embedding, T_low = s_min + (s_max - s_min) * alpha,
 * T_high = s_max - (s_max - s_min) * beta, and bits_i = 16 if sim_i > T_high,
 * 4 if T_low < sim_i <= T_high, else 2 (the page recommends alpha = 0.6,
 * beta = 0.1, §4.3.2).  Every similarity is a sequential binary64 sum over
 * d = 0 .. dim-1 with one rounding per operation, so results are
 * reproducible bit for bit by any such evaluation.
 *  q_emb:     device double [batch][dim], 8-byte aligned.
 *  chunk_emb: device double [batch][n_chunks][dim], 8-byte aligned.
 *  sims:      optional device double [batch][n_chunks] (NULL: not written).
 *  bits:      device uint8 [batch][n_chunks], the input of kvq_reorder_chunks.
 * alpha and beta must lie in [0, 1]; batch <= 65535.
 */
kvq_status kvq_chunk_bits(const double* q_emb, const double* chunk_emb, int32_t batch,
                          int32_t n_chunks, int32_t dim, double alpha, double beta, double* sims,
                          uint8_t* bits, void* stream);

/*
 * [Oaken] §3.1 offline stage, the distribution of sampled K or V values:
 * adds, for each of the n fp16 values of x, one count to hist[key], where
 * key orders fp16 bit patterns by value (h | 0x8000 for a positive sign
 * bit, 0xFFFF - h for a negative one, so -0 sorts just below +0).
 *  x:    device fp16 [n], 16-byte aligned; n <= 2^40.
 *  hist: device uint64 [65536], 8-byte aligned, accumulated into (the
 *        caller zeroes it before the first call of a calibration).
 */
kvq_status kvq_hist_f16(const void* x, int64_t n, uint64_t* hist, void* stream);

/*
 * Nearest-rank percentiles of a kvq_hist_f16 histogram of N values: for
 * each p_bp[i] (basis points, 0 .. 10000; e.g. 250 = 2.5 %), the value of
 * rank max(1, ceil(p * N / 10000)) in ascending order, as float.  These are
 * the Oaken thresholds (T_lo_outer, T_lo_inner, T_hi_inner, T_hi_outer at
 * 250, 1500, 8500, 9750 for the 5 % / 25 % / 70 % regions of §3.2.1).
 *  p_bp: host int32 [count], count <= 8.   out: device float [count]
 *  (NaN when the histogram is empty).
 */
kvq_status kvq_hist_percentiles(const uint64_t* hist, int32_t count, const int32_t* p_bp, float* out,
                                void* stream);

/* Static string naming a kvq_status value. */
const char* kvq_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
