/*
 * semkv.h -- C ABI of the SemKV mixed-precision KV-cache hot path (gfx950).
 *
 * The operations follow the problem statement of the page "SemKV: Semantic
 * Mixed-Precision KV Cache Quantization Guided by the Quality Cliff for
 * Long-Context LLM Inference" (abbreviated SemKV): a full-precision KV cache
 * and a per-token importance score go in; the tokens are ranked, the top-r
 * set gets the higher of two level counts, every K and V row is quantized and
 * packed, and decoding reads the packed cache (SemKV Fig. 1, Figs. 4-5);
 * newly generated tokens are quantized block-exactly (SemKV Fig. 6).
 *
 * Conventions for every entry point
 *  - Data pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or retains device memory.  Its only state besides its
 *    loaded code objects: per device, the decode kernel's resident workgroup
 *    count (taken from the occupancy query on first use, held in an atomic)
 *    and the address of the static scratch array of
 *    semkv_decode_attn_noalloc (part of the code object; looked up on first
 *    use).  Both are the same for every caller.  `stream` is a hipStream_t passed as
 *    void* (NULL = the null stream).  Calls enqueue work on `stream` and
 *    return without synchronising, except semkv_sync_check.
 *  - fp16 data is passed as uint16_t bit patterns so this header does not
 *    depend on HIP.
 *  - Arguments are validated on the host before anything is launched; an
 *    invalid call returns a negative status and enqueues nothing.  No
 *    exception crosses the ABI.  Asynchronous device errors surface at the
 *    next semkv_sync_check.
 *  - Calls that mutate one semkv_cache (quantize_pack, append_block) must not
 *    overlap; different caches may be used concurrently on different streams.
 *  - head_dim is 128; level counts L satisfy 3 <= L <= 65536.
 *
 * Packed row format (ours; SemKV Table 6 fixes only the code-bit rates):
 *  a row is the 128 values of one (sequence, token, layer, KV head, K-or-V).
 *  m = min, M = max, scale = smallest fp16 >= (M - m)/(L - 1) (0 when M == m),
 *  code_i = round-half-even((x_i - m)/scale) in [0, L-1]; meta = {scale, m}
 *  as two fp16 (scale first; a zero minimum is stored as +0).  g codes form
 *  one b-bit field sum_i code[g*j+i] * L^i, fields are laid LSB-first into a
 *  little-endian bit stream; (g, b) = (5,8) for L=3, (4,8) L=4, (3,7) L=5,
 *  (3,8) L=6, (1,3) L=8, (2,8) L=16, (1,16) L=65536, else (1, ceil(log2 L)).
 *  semkv_row_bytes(L) = ceil(ceil(128/g) * b / 8): 43 B for L=6, 38 B for L=5.
 */
#ifndef SEMKV_H
#define SEMKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t semkv_status;
enum {
  SEMKV_OK = 0,
  SEMKV_EINVAL = -1,       /* null/misaligned pointer, size or range error */
  SEMKV_EUNSUPPORTED = -2, /* valid but not supported (head_dim, L)          */
  SEMKV_ECAPACITY = -3,    /* a pool has no room for the rows to be written */
  SEMKV_EWORKSPACE = -4,   /* workspace missing or smaller than required    */
  SEMKV_EHIP = -5          /* the HIP runtime reported an error             */
};

/* Geometry of one cache.  One precision per token for all layers, KV heads,
 * K and V (SemKV Fig. 5).  Query head h reads KV head h / (q_heads/kv_heads)
 * (grouped-query attention of the backbones in SemKV Table 2). */
typedef struct {
  int32_t batch, layers, kv_heads, q_heads, head_dim; /* head_dim must be 128 */
  int32_t L_high, L_low;   /* 3 <= L_low <= L_high <= 65536                  */
  int32_t block;           /* generation block (SemKV Fig. 6), 1..1024       */
  int64_t cap_high, cap_low; /* rows per (b, layer, kv head, K|V); multiple of 16 */
  int32_t rotate;          /* 0, or 1: Hadamard rotation of every row before
                            * quantization (SemKV Table 2's quantizer; H is the
                            * normalized Sylvester H_128, applied in fp32 by
                            * index-bit butterflies; the row minimum is rounded
                            * down to fp16).  Decode rotates the queries in fp32
                            * (the matrix-core kernel then puts them on a
                            * fixed-point grid of 2^-27 of their largest
                            * component) for the pool rows and rotates their
                            * share of the output back; the fp16 tail of generation
                            * is not quantized, hence not rotated, and is read
                            * with the query as given.  Any level pair and
                            * query group; rotated rows must stay within the
                            * fp16 range. */
} semkv_geom;

/* A mixed-precision cache.  All buffers are caller-owned device memory whose
 * sizes semkv_cache_sizes reports; every base pointer is 256-byte aligned.
 *  codes_*  uint8  [B][layers][kv][2][cap * row_bytes(L)]  one plane per
 *           (b, layer, kv head, K|V).  K planes hold rows back to back (row r
 *           at r*R).  V planes are byte-planar in 16-row tiles: byte j of row
 *           r is at (r/16)*16*R + 16*j + r%16, so one code byte of 16
 *           consecutive tokens is contiguous.  R = semkv_row_bytes(L).
 *  meta_*   fp16   [B][layers][kv][2][cap][2]              {scale, min}
 *  tok_*    int32  [B][cap]      slot -> token index (written with the rows)
 *  tail_kv  fp16   [B][layers][kv][2][block][128]  newest tokens, unquantized
 *  tail_score fp32 [B][block]    their importance scores
 *  index 2 of the [..][2] axes: 0 = K, 1 = V.
 *  The counters are HOST-side and shared by every sequence of the batch:
 *  rows [0, n_high) / [0, n_low) of each pool are valid, tail rows
 *  [0, n_tail) are valid, and n_high + n_low + n_tail == n_tokens.  A cache
 *  driven by the semkv_ragged_* calls keeps them at 0 and holds each
 *  sequence's counters in a device array instead (see below). */
typedef struct {
  semkv_geom g;
  uint8_t* codes_high;
  uint8_t* codes_low;
  uint16_t* meta_high;
  uint16_t* meta_low;
  int32_t* tok_high;
  int32_t* tok_low;
  uint16_t* tail_kv;
  float* tail_score;
  int64_t n_high, n_low, n_tail, n_tokens;
} semkv_cache;

/* Packed bytes of one 128-value row at L levels; < 0 if L is unsupported. */
int64_t semkv_row_bytes(int32_t L);

/* Top-r count k = floor(r*n + 1/2) computed in double (SemKV Fig. 4: the
 * allocation is the top-r ranking; the integer rounding is our reading).
 * Returns < 0 if n < 0 or r is outside [0, 1]. */
int64_t semkv_topr_count(int64_t n, double r);

/* Bytes of each cache buffer for geometry *g, in this order:
 * codes_high, codes_low, meta_high, meta_low, tok_high, tok_low, tail_kv,
 * tail_score.  Validates *g. */
semkv_status semkv_cache_sizes(const semkv_geom* g, int64_t bytes_out[8]);

/* Workspace bytes needed by semkv_decode_* for `nlayers` layers and up to
 * `max_tokens` cached tokens per sequence, and by semkv_append_block.
 * Returns < 0 if *g is invalid. */
int64_t semkv_workspace_bytes(const semkv_geom* g, int32_t nlayers, int64_t max_tokens);

/* Rank (SemKV Figs. 2 and 4: rank within each prompt, no threshold; top-r
 * forms the high-precision set H).
 *  scores  fp32 [batch][ld_scores], the first n entries of each row are used
 *  k       0 <= k <= n, the size of H for every sequence
 *  perm    int32 [batch][n] out: H in ascending token order, then the other
 *          tokens ascending (so slot j of the high pool holds perm[j])
 *  mask    uint32 [batch][ceil(n/32)] out, nullable: bit t%32 of word t/32 is
 *          set iff token t is in H
 * Order: score descending, ties to the lower index, -0 == +0, NaN below
 * every number.  Errors: EINVAL (null scores/perm, n < 1, k outside [0, n],
 * ld_scores < n, batch < 1, n > 2^31 - 1). */
semkv_status semkv_rank_topr(const float* scores, int32_t batch, int64_t n, int64_t ld_scores,
                             int64_t k, int32_t* perm, uint32_t* mask, void* stream);

/* Key-norm token scores (SemKV Fig. 2: a per-token importance score from one
 * model-internal indicator, ranked within the prompt; SemKV Table 3 lists the
 * key-norm indicator; its form and layer window are not given there, and
 * the reading here is the sum of the key rows' Euclidean norms).
 *   scores[b * ld_scores + t] = sum over layers layer0 .. layer0+nlayers-1
 *     and KV heads 0 .. kv_heads-1 of sqrt(sum_d k[b,layer,head,t,d]^2)
 * accumulated in fp32, layer-major.  The result feeds semkv_rank_topr.
 *  k        fp16 keys; element (b, layer, head, token, d) is at
 *           k + b*strides[0] + layer*strides[1] + head*strides[2]
 *             + token*strides[3] + d   (strides in elements, d contiguous;
 *           every layer of the window must exist)
 *  scores   fp32 [batch][ld_scores] device memory, first n of each row written
 * Errors: EINVAL (null or misaligned pointers: k 16-byte, scores 4-byte;
 * strides negative or not multiples of 8; batch outside [1, 65535];
 * kv_heads, nlayers < 1; layer0 < 0; n < 1; ld_scores < n). */
semkv_status semkv_score_keynorm(const uint16_t* k, const int64_t strides[4], int32_t batch,
                                 int32_t kv_heads, int64_t n, int32_t layer0, int32_t nlayers,
                                 float* scores, int64_t ld_scores, void* stream);

/* Hidden-state delta-norm token scores, the pages' default indicator (SemKV
 * Table 2: hidden-state delta norm over the last 4 layers; Fig. 10: O(1) per
 * token; the formula is not given there, and the reading here is the sum of
 * the Euclidean norms of the last layers' updates to the token's hidden state):
 *   scores[b * ld_scores + t] = sum_{j=1..nstates-1} ||h_j[t] - h_{j-1}[t]||_2
 * where h_0 .. h_{nstates-1} are the hidden states entering and leaving those
 * layers (nstates = 5 for the last 4 layers).  Each update is formed in fp32
 * from the fp16 states and its squares are summed in fp32.  The result feeds
 * semkv_rank_topr.
 *  h        fp16 hidden states; element (b, state, token, k) is at
 *           h + b*strides[0] + state*strides[1] + token*strides[2] + k
 *           (strides in elements, k contiguous), k < d_model
 *  scores   fp32 [batch][ld_scores] device memory, first n of each row written
 * Errors: EINVAL (null or misaligned pointers: h 16-byte, scores 4-byte;
 * strides negative or not multiples of 8; batch outside [1, 65535]; nstates
 * outside [2, 9]; d_model not a multiple of 8 in [8, 65536]; n < 1;
 * ld_scores < n). */
semkv_status semkv_score_hidden_delta(const uint16_t* h, const int64_t strides[3], int32_t batch,
                                      int32_t nstates, int64_t n, int32_t d_model, float* scores,
                                      int64_t ld_scores, void* stream);

/* Quantize and pack a prompt (SemKV Fig. 5 and Table 6).
 *  k, v     fp16 rows; element (b, layer, head, token, d) is at
 *           base + b*strides[0] + layer*strides[1] + head*strides[2]
 *                + token*strides[3] + d        (strides in elements, d contiguous)
 *  n        tokens per sequence; perm int32 [batch][n] as from semkv_rank_topr
 *  k_high   |H|: tokens perm[b][0..k_high) go to the high pool at L_high, the
 *           rest to the low pool at L_low
 * Rows are written at slots n_high.. and n_low.. of each pool (K and V of
 * every layer and KV head); tok_* records n_tokens + token.  On success the
 * host counters advance: n_high += k_high, n_low += n - k_high,
 * n_tokens += n.  Requires an empty tail (n_tail == 0).
 * Errors: EINVAL (null/misaligned pointers, n < 1, k_high outside [0, n],
 * n_tail != 0), ECAPACITY (a pool would overflow), EUNSUPPORTED (geometry). */
semkv_status semkv_quantize_pack(semkv_cache* c, const uint16_t* k, const uint16_t* v,
                                 const int64_t strides[4], int64_t n, const int32_t* perm,
                                 int64_t k_high, void* stream);

/* Generation-time block-exact quantization (SemKV Fig. 6).
 *  k_new, v_new  fp16, t_new tokens per sequence, strides as in
 *                semkv_quantize_pack; score_new fp32 [batch][t_new]
 * The tokens are appended to the fp16 tail.  Each time the tail holds
 * `block` tokens, the block is ranked on its own scores with
 * k_b = semkv_topr_count(block, r), quantized, packed and appended to the
 * pools (ascending token order within each pool), and the tail empties.
 * With flush != 0 the residual tail is then processed the same way with
 * k = semkv_topr_count(n_tail, r) (end of a generation turn).  Host counters
 * are updated.  workspace: device memory of at least
 * semkv_workspace_bytes(g, 0, 0) bytes.
 * Errors: EINVAL, ECAPACITY, EWORKSPACE. */
semkv_status semkv_append_block(semkv_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                                const int64_t strides[4], const float* score_new, int32_t t_new,
                                double r, int32_t flush, void* workspace, int64_t ws_bytes,
                                void* stream);

/* Decode attention over the packed mixed-precision cache (SemKV Figs. 1 and
 * 5: the quantized cache is what decoding reads).  For each sequence b,
 * layer layer0 + i (0 <= i < nlayers) and query head h:
 *   out[b][i][h] = sum_t softmax_t(sm_scale * q[b][i][h] . k_t) v_t
 * over every cached token t -- high pool rows, low pool rows and the fp16
 * tail rows -- of KV head h / (q_heads/kv_heads); packed rows are
 * dequantized on the fly (x = min + code * scale).
 *  q    fp16 [batch][nlayers][q_heads][128]
 *  out  fp32 [batch][nlayers][q_heads][128]
 *  workspace  >= semkv_workspace_bytes(g, nlayers, n_tokens) bytes
 * Errors: EINVAL (pointers, layer range, empty cache), EWORKSPACE. */
semkv_status semkv_decode_attn(const semkv_cache* c, const uint16_t* q, int32_t layer0,
                               int32_t nlayers, float sm_scale, float* out, void* workspace,
                               int64_t ws_bytes, void* stream);

/* The two halves of semkv_decode_attn, for callers that combine partial
 * results themselves (e.g. a context split across devices):
 * semkv_decode_partials writes per-chunk (max logit, sum of exponentials,
 * unnormalised output) into the workspace; semkv_decode_merge combines them
 * with a log-sum-exp merge into `out`.  Same arguments and errors as
 * semkv_decode_attn; the merge must use the same cache counters, layer range
 * and workspace as the partials call before it. */
semkv_status semkv_decode_partials(const semkv_cache* c, const uint16_t* q, int32_t layer0,
                                   int32_t nlayers, float sm_scale, void* workspace,
                                   int64_t ws_bytes, void* stream);
semkv_status semkv_decode_merge(const semkv_cache* c, int32_t nlayers, float* out,
                                void* workspace, int64_t ws_bytes, void* stream);

/* Reconstructed pool rows, for inspection and quality measurement (the
 * quantizer of SemKV Table 6 undone: x = min + code * scale per value in
 * fp32; for a rotated cache, SemKV Table 2's rotation, the row is rotated
 * back by H in fp32).  Decoding never needs this.
 *  pool   0 = high pool (L_high), 1 = low pool (L_low)
 *  layer  0 <= layer < layers
 *  rows   [row0, row0 + nrows) of every (sequence, KV head, K|V) plane of that
 *         pool and layer; they must be valid (row0 + nrows <= n_high or n_low).
 *         Slot j of the pool holds token tok_*[b][j] (see semkv_cache).
 *  out    fp32 [batch][kv_heads][2][nrows][128] device memory, 16-byte aligned
 * Errors: EINVAL (pool, layer or row range, null or misaligned out). */
semkv_status semkv_dequantize_rows(const semkv_cache* c, int32_t pool, int32_t layer,
                                   int64_t row0, int64_t nrows, float* out, void* stream);

/* semkv_decode_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The split-K partials live in a static device array
 * of semkv_decode_noalloc_scratch_bytes() = 64 MiB that the library holds on
 * each device it runs on until the process ends; no call allocates or frees.
 * Same arguments, output and errors as semkv_decode_attn, except: EWORKSPACE
 * when this call's partials (2080 bytes per (sequence, layer, KV head, chunk)
 * with 4 query heads per KV head; about 16k such records) exceed that array;
 * EHIP if the array's device address cannot be looked up.  Every call on one
 * device shares that device's array and nothing in it needs to start at
 * zero; calls that overlap on one device (concurrent streams, or threads)
 * race on it and must be serialised by the caller. */
semkv_status semkv_decode_attn_noalloc(const semkv_cache* c, const uint16_t* q, int32_t layer0,
                                       int32_t nlayers, float sm_scale, float* out, void* stream);
int64_t semkv_decode_noalloc_scratch_bytes(void);

/* ---- Ragged batches: sequences of one cache advance independently (SemKV
 * Fig. 6: each prompt is ranked and quantized on its own and each sequence's
 * generation blocks fill at their own pace; Table 2: multi-turn use with a
 * flush at every turn's end).  Each sequence b owns SEMKV_SEQ_WORDS int64
 * counters in a caller-owned DEVICE array seq[batch][SEMKV_SEQ_WORDS]:
 *   [SEMKV_SEQ_HIGH] n_high  [SEMKV_SEQ_LOW] n_low  [SEMKV_SEQ_TAIL] n_tail
 *   [SEMKV_SEQ_TOKENS] n_tokens  [SEMKV_SEQ_STATUS] status bits (sticky)
 * with n_high + n_low + n_tail == n_tokens; rows [0, n_high) / [0, n_low) of
 * sequence b's pool planes and [0, n_tail) of its tail are valid, tok_* of
 * its slots hold its own token indices.  The kernels read them as offsets and
 * advance them in stream order, so ragged calls need no host
 * synchronisation and may be captured in a HIP graph.  A cache used this way
 * keeps its host counters at 0 (EINVAL otherwise).  Capacity is checked on
 * the device: a sequence whose rows would not fit writes nothing and gets
 * SEMKV_SEQ_CAPACITY in its status (its counters stay as they were); read
 * the array after semkv_sync_check to see it. */
#define SEMKV_SEQ_WORDS 8
enum { SEMKV_SEQ_HIGH = 0, SEMKV_SEQ_LOW = 1, SEMKV_SEQ_TAIL = 2, SEMKV_SEQ_TOKENS = 3,
       SEMKV_SEQ_STATUS = 4 };
enum {
  SEMKV_SEQ_CAPACITY = 1,  /* rows skipped: a pool had no room                */
  SEMKV_SEQ_TAIL_BUSY = 2, /* prompt skipped: the sequence's tail is not empty */
  SEMKV_SEQ_TAIL_FULL = 4  /* token dropped: the tail was full (after a
                            * capacity failure)                               */
};

/* Zero the counters of `batch` sequences (a fill kernel on `stream`). */
semkv_status semkv_seq_reset(int64_t* seq, int32_t batch, void* stream);

/* semkv_rank_topr for prompts of different lengths: sequence b ranks the
 * first n_seq[b] <= n_max scores of its row with k = floor(r n_seq[b] + 1/2).
 *  n_seq  int32 [batch] device memory
 *  perm   int32 [batch][n_max]: entries [0, n_seq[b]) of row b are written
 *  mask   nullable uint32 [batch][ceil(n_max/32)]: words [0, ceil(n_seq[b]/32))
 * Errors: EINVAL (pointers, sizes, r outside [0, 1]). */
semkv_status semkv_ragged_rank_topr(const float* scores, int32_t batch, int64_t n_max,
                                    int64_t ld_scores, const int32_t* n_seq, double r,
                                    int32_t* perm, uint32_t* mask, void* stream);

/* semkv_quantize_pack of one prompt per sequence: sequence b quantizes its
 * tokens 0 .. n_seq[b]-1 (K, V laid out as for semkv_quantize_pack, with room
 * for n_max tokens) with k = floor(r n_seq[b] + 1/2) high rows listed first in
 * row b of perm (stride n_max, as semkv_ragged_rank_topr writes it), appends
 * them after its own pool rows with token indices n_tokens + t, and advances
 * its counters.  A sequence with n_seq[b] = 0 is left as is; one whose tail is
 * not empty is skipped (SEMKV_SEQ_TAIL_BUSY).
 * Errors: EINVAL (pointers, strides, n_max < 1, r, host counters not 0). */
semkv_status semkv_ragged_quantize_pack(semkv_cache* c, int64_t* seq, const uint16_t* k,
                                        const uint16_t* v, const int64_t strides[4], int64_t n_max,
                                        const int32_t* n_seq, double r, const int32_t* perm,
                                        void* stream);

/* One generation step of a ragged batch (SemKV Fig. 6).  Every sequence with
 * active[b] != 0 appends one token (k_new, v_new: [batch][layers][kv][128]
 * fp16 with the given strides, token index 0; score_new: fp32 [batch]) to its
 * tail.  Then every sequence whose tail holds `block` rows, or that has
 * flush[b] != 0 and a non-empty tail (the end of its turn), ranks its tail
 * with k = floor(r n_tail + 1/2), quantizes and appends it to its pools and
 * empties its tail.  active may be NULL (no token appended: k_new, v_new,
 * score_new are then unused), flush may be NULL (no flush).  workspace as for
 * semkv_append_block (semkv_workspace_bytes).
 * Errors: EINVAL, EWORKSPACE. */
semkv_status semkv_ragged_append(semkv_cache* c, int64_t* seq, const uint16_t* k_new,
                                 const uint16_t* v_new, const int64_t strides[4],
                                 const float* score_new, const int32_t* active,
                                 const int32_t* flush, double r, void* workspace, int64_t ws_bytes,
                                 void* stream);

/* semkv_decode_attn over a ragged batch: sequence b attends over its own
 * n_high + n_low pool rows and n_tail tail rows.  max_high and max_low bound
 * n_high and n_low over the batch (they size the launch; cap_high and cap_low
 * always do); workspace: semkv_workspace_bytes(g, nlayers, max_high + max_low
 * + block).  Every sequence must hold at least one token.
 * Errors: as semkv_decode_attn; EINVAL if a bound exceeds its capacity. */
semkv_status semkv_ragged_decode_attn(const semkv_cache* c, const int64_t* seq, const uint16_t* q,
                                      int32_t layer0, int32_t nlayers, float sm_scale,
                                      int64_t max_high, int64_t max_low, float* out,
                                      void* workspace, int64_t ws_bytes, void* stream);

/* Synchronise `stream` and map a sticky HIP error to SEMKV_EHIP. */
semkv_status semkv_sync_check(void* stream);

/* Static string for a status code. */
const char* semkv_status_str(semkv_status s);

#ifdef __cplusplus
}
#endif

#endif /* SEMKV_H */
