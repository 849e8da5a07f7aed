// Launch interfaces between the C ABI layer (api.hip) and the kernels.
#pragma once

#include "semkv_common.h"

namespace semkv {

// ---------------------------------------------------------------- score
// Key-norm scores: scores[b * ld + t] = sum over layers layer0 ..
// layer0 + nlayers - 1 and heads 0 .. kv_heads - 1 of |k row|_2.
struct ScoreArgs {
  const uint16_t* k;        // layer 0, head 0, token 0 of sequence 0
  int64_t sb, sl, sh, st;   // element strides: batch, layer, head, token
  int64_t n;                // tokens per sequence
  int kv_heads, layer0, nlayers;
  float* scores;
  int64_t ld;               // row stride of scores
};
hipError_t launch_score_keynorm(const ScoreArgs& a, int batch, hipStream_t stream);

// Hidden-state delta norms: scores[b * ld + t] = sum_{j=1..S} ||h_j - h_{j-1}||
// of token t, h_j at h + b * sb + j * ss + t * st (d contiguous fp16 values).
struct DeltaArgs {
  const uint16_t* h;
  int64_t sb, ss, st;       // element strides: batch, state, token
  int64_t n;
  int32_t S, d;             // layers (states - 1), hidden size
  float* scores;
  int64_t ld;
};
hipError_t launch_score_hidden_delta(const DeltaArgs& a, int batch, hipStream_t stream);

// ---------------------------------------------------------------- ragged batches
// Per-sequence counters in device memory, kSeqWords int64 per sequence.
constexpr int kSeqWords = 8;
enum SeqWord { kSeqHigh = 0, kSeqLow = 1, kSeqTail = 2, kSeqTokens = 3, kSeqStatus = 4 };
enum SeqStatus { kSeqCapacity = 1, kSeqTailBusy = 2, kSeqTailFull = 4 };
// floor(r n + 1/2) in double, as semkv_topr_count
__host__ __device__ inline int64_t topr_count(int64_t n, double r) {
  return (int64_t)floor(r * (double)n + 0.5);
}

// ---------------------------------------------------------------- rank
// perm/mask of `batch` sequences of n scores each (row stride ld).  With
// n_seq, sequence b ranks its first n_seq[b] <= n scores with k = floor(r
// n_seq[b] + 1/2) and perm rows have stride ld_perm.
hipError_t launch_rank(const float* scores, int batch, int n, int64_t ld, int k,
                       int32_t* perm, uint32_t* mask, hipStream_t stream,
                       const int32_t* n_seq = nullptr, double r = 0.0, int64_t ld_perm = -1);

// ---------------------------------------------------------------- quantize
struct QuantArgs {
  const uint16_t* src[2];   // K rows, V rows
  int64_t sb, sl, sh, st;   // element strides: batch, layer, head, token
  const int32_t* perm;      // [batch][n]
  int32_t n, k_high;
  int32_t batch, layers, kv_heads;
  uint8_t* codes[2];        // [0] high pool, [1] low pool
  uint32_t* meta[2];        // {scale, min} fp16 pair as one word per row
  int32_t* tok[2];
  int64_t cap[2];
  int64_t start[2];         // first destination slot (n_high, n_low)
  RowFmt fmt[2];
  int64_t token_base;       // tok_* = token_base + token
  int32_t rotate;           // Hadamard-rotate every row before quantizing
  // ragged batches (seq != null): sequence b quantizes n_seq[b] tokens with
  // k = floor(r n_seq[b] + 1/2), at its own pool counters, token base
  // n_tokens - n_tail; perm rows have stride ld_perm.  tail_mode = 0: a
  // prompt (skipped while the sequence's tail is not empty); 1: a tail block.
  const int64_t* seq;
  const int32_t* n_seq;
  double r;
  int64_t ld_perm;
  int32_t tail_mode;
};
hipError_t launch_quantize_pack(const QuantArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- append
struct AppendArgs {
  const uint16_t* src[2];
  int64_t sb, sl, sh, st;
  const float* score_new;   // [batch][t_total]
  int32_t t_total, t_off, t_cnt;   // copy new tokens [t_off, t_off + t_cnt)
  int32_t batch, layers, kv_heads, block;
  int32_t pos;              // first tail row written
  uint16_t* tail_kv;
  float* tail_score;
  // ragged batches (seq != null): one token per sequence with active[b] != 0,
  // written at that sequence's n_tail (pos and t_cnt are then unused)
  const int64_t* seq;
  const int32_t* active;
};
hipError_t launch_append_tail(const AppendArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- dequantize
// Rows [row0, row0 + nrows) of every (sequence, KV head, K|V) plane of one
// layer of one pool -> fp32 out[b][head][K|V][row - row0][128].
struct DequantArgs {
  const uint8_t* codes;
  const uint32_t* meta;
  int64_t cap;
  RowFmt fmt;
  int32_t batch, layers, kv_heads, layer;
  int64_t row0, nrows;
  int32_t rotate;
  float* out;
};
hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- decode
struct DecodeArgs {
  const uint8_t* codes[2];
  const uint32_t* meta[2];
  int64_t cap[2];
  int64_t rows[2];          // valid rows per pool
  RowFmt fmt[2];
  const uint16_t* tail_kv;
  int64_t n_tail;
  int32_t block;
  const uint16_t* q;        // [batch][nl][Hq][128]
  float* out;               // [batch][nl][Hq][128]
  int32_t batch, layers, kv_heads, q_heads, group, layer0, nl;
  float sm_scale;
  int32_t chunk;            // tokens per chunk (multiple of 64)
  int32_t nch[3];           // chunks of high pool, low pool, tail
  int32_t nchunks;
  int32_t x0;               // first chunk index handled by a launch
  float* ws;                // partials
  int32_t rotate;           // rows are Hadamard-rotated: rotate q, rotate the output back
  // ragged batches (seq != null): sequence b has its own n_high, n_low and
  // n_tail there; rows[] and n_tail are bounds over the batch
  const int64_t* seq;
};
// rows of pool seg (0, 1) or of the tail (2) of sequence b
__device__ __forceinline__ int64_t seg_rows(const DecodeArgs& a, int seg, int b) {
  if (a.seq) return a.seq[(int64_t)b * kSeqWords + seg];
  return seg == 0 ? a.rows[0] : seg == 1 ? a.rows[1] : a.n_tail;
}
// Chunking rule shared by the launchers and the workspace query.
int decode_chunk_tokens(int64_t tokens_per_unit, int64_t units);
int64_t decode_partial_floats_per_chunk(int group);
hipError_t launch_decode_partials(const DecodeArgs& a, hipStream_t stream);
// Generic kernel over chunks [a.x0, a.x0 + count).
hipError_t launch_decode_generic(const DecodeArgs& a, int count, hipStream_t stream);
// Matrix-core kernel for the pool chunks [0, nch[0] + nch[1]) when both pool
// level counts are among 3, 4, 5, 6, 8 and 16 and the query group is 4.
bool decode_mfma_supported(const DecodeArgs& a);
// The matrix-core kernel will run for these arguments.
bool decode_use_mfma(const DecodeArgs& a);
// Pool chunk rows for the matrix-core kernel: enough chunks per (sequence,
// layer, KV head) to fill the device's resident wave slots once.
int decode_mfma_chunk_rows(int64_t n_high, int64_t n_low, int64_t units);
int64_t decode_mfma_resident_waves();
// The pool chunks, and with with_tail the fp16 tail chunk too (a tail of at
// most 128 rows in one chunk: nch[2] <= 1, block <= 128).
hipError_t launch_decode_mfma(const DecodeArgs& a, bool with_tail, hipStream_t stream);
// The matrix-core kernels of the pairs with 16 levels, of (6,3), (5,3) and
// of the 8-level pairs other than (8,8), (8,6).
hipError_t launch_decode_mfma_wide(int LA, int LB, bool rot, dim3 grid, const DecodeArgs& a,
                                   hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- ragged counters
hipError_t launch_seq_reset(int64_t* seq, int batch, hipStream_t stream);
// After a ragged prompt: advance each sequence's counters by what the
// quantize kernel wrote for it (the same capacity and tail decisions).
hipError_t launch_seq_prefill_advance(int64_t* seq, const int32_t* n_seq, double r, int batch,
                                      int64_t cap_high, int64_t cap_low, hipStream_t stream);
// After a ragged append: count the appended tokens, decide per sequence
// whether its tail is quantized now (full, or flushed), write that row count
// (0 if not) to nq.
hipError_t launch_seq_tail_plan(int64_t* seq, const int32_t* active, const int32_t* flush,
                                double r, int block, int batch, int64_t cap_high, int64_t cap_low,
                                int32_t* nq, hipStream_t stream);
// After the tail blocks were quantized: move their rows to the pool counters.
hipError_t launch_seq_tail_advance(int64_t* seq, const int32_t* nq, double r, int batch,
                                   hipStream_t stream);

}  // namespace semkv
