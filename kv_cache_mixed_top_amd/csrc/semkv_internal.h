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

// ---------------------------------------------------------------- rank
// perm/mask of `batch` sequences of n scores each (row stride ld).
hipError_t launch_rank(const float* scores, int batch, int n, int64_t ld, int k,
                       int32_t* perm, uint32_t* mask, hipStream_t stream);

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
};
hipError_t launch_append_tail(const AppendArgs& a, hipStream_t stream);

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
};
// Chunking rule shared by the launchers and the workspace query.
int decode_chunk_tokens(int64_t tokens_per_unit, int64_t units);
int64_t decode_partial_floats_per_chunk(int group);
hipError_t launch_decode_partials(const DecodeArgs& a, hipStream_t stream);
// Generic kernel over chunks [a.x0, a.x0 + count).
hipError_t launch_decode_generic(const DecodeArgs& a, int count, hipStream_t stream);
// Matrix-core kernel for the pool chunks [0, nch[0] + nch[1]) when both pool
// formats are 6- or 5-level and the query group is 4.
bool decode_mfma_supported(const DecodeArgs& a);
// The matrix-core kernel will run for these arguments (supported and not
// disabled with SEMKV_DECODE=generic).
bool decode_use_mfma(const DecodeArgs& a);
// Pool chunk rows for the matrix-core kernel: enough chunks per (sequence,
// layer, KV head) to fill the device's resident wave slots once.
int decode_mfma_chunk_rows(int64_t n_high, int64_t n_low, int64_t units);
int64_t decode_mfma_resident_waves();
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);

}  // namespace semkv
