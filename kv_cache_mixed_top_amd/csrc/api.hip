// C ABI of the SemKV hot path: host-side validation and kernel launches.
// Declarations and the contract of every entry point are in include/semkv.h.
#include <atomic>
#include <cmath>
#include <cstdint>

#include "semkv.h"
#include "semkv_internal.h"

using namespace semkv;

namespace {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

semkv_status check_geom(const semkv_geom* g) {
  if (!g) return SEMKV_EINVAL;
  if (g->head_dim != kHeadDim) return SEMKV_EUNSUPPORTED;
  if (g->batch < 1 || g->layers < 1 || g->kv_heads < 1 || g->q_heads < 1) return SEMKV_EINVAL;
  if (g->q_heads % g->kv_heads != 0) return SEMKV_EINVAL;
  if (g->q_heads / g->kv_heads > kMaxGroup) return SEMKV_EUNSUPPORTED;
  if ((int64_t)g->layers * g->kv_heads * 2 > 65535 || g->batch > 65535) return SEMKV_EUNSUPPORTED;
  if (g->L_low < 3 || g->L_high > 65536 || g->L_low > g->L_high) return SEMKV_EINVAL;
  if (g->block < 1 || g->block > 1024) return SEMKV_EINVAL;
  if (g->cap_high < 0 || g->cap_low < 0 || g->cap_high % 16 != 0 || g->cap_low % 16 != 0)
    return SEMKV_EINVAL;
  if (g->cap_high > (int64_t)INT32_MAX || g->cap_low > (int64_t)INT32_MAX) return SEMKV_EINVAL;
  if (g->rotate != 0 && g->rotate != 1) return SEMKV_EINVAL;
  return SEMKV_OK;
}

semkv_status check_cache(const semkv_cache* c) {
  if (!c) return SEMKV_EINVAL;
  const semkv_status st = check_geom(&c->g);
  if (st != SEMKV_OK) return st;
  const semkv_geom& g = c->g;
  auto pool_ok = [](const void* p, int64_t cap) { return cap == 0 || (p && aligned(p, 256)); };
  if (!pool_ok(c->codes_high, g.cap_high) || !pool_ok(c->meta_high, g.cap_high) ||
      !pool_ok(c->tok_high, g.cap_high))
    return SEMKV_EINVAL;
  if (!pool_ok(c->codes_low, g.cap_low) || !pool_ok(c->meta_low, g.cap_low) ||
      !pool_ok(c->tok_low, g.cap_low))
    return SEMKV_EINVAL;
  if (!c->tail_kv || !aligned(c->tail_kv, 256) || !c->tail_score || !aligned(c->tail_score, 16))
    return SEMKV_EINVAL;
  if (c->n_high < 0 || c->n_high > g.cap_high || c->n_low < 0 || c->n_low > g.cap_low)
    return SEMKV_EINVAL;
  if (c->n_tail < 0 || c->n_tail >= g.block) return SEMKV_EINVAL;
  if (c->n_high + c->n_low + c->n_tail != c->n_tokens) return SEMKV_EINVAL;
  return SEMKV_OK;
}

bool strides_ok(const int64_t* s) {
  if (!s) return false;
  for (int i = 0; i < 4; ++i)
    if (s[i] < 0 || s[i] % 8 != 0) return false;
  return true;
}

semkv_status from_hip(hipError_t e) { return e == hipSuccess ? SEMKV_OK : SEMKV_EHIP; }

// A cache used by ragged calls keeps its host counters at 0: each sequence's
// counters are in the device array seq.
semkv_status check_ragged(const semkv_cache* c, const int64_t* seq) {
  const semkv_status st = check_cache(c);
  if (st != SEMKV_OK) return st;
  if (!seq || !aligned(seq, 8)) return SEMKV_EINVAL;
  if (c->n_high != 0 || c->n_low != 0 || c->n_tail != 0 || c->n_tokens != 0) return SEMKV_EINVAL;
  return SEMKV_OK;
}

int64_t topr(int64_t n, double r) { return semkv::topr_count(n, r); }

// generation workspace: the block ranking's perm [batch][block], then (for a
// ragged batch) the row count of each sequence's tail quantized by a call
int64_t append_perm_bytes(const semkv_geom& g) {
  return ((int64_t)g.batch * g.block * 4 + 255) / 256 * 256;
}
int64_t append_ws_bytes(const semkv_geom& g) {
  return append_perm_bytes(g) + ((int64_t)g.batch * 4 + 255) / 256 * 256;
}

int64_t decode_chunks_bound(int64_t max_tokens, int64_t units) {
  const int64_t desired = (4096 + units - 1) / units;
  int64_t big = (max_tokens + 1023) / 1024;
  return (desired > big ? desired : big) + 3;
}

QuantArgs quant_args(const semkv_cache* c, const uint16_t* k, const uint16_t* v,
                     const int64_t s[4], int64_t n, const int32_t* perm, int64_t k_high,
                     int64_t token_base) {
  QuantArgs a;
  a.src[0] = k;
  a.src[1] = v;
  a.sb = s[0];
  a.sl = s[1];
  a.sh = s[2];
  a.st = s[3];
  a.perm = perm;
  a.n = (int32_t)n;
  a.k_high = (int32_t)k_high;
  a.batch = c->g.batch;
  a.layers = c->g.layers;
  a.kv_heads = c->g.kv_heads;
  a.codes[0] = c->codes_high;
  a.codes[1] = c->codes_low;
  a.meta[0] = reinterpret_cast<uint32_t*>(c->meta_high);
  a.meta[1] = reinterpret_cast<uint32_t*>(c->meta_low);
  a.tok[0] = c->tok_high;
  a.tok[1] = c->tok_low;
  a.cap[0] = c->g.cap_high;
  a.cap[1] = c->g.cap_low;
  a.start[0] = c->n_high;
  a.start[1] = c->n_low;
  a.fmt[0] = row_fmt(c->g.L_high);
  a.fmt[1] = row_fmt(c->g.L_low);
  a.token_base = token_base;
  a.rotate = c->g.rotate;
  a.seq = nullptr;
  a.n_seq = nullptr;
  a.r = 0.0;
  a.ld_perm = n;
  a.tail_mode = 0;
  return a;
}

// seq != null: a ragged batch; c's counters are then bounds over the batch
// and the tail bound is tail_rows.
semkv_status decode_args(const semkv_cache* c, const uint16_t* q, int32_t layer0, int32_t nl,
                         float sm_scale, float* out, void* ws, int64_t ws_bytes, DecodeArgs* a,
                         const int64_t* seq = nullptr, int64_t tail_rows = -1) {
  semkv_status st = check_cache(c);
  if (st != SEMKV_OK) return st;
  const semkv_geom& g = c->g;
  if (layer0 < 0 || nl < 1 || (int64_t)layer0 + nl > g.layers) return SEMKV_EINVAL;
  const int64_t n_tail = seq ? tail_rows : c->n_tail;
  const int64_t T = c->n_high + c->n_low + n_tail;
  if (T <= 0) return SEMKV_EINVAL;
  const int64_t units = (int64_t)g.batch * nl * g.kv_heads;
  const int chunk = decode_chunk_tokens(T, units);
  a->codes[0] = c->codes_high;
  a->codes[1] = c->codes_low;
  a->meta[0] = reinterpret_cast<const uint32_t*>(c->meta_high);
  a->meta[1] = reinterpret_cast<const uint32_t*>(c->meta_low);
  a->cap[0] = g.cap_high;
  a->cap[1] = g.cap_low;
  a->rows[0] = c->n_high;
  a->rows[1] = c->n_low;
  a->fmt[0] = row_fmt(g.L_high);
  a->fmt[1] = row_fmt(g.L_low);
  a->tail_kv = c->tail_kv;
  a->n_tail = n_tail;
  a->seq = seq;
  a->block = g.block;
  a->q = q;
  a->out = out;
  a->batch = g.batch;
  a->layers = g.layers;
  a->kv_heads = g.kv_heads;
  a->q_heads = g.q_heads;
  a->group = g.q_heads / g.kv_heads;
  a->layer0 = layer0;
  a->nl = nl;
  a->sm_scale = sm_scale;
  a->chunk = chunk;
  a->nch[0] = (int32_t)((c->n_high + chunk - 1) / chunk);
  a->nch[1] = (int32_t)((c->n_low + chunk - 1) / chunk);
  a->nch[2] = (int32_t)((n_tail + chunk - 1) / chunk);
  a->nchunks = a->nch[0] + a->nch[1] + a->nch[2];
  a->x0 = 0;
  const int64_t per_chunk_bytes = decode_partial_floats_per_chunk(a->group) * 4;
  auto set_chunk = [&](int cm) {
    a->chunk = cm;
    a->nch[0] = (int32_t)((c->n_high + cm - 1) / cm);
    a->nch[1] = (int32_t)((c->n_low + cm - 1) / cm);
    a->nch[2] = (int32_t)((n_tail + cm - 1) / cm);
    a->nchunks = a->nch[0] + a->nch[1] + a->nch[2];
  };
  if (decode_use_mfma(*a)) {
    // pool chunks fill whole rounds of the resident workgroup slots (the fp16
    // tail, < block <= 1024 rows, stays one generic chunk of the same size);
    // if the caller's workspace cannot hold that many partials, chunks no
    // finer than the generic ones, which semkv_workspace_bytes covers
    const int c2 = decode_mfma_chunk_rows(c->n_high, c->n_low, units);
    set_chunk(c2);
    if (units * a->nchunks * per_chunk_bytes > ws_bytes && c2 < chunk) set_chunk(chunk);
  }
  a->ws = reinterpret_cast<float*>(ws);
  a->rotate = g.rotate;
  const int64_t need = units * a->nchunks * per_chunk_bytes;
  if (!ws || !aligned(ws, 256) || ws_bytes < need) return SEMKV_EWORKSPACE;
  return SEMKV_OK;
}

// ---- scratch of the no-allocation decode entry point (semkv_decode_attn_noalloc)
// A file-scope device array holds that entry point's split-K partials, so it
// needs no caller workspace and never allocates.  Each device that runs the
// library holds its own copy until the process ends.  In host code the
// array's name is only a stand-in: its device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and only that
// address is ever handed to kernels.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> scratch_ptr[kMaxScratchDevices];

// Device address of the current device's scratch, or null on failure.
// Concurrent first calls look up the same address.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" {

int64_t semkv_row_bytes(int32_t L) {
  if (L < 3 || L > 65536) return -1;
  return row_fmt(L).R;
}

int64_t semkv_topr_count(int64_t n, double r) {
  if (n < 0 || !(r >= 0.0 && r <= 1.0)) return -1;
  return topr(n, r);
}

semkv_status semkv_cache_sizes(const semkv_geom* g, int64_t bytes_out[8]) {
  const semkv_status st = check_geom(g);
  if (st != SEMKV_OK) return st;
  if (!bytes_out) return SEMKV_EINVAL;
  const int64_t planes = (int64_t)g->batch * g->layers * g->kv_heads * 2;
  bytes_out[0] = planes * g->cap_high * row_fmt(g->L_high).R;
  bytes_out[1] = planes * g->cap_low * row_fmt(g->L_low).R;
  bytes_out[2] = planes * g->cap_high * 4;
  bytes_out[3] = planes * g->cap_low * 4;
  bytes_out[4] = (int64_t)g->batch * g->cap_high * 4;
  bytes_out[5] = (int64_t)g->batch * g->cap_low * 4;
  bytes_out[6] = planes * g->block * kHeadDim * 2;
  bytes_out[7] = (int64_t)g->batch * g->block * 4;
  return SEMKV_OK;
}

int64_t semkv_workspace_bytes(const semkv_geom* g, int32_t nlayers, int64_t max_tokens) {
  if (check_geom(g) != SEMKV_OK) return -1;
  if (nlayers < 0 || nlayers > g->layers || max_tokens < 0) return -1;
  int64_t need = append_ws_bytes(*g);
  if (nlayers > 0) {
    const int64_t units = (int64_t)g->batch * nlayers * g->kv_heads;
    const int64_t dec = units * decode_chunks_bound(max_tokens, units) *
                        decode_partial_floats_per_chunk(g->q_heads / g->kv_heads) * 4;
    if (dec > need) need = dec;
  }
  return need;
}

semkv_status semkv_rank_topr(const float* scores, int32_t batch, int64_t n, int64_t ld_scores,
                             int64_t k, int32_t* perm, uint32_t* mask, void* stream) {
  if (!scores || !perm || !aligned(scores, 4) || !aligned(perm, 4)) return SEMKV_EINVAL;
  if (mask && !aligned(mask, 4)) return SEMKV_EINVAL;
  if (batch < 1 || batch > 65535 || n < 1 || n > (int64_t)INT32_MAX || ld_scores < n)
    return SEMKV_EINVAL;
  if (k < 0 || k > n) return SEMKV_EINVAL;
  return from_hip(launch_rank(scores, batch, (int)n, ld_scores, (int)k, perm, mask,
                              (hipStream_t)stream));
}

semkv_status semkv_score_keynorm(const uint16_t* k, const int64_t strides[4], int32_t batch,
                                 int32_t kv_heads, int64_t n, int32_t layer0, int32_t nlayers,
                                 float* scores, int64_t ld_scores, void* stream) {
  if (!k || !aligned(k, 16) || !strides_ok(strides)) return SEMKV_EINVAL;
  if (batch < 1 || batch > 65535 || kv_heads < 1 || layer0 < 0 || nlayers < 1) return SEMKV_EINVAL;
  if ((int64_t)nlayers * kv_heads > (int64_t)INT32_MAX) return SEMKV_EINVAL;
  if (n < 1 || n > (int64_t)INT32_MAX || !scores || !aligned(scores, 4) || ld_scores < n)
    return SEMKV_EINVAL;
  ScoreArgs a;
  a.k = k;
  a.sb = strides[0];
  a.sl = strides[1];
  a.sh = strides[2];
  a.st = strides[3];
  a.n = n;
  a.kv_heads = kv_heads;
  a.layer0 = layer0;
  a.nlayers = nlayers;
  a.scores = scores;
  a.ld = ld_scores;
  return from_hip(launch_score_keynorm(a, batch, (hipStream_t)stream));
}

semkv_status semkv_score_hidden_delta(const uint16_t* h, const int64_t strides[3], int32_t batch,
                                      int32_t nstates, int64_t n, int32_t d_model, float* scores,
                                      int64_t ld_scores, void* stream) {
  if (!h || !aligned(h, 16) || !strides) return SEMKV_EINVAL;
  for (int i = 0; i < 3; ++i)
    if (strides[i] < 0 || strides[i] % 8 != 0) return SEMKV_EINVAL;
  if (batch < 1 || batch > 65535 || nstates < 2 || nstates > 9) return SEMKV_EINVAL;
  if (d_model < 8 || d_model > 65536 || d_model % 8 != 0) return SEMKV_EINVAL;
  if (n < 1 || n > (int64_t)INT32_MAX * 4 || !scores || !aligned(scores, 4) || ld_scores < n)
    return SEMKV_EINVAL;
  DeltaArgs a;
  a.h = h;
  a.sb = strides[0];
  a.ss = strides[1];
  a.st = strides[2];
  a.n = n;
  a.S = nstates - 1;
  a.d = d_model;
  a.scores = scores;
  a.ld = ld_scores;
  return from_hip(launch_score_hidden_delta(a, batch, (hipStream_t)stream));
}

semkv_status semkv_quantize_pack(semkv_cache* c, const uint16_t* k, const uint16_t* v,
                                 const int64_t strides[4], int64_t n, const int32_t* perm,
                                 int64_t k_high, void* stream) {
  semkv_status st = check_cache(c);
  if (st != SEMKV_OK) return st;
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16) || !strides_ok(strides)) return SEMKV_EINVAL;
  if (!perm || !aligned(perm, 4)) return SEMKV_EINVAL;
  if (n < 1 || n > (int64_t)INT32_MAX || k_high < 0 || k_high > n) return SEMKV_EINVAL;
  if (c->n_tail != 0) return SEMKV_EINVAL;
  if (c->n_high + k_high > c->g.cap_high || c->n_low + (n - k_high) > c->g.cap_low)
    return SEMKV_ECAPACITY;
  const QuantArgs a = quant_args(c, k, v, strides, n, perm, k_high, c->n_tokens);
  st = from_hip(launch_quantize_pack(a, (hipStream_t)stream));
  if (st != SEMKV_OK) return st;
  c->n_high += k_high;
  c->n_low += n - k_high;
  c->n_tokens += n;
  return SEMKV_OK;
}

semkv_status semkv_append_block(semkv_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                                const int64_t strides[4], const float* score_new, int32_t t_new,
                                double r, int32_t flush, void* workspace, int64_t ws_bytes,
                                void* stream) {
  semkv_status st = check_cache(c);
  if (st != SEMKV_OK) return st;
  if (t_new < 0 || !(r >= 0.0 && r <= 1.0)) return SEMKV_EINVAL;
  if (t_new > 0) {
    if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16) || !strides_ok(strides))
      return SEMKV_EINVAL;
    if (!score_new || !aligned(score_new, 4)) return SEMKV_EINVAL;
  }
  const semkv_geom& g = c->g;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < append_ws_bytes(g))
    return SEMKV_EWORKSPACE;

  // capacity for everything this call will write, checked before any launch
  const int64_t kb = topr(g.block, r);
  int64_t nt = c->n_tail, left = t_new, blocks = 0;
  while (left > 0) {
    const int64_t m = left < g.block - nt ? left : g.block - nt;
    nt += m;
    left -= m;
    if (nt == g.block) {
      ++blocks;
      nt = 0;
    }
  }
  int64_t add_high = blocks * kb, add_low = blocks * (g.block - kb);
  if (flush && nt > 0) {
    const int64_t kf = topr(nt, r);
    add_high += kf;
    add_low += nt - kf;
  }
  if (c->n_high + add_high > g.cap_high || c->n_low + add_low > g.cap_low) return SEMKV_ECAPACITY;

  hipStream_t s = (hipStream_t)stream;
  int32_t* wperm = reinterpret_cast<int32_t*>(workspace);
  const int64_t tb = (int64_t)g.layers * g.kv_heads * 2 * g.block * kHeadDim;
  const int64_t tstr[4] = {tb, (int64_t)g.kv_heads * 2 * g.block * kHeadDim,
                           (int64_t)2 * g.block * kHeadDim, kHeadDim};
  const uint16_t* tail_k = c->tail_kv;
  const uint16_t* tail_v = c->tail_kv + (int64_t)g.block * kHeadDim;

  auto quantize_tail = [&](int64_t ntail) -> semkv_status {
    const int64_t kk = topr(ntail, r);
    semkv_status e = from_hip(launch_rank(c->tail_score, g.batch, (int)ntail, g.block, (int)kk,
                                          wperm, nullptr, s));
    if (e != SEMKV_OK) return e;
    const QuantArgs qa = quant_args(c, tail_k, tail_v, tstr, ntail, wperm, kk,
                                    c->n_tokens - ntail);
    e = from_hip(launch_quantize_pack(qa, s));
    if (e != SEMKV_OK) return e;
    c->n_high += kk;
    c->n_low += ntail - kk;
    c->n_tail = 0;
    return SEMKV_OK;
  };

  int32_t off = 0;
  while (off < t_new) {
    const int32_t m = (int32_t)((t_new - off) < (g.block - c->n_tail) ? (t_new - off)
                                                                        : (g.block - c->n_tail));
    AppendArgs aa;
    aa.src[0] = k_new;
    aa.src[1] = v_new;
    aa.sb = strides[0];
    aa.sl = strides[1];
    aa.sh = strides[2];
    aa.st = strides[3];
    aa.score_new = score_new;
    aa.t_total = t_new;
    aa.t_off = off;
    aa.t_cnt = m;
    aa.batch = g.batch;
    aa.layers = g.layers;
    aa.kv_heads = g.kv_heads;
    aa.block = g.block;
    aa.pos = (int32_t)c->n_tail;
    aa.tail_kv = c->tail_kv;
    aa.tail_score = c->tail_score;
    aa.seq = nullptr;
    aa.active = nullptr;
    st = from_hip(launch_append_tail(aa, s));
    if (st != SEMKV_OK) return st;
    c->n_tail += m;
    c->n_tokens += m;
    off += m;
    if (c->n_tail == g.block) {
      st = quantize_tail(g.block);
      if (st != SEMKV_OK) return st;
    }
  }
  if (flush && c->n_tail > 0) {
    st = quantize_tail(c->n_tail);
    if (st != SEMKV_OK) return st;
  }
  return SEMKV_OK;
}

semkv_status semkv_decode_partials(const semkv_cache* c, const uint16_t* q, int32_t layer0,
                                   int32_t nlayers, float sm_scale, void* workspace,
                                   int64_t ws_bytes, void* stream) {
  if (!q || !aligned(q, 16)) return SEMKV_EINVAL;
  DecodeArgs a;
  const semkv_status st =
      decode_args(c, q, layer0, nlayers, sm_scale, nullptr, workspace, ws_bytes, &a);
  if (st != SEMKV_OK) return st;
  return from_hip(launch_decode_partials(a, (hipStream_t)stream));
}

semkv_status semkv_decode_merge(const semkv_cache* c, int32_t nlayers, float* out,
                                void* workspace, int64_t ws_bytes, void* stream) {
  if (!out || !aligned(out, 16)) return SEMKV_EINVAL;
  DecodeArgs a;
  const semkv_status st = decode_args(c, nullptr, 0, nlayers, 1.0f, out, workspace, ws_bytes, &a);
  if (st != SEMKV_OK) return st;
  return from_hip(launch_decode_merge(a, (hipStream_t)stream));
}

semkv_status semkv_decode_attn(const semkv_cache* c, const uint16_t* q, int32_t layer0,
                               int32_t nlayers, float sm_scale, float* out, void* workspace,
                               int64_t ws_bytes, void* stream) {
  if (!q || !aligned(q, 16) || !out || !aligned(out, 16)) return SEMKV_EINVAL;
  DecodeArgs a;
  semkv_status st = decode_args(c, q, layer0, nlayers, sm_scale, out, workspace, ws_bytes, &a);
  if (st != SEMKV_OK) return st;
  st = from_hip(launch_decode_partials(a, (hipStream_t)stream));
  if (st != SEMKV_OK) return st;
  return from_hip(launch_decode_merge(a, (hipStream_t)stream));
}

semkv_status semkv_decode_attn_noalloc(const semkv_cache* c, const uint16_t* q, int32_t layer0,
                                       int32_t nlayers, float sm_scale, float* out, void* stream) {
  if (!q || !aligned(q, 16) || !out || !aligned(out, 16)) return SEMKV_EINVAL;
  void* ws = device_scratch();
  if (!ws) return SEMKV_EHIP;
  DecodeArgs a;
  // the partials must fit the static scratch: decode_args picks the chunking
  // for kScratchBytes of workspace and reports EWORKSPACE if even the
  // coarsest chunking does not fit
  semkv_status st =
      decode_args(c, q, layer0, nlayers, sm_scale, out, ws, kScratchBytes, &a);
  if (st != SEMKV_OK) return st;
  st = from_hip(launch_decode_partials(a, (hipStream_t)stream));
  if (st != SEMKV_OK) return st;
  return from_hip(launch_decode_merge(a, (hipStream_t)stream));
}

int64_t semkv_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

semkv_status semkv_dequantize_rows(const semkv_cache* c, int32_t pool, int32_t layer,
                                   int64_t row0, int64_t nrows, float* out, void* stream) {
  semkv_status st = check_cache(c);
  if (st != SEMKV_OK) return st;
  const semkv_geom& g = c->g;
  if (pool != 0 && pool != 1) return SEMKV_EINVAL;
  if (layer < 0 || layer >= g.layers) return SEMKV_EINVAL;
  const int64_t valid = pool == 0 ? c->n_high : c->n_low;
  if (row0 < 0 || nrows < 0 || row0 + nrows > valid) return SEMKV_EINVAL;
  if (!out || !aligned(out, 16)) return SEMKV_EINVAL;
  DequantArgs a;
  a.codes = pool == 0 ? c->codes_high : c->codes_low;
  a.meta = reinterpret_cast<const uint32_t*>(pool == 0 ? c->meta_high : c->meta_low);
  a.cap = pool == 0 ? g.cap_high : g.cap_low;
  a.fmt = row_fmt(pool == 0 ? g.L_high : g.L_low);
  a.batch = g.batch;
  a.layers = g.layers;
  a.kv_heads = g.kv_heads;
  a.layer = layer;
  a.row0 = row0;
  a.nrows = nrows;
  a.rotate = g.rotate;
  a.out = out;
  return from_hip(launch_dequant(a, (hipStream_t)stream));
}

// ---- ragged batches: per-sequence counters in device memory

semkv_status semkv_seq_reset(int64_t* seq, int32_t batch, void* stream) {
  if (!seq || !aligned(seq, 8) || batch < 1 || batch > 65535) return SEMKV_EINVAL;
  return from_hip(launch_seq_reset(seq, batch, (hipStream_t)stream));
}

semkv_status semkv_ragged_rank_topr(const float* scores, int32_t batch, int64_t n_max,
                                    int64_t ld_scores, const int32_t* n_seq, double r,
                                    int32_t* perm, uint32_t* mask, void* stream) {
  if (!scores || !perm || !aligned(scores, 4) || !aligned(perm, 4)) return SEMKV_EINVAL;
  if (!n_seq || !aligned(n_seq, 4) || (mask && !aligned(mask, 4))) return SEMKV_EINVAL;
  if (batch < 1 || batch > 65535 || n_max < 1 || n_max > (int64_t)INT32_MAX || ld_scores < n_max)
    return SEMKV_EINVAL;
  if (!(r >= 0.0 && r <= 1.0)) return SEMKV_EINVAL;
  return from_hip(launch_rank(scores, batch, (int)n_max, ld_scores, 0, perm, mask,
                              (hipStream_t)stream, n_seq, r, n_max));
}

semkv_status semkv_ragged_quantize_pack(semkv_cache* c, int64_t* seq, const uint16_t* k,
                                        const uint16_t* v, const int64_t strides[4], int64_t n_max,
                                        const int32_t* n_seq, double r, const int32_t* perm,
                                        void* stream) {
  semkv_status st = check_ragged(c, seq);
  if (st != SEMKV_OK) return st;
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16) || !strides_ok(strides)) return SEMKV_EINVAL;
  if (!perm || !aligned(perm, 4) || !n_seq || !aligned(n_seq, 4)) return SEMKV_EINVAL;
  if (n_max < 1 || n_max > (int64_t)INT32_MAX || !(r >= 0.0 && r <= 1.0)) return SEMKV_EINVAL;
  // launch bounds: both pool counts are non-decreasing in n, so n_max bounds them
  QuantArgs a = quant_args(c, k, v, strides, n_max, perm, topr(n_max, r), 0);
  a.seq = seq;
  a.n_seq = n_seq;
  a.r = r;
  a.ld_perm = n_max;
  a.tail_mode = 0;
  hipStream_t s = (hipStream_t)stream;
  st = from_hip(launch_quantize_pack(a, s));
  if (st != SEMKV_OK) return st;
  return from_hip(launch_seq_prefill_advance(seq, n_seq, r, c->g.batch, c->g.cap_high,
                                             c->g.cap_low, s));
}

semkv_status semkv_ragged_append(semkv_cache* c, int64_t* seq, const uint16_t* k_new,
                                 const uint16_t* v_new, const int64_t strides[4],
                                 const float* score_new, const int32_t* active,
                                 const int32_t* flush, double r, void* workspace, int64_t ws_bytes,
                                 void* stream) {
  semkv_status st = check_ragged(c, seq);
  if (st != SEMKV_OK) return st;
  if (!(r >= 0.0 && r <= 1.0)) return SEMKV_EINVAL;
  if (active) {
    if (!aligned(active, 4) || !k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16) ||
        !strides_ok(strides) || !score_new || !aligned(score_new, 4))
      return SEMKV_EINVAL;
  }
  if (flush && !aligned(flush, 4)) return SEMKV_EINVAL;
  const semkv_geom& g = c->g;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < append_ws_bytes(g))
    return SEMKV_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  int32_t* wperm = reinterpret_cast<int32_t*>(workspace);
  int32_t* nq = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(workspace) + append_perm_bytes(g));
  if (active) {
    AppendArgs aa;
    aa.src[0] = k_new;
    aa.src[1] = v_new;
    aa.sb = strides[0];
    aa.sl = strides[1];
    aa.sh = strides[2];
    aa.st = strides[3];
    aa.score_new = score_new;
    aa.t_total = 1;
    aa.t_off = 0;
    aa.t_cnt = 1;
    aa.batch = g.batch;
    aa.layers = g.layers;
    aa.kv_heads = g.kv_heads;
    aa.block = g.block;
    aa.pos = 0;
    aa.tail_kv = c->tail_kv;
    aa.tail_score = c->tail_score;
    aa.seq = seq;
    aa.active = active;
    st = from_hip(launch_append_tail(aa, s));
    if (st != SEMKV_OK) return st;
  }
  st = from_hip(launch_seq_tail_plan(seq, active, flush, r, g.block, g.batch, g.cap_high,
                                     g.cap_low, nq, s));
  if (st != SEMKV_OK) return st;
  // rank and quantize every tail with nq[b] > 0 rows (the others write nothing)
  st = from_hip(launch_rank(c->tail_score, g.batch, g.block, g.block, 0, wperm, nullptr, s, nq, r,
                            g.block));
  if (st != SEMKV_OK) return st;
  const int64_t tb = (int64_t)g.layers * g.kv_heads * 2 * g.block * kHeadDim;
  const int64_t tstr[4] = {tb, (int64_t)g.kv_heads * 2 * g.block * kHeadDim,
                           (int64_t)2 * g.block * kHeadDim, kHeadDim};
  QuantArgs qa = quant_args(c, c->tail_kv, c->tail_kv + (int64_t)g.block * kHeadDim, tstr,
                            g.block, wperm, topr(g.block, r), 0);
  qa.seq = seq;
  qa.n_seq = nq;
  qa.r = r;
  qa.ld_perm = g.block;
  qa.tail_mode = 1;
  st = from_hip(launch_quantize_pack(qa, s));
  if (st != SEMKV_OK) return st;
  return from_hip(launch_seq_tail_advance(seq, nq, r, g.batch, s));
}

semkv_status semkv_ragged_decode_attn(const semkv_cache* c, const int64_t* seq, const uint16_t* q,
                                      int32_t layer0, int32_t nlayers, float sm_scale,
                                      int64_t max_high, int64_t max_low, float* out,
                                      void* workspace, int64_t ws_bytes, void* stream) {
  semkv_status st = check_ragged(c, seq);
  if (st != SEMKV_OK) return st;
  if (!q || !aligned(q, 16) || !out || !aligned(out, 16)) return SEMKV_EINVAL;
  if (max_high < 0 || max_high > c->g.cap_high || max_low < 0 || max_low > c->g.cap_low)
    return SEMKV_EINVAL;
  // launch over the bounds; every kernel reads its sequence's own rows
  semkv_cache view = *c;
  view.n_high = max_high;
  view.n_low = max_low;
  view.n_tokens = max_high + max_low;
  DecodeArgs a;
  st = decode_args(&view, q, layer0, nlayers, sm_scale, out, workspace, ws_bytes, &a, seq,
                   c->g.block);
  if (st != SEMKV_OK) return st;
  st = from_hip(launch_decode_partials(a, (hipStream_t)stream));
  if (st != SEMKV_OK) return st;
  return from_hip(launch_decode_merge(a, (hipStream_t)stream));
}

semkv_status semkv_sync_check(void* stream) {
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return SEMKV_EHIP;
  e = hipGetLastError();
  return e == hipSuccess ? SEMKV_OK : SEMKV_EHIP;
}

const char* semkv_status_str(semkv_status s) {
  switch (s) {
    case SEMKV_OK: return "ok";
    case SEMKV_EINVAL: return "invalid argument";
    case SEMKV_EUNSUPPORTED: return "unsupported geometry or level count";
    case SEMKV_ECAPACITY: return "pool capacity exceeded";
    case SEMKV_EWORKSPACE: return "workspace missing or too small";
    case SEMKV_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
