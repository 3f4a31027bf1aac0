// hs_api.hip -- the extern "C" entry points declared in include/hysparse.h:
// argument validation (before anything is launched), error reporting and
// dispatch to the kernel launchers.
#include <math.h>
#include <stddef.h>
#include <stdarg.h>
#include <stdio.h>
#include <algorithm>
#include <mutex>
#include <string>

#include "hs_internal.h"
#include "hysparse.h"

// Scratch of hs_decode_select_attn_static: a fixed device array, one copy per
// GPU (each device loads its own copy of this code object).  Host code never
// uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[HS_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

hs_status fail(hs_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

hs_status ok() {
  g_err.clear();
  return HS_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

#define REQUIRE_PTR(p)                                                               \
  do {                                                                               \
    if (!(p)) return fail(HS_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);             \
    if (!aligned16(p)) return fail(HS_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

// hs_shape as first published ended after kv_scale; later fields are read
// only when the caller's struct_size covers them
constexpr size_t kShapeMinSize = offsetof(hs_shape, kv_scale) + sizeof(const float*);
const float* shape_q_scale(const hs_shape* s) {
  return s->struct_size >= offsetof(hs_shape, q_scale) + sizeof(const float*) ? s->q_scale : nullptr;
}
const float* shape_swa_scale(const hs_shape* s) {
  return s->struct_size >= offsetof(hs_shape, swa_scale) + sizeof(const float*) ? s->swa_scale : nullptr;
}
bool aligned4(const void* p) { return p && ((uintptr_t)p & 3u) == 0; }

// Common shape checks.  Returns HS_OK or an error (message set).
hs_status check_shape(const char* fn, const hs_shape* s) {
  if (!s) return fail(HS_ERR_INVALID_ARG, "%s: shape is NULL", fn);
  if (s->struct_size < kShapeMinSize)
    return fail(HS_ERR_INVALID_ARG, "%s: shape.struct_size %zu < %zu", fn, s->struct_size, kShapeMinSize);
  if (s->batch < 0 || s->q_len < 0 || s->kv_len < 0)
    return fail(HS_ERR_INVALID_ARG, "%s: negative batch/q_len/kv_len", fn);
  if (s->hq <= 0 || s->hkv <= 0 || s->hq % s->hkv != 0)
    return fail(HS_ERR_INVALID_ARG, "%s: hq=%d must be a positive multiple of hkv=%d", fn, s->hq, s->hkv);
  const int G = s->hq / s->hkv;
  if (!pow2(G) || G > 32)
    return fail(HS_ERR_UNSUPPORTED, "%s: group size hq/hkv=%d must be a power of two <= 32", fn, G);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(HS_ERR_UNSUPPORTED, "%s: head_dim=%d (supported: 64, 128)", fn, s->head_dim);
  if (!(s->scale >= 0.f) || isinf(s->scale))
    return fail(HS_ERR_INVALID_ARG, "%s: scale must be finite and >= 0", fn);
  if ((long long)s->batch * s->hq * (long long)(s->q_len > s->kv_len ? s->q_len : s->kv_len) * s->head_dim >
      (1ll << 40))
    return fail(HS_ERR_INVALID_ARG, "%s: problem too large", fn);
  return HS_OK;
}

hs_status check_prefill(const char* fn, const hs_shape* s) {
  hs_status st = check_shape(fn, s);
  if (st) return st;
  if (s->kv_lens) return fail(HS_ERR_INVALID_ARG, "%s: prefill call with kv_lens set", fn);
  if (s->q_len != s->kv_len)
    return fail(HS_ERR_INVALID_ARG, "%s: prefill needs q_len == kv_len (got %d, %d)", fn, s->q_len, s->kv_len);
  if (s->dtype != HS_F32 && s->dtype != HS_BF16 && s->dtype != HS_FP8_E4M3)
    return fail(HS_ERR_UNSUPPORTED, "%s: prefill dtype %d (supported: HS_F32, HS_BF16, HS_FP8_E4M3)", fn,
                s->dtype);
  if (s->kv_dtype != s->dtype)
    return fail(HS_ERR_UNSUPPORTED, "%s: prefill needs kv_dtype == dtype", fn);
  if (s->dtype == HS_FP8_E4M3 && (s->head_dim != 128 || s->hq / s->hkv > 16))
    return fail(HS_ERR_UNSUPPORTED, "%s: fp8 prefill needs head_dim 128 and hq/hkv <= 16", fn);
  return HS_OK;
}

hs_status check_decode(const char* fn, const hs_shape* s) {
  hs_status st = check_shape(fn, s);
  if (st) return st;
  if (!s->kv_lens) return fail(HS_ERR_INVALID_ARG, "%s: decode needs kv_lens", fn);
  if (!aligned16(s->kv_lens)) return fail(HS_ERR_INVALID_ARG, "%s: kv_lens not 16-byte aligned", fn);
  if (s->q_len != 1) return fail(HS_ERR_INVALID_ARG, "%s: decode needs q_len == 1", fn);
  if (s->kv_len <= 0 || s->kv_len % 64)
    return fail(HS_ERR_INVALID_ARG, "%s: cache capacity kv_len=%d must be a positive multiple of 64", fn,
                s->kv_len);
  if (s->dtype != HS_BF16) return fail(HS_ERR_UNSUPPORTED, "%s: decode query dtype must be HS_BF16", fn);
  if (s->kv_dtype != HS_BF16 && s->kv_dtype != HS_FP8_E4M3)
    return fail(HS_ERR_UNSUPPORTED, "%s: decode cache dtype %d is not available", fn, s->kv_dtype);
  if (s->kv_dtype == HS_FP8_E4M3 && (!s->kv_scale || ((uintptr_t)s->kv_scale & 3u)))
    return fail(HS_ERR_INVALID_ARG, "%s: fp8 caches need a 4-byte aligned kv_scale", fn);
  if (s->hq / s->hkv > 16) return fail(HS_ERR_UNSUPPORTED, "%s: decode group size > 16", fn);
  return HS_OK;
}

int decode_nch(const hs_shape* s) {
  const int span = 64 * hs::decode_chunk_blocks(s->kv_len);
  return (s->kv_len + span - 1) / span;
}
size_t decode_full_ws(const hs_shape* s) {
  return (size_t)s->batch * s->hq * decode_nch(s) * (s->head_dim + 2) * sizeof(float);
}
// keys [rows][C], histograms [rows][2 * 2048], counts [rows] (padded to 4),
// candidates [rows][kTokCap] keys and ids
int token_nseg(const hs_shape* s) { return (s->kv_len + hs::kTokSeg - 1) / hs::kTokSeg; }
size_t token_topk_ws(const hs_shape* s) {
  const size_t rows = (size_t)s->batch * s->hkv;
  return rows * ((size_t)s->kv_len + 2 * 2048 + 2 * hs::kTokCap + 2 * (size_t)token_nseg(s)) * sizeof(uint32_t) +
         ((rows + 3) / 4) * 4 * sizeof(uint32_t);
}
// hs_decode_token_select: split-K partials, the bounds (z per token, offsets
// per tile and head, the upper-bound term per tile) and the token selection's
// workspace (its key array serves the whole-row fallback)
struct TokenSelWs {
  size_t part, zb, ab, wb, topk, total;
};
TokenSelWs token_select_ws(const hs_shape* s) {
  TokenSelWs w{};
  const size_t rows = (size_t)s->batch * s->hkv, ntl = (size_t)s->kv_len / 64;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  w.part = take(decode_full_ws(s));
  w.zb = take(rows * s->kv_len * sizeof(float));
  w.ab = take(rows * ntl * (size_t)(s->hq / s->hkv) * sizeof(float));
  w.wb = take(rows * ntl * sizeof(float));
  w.topk = take(token_topk_ws(s));
  w.total = off;
  return w;
}
// token-mode sparse layer: partial states of up to kTokSplitMax work groups per
// (sequence, group)
size_t decode_select_ws(const hs_shape* s, int block) {
  if (block != 1 || s->hkv <= 0) return 0;
  return (size_t)s->batch * s->hkv * hs::kTokSplitMax * (s->hq / s->hkv) * (s->head_dim + 2) * sizeof(float);
}
// Token mode (block = 1) runs on fp8 caches with position-major values; block
// mode (block = 64) on bf16 caches with block-major values.
hs_status check_decode_block(const char* fn, const hs_shape* s, int block) {
  if (block != 64 && block != 1) return fail(HS_ERR_INVALID_ARG, "%s: decode block=%d (64 or 1)", fn, block);
  if (block == 64 && s->kv_dtype != HS_BF16)
    return fail(HS_ERR_UNSUPPORTED, "%s: block mode needs HS_BF16 caches", fn);
  if (block == 1 && s->kv_dtype != HS_FP8_E4M3)
    return fail(HS_ERR_UNSUPPORTED, "%s: token mode needs HS_FP8_E4M3 caches", fn);
  return HS_OK;
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[256];  // per device id; filled on the first call on that device

hs_status static_scratch_ptr(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 256)
    return fail(HS_ERR_LAUNCH, "%s: no current HIP device (%s)", fn, hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(HS_ERR_LAUNCH, "%s: hipGetSymbolAddress of the static scratch failed on device %d: %s", fn,
                  dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HS_OK;
}

std::mutex g_cu_mu;
int g_cu_count[256];  // per device id; filled on the first query on that device

// compute units of the current device (256 if it cannot be queried)
int device_cu_count() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return 256;
  std::lock_guard<std::mutex> lock(g_cu_mu);
  if (!g_cu_count[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

// bytes of the token-mode split partial states for nsp work groups per
// (sequence, kv head)
size_t split_partials_bytes(const hs_shape* s, int nsp) {
  return (size_t)s->batch * s->hkv * nsp * (s->hq / s->hkv) * (s->head_dim + 2) * sizeof(float);
}

// workspace of hs_offload_full_select: two staging buffers of `chunk`
// sequences at full capacity, then the split-K partials of one chunk
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t offload_ws(const hs_shape* s, int chunk) {
  hs_shape c = *s;
  c.batch = chunk;
  return 2 * align256(hs::offload_stage_bytes(chunk, s->hkv, s->kv_len, s->head_dim, 2)) + decode_full_ws(&c);
}

// backward workspace: layout copies of K and V, per-row terms, per-column
// statistics, the sparse branch's position lists
struct BwdWs {
  size_t vp[2], delta[2], sterm[2], cstat[2], colbits, plist, pcnt, poff, utab, ucount, soff, pbuf, total;
};
int bwd_nc(const hs_shape* s) {
  const long cols = (long)s->q_len * hs::bwd_gp(s->hq / s->hkv) + 32;
  return (int)((cols + 63) / 64 * 64);
}
BwdWs bwd_ws(const hs_shape* s, bool sparse, int topk) {
  BwdWs w{};
  const size_t B = s->batch, T = s->q_len, D = s->head_dim, Hkv = s->hkv, Hq = s->hq;
  const size_t nblk = (T + 63) / 64, nw32 = (nblk + 31) / 32;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const int nbr = sparse ? 2 : 1;
  for (int i = 0; i < nbr; ++i) {
    w.vp[i] = take(B * Hkv * nblk * 64 * D * 2);
  }
  for (int i = 0; i < nbr; ++i) w.delta[i] = take(B * Hq * T * 4);
  for (int i = 0; i < nbr; ++i) w.cstat[i] = take(B * Hkv * 3 * (size_t)bwd_nc(s) * 4);
  if (sparse) {
    (void)nw32;
    for (int i = 0; i < 2; ++i) w.sterm[i] = take(B * Hq * T * 4);
    w.colbits = take(B * Hkv * nblk * ((T + 31) / 32) * 4);
    w.plist = take(B * Hkv * T * (size_t)(topk > 0 ? topk : 1) * 4);
    w.pcnt = take(B * Hkv * nblk * 4);
    w.poff = take(B * Hkv * nblk * 4);
    const int tk = topk > 0 ? topk : 1;
    w.utab = take(B * Hkv * (size_t)hs::kv_umax((int)nblk, (int)T, tk) * 4);
    w.ucount = take(B * Hkv * 4);
    w.soff = take(B * Hkv * nblk * 4);
    w.pbuf = take(B * Hkv * (size_t)hs::kv_smax((int)T, tk) * 2 * 64 * D * 4);
  }
  w.total = off;
  return w;
}

float scale_log2(const hs_shape* s) {
  const float tau = s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)s->head_dim);
  return tau * 1.4426950408889634f;
}

hs_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(HS_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int hs_version(void) { return 100; }

const char* hs_last_error(void) { return g_err.c_str(); }

size_t hs_workspace_size(int fn_id, const hs_shape* shape, int block, int topk, int window) {
  (void)block;
  (void)window;
  if (!shape || shape->struct_size < kShapeMinSize || shape->hkv <= 0 || shape->hq <= 0) return 0;
  if (!shape->kv_lens && (fn_id == HS_FN_FULL_ATTN_BWD || fn_id == HS_FN_SPARSE_ATTN_BWD))
    return bwd_ws(shape, fn_id == HS_FN_SPARSE_ATTN_BWD, topk < 0 ? 0 : topk).total;
  if (!shape->kv_lens) return 0;
  if (fn_id == HS_FN_FULL_ATTN) return decode_full_ws(shape);
  if (fn_id == HS_FN_BLOCK_TOPK && block == 1) return token_topk_ws(shape);
  if (fn_id == HS_FN_DECODE_TOKEN_SELECT) return token_select_ws(shape).total;
  if (fn_id == HS_FN_DECODE_SELECT) return decode_select_ws(shape, block);
  return 0;
}

hs_status hs_full_attn_fwd_scores(const hs_shape* s, const void* q, const void* k, const void* v,
                                  void* o, float* lse, float* blk_raw, int block, int flags,
                                  void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "hs_full_attn_fwd_scores";
  (void)ws;
  (void)ws_bytes;
  hs_status st = check_shape(fn, s);
  if (st) return st;
  if (flags != HS_SCORE_MAX && flags != HS_SCORE_LSE)
    return fail(HS_ERR_INVALID_ARG, "%s: flags=%d (HS_SCORE_MAX or HS_SCORE_LSE)", fn, flags);
  if (s->kv_lens) {
    st = check_decode(fn, s);
    if (st) return st;
    st = check_decode_block(fn, s, block);
    if (st) return st;
    if (flags != HS_SCORE_MAX) return fail(HS_ERR_UNSUPPORTED, "%s: decode supports HS_SCORE_MAX only", fn);
    if (s->batch == 0) return ok();
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(o);
    REQUIRE_PTR(lse);
    REQUIRE_PTR(blk_raw);
    const size_t need = decode_full_ws(s);
    if (!ws || ws_bytes < need)
      return fail(HS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, ws_bytes);
    if (!aligned16(ws)) return fail(HS_ERR_INVALID_ARG, "%s: ws not 16-byte aligned", fn);
    hs::DecodeFullArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.raw = blk_raw;
    a.part = (float*)ws;
    a.lens = s->kv_lens;
    a.B = s->batch;
    a.Hq = s->hq;
    a.Hkv = s->hkv;
    a.C = s->kv_len;
    a.nch = decode_nch(s);
    a.ch_blocks = hs::decode_chunk_blocks(s->kv_len);
    a.token = block == 1;
    a.kv_dtype = s->kv_dtype;
    a.kv_scale = s->kv_scale;
    a.sc2 = scale_log2(s);
    return launched(fn, hs::launch_decode_full(a, s->head_dim, (hipStream_t)stream));
  }
  st = check_prefill(fn, s);
  if (st) return st;
  if (block != 64) return fail(HS_ERR_UNSUPPORTED, "%s: prefill block=%d (only 64)", fn, block);
  if (s->batch == 0 || s->q_len == 0) return ok();
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(blk_raw);
  hs::FullPrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.raw = blk_raw;
  a.B = s->batch;
  a.T = s->q_len;
  a.Hq = s->hq;
  a.Hkv = s->hkv;
  a.nblk = (s->q_len + 63) / 64;
  a.sc2 = scale_log2(s);
  if (s->dtype == HS_FP8_E4M3) {
    a.q_scale = shape_q_scale(s);
    a.kv_scale = s->kv_scale;
    if (!aligned4(a.q_scale) || !aligned4(a.kv_scale))
      return fail(HS_ERR_INVALID_ARG, "%s: fp8 prefill needs shape.q_scale and shape.kv_scale", fn);
    return launched(fn, hs::launch_full_prefill_f8(a, flags == HS_SCORE_LSE, (hipStream_t)stream));
  }
  return launched(fn, hs::launch_full_prefill(a, s->dtype, s->head_dim, flags == HS_SCORE_LSE,
                                              (hipStream_t)stream));
}

hs_status hs_decode_token_select(const hs_shape* s, const void* q, const void* k, const void* v, void* o,
                                 float* lse, int topk, int n_recent, int32_t* idx, void* ws, size_t ws_bytes,
                                 void* stream) {
  const char* fn = "hs_decode_token_select";
  hs_status st = check_decode(fn, s);
  if (st) return st;
  st = check_decode_block(fn, s, 1);
  if (st) return st;
  if (topk < 1 || topk > 4096) return fail(HS_ERR_INVALID_ARG, "%s: topk=%d (1..4096 tokens)", fn, topk);
  if (n_recent < 0 || n_recent > 4096) return fail(HS_ERR_INVALID_ARG, "%s: n_recent=%d (0..4096)", fn, n_recent);
  if (s->batch == 0) return ok();
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(idx);
  if (!aligned16(k)) return fail(HS_ERR_INVALID_ARG, "%s: k not 16-byte aligned", fn);
  const TokenSelWs w = token_select_ws(s);
  if (!ws || ws_bytes < w.total)
    return fail(HS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, w.total, ws_bytes);
  if (!aligned16(ws)) return fail(HS_ERR_INVALID_ARG, "%s: ws not 16-byte aligned", fn);
  char* W = (char*)ws;
  hipStream_t strm = (hipStream_t)stream;
  hs::DecodeFullArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.raw = nullptr;
  a.part = (float*)(W + w.part);
  a.lens = s->kv_lens;
  a.B = s->batch;
  a.Hq = s->hq;
  a.Hkv = s->hkv;
  a.C = s->kv_len;
  a.nch = decode_nch(s);
  a.ch_blocks = hs::decode_chunk_blocks(s->kv_len);
  a.token = 2;
  a.kv_dtype = s->kv_dtype;
  a.kv_scale = s->kv_scale;
  a.sc2 = scale_log2(s);
  a.zb = (float*)(W + w.zb);
  a.ab = (float*)(W + w.ab);
  const size_t rows = (size_t)s->batch * s->hkv;
  uint32_t* keys = (uint32_t*)(W + w.topk);
  uint32_t* hist = keys + rows * s->kv_len;
  // the merge kernel of the full layer clears the selection's two histograms
  // per row and its per-row counters
  a.clear = hist;
  a.nclear = (long)rows * 2 * 2048 + (long)rows;
  hipError_t e = hs::launch_decode_full(a, s->head_dim, strm);
  if (e != hipSuccess) return launched(fn, e);
  hs::TokenTopkArgs t{};
  t.lse = lse;
  t.idx = idx;
  t.lens = s->kv_lens;
  t.keys = keys;
  t.hist = hist;
  t.cand_key = t.hist + rows * 2 * 2048 + ((rows + 3) / 4) * 4;
  t.cand_idx = (int32_t*)(t.cand_key + rows * hs::kTokCap);
  t.nseg = token_nseg(s);
  t.seg = (uint32_t*)(t.cand_idx + rows * hs::kTokCap);
  t.B = s->batch;
  t.Hq = s->hq;
  t.Hkv = s->hkv;
  t.C = s->kv_len;
  t.kb = topk;
  t.n_recent = n_recent;
  t.zb = a.zb;
  t.ab = a.ab;
  t.wb = (float*)(W + w.wb);
  t.q = q;
  t.k = (const uint8_t*)k;
  t.kv_scale = s->kv_scale;
  t.sc2 = a.sc2;
  t.D = s->head_dim;
  return launched(fn, hs::launch_token_topk_bounds(t, strm));
}

hs_status hs_block_topk(const hs_shape* s, const float* blk_raw, const float* lse, int block,
                        int topk, int n_recent, int flags, float* grp_score, int32_t* idx,
                        void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "hs_block_topk";
  (void)ws;
  (void)ws_bytes;
  hs_status st = check_shape(fn, s);
  if (st) return st;
  if (flags != HS_SEL_FULLY_PAST && flags != HS_SEL_INCLUDE_DIAG)
    return fail(HS_ERR_INVALID_ARG, "%s: flags=%d", fn, flags);
  if (n_recent < 0) return fail(HS_ERR_INVALID_ARG, "%s: n_recent < 0", fn);
  if (block == 1) {
    // token-level selection (decode only)
    st = check_decode(fn, s);
    if (st) return st;
    st = check_decode_block(fn, s, block);
    if (st) return st;
    if (flags != HS_SEL_FULLY_PAST) return fail(HS_ERR_INVALID_ARG, "%s: token mode takes no flags", fn);
    if (topk < 1 || topk > 4096) return fail(HS_ERR_INVALID_ARG, "%s: topk=%d (1..4096 tokens)", fn, topk);
    if (n_recent > 4096) return fail(HS_ERR_INVALID_ARG, "%s: n_recent=%d (0..4096)", fn, n_recent);
    if (s->batch == 0) return ok();
    REQUIRE_PTR(blk_raw);
    REQUIRE_PTR(lse);
    REQUIRE_PTR(idx);
    if (grp_score && !aligned16(grp_score)) return fail(HS_ERR_INVALID_ARG, "%s: grp_score misaligned", fn);
    const size_t need = token_topk_ws(s);
    if (!ws || ws_bytes < need)
      return fail(HS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, ws_bytes);
    if (!aligned16(ws)) return fail(HS_ERR_INVALID_ARG, "%s: ws not 16-byte aligned", fn);
    hs::TokenTopkArgs a{};
    a.raw = blk_raw;
    a.lse = lse;
    a.gs = grp_score;
    a.idx = idx;
    a.lens = s->kv_lens;
    const size_t rows = (size_t)s->batch * s->hkv;
    a.keys = (uint32_t*)ws;
    a.hist = a.keys + rows * s->kv_len;
    a.cand_key = a.hist + rows * 2 * 2048 + ((rows + 3) / 4) * 4;
    a.cand_idx = (int32_t*)(a.cand_key + rows * hs::kTokCap);
    a.nseg = token_nseg(s);
    a.seg = (uint32_t*)(a.cand_idx + rows * hs::kTokCap);
    a.B = s->batch;
    a.Hq = s->hq;
    a.Hkv = s->hkv;
    a.C = s->kv_len;
    a.kb = topk;
    a.n_recent = n_recent;
    return launched(fn, hs::launch_token_topk(a, (hipStream_t)stream));
  }
  if (block != 64) return fail(HS_ERR_INVALID_ARG, "%s: block=%d (64 or 1)", fn, block);
  if (topk < 1 || topk > 1024) return fail(HS_ERR_INVALID_ARG, "%s: topk=%d (1..1024 blocks)", fn, topk);
  if (n_recent != 0) return fail(HS_ERR_INVALID_ARG, "%s: n_recent applies to token mode only", fn);
  hs::TopkArgs a{};
  if (s->kv_lens) {
    st = check_decode(fn, s);
    if (st) return st;
    st = check_decode_block(fn, s, block);
    if (st) return st;
    a.R = 1;
    a.raw_stride = s->kv_len / 64;
  } else {
    st = check_prefill(fn, s);
    if (st) return st;
    a.R = s->q_len;
    a.raw_stride = (s->q_len + 63) / 64;
  }
  if (a.raw_stride > 4096)
    return fail(HS_ERR_UNSUPPORTED, "%s: more than 4096 candidate blocks per row", fn);
  if (s->batch == 0 || a.R == 0) return ok();
  REQUIRE_PTR(blk_raw);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(idx);
  if (grp_score && !aligned16(grp_score)) return fail(HS_ERR_INVALID_ARG, "%s: grp_score misaligned", fn);
  a.raw = blk_raw;
  a.lse = lse;
  a.gs = grp_score;
  a.idx = idx;
  a.kv_lens = s->kv_lens;
  a.B = s->batch;
  a.Hq = s->hq;
  a.Hkv = s->hkv;
  a.kb = topk;
  a.diag = flags == HS_SEL_INCLUDE_DIAG;
  return launched(fn, hs::launch_block_topk(a, a.raw_stride, (hipStream_t)stream));
}

}  // extern "C"

namespace {
hs_status sparse_fwd_impl(const char* fn, const hs_shape* s, const void* q_sp, const void* k, const void* v,
                          const int32_t* idx, int topk, const void* k_swa, const void* v_swa, int window,
                          const float* gate_logits, const float* sinks, void* o, void* o_br, float* lse_br,
                          void* stream) {
  hs_status st = check_prefill(fn, s);
  if (st) return st;
  if (topk < 0 || topk > 1024) return fail(HS_ERR_INVALID_ARG, "%s: topk=%d (0..1024)", fn, topk);
  if (window < 0) return fail(HS_ERR_INVALID_ARG, "%s: window < 0", fn);
  if (s->batch == 0 || s->q_len == 0) return ok();
  if (s->hq / s->hkv > 16) return fail(HS_ERR_UNSUPPORTED, "%s: group size > 16", fn);
  if (hs::sparse_prefill_lds_bytes(s->q_len, s->hq / s->hkv) > 48 * 1024)
    return fail(HS_ERR_UNSUPPORTED, "%s: sequence too long for the selection bitsets", fn);
  REQUIRE_PTR(q_sp);
  REQUIRE_PTR(o);
  if (topk > 0) {
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(idx);
  }
  if (window > 0) {
    REQUIRE_PTR(k_swa);
    REQUIRE_PTR(v_swa);
  }
  if (gate_logits && ((uintptr_t)gate_logits & 7u))
    return fail(HS_ERR_INVALID_ARG, "%s: gate_logits not 8-byte aligned", fn);
  hs::SparsePrefillArgs a{};
  a.q = q_sp;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.ks = k_swa;
  a.vs = v_swa;
  a.gates = gate_logits;
  a.sinks = sinks;
  a.o = o;
  a.B = s->batch;
  a.T = s->q_len;
  a.Hq = s->hq;
  a.Hkv = s->hkv;
  a.nblk = (s->q_len + 63) / 64;
  a.topk = topk;
  a.W = window;
  a.sc2 = scale_log2(s);
  a.o_br = o_br;
  a.lse_br = lse_br;
  if (s->dtype == HS_FP8_E4M3) {
    a.q_scale = shape_q_scale(s);
    a.kv_scale = s->kv_scale;
    a.swa_scale = shape_swa_scale(s);
    if (!aligned4(a.q_scale)) return fail(HS_ERR_INVALID_ARG, "%s: fp8 prefill needs shape.q_scale", fn);
    if (topk > 0 && !aligned4(a.kv_scale))
      return fail(HS_ERR_INVALID_ARG, "%s: fp8 prefill with topk > 0 needs shape.kv_scale", fn);
    if (window > 0 && !aligned4(a.swa_scale))
      return fail(HS_ERR_INVALID_ARG, "%s: fp8 prefill with a window needs shape.swa_scale", fn);
    return launched(fn, hs::launch_sparse_prefill_f8(a, (hipStream_t)stream));
  }
  return launched(fn, hs::launch_sparse_prefill(a, s->dtype, s->head_dim, (hipStream_t)stream));
}
}  // namespace

extern "C" {

hs_status hs_sparse_attn_fwd(const hs_shape* s, const void* q_sp, const void* k, const void* v,
                             const int32_t* idx, int topk, const void* k_swa, const void* v_swa,
                             int window, const float* gate_logits, const float* sinks, void* o,
                             void* stream) {
  return sparse_fwd_impl("hs_sparse_attn_fwd", s, q_sp, k, v, idx, topk, k_swa, v_swa, window, gate_logits, sinks,
                         o, nullptr, nullptr, stream);
}

}  // extern "C"

namespace {

hs_status decode_select_impl(const char* fn, const hs_shape* s, const void* q_sp, const void* k, const void* v,
                             const int32_t* idx, int n_sel, int block, const void* k_ring, const void* v_ring,
                             int window, const float* gate_logits, const float* sinks, void* o, void* ws,
                             size_t ws_bytes, bool static_scratch, void* stream) {
  hs_status st = check_decode(fn, s);
  if (st) return st;
  st = check_decode_block(fn, s, block);
  if (st) return st;
  if (n_sel < 0 || n_sel > 8192) return fail(HS_ERR_INVALID_ARG, "%s: n_sel=%d (0..8192)", fn, n_sel);
  if (block == 1 && (window != 0 || gate_logits))
    return fail(HS_ERR_INVALID_ARG, "%s: token mode has no window branch and no gate", fn);
  if (window < 0 || window > s->kv_len) return fail(HS_ERR_INVALID_ARG, "%s: window=%d", fn, window);
  if (s->batch == 0) return ok();
  REQUIRE_PTR(q_sp);
  REQUIRE_PTR(o);
  if (n_sel > 0) {
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(idx);
  }
  if (window > 0) {
    REQUIRE_PTR(k_ring);
    REQUIRE_PTR(v_ring);
  }
  if (gate_logits && ((uintptr_t)gate_logits & 7u))
    return fail(HS_ERR_INVALID_ARG, "%s: gate_logits not 8-byte aligned", fn);
  hs::DecodeSparseArgs a{};
  a.q = q_sp;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.kr = k_ring;
  a.vr = v_ring;
  a.gates = gate_logits;
  a.sinks = sinks;
  a.o = o;
  a.lens = s->kv_lens;
  a.B = s->batch;
  a.Hq = s->hq;
  a.Hkv = s->hkv;
  a.C = s->kv_len;
  a.nsel = n_sel;
  a.W = window;
  a.kv_scale = s->kv_scale;
  a.sc2 = scale_log2(s);
  a.nsplit = 1;
  if (block == 1) {
    // with a workspace, each (sequence, group) is spread over several work
    // groups of eight waves, about one 64-token tile per wave, and merged by
    // a second kernel.  One such group takes a compute unit's registers, so
    // there are no more groups than compute units: all run at once.
    const int ntile = (n_sel + 63) / 64;
    int nsp = std::min(hs::kTokSplitMax, std::max(1, (ntile + 7) / 8));
    while (nsp > 1 && (long)s->batch * s->hkv * nsp > device_cu_count()) --nsp;
    if (static_scratch) {
      // the split partial states go to this device's static scratch array
      const size_t need = split_partials_bytes(s, nsp);
      if (nsp > 1) {
        if (need > HS_STATIC_SCRATCH_BYTES)
          return fail(HS_ERR_WORKSPACE,
                      "%s: this shape needs %zu bytes of scratch; the static scratch holds %zu "
                      "(use hs_decode_select_attn with a workspace)",
                      fn, need, (size_t)HS_STATIC_SCRATCH_BYTES);
        void* scr = nullptr;
        st = static_scratch_ptr(fn, &scr);
        if (st) return st;
        a.part = (float*)scr;
        a.nsplit = nsp;
      }
    } else if (nsp > 1 && ws && ws_bytes >= decode_select_ws(s, block)) {
      if (!aligned16(ws)) return fail(HS_ERR_INVALID_ARG, "%s: ws not 16-byte aligned", fn);
      a.part = (float*)ws;
      a.nsplit = nsp;
    }
    return launched(fn, hs::launch_decode_sparse_token(a, s->head_dim, (hipStream_t)stream));
  }
  return launched(fn, hs::launch_decode_sparse(a, s->head_dim, (hipStream_t)stream));
}

}  // namespace

extern "C" {

hs_status hs_decode_select_attn(const hs_shape* s, const void* q_sp, const void* k, const void* v,
                                const int32_t* idx, int n_sel, int block, const void* k_ring,
                                const void* v_ring, int window, const float* gate_logits,
                                const float* sinks, void* o, void* ws, size_t ws_bytes,
                                void* stream) {
  return decode_select_impl("hs_decode_select_attn", s, q_sp, k, v, idx, n_sel, block, k_ring, v_ring,
                            window, gate_logits, sinks, o, ws, ws_bytes, false, stream);
}

hs_status hs_decode_select_attn_static(const hs_shape* s, const void* q_sp, const void* k, const void* v,
                                       const int32_t* idx, int n_sel, int block, const void* k_ring,
                                       const void* v_ring, int window, const float* gate_logits,
                                       const float* sinks, void* o, void* stream) {
  return decode_select_impl("hs_decode_select_attn_static", s, q_sp, k, v, idx, n_sel, block, k_ring,
                            v_ring, window, gate_logits, sinks, o, nullptr, 0, true, stream);
}

hs_status hs_gather_blocks(const hs_shape* s, const void* k, const void* v, const int32_t* idx, int n_sel,
                           void* k_sel, void* v_sel, int32_t* idx_sel, void* stream) {
  const char* fn = "hs_gather_blocks";
  hs_status st = check_decode(fn, s);
  if (st) return st;
  st = check_decode_block(fn, s, 64);
  if (st) return st;
  if (n_sel < 1 || n_sel > 8192) return fail(HS_ERR_INVALID_ARG, "%s: n_sel=%d (1..8192)", fn, n_sel);
  if (s->batch == 0) return ok();
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(k_sel);
  REQUIRE_PTR(v_sel);
  REQUIRE_PTR(idx_sel);
  hs::GatherArgs g{};
  g.k = k;
  g.v = v;
  g.idx = idx;
  g.lens = s->kv_lens;
  g.k_sel = k_sel;
  g.v_sel = v_sel;
  g.idx_sel = idx_sel;
  g.B = s->batch;
  g.Hkv = s->hkv;
  g.C = s->kv_len;
  g.D = s->head_dim;
  g.nsel = n_sel;
  g.es = 2;
  return launched(fn, hs::launch_gather_blocks(g, (hipStream_t)stream));
}

size_t hs_offload_workspace_size(const hs_shape* shape, int chunk) {
  if (!shape || shape->struct_size < sizeof(hs_shape) || chunk < 1 || shape->hkv <= 0) return 0;
  return offload_ws(shape, chunk);
}

hs_status hs_offload_full_select(const hs_shape* s, const int32_t* lens_host, const void* q, const void* k_host,
                                 const void* v_host, void* o, float* lse, float* blk_raw, int topk, int32_t* idx,
                                 void* k_sel, void* v_sel, int32_t* idx_sel, int chunk, void* ws,
                                 size_t ws_bytes, void* stream, void* copy_stream) {
  const char* fn = "hs_offload_full_select";
  hs_status st = check_decode(fn, s);
  if (st) return st;
  st = check_decode_block(fn, s, 64);
  if (st) return st;
  if (topk < 1 || topk > 1024) return fail(HS_ERR_INVALID_ARG, "%s: topk=%d (1..1024 blocks)", fn, topk);
  if (s->kv_len / 64 > 4096) return fail(HS_ERR_UNSUPPORTED, "%s: more than 4096 candidate blocks per row", fn);
  if (chunk < 1) return fail(HS_ERR_INVALID_ARG, "%s: chunk=%d", fn, chunk);
  if (s->batch == 0) return ok();
  if (!lens_host) return fail(HS_ERR_INVALID_ARG, "%s: lens_host is NULL", fn);
  if (!k_host || !v_host) return fail(HS_ERR_INVALID_ARG, "%s: host caches are NULL", fn);
  REQUIRE_PTR(q);
  REQUIRE_PTR(o);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(blk_raw);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(k_sel);
  REQUIRE_PTR(v_sel);
  REQUIRE_PTR(idx_sel);
  if (chunk > s->batch) chunk = s->batch;
  const size_t need = offload_ws(s, chunk);
  if (!ws || ws_bytes < need)
    return fail(HS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, ws_bytes);
  if (((uintptr_t)ws & 255u)) return fail(HS_ERR_INVALID_ARG, "%s: ws not 256-byte aligned", fn);
  hs::OffloadArgs a{};
  const size_t stage = align256(hs::offload_stage_bytes(chunk, s->hkv, s->kv_len, s->head_dim, 2));
  a.stage[0] = ws;
  a.stage[1] = (char*)ws + stage;
  a.chunk = chunk;
  a.lens_host = lens_host;
  hs_shape cs = *s;
  cs.batch = chunk;
  a.full.q = q;
  a.full.k = k_host;
  a.full.v = v_host;
  a.full.o = o;
  a.full.lse = lse;
  a.full.raw = blk_raw;
  a.full.part = (float*)((char*)ws + 2 * stage);
  a.full.lens = s->kv_lens;
  a.full.B = s->batch;
  a.full.Hq = s->hq;
  a.full.Hkv = s->hkv;
  a.full.C = s->kv_len;
  a.full.nch = decode_nch(s);
  a.full.ch_blocks = hs::decode_chunk_blocks(s->kv_len);
  a.full.token = 0;
  a.full.kv_dtype = HS_BF16;
  a.full.sc2 = scale_log2(s);
  a.topk.idx = idx;
  a.topk.B = s->batch;
  a.topk.Hq = s->hq;
  a.topk.Hkv = s->hkv;
  a.topk.R = 1;
  a.topk.raw_stride = s->kv_len / 64;
  a.topk.kb = topk;
  a.topk.diag = 0;
  a.gather.k_sel = k_sel;
  a.gather.v_sel = v_sel;
  a.gather.idx_sel = idx_sel;
  a.gather.B = s->batch;
  a.gather.Hkv = s->hkv;
  a.gather.C = s->kv_len;
  a.gather.D = s->head_dim;
  a.gather.nsel = topk;
  a.gather.es = 2;
  return launched(fn, hs::offload_pipeline(a, s->head_dim, (hipStream_t)stream, (hipStream_t)copy_stream));
}

hs_status hs_sparse_attn_fwd_train(const hs_shape* s, const void* q_sp, const void* k, const void* v,
                                   const int32_t* idx, int topk, const void* k_swa, const void* v_swa,
                                   int window, const float* gate_logits, const float* sinks, void* o,
                                   void* o_branch, float* lse_branch, void* stream) {
  const char* fn = "hs_sparse_attn_fwd_train";
  hs_status st = check_prefill(fn, s);
  if (st) return st;
  if (s->dtype != HS_BF16) return fail(HS_ERR_UNSUPPORTED, "%s: training forward takes bf16", fn);
  if (s->batch == 0 || s->q_len == 0) return ok();
  REQUIRE_PTR(o_branch);
  REQUIRE_PTR(lse_branch);
  hs::SparsePrefillArgs probe{};
  probe.Hq = s->hq;
  probe.Hkv = s->hkv;
  probe.nblk = (s->q_len + 63) / 64;
  if (!hs::sparse_prefill_dual_ok(probe, s->dtype, s->head_dim))
    return fail(HS_ERR_UNSUPPORTED, "%s: sequence too long for the training forward", fn);
  return sparse_fwd_impl(fn, s, q_sp, k, v, idx, topk, k_swa, v_swa, window, gate_logits, sinks, o, o_branch,
                         lse_branch, stream);
}

hs_status hs_full_attn_bwd(const hs_shape* s, const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv, void* ws,
                           size_t ws_bytes, void* stream) {
  const char* fn = "hs_full_attn_bwd";
  hs_status st = check_prefill(fn, s);
  if (st) return st;
  if (s->dtype != HS_BF16) return fail(HS_ERR_UNSUPPORTED, "%s: the backward takes bf16", fn);
  if (s->hq / s->hkv > 16) return fail(HS_ERR_UNSUPPORTED, "%s: group size > 16", fn);
  if (s->batch == 0 || s->q_len == 0) return ok();
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(dout);
  REQUIRE_PTR(dq);
  REQUIRE_PTR(dk);
  REQUIRE_PTR(dv);
  const BwdWs w = bwd_ws(s, false, 0);
  if (!ws || ws_bytes < w.total)
    return fail(HS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, w.total, ws_bytes);
  if ((uintptr_t)ws & 255u) return fail(HS_ERR_INVALID_ARG, "%s: ws not 256-byte aligned", fn);
  if (hs::bwd_q_lds_bytes(s->q_len, s->hq / s->hkv) > 64 * 1024)
    return fail(HS_ERR_UNSUPPORTED, "%s: sequence too long", fn);
  char* W = (char*)ws;
  hipStream_t strm = (hipStream_t)stream;
  const int nblk = (s->q_len + 63) / 64;
  hs::BwdLayoutArgs l{};
  l.v[0] = v;
  l.vp[0] = W + w.vp[0];
  l.B = s->batch;
  l.T = s->q_len;
  l.Hq = s->hq;
  l.Hkv = s->hkv;
  l.nblk = nblk;
  const int NC = bwd_nc(s), Gp = hs::bwd_gp(s->hq / s->hkv);
  hipError_t e = hs::launch_bwd_layouts(l, s->head_dim, strm);
  if (e != hipSuccess) return launched(fn, e);
  hs::BwdRowArgs r{};
  r.o[0] = o;
  r.dout = dout;
  r.delta[0] = (float*)(W + w.delta[0]);
  r.lse_col[0] = lse;
  r.cstat[0] = (float*)(W + w.cstat[0]);
  r.B = s->batch;
  r.T = s->q_len;
  r.Hq = s->hq;
  r.Hkv = s->hkv;
  r.Gp = Gp;
  r.NC = NC;
  r.D = s->head_dim;
  r.nbr = 1;
  e = hs::launch_bwd_rows(r, strm);
  if (e != hipSuccess) return launched(fn, e);
  const float tau = s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)s->head_dim);
  hs::BwdKVArgs a{};
  a.q = q;
  a.dout = dout;
  a.k = k;
  a.vp = l.vp[0];
  a.cstat = r.cstat[0];
  a.dk = dk;
  a.dv = dv;
  a.B = s->batch;
  a.T = s->q_len;
  a.Hq = s->hq;
  a.Hkv = s->hkv;
  a.nblk = nblk;
  a.NC = NC;
  a.Gp = Gp;
  a.sc2 = scale_log2(s);
  a.tau = tau;
  e = hs::launch_bwd_kv(a, 0, s->head_dim, strm);
  if (e != hipSuccess) return launched(fn, e);
  hs::BwdQArgs b{};
  b.q = q;
  b.dout = dout;
  b.k0 = k;
  b.vp0 = l.vp[0];
  b.lse0 = lse;
  b.delta0 = r.delta[0];
  b.dq = dq;
  b.B = s->batch;
  b.T = s->q_len;
  b.Hq = s->hq;
  b.Hkv = s->hkv;
  b.nblk = nblk;
  b.sc2 = a.sc2;
  b.tau = tau;
  return launched(fn, hs::launch_bwd_q(b, 0, s->head_dim, strm));
}

hs_status hs_sparse_attn_bwd(const hs_shape* s, const void* q_sp, const void* k, const void* v,
                             const int32_t* idx, int topk, const void* k_swa, const void* v_swa, int window,
                             const float* gate_logits, const float* sinks, const void* o_branch,
                             const float* lse_branch, const void* dout, float* dq_sp, float* dk, float* dv,
                             float* dk_swa, float* dv_swa, float* dgate, float* dsinks, void* ws, size_t ws_bytes,
                             void* stream) {
  const char* fn = "hs_sparse_attn_bwd";
  hs_status st = check_prefill(fn, s);
  if (st) return st;
  if (s->dtype != HS_BF16) return fail(HS_ERR_UNSUPPORTED, "%s: the backward takes bf16", fn);
  if (s->hq / s->hkv > 16) return fail(HS_ERR_UNSUPPORTED, "%s: group size > 16", fn);
  if (topk < 0 || topk > 1024) return fail(HS_ERR_INVALID_ARG, "%s: topk=%d (0..1024)", fn, topk);
  if (window < 0) return fail(HS_ERR_INVALID_ARG, "%s: window < 0", fn);
  if (s->batch == 0 || s->q_len == 0) return ok();
  REQUIRE_PTR(q_sp);
  REQUIRE_PTR(o_branch);
  REQUIRE_PTR(lse_branch);
  REQUIRE_PTR(dout);
  REQUIRE_PTR(dq_sp);
  if (topk > 0) {
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(idx);
    REQUIRE_PTR(dk);
    REQUIRE_PTR(dv);
  }
  if (window > 0) {
    REQUIRE_PTR(k_swa);
    REQUIRE_PTR(v_swa);
    REQUIRE_PTR(dk_swa);
    REQUIRE_PTR(dv_swa);
  }
  if (gate_logits && !dgate) return fail(HS_ERR_INVALID_ARG, "%s: gate_logits given without dgate", fn);
  if (sinks && !dsinks) return fail(HS_ERR_INVALID_ARG, "%s: sinks given without dsinks", fn);
  const BwdWs w = bwd_ws(s, true, topk);
  if (!ws || ws_bytes < w.total)
    return fail(HS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, w.total, ws_bytes);
  if ((uintptr_t)ws & 255u) return fail(HS_ERR_INVALID_ARG, "%s: ws not 256-byte aligned", fn);
  if (hs::bwd_q_lds_bytes(s->q_len, s->hq / s->hkv) > 64 * 1024)
    return fail(HS_ERR_UNSUPPORTED, "%s: sequence too long", fn);
  char* W = (char*)ws;
  hipStream_t strm = (hipStream_t)stream;
  const int T = s->q_len, nblk = (T + 63) / 64;
  const size_t brs = (size_t)s->batch * T * s->hq;  // rows of one branch
  hs::BwdLayoutArgs l{};
  if (topk > 0) {
    l.v[0] = v;
  }
  if (window > 0) {
    l.v[1] = v_swa;
  }
  for (int i = 0; i < 2; ++i) {
    l.vp[i] = W + w.vp[i];
  }
  l.B = s->batch;
  l.T = T;
  l.Hq = s->hq;
  l.Hkv = s->hkv;
  l.nblk = nblk;
  const int NC = bwd_nc(s), Gp = hs::bwd_gp(s->hq / s->hkv);
  hipError_t e = hs::launch_bwd_layouts(l, s->head_dim, strm);
  if (e != hipSuccess) return launched(fn, e);
  int32_t* plist = (int32_t*)(W + w.plist);
  int32_t* pcnt = (int32_t*)(W + w.pcnt);
  int32_t* poff = (int32_t*)(W + w.poff);
  if (topk > 0) {
    e = hs::launch_pos_lists(idx, (uint32_t*)(W + w.colbits), plist, pcnt, poff, s->batch, s->hkv, T, topk, nblk,
                             strm);
    if (e != hipSuccess) return launched(fn, e);
    e = hs::launch_kv_units(pcnt, (int32_t*)(W + w.utab), (int32_t*)(W + w.ucount), (int32_t*)(W + w.soff),
                            s->batch * s->hkv, nblk, hs::kv_umax(nblk, T, topk), strm);
    if (e != hipSuccess) return launched(fn, e);
  }
  hs::BwdRowArgs r{};
  r.o[0] = o_branch;
  r.o[1] = (const char*)o_branch + brs * s->head_dim * 2;
  r.dout = dout;
  r.lse[0] = lse_branch;
  r.lse[1] = lse_branch + brs;
  r.gates = gate_logits;
  r.sinks = sinks;
  r.delta[0] = (float*)(W + w.delta[0]);
  r.delta[1] = (float*)(W + w.delta[1]);
  r.dgates = dgate;
  r.sterm[0] = (float*)(W + w.sterm[0]);
  r.sterm[1] = (float*)(W + w.sterm[1]);
  r.dsinks = dsinks;
  r.lse_col[0] = r.lse[0];
  r.lse_col[1] = r.lse[1];
  if (topk > 0) r.cstat[0] = (float*)(W + w.cstat[0]);
  if (window > 0) r.cstat[1] = (float*)(W + w.cstat[1]);
  r.B = s->batch;
  r.T = T;
  r.Hq = s->hq;
  r.Hkv = s->hkv;
  r.Gp = Gp;
  r.NC = NC;
  r.D = s->head_dim;
  r.nbr = 2;
  e = hs::launch_bwd_rows(r, strm);
  if (e != hipSuccess) return launched(fn, e);
  const float tau = s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)s->head_dim);
  hs::BwdKVArgs a{};
  a.q = q_sp;
  a.dout = dout;
  a.B = s->batch;
  a.T = T;
  a.Hq = s->hq;
  a.Hkv = s->hkv;
  a.nblk = nblk;
  a.W = window;
  a.NC = NC;
  a.Gp = Gp;
  a.topk = topk;
  a.sc2 = scale_log2(s);
  a.tau = tau;
  if (topk > 0) {  // the sparse branch adds into the shared K/V's gradients
    a.k = k;
    a.vp = l.vp[0];
    a.cstat = r.cstat[0];
    a.plist = plist;
    a.pcnt = pcnt;
    a.poff = poff;
    a.utab = (const int32_t*)(W + w.utab);
    a.ucount = (const int32_t*)(W + w.ucount);
    a.soff = (const int32_t*)(W + w.soff);
    a.pbuf = (float*)(W + w.pbuf);
    a.umax = hs::kv_umax(nblk, T, topk);
    a.smax = hs::kv_smax(T, topk);
    a.dk = dk;
    a.dv = dv;
    a.accumulate = 1;
    e = hs::launch_bwd_kv(a, 2, s->head_dim, strm);
    if (e != hipSuccess) return launched(fn, e);
  }
  if (window > 0) {
    a.k = k_swa;
    a.vp = l.vp[1];
    a.cstat = r.cstat[1];
    a.plist = nullptr;
    a.dk = dk_swa;
    a.dv = dv_swa;
    a.accumulate = 0;
    e = hs::launch_bwd_kv(a, 1, s->head_dim, strm);
    if (e != hipSuccess) return launched(fn, e);
  }
  hs::BwdQArgs b{};
  b.q = q_sp;
  b.dout = dout;
  b.k0 = k;
  b.vp0 = l.vp[0];
  b.k1 = k_swa;
  b.vp1 = l.vp[1];
  b.lse0 = r.lse[0];
  b.lse1 = r.lse[1];
  b.delta0 = r.delta[0];
  b.delta1 = r.delta[1];
  b.gates = gate_logits;
  b.idx = idx;
  b.topk = topk;
  b.dq = dq_sp;
  b.B = s->batch;
  b.T = T;
  b.Hq = s->hq;
  b.Hkv = s->hkv;
  b.nblk = nblk;
  b.W = window;
  b.sc2 = a.sc2;
  b.tau = tau;
  return launched(fn, hs::launch_bwd_q(b, 1, s->head_dim, strm));
}

}  // extern "C"
