// hs_api.hip -- the extern "C" entry points declared in include/hysparse.h:
// argument validation (before anything is launched), error reporting and
// dispatch to the kernel launchers.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string>

#include "hs_internal.h"
#include "hysparse.h"

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

// Common shape checks.  Returns HS_OK or an error (message set).
hs_status check_shape(const char* fn, const hs_shape* s) {
  if (!s) return fail(HS_ERR_INVALID_ARG, "%s: shape is NULL", fn);
  if (s->struct_size < sizeof(hs_shape))
    return fail(HS_ERR_INVALID_ARG, "%s: shape.struct_size %zu < %zu", fn, s->struct_size, sizeof(hs_shape));
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
  if (s->dtype != HS_F32 && s->dtype != HS_BF16)
    return fail(HS_ERR_UNSUPPORTED, "%s: prefill dtype %d (supported: HS_F32, HS_BF16)", fn, s->dtype);
  if (s->kv_dtype != s->dtype)
    return fail(HS_ERR_UNSUPPORTED, "%s: prefill needs kv_dtype == dtype", fn);
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
  (void)topk;
  (void)window;
  if (!shape || shape->struct_size < sizeof(hs_shape) || !shape->kv_lens) return 0;
  if (fn_id == HS_FN_FULL_ATTN) return decode_full_ws(shape);
  if (fn_id == HS_FN_BLOCK_TOPK && block == 1) return token_topk_ws(shape);
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
  return launched(fn, hs::launch_full_prefill(a, s->dtype, s->head_dim, flags == HS_SCORE_LSE,
                                              (hipStream_t)stream));
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

hs_status hs_sparse_attn_fwd(const hs_shape* s, const void* q_sp, const void* k, const void* v,
                             const int32_t* idx, int topk, const void* k_swa, const void* v_swa,
                             int window, const float* gate_logits, const float* sinks, void* o,
                             void* stream) {
  const char* fn = "hs_sparse_attn_fwd";
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
  return launched(fn, hs::launch_sparse_prefill(a, s->dtype, s->head_dim, (hipStream_t)stream));
}

hs_status hs_decode_select_attn(const hs_shape* s, const void* q_sp, const void* k, const void* v,
                                const int32_t* idx, int n_sel, int block, const void* k_ring,
                                const void* v_ring, int window, const float* gate_logits,
                                const float* sinks, void* o, void* ws, size_t ws_bytes,
                                void* stream) {
  const char* fn = "hs_decode_select_attn";
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
    // groups (about eight 64-token tiles each) and merged by a second kernel
    const int ntile = (n_sel + 63) / 64;
    const int nsp = ntile / 8 < 1 ? 1 : (ntile / 8 > hs::kTokSplitMax ? hs::kTokSplitMax : ntile / 8);
    if (nsp > 1 && ws && ws_bytes >= decode_select_ws(s, block)) {
      if (!aligned16(ws)) return fail(HS_ERR_INVALID_ARG, "%s: ws not 16-byte aligned", fn);
      a.part = (float*)ws;
      a.nsplit = nsp;
    }
    return launched(fn, hs::launch_decode_sparse_token(a, s->head_dim, (hipStream_t)stream));
  }
  return launched(fn, hs::launch_decode_sparse(a, s->head_dim, (hipStream_t)stream));
}

}  // extern "C"
