// hs_internal.h -- launcher interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hs {

struct FullPrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* raw;
  int B, T, Hq, Hkv, nblk;
  float sc2;  // softmax scale * log2(e)
};

struct TopkArgs {
  const float* raw;
  const float* lse;
  float* gs;
  int32_t* idx;
  const int32_t* kv_lens;  // decode: context lengths; NULL in prefill
  int B, Hq, Hkv;
  int R;           // query rows per sequence (T in prefill, 1 in decode)
  int raw_stride;  // floats per (b, h, row) score row
  int kb;          // top-k
  int diag;        // include the diagonal block
};

struct SparsePrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  const void* ks;
  const void* vs;
  const float* gates;
  const float* sinks;  // [2][Hq] sink logits (sparse, window branch) or NULL
  void* o;
  int B, T, Hq, Hkv, nblk, topk, W;
  int nwg;  // work groups (kv groups x position blocks)
  float sc2;
};

// split-K chunking of the decode full layer: at most this many 64-key tiles
// per chunk (the kernel keeps one block maximum per tile in registers until
// the chunk ends); the host picks 16 or 32 by context capacity
constexpr int kDecodeChunkBlocksMax = 32;
static_assert(kDecodeChunkBlocksMax % 4 == 0, "chunk tiles are spread over four lane groups");
inline int decode_chunk_blocks(int capacity) { return capacity > 131072 ? 32 : 16; }

struct DecodeFullArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* raw;
  float* part;            // workspace: [B][Hq][nch][D+2] partial (o, m, l)
  const int32_t* lens;
  int B, Hq, Hkv;
  int C;                  // cache capacity per sequence (multiple of 64)
  int nch;                // chunks per sequence at capacity
  int ch_blocks;          // 64-key blocks per chunk
  int token;              // 1: raw holds per-token logits; 0: per-block maxima
  int kv_dtype;           // HS_BF16 (block-major V) or HS_FP8_E4M3 (position-major V)
  const float* kv_scale;  // fp8: device [2][Hkv]
  float sc2;
};

struct DecodeSparseArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  const void* kr;
  const void* vr;
  const float* gates;
  const float* sinks;     // [2][Hq] sink logits (sparse, window branch) or NULL
  void* o;
  const int32_t* lens;
  const float* kv_scale;  // fp8 token mode: device [2][Hkv]
  float* part;            // token mode, nsplit > 1: workspace [B*Hkv][nsplit][G][D+2]
  int B, Hq, Hkv, C, nsel, W, nsplit;
  float sc2;
};
// token-mode sparse decode: work groups per (sequence, group) at most
constexpr int kTokSplitMax = 8;

struct TokenTopkArgs {
  const float* raw;       // [B][Hq][C] per-token logits
  const float* lse;       // [B][Hq]
  float* gs;              // nullable [B][Hkv][C]
  int32_t* idx;           // [B][Hkv][kb + n_recent]
  const int32_t* lens;
  uint32_t* keys;         // workspace [B*Hkv][C]
  uint32_t* hist;         // workspace [B*Hkv][2048] level-1, then [B*Hkv][2048] level-2,
                          // then [B*Hkv] candidate counts (zeroed together)
  uint32_t* cand_key;     // workspace [B*Hkv][kTokCap]
  int32_t* cand_idx;      // workspace [B*Hkv][kTokCap]
  uint32_t* seg;          // workspace [B*Hkv][nseg][2]: (first slot, count) of each
                          // key segment's candidates in cand_key / cand_idx
  int nseg;               // key segments per row, ceil(C / kTokSeg)
  int B, Hq, Hkv, C, kb, n_recent;
};
// candidates kept per row for the final exact selection (rows with more fall
// back to a radix select over the whole row)
constexpr int kTokCap = 8192;
constexpr int kTokSeg = 16384;  // keys per work group in the histogram and candidate passes

hipError_t launch_token_topk(const TokenTopkArgs& a, hipStream_t s);
hipError_t launch_decode_sparse_token(const DecodeSparseArgs& a, int D, hipStream_t s);

hipError_t launch_decode_full(const DecodeFullArgs& a, int D, hipStream_t s);
hipError_t launch_decode_sparse(const DecodeSparseArgs& a, int D, hipStream_t s);

hipError_t launch_full_prefill(const FullPrefillArgs& a, int dtype, int D, int score_lse,
                               hipStream_t s);
hipError_t launch_block_topk(const TopkArgs& a, int max_blocks, hipStream_t s);
hipError_t launch_sparse_prefill(const SparsePrefillArgs& a, int dtype, int D, hipStream_t s);
// dynamic LDS of the sparse prefill kernel (bitsets + block list)
size_t sparse_prefill_lds_bytes(int T, int G);

}  // namespace hs
