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
  const float* q_scale;   // fp8: [Hq] query scales
  const float* kv_scale;  // fp8: [2][Hkv] key and value scales
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
  const float* q_scale;    // fp8: [Hq] scales of the layer's queries
  const float* kv_scale;   // fp8: [2][Hkv] scales of the shared K, V
  const float* swa_scale;  // fp8: [2][Hkv] scales of the window K', V'
  // training forward (optional): each branch's ungated output [2][B][T][Hq][D]
  // (0: sparse branch, 1: window branch, output dtype) and its LSE
  // [2][B][Hq][T] (natural log, sink included)
  void* o_br;
  float* lse_br;
};
// whether hs_sparse_attn_fwd runs sparse_prefill_dual_kernel for this shape
// (the kernel that also writes the training-forward branch outputs)
bool sparse_prefill_dual_ok(const SparsePrefillArgs& a, int dtype, int D);

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
  int token;              // 1: raw holds per-token logits; 0: per-block maxima;
                          // 2: selection bounds in zb / ab (raw unused)
  int kv_dtype;           // HS_BF16 (block-major V) or HS_FP8_E4M3 (position-major V)
  const float* kv_scale;  // fp8: device [2][Hkv]
  float sc2;
  // token == 2: per (sequence, kv group) row, zb [rows][C] = max over the
  // group's heads of (logit - a) and ab [rows][C/64][G] = the offsets a of
  // each tile and head (log2 units; a is the chunk's LSE over its earlier
  // tiles, or the tile's own maximum for a chunk's first tile)
  float* zb;
  float* ab;
  // nclear words at clear are set to zero by the merge kernel (the fused
  // selection's histograms and counters, which the next kernel accumulates)
  uint32_t* clear;
  long nclear;
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
                          // then [B*Hkv] candidate counts (zeroed together); from
                          // bounds, the first part holds the lower bounds' bins
  uint32_t* cand_key;     // workspace [B*Hkv][kTokCap]
  int32_t* cand_idx;      // workspace [B*Hkv][kTokCap]
  uint32_t* seg;          // workspace [B*Hkv][nseg][2]: (first slot, count) of each
                          // key segment's candidates in cand_key / cand_idx
  int nseg;               // key segments per row, ceil(C / kTokSeg)
  int B, Hq, Hkv, C, kb, n_recent;
  // selection from bounds (raw unused): zb, ab as written by the full layer
  // with token == 2, wb [rows][C/64] scratch (per tile, min over the heads of
  // LSE_h - offset_h: hi = z - wb), and what the exact rescoring reads
  const float* zb;
  const float* ab;
  float* wb;
  const void* q;          // [B][Hq][D] bf16
  const uint8_t* k;       // [B][Hkv][C][D] fp8 e4m3 key cache
  const float* kv_scale;  // [2][Hkv]
  float sc2;              // softmax scale * log2(e)
  int D;
};
// candidates kept per row for the final exact selection (rows with more fall
// back to a radix select over the whole row)
constexpr int kTokCap = 8192;
constexpr int kTokSeg = 16384;  // keys per work group in the histogram and candidate passes

// Gather of the selected 64-token blocks of a block-mode decode cache into a
// compact per-(sequence, kv head) cache (explainer 3.4.3 eq. K~,V~).
struct GatherArgs {
  const void* k;          // [B][Hkv][C][D] keys
  const void* v;          // [B][Hkv][C/64][D][64] values (block-major)
  const int32_t* idx;     // [B][Hkv][nsel] block ids (read as a set)
  const int32_t* lens;    // [B] context lengths
  void* k_sel;            // [B][Hkv][nsel*64][D]
  void* v_sel;            // [B][Hkv][nsel][D][64]
  int32_t* idx_sel;       // [B][Hkv][nsel]: 0 .. n-1 for the live blocks, then -1
  int B, Hkv, C, D, nsel;
  int es;                 // bytes per cache element
};
hipError_t launch_gather_blocks(const GatherArgs& a, hipStream_t s);

// One decode step's full layer over a cache held in host memory: chunks of
// sequences are copied to one of two device staging buffers on copy_stream
// while the full layer, the selection and the gather of the previous chunk
// run on stream.
struct OffloadArgs {
  DecodeFullArgs full;    // the whole batch; k, v are the host caches, part the split-K workspace of a chunk
  TopkArgs topk;          // the whole batch
  GatherArgs gather;      // the whole batch; k, v are ignored (the staging buffers are read)
  const int32_t* lens_host;
  void* stage[2];         // each [chunk][Hkv][C][D] keys then [chunk][Hkv][C/64][D][64] values
  int chunk;              // sequences per chunk
};
hipError_t offload_pipeline(const OffloadArgs& a, int D, hipStream_t s, hipStream_t copy_s);
size_t offload_stage_bytes(int chunk, int Hkv, int C, int D, int es);

// ------------------------------------------------------------ backward
// layout copies for the backward (hs_backward.hip)
struct BwdLayoutArgs {
  const void* v[2];  // block-major value caches [B][Hkv][nblk][D][64] (NULL: skip)
  void* vp[2];       // out: values position-major [B][Hkv][nblk*64][D]
  int B, T, Hq, Hkv, nblk;
};
// query columns per position on the key side: the group size rounded up to a
// power of two (columns of the extra heads are switched off)
inline int bwd_gp(int G) {
  int p = 1;
  while (p < G) p <<= 1;
  return p;
}
struct BwdRowArgs {
  const void* o[2];     // branch outputs [B][T][Hq][D] bf16 (the layer output for the full layer)
  const void* dout;
  const float* lse[2];  // [B][Hq][T] (sinks only)
  const float* gates;   // [B][T][Hq][2] or NULL
  const float* sinks;   // [2][Hq] or NULL
  float* delta[2];      // out: [B][Hq][T] dO . o_br
  float* dgates;        // out (gated layers): [B][T][Hq][2]
  float* sterm[2];      // scratch (sinks): [B][Hq][T]
  float* dsinks;        // out (sinks): [2][Hq]
  // per-column statistics for the key side, in the column order of the
  // d-major copies: [B*Hkv][3][NC] = lse * log2(e), dO . o_br, sigma(gate)
  const float* lse_col[2];  // the branch's row LSE [B][Hq][T] (natural log)
  float* cstat[2];
  int B, T, Hq, D, nbr, Hkv, Gp, NC;
};
struct BwdKVArgs {
  const void* q;
  const void* dout;
  const void* k;        // this branch's keys [B][Hkv][T][D]
  const void* vp;       // this branch's values, position-major
  const float* cstat;   // this branch's per-column statistics (BwdRowArgs::cstat)
  const int32_t* plist; // sparse branch: positions that selected each block, ascending
  const int32_t* pcnt;  // [B*Hkv][nblk] list lengths
  const int32_t* poff;  // [B*Hkv][nblk] list offsets within the kv group's T*topk slots
  // sparse branch: work units of at most kUnitPos list entries.  utab
  // [B*Hkv][umax]: unit u of a kv group is part (code & 0xffff) of block
  // (code >> 16); ucount [B*Hkv] units per kv group; soff [B*Hkv][nblk] the
  // first partial slot of a block of several parts; pbuf [B*Hkv][smax][2][64][D]
  // the parts' dK (times tau) and dV, summed in part order by kv_part_sum_kernel
  const int32_t* utab;
  const int32_t* ucount;
  const int32_t* soff;
  float* pbuf;
  int umax, smax;
  float* dk;
  float* dv;
  int B, T, Hq, Hkv, nblk, W, NC, Gp, topk, accumulate;
  float sc2, tau;
};
// list entries per work unit of the sparse branch's key side: a block selected
// by more positions is split over several work groups
constexpr int kUnitPos = 1024;
inline int kv_umax(int nblk, int T, int topk) { return nblk + (int)((long)T * topk / kUnitPos) + 1; }
inline int kv_smax(int T, int topk) { return (int)(2L * T * topk / kUnitPos) + 1; }
// units of the sparse branch from the list lengths
hipError_t launch_kv_units(const int32_t* pcnt, int32_t* utab, int32_t* ucount, int32_t* soff, int nbg, int nblk,
                           int umax, hipStream_t s);
struct BwdQArgs {
  const void* q;
  const void* dout;
  const void* k0;   // branch 0 (full layer / sparse branch): keys [B][Hkv][T][D], values position-major
  const void* vp0;
  const void* k1;   // branch 1 (window): the layer's own cache
  const void* vp1;
  const float* lse0;
  const float* lse1;
  const float* delta0;
  const float* delta1;
  const float* gates;
  const int32_t* idx;
  int topk;
  float* dq;
  int B, T, Hq, Hkv, nblk, W;
  float sc2, tau;
};
hipError_t launch_bwd_layouts(const BwdLayoutArgs& l, int D, hipStream_t s);
hipError_t launch_bwd_rows(const BwdRowArgs& a, hipStream_t s);
// per (kv group, block) lists of the positions that selected the block (the
// forward's rule), ascending: colbits [B*Hkv][nblk][ceil(T/32)] scratch,
// plist [B*Hkv][T*topk], pcnt and poff [B*Hkv][nblk]
hipError_t launch_pos_lists(const int32_t* idx, uint32_t* colbits, int32_t* plist, int32_t* pcnt, int32_t* poff,
                            int B, int Hkv, int T, int topk, int nblk, hipStream_t s);
hipError_t launch_bwd_kv(const BwdKVArgs& a, int mode, int D, hipStream_t s);  // mode 0 full, 1 window, 2 sparse
hipError_t launch_bwd_q(const BwdQArgs& a, int mode, int D, hipStream_t s);    // mode 0 full, 1 sparse layer
size_t bwd_q_lds_bytes(int T, int G);

hipError_t launch_token_topk(const TokenTopkArgs& a, hipStream_t s);
// the same selection from the bounds of a token == 2 full layer
hipError_t launch_token_topk_bounds(const TokenTopkArgs& a, hipStream_t s);
hipError_t launch_decode_sparse_token(const DecodeSparseArgs& a, int D, hipStream_t s);

hipError_t launch_decode_full(const DecodeFullArgs& a, int D, hipStream_t s);
hipError_t launch_decode_sparse(const DecodeSparseArgs& a, int D, hipStream_t s);

hipError_t launch_full_prefill(const FullPrefillArgs& a, int dtype, int D, int score_lse,
                               hipStream_t s);
// fp8 e4m3 Q, K, V (head_dim 128, G <= 16): bf16 O
hipError_t launch_full_prefill_f8(const FullPrefillArgs& a, int score_lse, hipStream_t s);
hipError_t launch_sparse_prefill_f8(const SparsePrefillArgs& a, hipStream_t s);
hipError_t launch_block_topk(const TopkArgs& a, int max_blocks, hipStream_t s);
hipError_t launch_sparse_prefill(const SparsePrefillArgs& a, int dtype, int D, hipStream_t s);
// dynamic LDS of the sparse prefill kernel (bitsets + block list)
size_t sparse_prefill_lds_bytes(int T, int G);

}  // namespace hs
