// hs_device_f8.h -- fp8 (OCP e4m3) attention engine for gfx950, head_dim 128.
//
// Scores: S^T = K Q^T with v_mfma_f32_16x16x128_f8f6f4: one product covers a
// 16-key x 16-column chunk over the whole head_dim.  Values: O^T = V^T P^T
// with v_mfma_f32_32x32x64_f8f6f4: one product covers 32 head_dim rows x 32
// query columns (the wave's two column tiles) over one 64-key block.
//
// Operand layouts (lane l, q = l/16, r = l%16, h = l/32):
//   16x16x128  A: row r, 32 k-slots of lane group q   B: column r, same slots
//              C: column r, rows 4q .. 4q+3
//   32x32x64   A: row l%32, 32 k-slots of lane half h  B: column l%32, same
//              C: column l%32, value v = row 8(v/4) + 4h + v%4
// (which k index a slot holds does not matter as long as A and B agree).
//
// S^T chunk c row rho holds key 16*(rho/4) + 4c + rho%4, so lane group q
// holds keys 16q .. 16q+15 of the tile (4c+i for its logit s[c][i]).  After
// the softmax each lane packs its 16 probabilities of a column tile into four
// dwords, in key order.  The P operand of the 32x32x64 product wants, in lane
// half h, the 32 keys 32h .. 32h+31 of column l%32 (column tile (l/16)%2):
// one v_permlane16_swap per dword pair (column tile 0, column tile 1) swaps
// column tile 1 of lane groups 0/2 with column tile 0 of groups 1/3, which
// leaves every lane holding keys 32h .. 32h+31 of its own column.  The value
// operand is then 32 consecutive keys of one head_dim row: 32 contiguous
// bytes of a [head_dim][64] (block-major) fp8 value tile.
//
// Logits are exact fp32 sums of products of e4m3 values; the scales of Q and
// K enter the softmax scale and the scale of V the output.  P is rounded to
// e4m3 (round to nearest even) for the value product.  The denominators are
// fp32 sums of the unrounded probabilities (so the LSE and the block scores
// are those of the exact logits), or, with LSUM (no LSE wanted), the matrix
// unit's sums of the same rounded P against an all-ones operand, so that the
// output is an exactly normalised mean under the rounded weights.
#pragma once

#include "hs_device.h"

namespace hs {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// 32 fp8 codes of one lane
struct F8x32 {
  uint4 a, b;
};

__device__ __forceinline__ i32x8 f8_vec(const F8x32& f) {
  return i32x8{(int)f.a.x, (int)f.a.y, (int)f.a.z, (int)f.a.w, (int)f.b.x, (int)f.b.y, (int)f.b.z, (int)f.b.w};
}
__device__ __forceinline__ void mma16_f8(f32x4& acc, const F8x32& a, const F8x32& b) {
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f8_vec(a), f8_vec(b), acc, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ void mma32_f8(f32x16& acc, const F8x32& a, const F8x32& b) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f8_vec(a), f8_vec(b), acc, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ F8x32 f8_ld(const void* p) {
  F8x32 f;
  f.a = reinterpret_cast<const uint4*>(p)[0];
  f.b = reinterpret_cast<const uint4*>(p)[1];
  return f;
}
__device__ __forceinline__ F8x32 f8_zero() {
  F8x32 f;
  f.a = make_uint4(0u, 0u, 0u, 0u);
  f.b = f.a;
  return f;
}

// key held in row (16c + rho) of the fp8 S^T tile
__host__ __device__ __forceinline__ int f8_tile_key(int c, int rho) { return ((rho >> 2) << 4) | (c << 2) | (rho & 3); }

// four floats -> four e4m3 codes (RNE), one dword, byte e = element e
__device__ __forceinline__ uint32_t f8x4_bits(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// ------------------------------------------------------ LDS tile staging
// One 64-key fp8 tile: K rows [64][128 B] in S^T row order, then the value
// tile [128][64 B] as it is in memory.  The 16-byte chunk c of a K row r is
// stored at chunk c ^ (r & 7), of a value row d at c ^ (d & 3).  Transfers
// are direct global -> LDS (global_load_lds_dwordx4, 1 KiB per wave
// instruction), NTHR threads.  Key rows past the valid count read the last
// valid row (their logits are masked); value bytes past it are zeroed by
// dma_fix once the data has landed.
template <int NTHR>
struct TileStageF8 {
  static constexpr int KS = 128;            // bytes per key row
  static constexpr int VS = 64;             // bytes per value row
  static constexpr int KB = 64 * KS;        // 8 KiB
  static constexpr int BYTES = KB + 128 * VS;  // 16 KiB
  static constexpr int NWV = NTHR / 64;
  static constexpr int NDMA = BYTES / 1024 / NWV;
  static constexpr int NDK = KB / 1024 / NWV;
  static_assert(NDMA * NWV * 1024 == BYTES && (KB / 1024) % NWV == 0, "tile does not split into wave chunks");
  int dkey[NDK > 0 ? NDK : 1];
  uint32_t doff[NDMA];
  int nk_;

  __device__ __forceinline__ static int k_lds(int row, int chunk) { return row * KS + ((chunk ^ (row & 7)) << 4); }
  __device__ __forceinline__ static int v_lds(int row, int chunk) { return KB + row * VS + ((chunk ^ (row & 3)) << 4); }

  __device__ __forceinline__ void dma_init() {
    const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int off = (w + NWV * n) * 1024 + 16 * lane;
      if (n < NDK) {
        const int r = off / KS, c = ((off % KS) >> 4) ^ (r & 7);
        dkey[n] = f8_tile_key(r >> 4, r & 15);
        doff[n] = dkey[n] * KS + c * 16;
      } else {
        const int v = off - KB, dd = v / VS, c = ((v % VS) >> 4) ^ (dd & 3);
        doff[n] = dd * VS + c * 16;
      }
    }
  }
  // krows: key row 0 of the tile (128-byte rows); vslab: [128][64] value
  // tile; nk: valid keys (>= 64: all).  All wave-uniform.
  __device__ __forceinline__ void dma(char* buf, const char* krows, const char* vslab, int nk) {
    nk_ = nk;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (nk >= 64) {
#pragma unroll
      for (int n = 0; n < NDMA; ++n) {
        const char* src = n < NDK ? krows + doff[n] : vslab + doff[n];
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(buf + (w + NWV * n) * 1024),
                                         16, 0, 0);
      }
    } else {
#pragma unroll
      for (int n = 0; n < NDMA; ++n) {
        const int kk = dkey[n < NDK ? n : 0];
        const char* src = n < NDK ? krows + (doff[n] - (uint32_t)((kk - min(kk, nk - 1)) * KS)) : vslab + doff[n];
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(buf + (w + NWV * n) * 1024),
                                         16, 0, 0);
      }
    }
  }
  // after this wave's transfers have landed: zero the value bytes past the
  // valid count in the chunks this lane fetched
  __device__ __forceinline__ void dma_fix(char* buf) const {
    if (nk_ >= 64) return;
    const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
    for (int n = NDK; n < NDMA; ++n) {
      const int k0 = ((int)doff[n] % VS);  // first key (byte) of the chunk
      if (k0 + 16 > nk_) {
        uint4* p = (uint4*)(buf + (w + NWV * n) * 1024 + 16 * lane);
        const uint4 x = *p;
        uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = nk_ - (k0 + 4 * i);  // valid bytes left from this word on
          wd[i] &= r >= 4 ? 0xffffffffu : (r <= 0 ? 0u : (0xffffffffu >> (8 * (4 - r))));
        }
        *p = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    }
  }
  // A fragment of S^T chunk c: row 16c + r, head_dim bytes 32q .. 32q+31
  __device__ __forceinline__ static F8x32 ldK(const char* buf, int c) {
    const int lane = lane_id();
    const int row = 16 * c + (lane & 15), ch = 2 * (lane >> 4);
    F8x32 f;
    f.a = *(const uint4*)(buf + k_lds(row, ch));
    f.b = *(const uint4*)(buf + k_lds(row, ch + 1));
    return f;
  }
  // A fragment of O^T rows 32mb .. 32mb+31: value row 32mb + l%32, keys 32h .. 32h+31
  __device__ __forceinline__ static F8x32 ldV(const char* buf, int mb) {
    const int lane = lane_id();
    const int row = 32 * mb + (lane & 31), ch = 2 * (lane >> 5);
    F8x32 f;
    f.a = *(const uint4*)(buf + v_lds(row, ch));
    f.b = *(const uint4*)(buf + v_lds(row, ch + 1));
    return f;
  }
};

// ------------------------------------------------------------- the engine
// One wavefront, two column tiles of 16 query columns, head_dim 128.
// m[nt], l[nt]: running maximum (log2 units) and the lane's partial
// denominator of column tile nt; o[mb]: O^T rows 32mb .. 32mb+31 of the
// lane's column (l%32 of the 32 columns: column tile (l/16)%2, column l%16).
// sc2[nt]: the column's softmax scale in log2 units (tau * log2(e) times the
// query and key scales).
template <bool LSUM = false>
struct WaveAttnF8 {
  static constexpr int NT = 2;
  static constexpr int NMB = 4;  // 32-row blocks of O^T
  static constexpr unsigned kAll = 3u;

  F8x32 qf[NT];
  f32x16 o[NMB];
  f32x16 lacc;  // LSUM: the lane column's sum of the rounded P (every value)
  float m[NT], l[NT];

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m[nt] = kNegBig;
      l[nt] = 0.f;
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) o[mb] = f32x16{};
    if (LSUM) lacc = f32x16{};
  }

  // S^T of one 64-key tile (4 chunks x 2 column tiles); LA > 0 orders the
  // LDS reads ahead of the products (WaveAttn::lds_mfma_order)
  template <int LA = 0, class LK>
  __device__ __forceinline__ void qk(const LK& ldK, f32x4 (&s)[NT][4]) const {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const F8x32 a = ldK(c);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        s[nt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        mma16_f8(s[nt][c], a, qf[nt]);
      }
    }
    WaveAttn<HS_BF16, 128, NT>::template lds_mfma_order<LA, 4, NT, 0>();
  }

  // Online softmax of a tile's logits (as WaveAttn::softmax, with the fp8 key
  // order and per-column scales), then the P operand: pf receives the 32
  // packed probabilities of the lane's column for the value product.
  template <bool MASK, bool WANT_SUM>
  __device__ __forceinline__ void softmax(f32x4 (&s)[NT][4], int kbase, const int* lo, const int* hi,
                                          const float* sc2, float* bmax, float* bsum, F8x32& pf,
                                          unsigned act = kAll) {
    const int lane = lane_id();
    bool ranged = false, off = false;
    if (MASK) {
      bool part = false, dis = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bool en = lo[nt] != kNoKey;
        dis = dis || !en;
        part = part || (en && (kbase < lo[nt] || kbase + 63 > hi[nt]));
      }
      ranged = __ballot(part) != 0ull;
      off = __ballot(dis) != 0ull;
    }
    uint32_t pk[NT][4];
    float alpha[NT];
    bool anyup = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      alpha[nt] = 1.f;
      if (!((act >> nt) & 1u)) {
        bmax[nt] = -INFINITY;
        if (WANT_SUM) bsum[nt] = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) pk[nt][c] = 0u;
        continue;
      }
      f32x4(&x)[4] = s[nt];
      const bool en = !MASK || lo[nt] != kNoKey;
      if (MASK && ranged) {
        // the lane's keys are kbase + 16*(lane/16) + 4c + i
        const int base = kbase + 16 * (lane >> 4);
        const int klo = en ? lo[nt] - base : 64;
        const int khi = hi[nt] - base;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = 4 * c + i;
            x[c][i] = (k < klo || k > khi) ? -INFINITY : x[c][i];
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[c][i]);
      if (MASK && off) mx = en ? mx : -INFINITY;
      mx = xlane_max(mx) * sc2[nt];
      bmax[nt] = mx;
      const bool up = mx > m[nt] + kSlack;
      const float mn = up ? mx : m[nt];
      alpha[nt] = up ? fast_exp2(m[nt] - mn) : 1.f;
      anyup = anyup || up;
      m[nt] = mn;
      const float nmn = (MASK && off && !en) ? -INFINITY : -mn;
      float ps = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[c][i] = fast_exp2(__builtin_fmaf(x[c][i], sc2[nt], nmn));
          if (!LSUM || WANT_SUM) ps = (c | i) ? ps + x[c][i] : x[c][i];
        }
      if (!LSUM) l[nt] = l[nt] * alpha[nt] + ps;
      if (WANT_SUM) bsum[nt] = xlane_sum(ps);
#pragma unroll
      for (int c = 0; c < 4; ++c) pk[nt][c] = f8x4_bits(x[c][0], x[c][1], x[c][2], x[c][3]);
    }
    // column tile 1 of lane groups 0/2 <-> column tile 0 of groups 1/3
    uint32_t w[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const auto r = __builtin_amdgcn_permlane16_swap(pk[0][c], pk[1][c], false, false);
      w[c] = r[0];
      w[4 + c] = r[1];
    }
    pf.a = make_uint4(w[0], w[1], w[2], w[3]);
    pf.b = make_uint4(w[4], w[5], w[6], w[7]);
    if (__ballot(anyup) != 0ull) {
      const float al = ((lane >> 4) & 1) ? alpha[1] : alpha[0];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) o[mb] *= al;
      if (LSUM) lacc *= al;
    }
  }

  // O += P V for one tile
  template <int LA = 0, class LV>
  __device__ __forceinline__ void pv(const F8x32& pf, const LV& ldV) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) mma32_f8(o[mb], ldV(mb), pf);
    if (LSUM) {
      F8x32 ones;
      ones.a = make_uint4(0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u);  // e4m3 1.0
      ones.b = ones.a;
      mma32_f8(lacc, ones, pf);
    }
    WaveAttn<HS_BF16, 128, NT>::template lds_mfma_order<LA, NMB, 1, LSUM ? 1 : 0>();
  }

  // LSUM: 1/denominator of the lane's own column (column tile (lane/16)%2),
  // with an optional sink logit (log2 units) in the maximum and the sum
  __device__ __forceinline__ float inv_own(float sink2 = -INFINITY) const {
    const bool t1 = (lane_id() >> 4) & 1;
    float lt = lacc[0];
    const float mm = t1 ? m[1] : m[0];
    float sc = 1.f;
    if (sink2 > -INFINITY) {
      const float M = fmaxf(mm, sink2);
      sc = fast_exp2(mm - M);
      lt = lt * sc + fast_exp2(sink2 - M);
    }
    return lt > 0.f ? sc / lt : 0.f;
  }

  // column totals of column tile nt, as WaveAttn::finish
  __device__ __forceinline__ void finish(int nt, float& inv_l, float& lse2, float sink2 = -INFINITY) const {
    float lt = xlane_sum(l[nt]);
    float mm = m[nt], sc = 1.f;
    if (sink2 > -INFINITY) {
      const float M = fmaxf(mm, sink2);
      sc = fast_exp2(mm - M);
      lt = lt * sc + fast_exp2(sink2 - M);
      mm = M;
    }
    inv_l = lt > 0.f ? sc / lt : 0.f;
    lse2 = lt > 0.f ? mm + fast_log2(lt) : -INFINITY;
  }
};

}  // namespace hs
