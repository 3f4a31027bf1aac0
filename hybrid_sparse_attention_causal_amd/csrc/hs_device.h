// hs_device.h -- device building blocks shared by the HySparse kernels (gfx950).
//
// The attention "engine" works on one wavefront (64 lanes) and one tile of 64
// keys at a time.  It computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (or
// 8x v_mfma_f32_16x16x4f32 for fp32 inputs), so that a lane holds 16 logits of
// ONE query column: the per-column softmax maximum and sum need only two
// cross-lane exchanges (xor 16, xor 32), and the 64-key tile maximum is exactly
// the per-block maximum of the modified FlashAttention pass (HySparse
// explainer, section 3.4.1 "Modified FlashAttention Kernel": the row-wise
// maximum of each key tile is stored as the block score).
//
// MFMA 16x16x32 operand layout (lane l, q = l/16, r = l%16):
//   A (16 x 32): row r, k-slots 8q..8q+7        B (32 x 16): col r, k-slots 8q..8q+7
//   C (16 x 16): col r, rows 4q..4q+3
// S^T chunk c (c = 0..3, 16 keys each) row r holds key tile_key(c, r).  The map
// is chosen so that, after the softmax, a lane's 8 probabilities of chunks
// {2u, 2u+1} are exactly the k-slots 8q..8q+7 of keys 32u+8q..32u+8q+7 of the
// P.V product: the P operand needs no shuffle, and the value operand is eight
// consecutive keys of one head_dim row, i.e. 16 contiguous bytes of a
// [head_dim][64] (block-major) value tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hysparse.h"

namespace hs {

// Context length of sequence b held to [0, C]: a length outside the cache
// then cannot send a kernel outside its buffers.
__device__ __forceinline__ int ctx_len(const int32_t* lens, int b, int C) { return min(max(lens[b], 0), C); }

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;
constexpr int kBlk = 64;
constexpr int kNoKey = 0x7fffffff;
constexpr float kSlack = 8.f;  // see WaveAttn::tile

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__host__ __device__ __forceinline__ int tile_key(int c, int r) {
  return ((c >> 1) << 5) | ((r >> 2) << 3) | ((c & 1) << 2) | (r & 3);
}
// inverse of tile_key: the S^T row (16*c + r) that holds key kk of the tile
__host__ __device__ __forceinline__ int tile_row(int kk) {
  const int u = kk >> 5, q = (kk >> 3) & 3, e = (kk >> 2) & 1, i = kk & 3;
  return ((2 * u + e) << 4) | (q << 2) | i;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Reductions over the four lanes {l, l^16, l^32, l^48} that hold one MFMA
// column, with the gfx950 row-swap instructions (no LDS traffic).  Every
// lane of the group gets the same result.
// max of two floats that are never NaN here (logits, -inf for masked keys):
// one v_max_f32.  The compiler's own max (maxnum) first quiets both inputs
// with two more v_max_f32 in IEEE mode when it cannot prove them canonical,
// as after a cross-lane swap.
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float xlane_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float xlane_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
// two floats -> packed bf16 pair (RNE), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ----------------------------------------------------------- element traits
// Wait until every vector memory load of this wave has returned.  Issued once
// after the prologue loads (queries, gates): the compiler otherwise cannot
// tell them apart from the tile prefetches in flight inside the main loop and
// waits for all of them at the first use of a query fragment.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int DT> struct Tr;

template <> struct Tr<HS_BF16> {
  static constexpr int ES = 2;  // bytes per element
  struct Frag { uint4 u; };
  __device__ __forceinline__ static Frag ld(const void* p) {
    Frag f;
    f.u = *reinterpret_cast<const uint4*>(p);
    return f;
  }
  __device__ __forceinline__ static Frag zero() {
    Frag f;
    f.u = make_uint4(0u, 0u, 0u, 0u);
    return f;
  }
  // keep elements e < n, zero the rest (n in 0..8)
  __device__ __forceinline__ static Frag keep(Frag f, int n) {
    uint32_t w[4] = {f.u.x, f.u.y, f.u.z, f.u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (2 * i >= n) w[i] = 0u;
      else if (2 * i + 1 >= n) w[i] &= 0xffffu;
    }
    f.u = make_uint4(w[0], w[1], w[2], w[3]);
    return f;
  }
  __device__ __forceinline__ static void mma(f32x4& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.u),
                                                  __builtin_bit_cast(bf16x8_t, b.u), acc, 0, 0, 0);
  }
  __device__ __forceinline__ static Frag pack(const float* p) {
    Frag f;
    f.u = make_uint4(bf16x2_bits(p[0], p[1]), bf16x2_bits(p[2], p[3]), bf16x2_bits(p[4], p[5]),
                     bf16x2_bits(p[6], p[7]));
    return f;
  }
  __device__ __forceinline__ static void store4(void* dst, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(bf16x2_bits(a, b), bf16x2_bits(c, d));
  }
  __device__ __forceinline__ static Frag ones() {
    Frag f;
    f.u = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
    return f;
  }
  // a lane's 16 probabilities (four f32x4) -> its two P fragments, stored in
  // place in x[0] and x[1]; p_frag reads fragment u back
  __device__ __forceinline__ static void pack_p(f32x4 (&x)[4]) {
    const Frag a = pack(reinterpret_cast<const float*>(&x[0]));
    const Frag b = pack(reinterpret_cast<const float*>(&x[2]));
    x[0] = __builtin_bit_cast(f32x4, a.u);
    x[1] = __builtin_bit_cast(f32x4, b.u);
  }
  __device__ __forceinline__ static Frag p_frag(const f32x4 (&x)[4], int u) {
    Frag f;
    f.u = __builtin_bit_cast(uint4, x[u]);
    return f;
  }
  __device__ __forceinline__ static f32x4 load4(const void* src) {
    const uint2 w = *reinterpret_cast<const uint2*>(src);
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                 __uint_as_float(w.y & 0xffff0000u)};
  }
};

template <> struct Tr<HS_F32> {
  static constexpr int ES = 4;
  struct Frag { float4 a, b; };
  __device__ __forceinline__ static Frag ld(const void* p) {
    Frag f;
    f.a = reinterpret_cast<const float4*>(p)[0];
    f.b = reinterpret_cast<const float4*>(p)[1];
    return f;
  }
  __device__ __forceinline__ static Frag zero() {
    Frag f;
    f.a = make_float4(0.f, 0.f, 0.f, 0.f);
    f.b = f.a;
    return f;
  }
  __device__ __forceinline__ static Frag keep(Frag f, int n) {
    float v[8] = {f.a.x, f.a.y, f.a.z, f.a.w, f.b.x, f.b.y, f.b.z, f.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i >= n) v[i] = 0.f;
    f.a = make_float4(v[0], v[1], v[2], v[3]);
    f.b = make_float4(v[4], v[5], v[6], v[7]);
    return f;
  }
  __device__ __forceinline__ static void mma(f32x4& acc, const Frag& a, const Frag& b) {
    // k-slot 8q+e of the 32-wide step is fed as k = q of sub-step e
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.x, b.a.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.y, b.a.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.z, b.a.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.w, b.a.w, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.x, b.b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.y, b.b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.z, b.b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.w, b.b.w, acc, 0, 0, 0);
  }
  __device__ __forceinline__ static Frag pack(const float* p) {
    Frag f;
    f.a = make_float4(p[0], p[1], p[2], p[3]);
    f.b = make_float4(p[4], p[5], p[6], p[7]);
    return f;
  }
  __device__ __forceinline__ static void store4(void* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
  }
  __device__ __forceinline__ static Frag ones() {
    Frag f;
    f.a = make_float4(1.f, 1.f, 1.f, 1.f);
    f.b = f.a;
    return f;
  }
  // fp32 P fragments are the probabilities themselves
  __device__ __forceinline__ static void pack_p(f32x4 (&)[4]) {}
  __device__ __forceinline__ static Frag p_frag(const f32x4 (&x)[4], int u) {
    Frag f;
    f.a = make_float4(x[2 * u][0], x[2 * u][1], x[2 * u][2], x[2 * u][3]);
    f.b = make_float4(x[2 * u + 1][0], x[2 * u + 1][1], x[2 * u + 1][2], x[2 * u + 1][3]);
    return f;
  }
  __device__ __forceinline__ static f32x4 load4(const void* src) {
    const float4 v = *reinterpret_cast<const float4*>(src);
    return f32x4{v.x, v.y, v.z, v.w};
  }
};

// ---------------------------------------------------------- fp8 e4m3 caches
// v_cvt_pk_f32_fp8 decodes OCP e4m3fn exactly on gfx950 (every code checked
// against an independent table); e4m3 values are exact in bf16, so a decoded
// code feeds the bf16 MFMA without rounding.
typedef __attribute__((ext_vector_type(2))) float f32x2;

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16x2(uint32_t w) {
  const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return bf16x2_bits(f[0], f[1]);
}

// 8 fp8 codes (byte e = element e) -> bf16 fragment of 8 elements
__device__ __forceinline__ Tr<HS_BF16>::Frag fp8x8_frag(uint2 c) {
  Tr<HS_BF16>::Frag f;
  f.u = make_uint4(fp8x2_bf16x2<false>(c.x), fp8x2_bf16x2<true>(c.x), fp8x2_bf16x2<false>(c.y),
                   fp8x2_bf16x2<true>(c.y));
  return f;
}

// Value fragments from a position-major fp8 cache.  Lane (q, r) of key step u
// loads the dword w[e] = V[key0 + e][dbase + 4r .. +3] of 8 consecutive keys
// (key0 = kbase + 32u + 8q).  A 4x4 byte transpose of w[0..3] and of w[4..7]
// yields, for k = 0..3, the 8 codes of head_dim row dbase + 4r + k over the 8
// keys: the A fragment of O^T row chunk mc = 4*(dbase/64) + k, whose row r is
// head_dim dbase + 4r + k (a permuted head_dim order, undone when storing).
__device__ __forceinline__ void fp8_vfrag4(const uint32_t* w, Tr<HS_BF16>::Frag* out) {
  uint32_t t[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w0 = w[4 * h], w1 = w[4 * h + 1], w2 = w[4 * h + 2], w3 = w[4 * h + 3];
    const uint32_t p = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // w0.0 w1.0 w0.1 w1.1
    const uint32_t q = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // w0.2 w1.2 w0.3 w1.3
    const uint32_t r = __builtin_amdgcn_perm(w3, w2, 0x05010400u);  // w2.0 w3.0 w2.1 w3.1
    const uint32_t s = __builtin_amdgcn_perm(w3, w2, 0x07030602u);  // w2.2 w3.2 w2.3 w3.3
    t[h][0] = __builtin_amdgcn_perm(r, p, 0x05040100u);  // byte 0 of w0..w3
    t[h][1] = __builtin_amdgcn_perm(r, p, 0x07060302u);  // byte 1
    t[h][2] = __builtin_amdgcn_perm(s, q, 0x05040100u);  // byte 2
    t[h][3] = __builtin_amdgcn_perm(s, q, 0x07060302u);  // byte 3
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = fp8x8_frag(make_uint2(t[0][k], t[1][k]));
}

// head_dim index held in row m of O^T chunk mc under the fp8 value order
__host__ __device__ __forceinline__ int fp8_vrow_d(int mc, int m) {
  return 64 * (mc >> 2) + 4 * m + (mc & 3);
}

// ------------------------------------------------------ LDS tile staging
// A 64-key tile (K rows + the matching [D][64] value tile) staged through LDS
// by NTHR threads: `gload` issues the global loads into registers, `sstore`
// writes them to one LDS buffer.  K rows are stored in S^T row order
// (tile_row).  Both tiles are unpadded; the 16-byte chunk c of row r is
// stored at chunk c ^ (r & SW), SW = min(chunks per row, 16) - 1.  Measured
// with the LDS bank-conflict counter on gfx950, this swizzle makes the
// fragment reads (16 rows x 4 chunks per wavefront) conflict-free, whereas
// padded row strides of 272 and 144 bytes conflict.  Keys at or after `nk`
// read as zero.
template <int DT, int D, int NTHR>
struct TileStage {
  using T = Tr<DT>;
  using Frag = typename T::Frag;
  static constexpr int ES = T::ES;
  static constexpr int KCH = D * ES / 16;   // 16-byte chunks per K row
  static constexpr int VCH = 64 * ES / 16;  // chunks per value row
  static constexpr int KS = D * ES;
  static constexpr int VS = 64 * ES;
  static constexpr int KSW = (KCH < 16 ? KCH : 16) - 1;
  static constexpr int VSW = (VCH < 16 ? VCH : 16) - 1;
  static constexpr int KB = 64 * KS;
  static constexpr int VB = D * VS;
  static constexpr int BYTES = KB + VB;
  static constexpr int NK = 64 * KCH / NTHR;
  static constexpr int NV = D * VCH / NTHR;
  static_assert(NK * NTHR == 64 * KCH && NV * NTHR == D * VCH, "tile does not split evenly");
  uint4 kr[NK], vr[NV];

  __device__ __forceinline__ static int k_lds(int row, int chunk) {
    return row * KS + ((chunk ^ (row & KSW)) << 4);
  }
  __device__ __forceinline__ static int v_lds(int row, int chunk) {
    return KB + row * VS + ((chunk ^ (row & VSW)) << 4);
  }

  // krows: key row 0 of the tile (row stride D elements); vslab: [D][64] tile;
  // nk: number of valid keys in the tile (>= 64 means all).  Key rows beyond
  // nk are not read; value columns beyond nk are zeroed in sstore, after the
  // data has arrived, so no wait is forced here.
  int nk_;
  __device__ __forceinline__ void gload(const char* krows, const char* vslab, int nk) {
    nk_ = nk;
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      const int ci = threadIdx.x + NTHR * n;
      const int kk = ci / KCH, col = ci % KCH;
      kr[n] = kk < nk ? *(const uint4*)(krows + kk * KS + col * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int ci = threadIdx.x + NTHR * n;
      const int dd = ci / VCH, col = ci % VCH;
      vr[n] = *(const uint4*)(vslab + dd * VS + col * 16);
    }
  }
  __device__ __forceinline__ void sstore(char* buf) {
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      const int ci = threadIdx.x + NTHR * n;
      *(uint4*)(buf + k_lds(tile_row(ci / KCH), ci % KCH)) = kr[n];
    }
    if (nk_ < 64) {  // uniform: only a ragged last tile
      constexpr int EPW = 4 / ES;  // elements per 32-bit word
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const int ci = threadIdx.x + NTHR * n;
        const int k0 = (ci % VCH) * (16 / ES);
        uint32_t w[4] = {vr[n].x, vr[n].y, vr[n].z, vr[n].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = nk_ - (k0 + EPW * i);  // valid elements left from this word on
          const uint32_t msk = r >= EPW ? 0xffffffffu : (r == 1 && EPW == 2 ? 0xffffu : 0u);
          w[i] &= msk;
        }
        vr[n] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int ci = threadIdx.x + NTHR * n;
      *(uint4*)(buf + v_lds(ci / VCH, ci % VCH)) = vr[n];
    }
  }
  // ---- direct global -> LDS staging (global_load_lds_dwordx4) ----------
  // A wave instruction writes 1 KiB of LDS: lane l's 16 bytes land at
  // base + 16 l.  Chunk q (1 KiB) of the tile goes to wave q % NW as its
  // instruction q / NW; each lane fetches the 16 source bytes that belong at
  // its LDS position under the row map and the chunk swizzle above.  Key rows
  // past the valid count are clamped to the last valid row (their logits are
  // masked); value columns past it are zeroed in LDS by dma_fix.
  static constexpr int NWV = NTHR / 64;
  static constexpr int NDMA = BYTES / 1024 / NWV;
  static_assert(NDMA * NWV * 1024 == BYTES && (KB / 1024) % NWV == 0, "tile does not split into wave chunks");
  static constexpr int NDK = KB / 1024 / NWV;  // instructions 0..NDK-1 are key rows
  int dkey[NDK > 0 ? NDK : 1];
  uint32_t doff[NDMA];  // source byte offset in the tile (key rows: of the unclamped row)
  __device__ __forceinline__ void dma_init() {
    const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int off = (w + NWV * n) * 1024 + 16 * lane;
      if (n < NDK) {
        const int r = off / KS, c = ((off % KS) >> 4) ^ (r & KSW);
        dkey[n] = tile_key(r >> 4, r & 15);
        doff[n] = dkey[n] * KS + c * 16;
      } else {
        const int v = off - KB, dd = v / VS, c = ((v % VS) >> 4) ^ (dd & VSW);
        doff[n] = dd * VS + c * 16;
      }
    }
  }
  // krows, vslab and nk must be wave-uniform.  The wave index is made
  // wave-uniform too, so each transfer's LDS destination (M0) is scalar
  // arithmetic instead of a vector add and a readfirstlane.
  __device__ __forceinline__ void dma(char* buf, const char* krows, const char* vslab, int nk) {
    nk_ = nk;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // (the source pointer goes through a named variable: passing the
    // conditional expression straight to the builtin makes the host pass of
    // this compiler drop the launch stubs of some kernel instantiations)
    if (nk >= 64) {  // whole tile: scalar base + per-lane offset
#pragma unroll
      for (int n = 0; n < NDMA; ++n) {
        const char* src = n < NDK ? krows + doff[n] : vslab + doff[n];
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(buf + (w + NWV * n) * 1024),
                                         16, 0, 0);
      }
    } else {  // ragged last tile: key rows past nk read row nk-1 instead
#pragma unroll
      for (int n = 0; n < NDMA; ++n) {
        const int kk = dkey[n < NDK ? n : 0];
        const char* src = n < NDK ? krows + (doff[n] - (uint32_t)((kk - min(kk, nk - 1)) * KS)) : vslab + doff[n];
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(buf + (w + NWV * n) * 1024),
                                         16, 0, 0);
      }
    }
  }
  // after this wave's transfers have landed (vmcnt 0): zero the value
  // columns past the valid count in the chunks this lane fetched
  __device__ __forceinline__ void dma_fix(char* buf) const {
    if (nk_ >= 64) return;  // uniform
    const int lane = lane_id(), w = threadIdx.x >> 6;
    constexpr int EPW = 4 / ES;
#pragma unroll
    for (int n = NDK; n < NDMA; ++n) {
      const int k0 = (((int)doff[n] % VS) >> 4) * (16 / ES);
      if (k0 + 16 / ES > nk_) {
        uint4* p = (uint4*)(buf + (w + NWV * n) * 1024 + 16 * lane);
        const uint4 x = *p;
        uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = nk_ - (k0 + EPW * i);
          wd[i] &= r >= EPW ? 0xffffffffu : (r == 1 && EPW == 2 ? 0xffffu : 0u);
        }
        *p = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    }
  }

  // A fragment of S^T chunk c, k-step ks: row 16c + r, elements 32ks + 8q .. +7
  __device__ __forceinline__ static Frag ldK(const char* buf, int c, int ks) {
    const int lane = lane_id();
    const int row = 16 * c + (lane & 15);
    const int ch = (32 * ks + 8 * (lane >> 4)) * ES / 16;
    if constexpr (ES == 2) {
      return T::ld(buf + k_lds(row, ch));
    } else {
      Frag f;
      f.a = *(const float4*)(buf + k_lds(row, ch));
      f.b = *(const float4*)(buf + k_lds(row, ch + 1));
      return f;
    }
  }
  // A fragment of O^T chunk mc, key step u: value row 16mc + r, keys 32u + 8q .. +7
  __device__ __forceinline__ static Frag ldV(const char* buf, int u, int mc) {
    const int lane = lane_id();
    const int row = 16 * mc + (lane & 15);
    const int ch = (32 * u + 8 * (lane >> 4)) * ES / 16;
    if constexpr (ES == 2) {
      return T::ld(buf + v_lds(row, ch));
    } else {
      Frag f;
      f.a = *(const float4*)(buf + v_lds(row, ch));
      f.b = *(const float4*)(buf + v_lds(row, ch + 1));
      return f;
    }
  }
};

// ------------------------------------------------------------- the engine
// One wavefront, NT column tiles of 16 query columns each, head_dim D.
// Online softmax state per column tile: running maximum m (log2 units, already
// scaled), the denominator, and O^T accumulators (o[nt][mc]: head_dim rows
// 16*mc + 4q .. +3 of the lane's column).  The denominator is a per-lane
// partial sum l of the fp32 probabilities, or, with LSUM, a column sum lacc
// that the matrix unit accumulates from the packed P against an all-ones
// fragment (two extra MFMAs per tile and column tile instead of 16 VALU adds
// per lane; numerator and denominator then use the same rounded P).
// softmax's `act` carries one bit per column tile; a clear bit (no live key
// in the tile for any of its columns, wave-uniform) skips that tile's
// softmax and sets its P to 0.
template <int DT, int D, int NT, bool LSUM = false>
struct WaveAttn {
  using T = Tr<DT>;
  using Frag = typename T::Frag;
  static constexpr int NS = D / 32;  // k-steps of S^T = K Q^T
  static constexpr int NM = D / 16;  // row chunks of O^T
  static constexpr unsigned kAll = (1u << NT) - 1;

  Frag qf[NT][NS];
  f32x4 o[NT][NM];
  f32x4 lacc[LSUM ? NT : 1];
  float m[NT], l[NT];

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m[nt] = kNegBig;
      l[nt] = 0.f;
      if (LSUM) lacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mc = 0; mc < NM; ++mc) o[nt][mc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  struct NoHook {
    __device__ __forceinline__ void operator()(int, const float*) const {}
  };

  // Issue order for NR operand fragments read from LDS, each used by NPER
  // matrix products (plus NTAIL more products at the end): the first LA reads,
  // then one read after every NPER products, so LA reads stay in flight ahead
  // of the products that need them.  Left to itself the compiler keeps about
  // one read in flight and waits for it before every few products.  LA = 0
  // leaves the order to the compiler (operands already in registers).
  template <int LA, int NR, int NPER, int NTAIL>
  __device__ __forceinline__ static void lds_mfma_order() {
    if constexpr (LA > 0) {
      __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);  // LDS reads
#pragma unroll
      for (int i = 0; i < NR - LA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, NPER, 0);  // matrix products
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NPER * LA + NTAIL, 0);
    }
  }

  // S^T of one 64-key tile: s[nt][c] (rows = keys tile_key(c, 4q+i), column = lane's).
  // LA > 0: ldK reads LDS, ordered by lds_mfma_order.
  template <int LA = 0, class LK>
  __device__ __forceinline__ void qk(const LK& ldK, f32x4 (&s)[NT][4]) const {
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const Frag a = ldK(c, ks);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (ks == 0) s[nt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
          T::mma(s[nt][c], a, qf[nt][ks]);
        }
      }
    }
    lds_mfma_order<LA, 4 * NS, NT, 0>();
  }

  // Online-softmax update with the logits s of a tile, then O += P V.
  // `hook(nt, x)` sees the lane's 16 masked, scaled logits (log2 units; x[4c+i]
  // belongs to key kbase + tile_key(c, 4q+i)) before the exponentials; those
  // of a switched-off column are not masked.
  // Masking is decided per wavefront: a column with lo == kNoKey is switched
  // off (its maximum and exponent offset are replaced, two selects per lane);
  // key-by-key range checks only when some live column's [lo, hi] does not
  // cover the whole tile.
  template <bool MASK, bool WANT_SUM, class HK = NoHook>
  __device__ __forceinline__ void softmax(f32x4 (&s)[NT][4], int kbase, const int* lo, const int* hi, float sc2,
                                          float* bmax, float* bsum, const HK& hook = HK(), unsigned act = kAll) {
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
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (!((act >> nt) & 1u)) {  // no live key for this column tile: P = 0
        bmax[nt] = -INFINITY;
        if (WANT_SUM) bsum[nt] = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) s[nt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        continue;
      }
      // masking, exponentials and packing work in place on the logits
      f32x4(&x)[4] = s[nt];
      const bool en = !MASK || lo[nt] != kNoKey;
      if (MASK && ranged) {
        // the lane's keys are kbase + 8*(lane/16) + k, k = 32(c/2) + 4(c%2) + i
        const int base = kbase + 8 * (lane >> 4);
        const int klo = en ? lo[nt] - base : 64;
        const int khi = hi[nt] - base;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = 32 * (c >> 1) + 4 * (c & 1) + i;
            x[c][i] = (k < klo || k > khi) ? -INFINITY : x[c][i];
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[c][i]);
      // a switched-off column (lo == kNoKey) keeps its raw logits; its maximum
      // is -inf and its exponentials are forced to 0 below
      if (MASK && off) mx = en ? mx : -INFINITY;
      if constexpr (!__is_same(HK, NoHook)) {
        float xs[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) xs[e] = x[e >> 2][e & 3] * sc2;
        hook(nt, xs);
      }
      mx = xlane_max(mx) * sc2;  // raw logits are unscaled; sc2 > 0
      bmax[nt] = mx;
      // The running maximum is only raised when the tile exceeds it by more
      // than kSlack (log2 units): the exponentials then stay <= 2^kSlack, exact
      // enough in fp32 and bf16, and the O rescale is rare.  m + log2(l) is
      // the LSE whichever maximum is kept.
      const bool up = mx > m[nt] + kSlack;
      const float mn = up ? mx : m[nt];
      const float alpha = up ? fast_exp2(m[nt] - mn) : 1.f;
      m[nt] = mn;
      const float nmn = (MASK && off && !en) ? -INFINITY : -mn;
      float ps = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[c][i] = fast_exp2(__builtin_fmaf(x[c][i], sc2, nmn));
          if (!LSUM || WANT_SUM) ps = (c | i) ? ps + x[c][i] : x[c][i];  // no 0 + x
        }
      if (!LSUM) l[nt] = l[nt] * alpha + ps;
      if (WANT_SUM) bsum[nt] = xlane_sum(ps);
      T::pack_p(x);
      if (__ballot(up) != 0ull) {
#pragma unroll
        for (int mc = 0; mc < NM; ++mc) o[nt][mc] *= alpha;
        if (LSUM) lacc[nt] *= alpha;
      }
    }
  }

  // O += P V with the P fragments that softmax left in s.
  // LA > 0: ldV reads LDS, ordered by lds_mfma_order.
  template <int LA = 0, class LV>
  __device__ __forceinline__ void pv(const f32x4 (&s)[NT][4], const LV& ldV) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int mc = 0; mc < NM; ++mc) {
        const Frag a = ldV(u, mc);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) T::mma(o[nt][mc], a, T::p_frag(s[nt], u));
      }
      if (LSUM) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) T::mma(lacc[nt], T::ones(), T::p_frag(s[nt], u));
      }
    }
    lds_mfma_order<LA, 2 * NM, NT, LSUM ? 2 * NT : 0>();
  }

  template <bool MASK, bool WANT_SUM, class LV, class HK = NoHook>
  __device__ __forceinline__ void softmax_pv(f32x4 (&s)[NT][4], const LV& ldV, int kbase, const int* lo,
                                             const int* hi, float sc2, float* bmax, float* bsum,
                                             const HK& hook = HK()) {
    softmax<MASK, WANT_SUM>(s, kbase, lo, hi, sc2, bmax, bsum, hook);
    pv(s, ldV);
  }

  // One whole 64-key tile whose first key has absolute index kbase.
  //   ldK(c, s)  -> A fragment of S^T chunk c, k-step s (key kbase+tile_key(c, r))
  //   ldV(u, mc) -> A fragment of O^T chunk mc, key step u (keys kbase+32u+8q..+7)
  //   lo[nt], hi[nt]: inclusive absolute key range valid for the lane's column
  //   (lo = kNoKey disables the column for this tile); sc2 = scale * log2(e).
  // Outputs per column tile: bmax = max scaled logit of the tile (log2 units,
  // -inf when no key is valid) and, when WANT_SUM, bsum = sum over the tile of
  // exp2(logit - m_new) (m_new = running max after this tile).
  template <bool MASK, bool WANT_SUM, class LK, class LV, class HK = NoHook>
  __device__ __forceinline__ void tile(const LK& ldK, const LV& ldV, int kbase, const int* lo,
                                       const int* hi, float sc2, float* bmax, float* bsum,
                                       const HK& hook = HK()) {
    f32x4 s[NT][4];
    qk(ldK, s);
    softmax_pv<MASK, WANT_SUM>(s, ldV, kbase, lo, hi, sc2, bmax, bsum, hook);
  }

  // Column totals: 1/l (0 when the column saw no key) and the log2-domain LSE.
  // sink2: an extra logit with no value (log2 units; -inf: none) joins the
  // maximum and the denominator, so inv_l also carries the o rescale.
  __device__ __forceinline__ void finish(int nt, float& inv_l, float& lse2, float sink2 = -INFINITY) const {
    float lt = LSUM ? lacc[nt][0] : xlane_sum(l[nt]);
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

// ------------------------------------------------ prefill work-group order
// LDS fragment reads kept in flight ahead of the matrix products that use
// them (WaveAttn::lds_mfma_order), per kernel: the deepest that measured
// fastest without register spills (full layer: 4 spills at 4, about 1 %
// faster; sparse layer: 6, 7 % faster than the compiler's own order)
constexpr int kFullLA = 3;
constexpr int kSparseLA = 6;

// Work-group order for position-block kernels: block id i takes kv group
// (sequence, group) bg = i % nbg and the rank-th latest position block, rank
// = i / nbg.  Consecutive ids are dealt round-robin over the 8 XCDs, so with
// nbg a multiple of 8 each XCD keeps to nbg/8 kv groups (their K/V stays in
// its L2); with fewer groups a group's position blocks alternate over several
// XCDs, and every XCD gets late (long) and early (short) blocks alike.  Each
// XCD starts with the latest blocks.
struct WgSlot {
  int bg, pblk;
  bool live;
};
__device__ __forceinline__ WgSlot wg_slot(int nbg, int npblk) {
  const int i = blockIdx.x;
  const int rank = i / nbg;
  WgSlot w;
  w.bg = i % nbg;
  w.live = rank < npblk;
  w.pblk = w.live ? npblk - 1 - rank : 0;
  return w;
}

}  // namespace hs
