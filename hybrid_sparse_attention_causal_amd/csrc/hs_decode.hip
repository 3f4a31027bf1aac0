// hs_decode.hip -- decode kernels of the hybrid block on gfx950 (one new query
// token per sequence; the query sits at position L-1 of an L-token context).
//
//  decode_full_kernel     split-K full attention over the cache: every wave
//                         streams one chunk of 64-key tiles for the G query heads
//                         of a kv group, emits the block scores (or, in the
//                         token-level variant, every token's logit) and a
//                         partial (m, l, o) (HySparse explainer 3.4.1; HySparse2
//                         explainer, decode_one_token: causal_scores(q, K))
//  decode_combine_kernel  merges the partials into o and LSE
//  token_*_kernel         token-level selection (HySparse2 explainer,
//                         decode_one_token): order keys and a level-1
//                         histogram, a level-2 histogram, candidate compaction,
//                         the exact pick
//  decode_sparse_kernel   one sparse layer: the selected blocks of the shared
//                         cache plus the layer's own window ring, merged by the
//                         sigmoid gates (explainer 3.4.3)
//  decode_sparse_token_kernel + decode_token_combine_kernel
//                         one token-level sparse layer over gathered fp8 rows
#include <type_traits>

#include "hs_device.h"
#include "hs_internal.h"
#include "hs_sel_list.h"

namespace hs {

// head_dim order of the QK^T operands from a position-major fp8 cache: lane
// group q = lane/16 holds, at k-step ks, head_dim (D/4) q + 8 ks .. +7, so a
// lane's keys over all k-steps are one contiguous D/4-byte run of the row
// (16-byte loads, two k-steps each) and every load touches 64 bytes of each
// of its 16 rows.  The queries are read in the same order; the dot products
// are the same sums.
template <int D>
__device__ __forceinline__ int fp8_kdim(int lane, int ks) {
  return (D / 4) * (lane >> 4) + 8 * ks;
}
// the 8 bytes of k-step 2j + hi from a 16-byte load
__device__ __forceinline__ uint2 half_u4(uint4 v, int hi) {
  return hi ? make_uint2(v.z, v.w) : make_uint2(v.x, v.y);
}

// Value rows from a position-major fp8 cache: lane (q, r) of key step u loads
// the D/16 bytes V[key0 + e][(D/16) r ..] of 8 consecutive keys (key0 =
// kbase + 32u + 8q), one load per key: 16 lanes cover a whole row.  A 4x4
// byte transpose of each dword column (fp8_vfrag4) gives the A fragments of
// O^T row chunks mc = 4h + k (h: which dword), whose row m is head_dim
// fp8_vrow_dv(mc, m); that order is undone when storing.
template <int D>
using Fp8VRow = std::conditional_t<D == 128, uint2, uint32_t>;
template <int D>
__host__ __device__ __forceinline__ int fp8_vrow_dv(int mc, int m) {
  return (D / 16) * m + 4 * (mc >> 2) + (mc & 3);
}
// the 4 fragments of chunks 4h .. 4h+3 from the 8 keys' rows
template <int D>
__device__ __forceinline__ void fp8_vfrag4_rows(const Fp8VRow<D> (&v)[8], int h, Tr<HS_BF16>::Frag* out) {
  uint32_t w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (D == 128) w[e] = h ? v[e].y : v[e].x;
    else w[e] = v[e];
  }
  fp8_vfrag4(w, out);
}

// Maximum over the 16 lanes of a row for 16 values at once, scattered: lane
// i of the row returns max over the row of v[i].  Four exchange steps halve
// the values a lane holds, each lane keeping the half whose next index bit
// matches its own (partners: row mirror, half-row mirror, then swaps within
// quads; each flips that bit and keeps the bits already settled): 15 moves
// instead of 16 full reductions of 4 moves each.
__device__ __forceinline__ float row16_max_scatter(const float (&v)[16], int i) {
#define HS_DPP_MOVE(x, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false))
  float w8[8], w4[4], w2[2];
  const bool b3 = i & 8, b2 = i & 4, b1 = i & 2, b0 = i & 1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float keep = b3 ? v[8 + e] : v[e], send = b3 ? v[e] : v[8 + e];
    w8[e] = max2(keep, HS_DPP_MOVE(send, 0x140));  // row mirror: lane 15 - i
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float keep = b2 ? w8[4 + e] : w8[e], send = b2 ? w8[e] : w8[4 + e];
    w4[e] = max2(keep, HS_DPP_MOVE(send, 0x141));  // half-row mirror: lane i ^ 7
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float keep = b1 ? w4[2 + e] : w4[e], send = b1 ? w4[e] : w4[2 + e];
    w2[e] = max2(keep, HS_DPP_MOVE(send, 0x4E));  // lane i ^ 2
  }
  const float keep = b0 ? w2[1] : w2[0], send = b0 ? w2[0] : w2[1];
  return max2(keep, HS_DPP_MOVE(send, 0xB1));  // lane i ^ 1
#undef HS_DPP_MOVE
}

// ======================================================== split-K full layer
// Unit (b, g, ch) covers keys [ch*CH*64, min(L, (ch+1)*CH*64)), CH =
// ch_blocks (16 or 32 tiles, chosen by the host).  MFMA columns
// 0..G-1 are the G query heads of kv group g (G <= 16).
// KV = HS_BF16: key cache [C][D] and block-major value cache [C/64][D][64];
// KV = HS_FP8_E4M3: position-major fp8 key and value caches [C][D] with one
// scale per (K|V, kv head); the value fragments are byte-transposed in
// registers (fp8_vfrag4), so their head_dim rows come in fp8_vrow_d order.
template <int D, int TOKEN, int KV>
__global__ __launch_bounds__(256, KV == HS_FP8_E4M3 ? 3 : 2) void decode_full_kernel(DecodeFullArgs a) {
  using Tt = Tr<HS_BF16>;
  using Frag = Tt::Frag;
  using Eng = WaveAttn<HS_BF16, D, 1>;
  constexpr int KES = KV == HS_FP8_E4M3 ? 1 : 2;  // cache bytes per element
  // bounds (TOKEN == 2): each wave's z and offsets of its chunk are gathered
  // here and written out when the chunk ends, in wide contiguous stores
  // instead of small stores interleaved with the cache reads
  __shared__ __attribute__((aligned(16))) float zst[TOKEN == 2 ? 4 * kDecodeChunkBlocksMax * 64 : 1];
  __shared__ float ast[TOKEN == 2 ? 4 * kDecodeChunkBlocksMax * 16 : 1];
  const int lane = threadIdx.x & 63;
  const int span = a.ch_blocks * 64;  // ch_blocks <= kDecodeChunkBlocksMax
  // Wave id -> live unit: sequence b owns Hkv * ceil(L_b / span) consecutive
  // ids in (b, g, ch) order, found by a wave prefix over the lengths.  The
  // grid is sized for full caches; the ids past the live total exit at the
  // end of the grid.  Numbering only live units keeps consecutive work groups
  // busy, so the round-robin placement over the XCDs stays even whatever the
  // length mix (numbering every (b, g, ch) and skipping dead ones leaves the
  // low XCDs with the long sequences' extra chunks).  Unit, sequence and
  // length are wave-uniform; saying so keeps the tile loop a scalar loop.
  const int id = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int b = -1, base = 0, nchb = 1;
  for (int b0 = 0, carry = 0; b0 < a.B; b0 += 64) {
    const int bl = b0 + lane;
    const int cnt = bl < a.B ? a.Hkv * ((ctx_len(a.lens, bl, a.C) + span - 1) / span) : 0;
    int inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    const int ex = carry + inc - cnt;
    const unsigned long long hit = __ballot(cnt > 0 && id >= ex && id < ex + cnt);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      b = b0 + src;
      base = __shfl(ex, src);
      nchb = __shfl(cnt, src) / a.Hkv;
      break;
    }
    carry += __shfl(inc, 63);
  }
  b = __builtin_amdgcn_readfirstlane(b);
  if (b < 0) return;
  base = __builtin_amdgcn_readfirstlane(base);
  nchb = __builtin_amdgcn_readfirstlane(nchb);
  const int g = (id - base) / nchb, ch = (id - base) % nchb;
  const int L = __builtin_amdgcn_readfirstlane(ctx_len(a.lens, b, a.C));
  const int kstart = ch * span;
  const int kend = min(L, kstart + span);
  const int G = a.Hq / a.Hkv;
  const int col = lane & 15;
  const int r16 = lane & 15, q8 = 8 * (lane >> 4);
  const int q4 = (lane >> 4) << 2;
  const int h = g * G + col;
  const float sk = KV == HS_FP8_E4M3 ? a.kv_scale[g] : 1.f;
  const float sv = KV == HS_FP8_E4M3 ? a.kv_scale[a.Hkv + g] : 1.f;
  const float sc2 = a.sc2 * sk;

  Eng eng;
  eng.reset();
  int lo[1], hi[1];
  lo[0] = col < G ? 0 : kNoKey;
  hi[0] = L - 1;
  // unconditional loads (columns past G read head g*G and are zeroed): a
  // load under a branch would make the compiler drain every later wait.
  // The fp8 path takes head_dim in the order of fp8_kdim (keys and queries
  // alike, so the logits are unchanged).
#pragma unroll
  for (int ks = 0; ks < Eng::NS; ++ks) {
    const int dq = KV == HS_FP8_E4M3 ? fp8_kdim<D>(lane, ks) : 32 * ks + q8;
    const Frag f = Tt::ld((const char*)a.q + ((size_t)(b * a.Hq + (col < G ? h : g * G)) * D + dq) * 2);
    eng.qf[0][ks] = col < G ? f : Tt::zero();
  }
  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * a.C * D * KES;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * a.C * D * KES;
  float* rawrow = TOKEN == 2 ? nullptr : a.raw + (size_t)(b * a.Hq + h) * (TOKEN ? a.C : a.C / 64);

  // Raw fragments of one tile: bf16: 16 K and 16 V fragments of 16 bytes;
  // fp8: 4 x D/64 K loads of 16 bytes (two fragments each) and 2x(D/64)x8
  // value dwords (decoded at use).  The key and value halves of a tile are separate register sets, so
  // the next tile's keys load while this tile's values are still in flight
  // and consumed, and its values load during the next tile's QK^T.
  constexpr bool F8 = KV == HS_FP8_E4M3;
  struct RawKB {
    uint4 k[4][Eng::NS];
  };
  struct RawK8 {
    uint4 k8[4][Eng::NS / 2];
  };
  struct RawVB {
    uint4 v[2][Eng::NM];
  };
  struct RawV8 {
    Fp8VRow<D> v8[2][8];
  };
  using RawK = std::conditional_t<F8, RawK8, RawKB>;
  using RawV = std::conditional_t<F8, RawV8, RawVB>;
  // Every load is unconditional: the capacity C is a multiple of 64, so a
  // tile's rows all lie inside the cache even past L.  Keys at or past L are
  // masked out of the logits by selects; values there are zeroed, since
  // P = 0 times a stale non-finite value would not vanish.
  auto loadK = [&](int kb0, RawK& r) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int key = kb0 + tile_key(c, r16);
      if constexpr (F8) {
#pragma unroll
        for (int j = 0; j < Eng::NS / 2; ++j)
          r.k8[c][j] = *(const uint4*)(kg + (size_t)key * D + fp8_kdim<D>(lane, 2 * j));
      } else {
#pragma unroll
        for (int ks = 0; ks < Eng::NS; ++ks)
          r.k[c][ks] = *(const uint4*)(kg + ((size_t)key * D + 32 * ks + q8) * 2);
      }
    }
  };
  auto loadV = [&](int kb0, RawV& r) {
    const int j = kb0 >> 6;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int key0 = kb0 + 32 * u + q8;
      if constexpr (F8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) r.v8[u][e] = *(const Fp8VRow<D>*)(vg + (size_t)(key0 + e) * D + (D / 16) * r16);
      } else {
#pragma unroll
        for (int mc = 0; mc < Eng::NM; ++mc)
          r.v[u][mc] = *(const uint4*)(vg + (((size_t)j * D + 16 * mc + r16) * 64 + 32 * u + q8) * 2);
      }
    }
  };
  // zero the value entries of keys >= L (last tile of a sequence only)
  auto clipV = [&](int kb0, RawV& r) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int key0 = kb0 + 32 * u + q8;
      if constexpr (F8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) r.v8[u][e] = key0 + e < L ? r.v8[u][e] : Fp8VRow<D>{};
      } else {
#pragma unroll
        for (int mc = 0; mc < Eng::NM; ++mc) {
          Frag f;
          f.u = r.v[u][mc];
          r.v[u][mc] = Tt::keep(f, L - key0).u;
        }
      }
    }
  };
  float bkeep[kDecodeChunkBlocksMax / 4];
#pragma unroll
  for (int r = 0; r < kDecodeChunkBlocksMax / 4; ++r) bkeep[r] = -INFINITY;
  RawK rk;
  RawV rv;
  // One tile: QK^T on the keys in rk, the keys of tile nx are requested,
  // softmax, PV with the values in rv, the values of tile nx are requested
  // (no requests when `more` is false: the last tile).
  auto body = [&](int kb0, int nx, auto more) {
    constexpr bool MORE = decltype(more)::value;
    const int j = kb0 >> 6;
    auto ldK = [&](int c, int ks) {
      if constexpr (F8) {
        return fp8x8_frag(half_u4(rk.k8[c][ks >> 1], ks & 1));
      } else {
        Frag f;
        f.u = rk.k[c][ks];
        return f;
      }
    };
    Frag vc[4];
    auto ldV = [&](int u, int mc) {
      if constexpr (F8) {
        if ((mc & 3) == 0) fp8_vfrag4_rows<D>(rv.v8[u], mc >> 2, vc);
        return vc[mc & 3];
      } else {
        Frag f;
        f.u = rv.v[u][mc];
        return f;
      }
    };
    f32x4 s[1][4];
    eng.qk(ldK, s);
    if constexpr (MORE) loadK(nx, rk);
    float bmax[1], bsum[1];
    if constexpr (TOKEN == 2) {
      // Selection bounds instead of logits.  The tile's offset per head is the
      // chunk's LSE over its earlier tiles (m + log2 l of the running state,
      // before this tile joins it), or the tile's own maximum for the
      // chunk's first tile; z of a key is the maximum over the group's heads
      // of (logit - offset).  With the heads' final LSEs, every token's score
      // max_h (logit - LSE_h) then lies in [z - max_h d_h, z - min_h d_h],
      // d_h = LSE_h - offset_h.
      auto hook = [&](int, const float* x) {
        float off;
        if (kb0 == kstart) {
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = max2(mx, x[e]);
          off = xlane_max(mx);
        } else {
          off = eng.m[0] + fast_log2(xlane_sum(eng.l[0]));
        }
        // x[e] is the logit of key tile_key(e / 4, q4 + e % 4); lane (q, i)
        // ends up with z of e = i, and the wave stores the tile's 64 z in one
        // instruction
        float xm[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) xm[e] = col < G ? x[e] - off : -INFINITY;
        const float z = row16_max_scatter(xm, col);
        const int slot = (threadIdx.x >> 6) * kDecodeChunkBlocksMax + ((kb0 - kstart) >> 6);
        zst[slot * 64 + tile_key(col >> 2, q4 + (col & 3))] = z;
        if (col < G) ast[slot * 16 + col] = off;
      };
      eng.template softmax<true, false>(s, kb0, lo, hi, sc2, bmax, bsum, hook);
    } else if constexpr (TOKEN == 1) {
      auto hook = [&](int, const float* x) {
        if (col < G) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int key = kb0 + tile_key(c, q4);
            if (key + 3 < L) {
              *(float4*)(rawrow + key) = make_float4(x[4 * c] * kLn2, x[4 * c + 1] * kLn2,
                                                     x[4 * c + 2] * kLn2, x[4 * c + 3] * kLn2);
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (key + i < L) rawrow[key + i] = x[4 * c + i] * kLn2;
            }
          }
        }
      };
      eng.template softmax<true, false>(s, kb0, lo, hi, sc2, bmax, bsum, hook);
    } else {
      eng.template softmax<true, false>(s, kb0, lo, hi, sc2, bmax, bsum);
      // block maxima are held until the chunk ends (lane group q keeps the
      // chunk's tiles q, q + 4, ...) and then written with one store per
      // lane group instead of one per tile
      const int tt = (kb0 - kstart) >> 6;
#pragma unroll
      for (int r = 0; r < kDecodeChunkBlocksMax / 4; ++r)
        if (tt == 4 * r + (lane >> 4)) bkeep[r] = bmax[0];
      (void)j;
    }
    eng.pv(s, ldV);
    if constexpr (MORE) loadV(nx, rv);
  };
  // Every tile but the last in a loop whose loads are the same every
  // iteration, so the compiler's waits stay counts instead of drains; the
  // last tile (the only one that can hold keys past L) is peeled off and
  // requests nothing.
  const int ntile = (kend - kstart + 63) >> 6;
  if (ntile > 0) {
    loadK(kstart, rk);
    loadV(kstart, rv);
  }
  for (int t = 0; t + 1 < ntile; ++t) {
    const int kb0 = kstart + 64 * t;
    body(kb0, kb0 + 64, std::true_type{});
  }
  if (ntile > 0) {
    const int kb0 = kstart + 64 * (ntile - 1);
    clipV(kb0, rv);
    body(kb0, kb0, std::false_type{});
  }

  if constexpr (TOKEN == 2) {
    // the chunk's bounds: z of its keys (contiguous in the row) and the
    // offsets of its tiles, from this wave's staging rows
    const size_t brow = (size_t)b * a.Hkv + g;
    const int w4 = threadIdx.x >> 6;
    float4* zg = (float4*)(a.zb + brow * a.C + kstart);
    const float4* zs = (const float4*)(zst + w4 * kDecodeChunkBlocksMax * 64);
    for (int i = lane; i < ntile * 16; i += 64) zg[i] = zs[i];
    float* ag = a.ab + (brow * (a.C / 64) + (kstart >> 6)) * G;
    for (int i = lane; i < ntile * G; i += 64) ag[i] = ast[(w4 * kDecodeChunkBlocksMax + i / G) * 16 + i % G];
  }
  if (!TOKEN && col < G) {
#pragma unroll
    for (int r = 0; r < kDecodeChunkBlocksMax / 4; ++r) {
      const int kb = kstart + 64 * (4 * r + (lane >> 4));
      if (kb < kend) rawrow[kb >> 6] = bkeep[r] * kLn2;
    }
  }

  // partial state: unnormalised o (head_dim floats, natural order), m (log2), l
  const float lt = xlane_sum(eng.l[0]);
  if (col < G) {
    float* pp = a.part + ((size_t)(b * a.Hq + h) * a.nch + ch) * (D + 2);
    if (KV == HS_FP8_E4M3) {
      // rows 4q+i of chunk mc hold head_dim fp8_vrow_dv(mc, 4q+i): this
      // lane's D/4 values are the contiguous run from (D/4) q
      float v[D / 4];
#pragma unroll
      for (int mc = 0; mc < Eng::NM; ++mc)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[fp8_vrow_dv<D>(mc, i)] = eng.o[0][mc][i] * sv;
      float4* dst = (float4*)(pp + (D / 4) * (lane >> 4));
#pragma unroll
      for (int j = 0; j < D / 16; ++j) dst[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    } else {
#pragma unroll
      for (int mc = 0; mc < Eng::NM; ++mc) *(float4*)(pp + 16 * mc + q4) = *(const float4*)&eng.o[0][mc];
    }
    if (lane < 16) {
      pp[D] = eng.m[0];
      pp[D + 1] = lt;
    }
  }
}

// One work group of 4 waves per (b, h) merges the nchb = ceil(L / (CH*64))
// partials: the group finds the common maximum, wave w sums the chunks
// c = w, w+4, ... (independent loads, unrolled), and the four partial sums
// are added through LDS.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeFullArgs a) {
  constexpr int PER = D / 64;
  __shared__ float red[4];
  __shared__ float accs[4][D + 1];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < a.nclear; i += (long)gridDim.x * 256) a.clear[i] = 0u;
  const long bh = blockIdx.x;
  const int b = (int)(bh / a.Hq);
  const int L = ctx_len(a.lens, b, a.C);
  const int span = a.ch_blocks * 64;
  const int nchb = L > 0 ? (L + span - 1) / span : 0;
  const float* pp = a.part + (size_t)bh * a.nch * (D + 2);
  // One pass: wave w takes chunks w, w + 4, ... with a running maximum, U
  // chunks' loads in flight at a time (every load unconditional: chunks past
  // the sequence reread chunk w and are weighted 0); the four waves' states
  // are then merged through LDS.
  constexpr int U = 8;
  float mw = kNegBig, lsum = 0.f, acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int c0 = w; c0 < nchb; c0 += 4 * U) {
    float pm[U], pl[U], po[U][PER];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 4 * u < nchb ? c0 + 4 * u : c0;
      const float* p = pp + (size_t)c * (D + 2);
      pm[u] = p[D];
      pl[u] = p[D + 1];
#pragma unroll
      for (int i = 0; i < PER; ++i) po[u][i] = p[lane + 64 * i];
    }
    float mn = mw;
#pragma unroll
    for (int u = 0; u < U; ++u) mn = c0 + 4 * u < nchb ? fmaxf(mn, pm[u]) : mn;
    const float sc = fast_exp2(mw - mn);
    lsum *= sc;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] *= sc;
    mw = mn;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wt = c0 + 4 * u < nchb ? fast_exp2(pm[u] - mn) : 0.f;
      lsum += wt * pl[u];
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += wt * po[u][i];
    }
  }
  if (lane == 0) red[w] = mw;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sw = fast_exp2(mw - M);
#pragma unroll
  for (int i = 0; i < PER; ++i) accs[w][lane + 64 * i] = acc[i] * sw;
  if (lane == 0) accs[w][D] = lsum * sw;
  __syncthreads();
  if (w == 0) {
    const float lt = accs[0][D] + accs[1][D] + accs[2][D] + accs[3][D];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* o = (uint16_t*)a.o + (size_t)bh * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = lane + 64 * i;
      o[d] = (uint16_t)bf16_bits((accs[0][d] + accs[1][d] + accs[2][d] + accs[3][d]) * inv);
    }
    if (lane == 0) a.lse[bh] = lt > 0.f ? (M + fast_log2(lt)) * kLn2 : -INFINITY;
  }
}

// ============================================================ sparse layer
// One work group (8 waves) per (b, g).  Work items: the ceil(min(L, W)/64)
// tiles of the window ring, then the n_sel selected blocks of the shared
// cache; item i goes to wave i % 8, so each wave meets its window items
// first.  A wave parks its window-branch state in LDS when it moves on to
// the selected blocks and reuses the same registers for the sparse branch.
// The 8 partial states of each branch are merged through LDS and the two
// branches combined with the gates.
template <int D>
__global__ __launch_bounds__(512) void decode_sparse_kernel(DecodeSparseArgs a) {
  using Tt = Tr<HS_BF16>;
  using Frag = typename Tt::Frag;
  using Eng = WaveAttn<HS_BF16, D, 1>;
  constexpr int ES = 2;
  constexpr int NW = 8;
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  // rows padded by 16 bytes: a 16-byte store of the 64 lanes then takes the
  // minimum four passes instead of one per column
  __shared__ __attribute__((aligned(16))) float sm_o[NW][16][D + 4];

  __shared__ int sm_wtot[NW];
  extern __shared__ uint32_t dyn[];  // canonical selection list: 2 x cap words

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bg = blockIdx.x;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int L = __builtin_amdgcn_readfirstlane(ctx_len(a.lens, b, a.C));
  const int G = a.Hq / a.Hkv;
  const int col = lane & 15;
  const int h = g * G + col;
  const int r16 = lane & 15, q8 = 8 * (lane >> 4), q4 = (lane >> 4) << 2;
  const int nring = a.W > 0 ? (min(L, a.W) + 63) / 64 : 0;
  const int nslots = min(L, a.W);
  // live selected blocks: ids j with 64 j < L, each once, ascending
  const int cap = sel_list_cap(a.nsel);
  const uint32_t* sel = dyn + cap;
  const int nlive = __builtin_amdgcn_readfirstlane(
      canon_sel_list<64 * NW>(a.idx + (size_t)(b * a.Hkv + g) * a.nsel, a.nsel, (uint32_t)((L + 63) / 64), cap,
                              dyn, dyn + cap, sm_wtot));
  const int nitem = nring + nlive;

  Eng eng;
  eng.reset();
  // Every global load below is unconditional: a load under a branch would
  // turn the compiler's later waits into full drains.  Columns past G read
  // head g*G and are zeroed.
#pragma unroll
  for (int ks = 0; ks < Eng::NS; ++ks) {
    const Frag f = Tt::ld((const char*)a.q + ((size_t)(b * a.Hq + (col < G ? h : g * G)) * D + 32 * ks + q8) * ES);
    eng.qf[0][ks] = col < G ? f : Tt::zero();
  }
  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * a.C * D * ES;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * (a.C / 64) * D * 64 * ES;
  const char* krg = (const char*)a.kr + (size_t)(b * a.Hkv + g) * a.W * D * ES;
  const char* vrg = (const char*)a.vr + (size_t)(b * a.Hkv + g) * ((a.W + 63) / 64) * D * 64 * ES;

  // Item it < nring: ring tile it (slots 64*it ..); otherwise live selected
  // block sel[it - nring].  All fields are wave-uniform, so one load path
  // serves both kinds.
  struct Item {
    const char* kp;  // first key row of the tile
    const char* vp;  // [D][64] value slab of the tile
    int rows;        // key rows addressable from kp
    int kbase;       // first key (cache position or ring slot)
    int hi;          // last valid key
    bool ring, on;
  };
  auto item = [&](int it) {
    Item r;
    r.ring = it < nring;
    if (r.ring) {
      r.on = true;
      r.kp = krg + (size_t)64 * it * D * ES;
      r.vp = vrg + (size_t)it * D * 64 * ES;
      r.rows = a.W - 64 * it;  // the ring's last tile may be short
      r.kbase = 64 * it;
      r.hi = nslots - 1;
    } else {
      // it < nitem whenever the item is used; a clamped read otherwise
      const int j = nlive > 0 ? __builtin_amdgcn_readfirstlane((int)sel[min(it - nring, nlive - 1)]) : 0;
      r.on = nlive > 0;
      r.kp = kg + (size_t)64 * j * D * ES;
      r.vp = vg + (size_t)j * D * 64 * ES;
      r.rows = 64;
      r.kbase = 64 * j;
      r.hi = L - 1;
    }
    return r;
  };
  uint4 rk[4][Eng::NS], rv[2][Eng::NM];
  auto loadK = [&](const Item& t) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int row = min(tile_key(c, r16), t.rows - 1);
#pragma unroll
      for (int ks = 0; ks < Eng::NS; ++ks) rk[c][ks] = *(const uint4*)(t.kp + ((size_t)row * D + 32 * ks + q8) * ES);
    }
  };
  auto loadV = [&](const Item& t) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int mc = 0; mc < Eng::NM; ++mc)
        rv[u][mc] = *(const uint4*)(t.vp + (((size_t)16 * mc + r16) * 64 + 32 * u + q8) * ES);
  };
  // a wave's partial state -> LDS slice w
  auto park = [&]() {
    const float lt = xlane_sum(eng.l[0]);
    if (lane < 16) {
      sm_m[w][col] = eng.m[0];
      sm_l[w][col] = lt;
    }
#pragma unroll
    for (int mc = 0; mc < Eng::NM; ++mc) *(float4*)&sm_o[w][col][16 * mc + q4] = *(const float4*)&eng.o[0][mc];
  };

  float bmax[1], bsum[1];
  int lo[1], hi[1];
  bool parked = false;  // window branch of this wave already in LDS
  Item cur = item(w < nitem ? w : 0);
  if (w < nitem) {
    loadK(cur);
    loadV(cur);
  }
  // One item: QK^T on rk, the next item's keys are requested, softmax, PV
  // with rv, the next item's values are requested (none when `more` is
  // false: this wave's last item).
  auto step = [&](int it, auto more) {
    constexpr bool MORE = decltype(more)::value;
    if (!parked && !cur.ring) {  // first selected block: the window branch is complete
      park();
      eng.reset();
      parked = true;
    }
    const Item nxt = MORE ? item(it + NW) : cur;
    auto ldK = [&](int c, int ks) {
      Frag f;
      f.u = rk[c][ks];
      return f;
    };
    auto ldV = [&](int u, int mc) {
      Frag f;
      f.u = rv[u][mc];
      // values of keys past the last valid one are zeroed (selects only):
      // P = 0 there, but a stale non-finite value would not vanish
      return Tt::keep(f, cur.hi + 1 - (cur.kbase + 32 * u + q8));
    };
    f32x4 sx[1][4];
    eng.qk(ldK, sx);
    if constexpr (MORE) loadK(nxt);
    lo[0] = col < G && cur.on ? 0 : kNoKey;
    hi[0] = cur.hi;
    eng.template softmax<true, false>(sx, cur.kbase, lo, hi, a.sc2, bmax, bsum);
    eng.pv(sx, ldV);
    if constexpr (MORE) loadV(nxt);
    cur = nxt;
  };
  // every item but the last in a loop with the same loads each iteration
  // (the compiler's waits stay counts), the last one peeled off
  int it = w;
  for (; it + NW < nitem; it += NW) step(it, std::true_type{});
  if (it < nitem) step(it, std::false_type{});
  if (!parked) {  // no selected block reached this wave
    park();
    eng.reset();
  }

  // Merge the partial states of one branch (the window branch sits in LDS
  // now; the sparse branch follows); thread -> (head column, d) outputs.
  constexpr int PER = (16 * D + 64 * NW - 1) / (64 * NW);
  float out[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) out[i] = 0.f;
  auto merge = [&](int br) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int el = threadIdx.x + 64 * NW * i;
      const int c = el / D, d = el % D;
      if (c < G) {
        // the branch's sink logit (log2 units) joins the maximum and the sum
        const float sk = a.sinks ? a.sinks[br * a.Hq + g * G + c] * kLog2e : -INFINITY;
        float M = fmaxf(kNegBig, sk);
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww][c]);
        float ls = fast_exp2(sk - M), os = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          const float wt = fast_exp2(sm_m[ww][c] - M);
          ls += wt * sm_l[ww][c];
          os += wt * sm_o[ww][c][d];
        }
        float gate = 1.f;
        if (a.gates) gate = 1.f / (1.f + expf(-a.gates[((size_t)b * a.Hq + g * G + c) * 2 + br]));
        out[i] += ls > 0.f ? gate * os / ls : 0.f;
      }
    }
  };
  __syncthreads();
  merge(1);
  __syncthreads();
  park();
  __syncthreads();
  merge(0);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int el = threadIdx.x + 64 * NW * i;
    const int c = el / D, d = el % D;
    if (c < G) ((uint16_t*)a.o)[((size_t)b * a.Hq + g * G + c) * D + d] = (uint16_t)bf16_bits(out[i]);
  }
}

// ========================================================= token-level top-k
// HySparse2 explainer, "Precise retrieval without a separate indexer" and the
// decode_one_token pseudocode: selected = newest n_recent tokens united with
// the top-k older tokens by full-layer score.  The token score is the group
// maximum of the post-softmax weights, x_i = max_h (logit_hi - LSE_h) in the
// log domain.  Selection is a three-level radix select on the order-preserving
// 32-bit key of x (11 + 11 + 10 bits), then one pass that emits the winners in
// ascending token order, equal keys resolved towards the smaller token id.
__device__ __forceinline__ uint32_t order_key_f(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// the slack of the selection from bounds (below, token_zcand_kernel)
constexpr float kBoundSlack = 1e-3f;

// hist[bin] += 1 for every active lane, one LDS atomic per distinct bin of the
// wave: the scores of a row are close together, so most lanes of a wave share
// a handful of bins and per-lane atomics would queue on the same addresses
__device__ __forceinline__ void wave_hist_add(uint32_t* hist, uint32_t bin, bool act) {
  const int lane = lane_id();
  for (;;) {
    const uint64_t am = __ballot(act);
    if (!am) break;
    const int leader = __builtin_ctzll(am);
    const uint32_t lb = (uint32_t)__shfl((int)bin, leader);
    const uint64_t m = __ballot(act && bin == lb);
    if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(m));
    act = act && bin != lb;
  }
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* p, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) p[i] = 0u;
}

// grid (rows, C/4096): keys for 4096 tokens and the level-1 histogram (top 11
// bits).  Thread t takes the token quads t, t + 256, t + 512, t + 768 of the
// group's 4096 tokens: 16-byte loads of each head's logits, all in flight.
__global__ __launch_bounds__(256) void token_keys_kernel(TokenTopkArgs a) {
  __shared__ uint32_t hist[2048];
  const int row = blockIdx.x;
  const int g = row % a.Hkv, b = row / a.Hkv;
  const int L = ctx_len(a.lens, b, a.C);
  const int ncand = max(0, L - a.n_recent);
  const int G = a.Hq / a.Hkv;
  for (int i = threadIdx.x; i < 2048; i += 256) hist[i] = 0u;
  __syncthreads();
  const int base = blockIdx.y * 4096;
  uint32_t* keys = a.keys + (size_t)row * a.C;
  const float* rg = a.raw + ((size_t)b * a.Hq + g * G) * a.C;
  const float* lse = a.lse + (size_t)b * a.Hq + g * G;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int i0 = base + 4 * (threadIdx.x + 256 * n);
    if (i0 >= a.C) break;  // C is a multiple of 64
    float4 x = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    if (i0 < L) {
      for (int hh = 0; hh < G; ++hh) {
        const float4 r = *(const float4*)(rg + (size_t)hh * a.C + i0);
        const float l = lse[hh];
        x.x = fmaxf(x.x, r.x - l);
        x.y = fmaxf(x.y, r.y - l);
        x.z = fmaxf(x.z, r.z - l);
        x.w = fmaxf(x.w, r.w - l);
      }
    }
    const float xs[4] = {x.x, x.y, x.z, x.w};
    uint32_t kq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + e;
      kq[e] = 0u;
      if (i < L) {
        if (a.gs) a.gs[(size_t)row * a.C + i] = expf(xs[e]);
        if (i < ncand) kq[e] = order_key_f(xs[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) wave_hist_add(hist, kq[e] >> 21, i0 + e < ncand);
    *(uint4*)(keys + i0) = make_uint4(kq[0], kq[1], kq[2], kq[3]);
  }
  __syncthreads();
  uint32_t* gh = a.hist + (size_t)row * 2048;
  for (int i = threadIdx.x; i < 2048; i += 256)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// Block-wide search in a histogram of nb bins (nb = 1024 or 2048, 1024 threads):
// the bin b with count(> b) < k <= count(>= b); returns b and count(> b).
__device__ void find_bin(const uint32_t* h, int nb, int k, uint32_t* scan, int* res) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int per = nb / 1024;
  // thread t owns bins [nb - (t+1)*per, nb - t*per), i.e. descending order
  uint32_t own = 0;
  for (int e = 0; e < per; ++e) own += h[nb - t * per - 1 - e];
  // inclusive scan: within the wave by shuffles, then over the 16 wave totals
  uint32_t incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) scan[w] = incl;
  __syncthreads();
  for (int v = 0; v < w; ++v) incl += scan[v];
  const uint32_t excl = incl - own;
  if (excl < (uint32_t)k && incl >= (uint32_t)k) {
    uint32_t above = excl;
    for (int e = 0; e < per; ++e) {
      const int bin = nb - t * per - 1 - e;
      if (above + h[bin] >= (uint32_t)k) {
        res[0] = bin;
        res[1] = (int)above;
        break;
      }
      above += h[bin];
    }
  }
  __syncthreads();
}

// grid (rows, ceil(C / kTokSeg)), 1024 threads: the level-2 histogram (bits
// 20..10 of the keys whose top 11 bits are the level-1 threshold bin); every
// group of a row finds that bin again from the level-1 histogram
__global__ __launch_bounds__(1024) void token_hist2_kernel(TokenTopkArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scan[1024];
  __shared__ int res[2];
  const int row = blockIdx.x, t = threadIdx.x;
  const int L = ctx_len(a.lens, row / a.Hkv, a.C);
  const int ncand = max(0, L - a.n_recent);
  const int s0 = blockIdx.y * kTokSeg;
  if (ncand <= a.kb || s0 >= ncand) return;  // uniform
  const uint32_t* gh = a.hist + (size_t)row * 2048;
  for (int i = t; i < 2048; i += 1024) hist[i] = gh[i];
  __syncthreads();
  find_bin(hist, 2048, a.kb, scan, res);
  const uint32_t b1 = (uint32_t)res[0];
  for (int i = t; i < 2048; i += 1024) hist[i] = 0u;
  __syncthreads();
  const uint32_t* keys = a.keys + (size_t)row * a.C;
  const int s1 = min(ncand, s0 + kTokSeg);
  for (int i = s0 + t; i < s1; i += 1024) {
    const uint32_t k = keys[i];
    // (plain atomics: inside the threshold bin the next 11 bits spread over
    // many bins, where the per-bin ballot loop of wave_hist_add runs long)
    if ((k >> 21) == b1) atomicAdd(&hist[(k >> 10) & 2047u], 1u);
  }
  __syncthreads();
  uint32_t* h2 = a.hist + (size_t)a.B * a.Hkv * 2048 + (size_t)row * 2048;
  for (int i = t; i < 2048; i += 1024)
    if (hist[i]) atomicAdd(&h2[i], hist[i]);
}

// grid (rows, ceil(C / kTokSeg)), 1024 threads: compacts the candidates, the
// keys whose top 22 bits are at least the level-2 threshold prefix (fewer
// than kb above it plus that prefix's bin), as (key, token id) pairs; each
// segment's candidates form one run in token order, the runs lie in arbitrary
// order and seg records where each one went.  The count may exceed kTokCap
// (then only the count is kept).
__global__ __launch_bounds__(1024) void token_cand_kernel(TokenTopkArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scan[1024];
  __shared__ int res[2];
  __shared__ uint32_t base_s;
  const int row = blockIdx.x, t = threadIdx.x;
  const int L = ctx_len(a.lens, row / a.Hkv, a.C);
  const int ncand = max(0, L - a.n_recent);
  const int s0 = blockIdx.y * kTokSeg;
  if (ncand <= a.kb || s0 >= ncand) return;  // uniform
  const size_t rows = (size_t)a.B * a.Hkv;
  for (int i = t; i < 2048; i += 1024) hist[i] = a.hist[(size_t)row * 2048 + i];
  __syncthreads();
  find_bin(hist, 2048, a.kb, scan, res);
  const uint32_t b1 = (uint32_t)res[0];
  const int need = a.kb - res[1];
  for (int i = t; i < 2048; i += 1024) hist[i] = a.hist[rows * 2048 + (size_t)row * 2048 + i];
  __syncthreads();
  find_bin(hist, 2048, need, scan, res);
  const uint32_t pfx = (b1 << 11) | (uint32_t)res[0];
  const uint32_t* keys = a.keys + (size_t)row * a.C;
  // thread t takes the PER consecutive keys s0 + PER*t .. (16-byte loads),
  // so the block's exclusive scan below keeps the candidates in token order
  constexpr int PER = kTokSeg / 1024;
  static_assert(PER % 4 == 0, "keys are read four at a time");
  uint32_t kv[PER];
  const int i0 = s0 + PER * t;
#pragma unroll
  for (int n = 0; n < PER; n += 4) {
    // a row holds C keys, C a multiple of 64, so a quad never leaves it
    const uint4 q = i0 + n < ncand ? *(const uint4*)(keys + i0 + n) : make_uint4(0u, 0u, 0u, 0u);
    kv[n] = q.x;
    kv[n + 1] = q.y;
    kv[n + 2] = q.z;
    kv[n + 3] = q.w;
  }
  uint32_t flags = 0u, cnt = 0u;
#pragma unroll
  for (int n = 0; n < PER; ++n) {
    if (i0 + n < ncand && (kv[n] >> 10) >= pfx) {
      flags |= 1u << n;
      ++cnt;
    }
  }
  // block exclusive scan of the per-thread counts
  scan[t] = cnt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const uint32_t x = t >= off ? scan[t - off] : 0u;
    __syncthreads();
    scan[t] += x;
    __syncthreads();
  }
  const uint32_t excl = scan[t] - cnt;
  if (t == 1023) {
    base_s = atomicAdd(a.hist + rows * 2 * 2048 + row, scan[1023]);
    // this segment's run: its candidates in ascending token order
    a.seg[((size_t)row * a.nseg + blockIdx.y) * 2] = base_s;
    a.seg[((size_t)row * a.nseg + blockIdx.y) * 2 + 1] = scan[1023];
  }
  __syncthreads();
  uint32_t pos = base_s + excl;
  uint32_t* ck = a.cand_key + (size_t)row * kTokCap;
  int32_t* ci = a.cand_idx + (size_t)row * kTokCap;
#pragma unroll
  for (int n = 0; n < PER; ++n) {
    if ((flags >> n) & 1u) {
      if (pos < (uint32_t)kTokCap) {
        ck[pos] = kv[n];
        ci[pos] = i0 + n;
      }
      ++pos;
    }
  }
}

// Writes, in ascending order of position, the ids of the n entries whose key
// is above thr and of the first need_eq entries whose key equals thr (1024
// threads).  Wave w owns the contiguous entries [w*wseg, (w+1)*wseg) and walks
// them 64 at a time; ballots give each lane its rank among the keys > thr and
// == thr of its wave, and the 16 waves' counts give every wave its first
// output slot and its first tie rank.
template <class KF, class IF>
__device__ void emit_selected(int n, uint32_t thr, int need_eq, const KF& key_of, const IF& id_of, int32_t* out,
                              uint32_t* wsum) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const uint64_t lt_mask = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int wseg = ((n + 1023) / 1024) * 64;
  const int i0 = min(n, w * wseg), i1 = min(n, i0 + wseg);
  uint32_t ngt = 0, neq = 0;
  for (int i = i0; i < i1; i += 64) {
    const bool in = i + lane < i1;
    const uint32_t k = in ? key_of(i + lane) : 0u;
    ngt += __popcll(__ballot(in && k > thr));
    neq += __popcll(__ballot(in && k == thr));
  }
  if (lane == 0) {
    wsum[w] = ngt;
    wsum[16 + w] = neq;
  }
  __syncthreads();
  uint32_t gt_base = 0, eq_base = 0;
  for (int v = 0; v < w; ++v) {
    gt_base += wsum[v];
    eq_base += wsum[16 + v];
  }
  uint32_t pos = gt_base + min(eq_base, (uint32_t)need_eq);
  for (int i = i0; i < i1; i += 64) {
    const bool in = i + lane < i1;
    const uint32_t k = in ? key_of(i + lane) : 0u;
    const uint64_t eqm = __ballot(in && k == thr);
    const uint32_t eq_rank = eq_base + __popcll(eqm & lt_mask);
    const bool take = in && (k > thr || (k == thr && eq_rank < (uint32_t)need_eq));
    const uint64_t tm = __ballot(take);
    if (take) out[pos + __popcll(tm & lt_mask)] = id_of(i + lane);
    pos += __popcll(tm);
    eq_base += __popcll(eqm);
  }
}

// one work group (1024 threads) per (sequence, kv group) row
__global__ __launch_bounds__(1024) void token_select_kernel(TokenTopkArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scan[1024];
  __shared__ int res[2];
  __shared__ uint32_t wsum[32];
  __shared__ uint32_t cand_k[kTokCap];
  __shared__ int32_t cand_i[kTokCap];
  const int row = blockIdx.x;
  const int b = row / a.Hkv;
  const int L = ctx_len(a.lens, b, a.C);
  const int ncand = max(0, L - a.n_recent);
  const int nrec = min(L, a.n_recent);
  const int kb = a.kb;
  const int t = threadIdx.x;
  const uint32_t* keys = a.keys + (size_t)row * a.C;
  int32_t* out = a.idx + (size_t)row * (kb + a.n_recent);
  int nsel;

  const uint32_t ncnd = a.hist[(size_t)a.B * a.Hkv * 2 * 2048 + row];
  if (ncand <= kb) {
    for (int i = t; i < ncand; i += 1024) out[i] = i;
    nsel = ncand;
  } else if (ncnd <= (uint32_t)kTokCap) {
    // the candidates (at least kb: all keys whose top 22 bits reach the
    // level-2 threshold prefix): gathered in ascending token order (each key
    // segment's run is in order, and runs follow their segments), then the
    // last 10 bits decide inside the threshold prefix and ties go to the
    // smaller token
    const uint32_t* gh = a.hist + (size_t)row * 2048;
    for (int i = t; i < 2048; i += 1024) hist[i] = gh[i];
    __syncthreads();
    find_bin(hist, 2048, kb, scan, res);
    const uint32_t b1 = (uint32_t)res[0];
    int need = kb - res[1];
    const uint32_t* gh2 = a.hist + (size_t)a.B * a.Hkv * 2048 + (size_t)row * 2048;
    for (int i = t; i < 2048; i += 1024) hist[i] = gh2[i];
    __syncthreads();
    find_bin(hist, 2048, need, scan, res);
    const uint32_t pfx = (b1 << 11) | (uint32_t)res[0];
    need -= res[1];
    const uint32_t* ck = a.cand_key + (size_t)row * kTokCap;
    const int32_t* ci = a.cand_idx + (size_t)row * kTokCap;
    const uint32_t* sg = a.seg + (size_t)row * a.nseg * 2;
    const int nsg = (ncand + kTokSeg - 1) / kTokSeg;
    int off = 0;
    for (int q = 0; q < nsg; ++q) {
      const int base = (int)sg[2 * q], cnt = (int)sg[2 * q + 1];
      for (int e = t; e < cnt; e += 1024) {
        cand_k[off + e] = ck[base + e];
        cand_i[off + e] = ci[base + e];
      }
      off += cnt;
    }
    for (int i = t; i < 1024; i += 1024) hist[i] = 0u;
    __syncthreads();
    for (int e = t; e < (int)ncnd; e += 1024)
      if ((cand_k[e] >> 10) == pfx) atomicAdd(&hist[cand_k[e] & 1023u], 1u);
    __syncthreads();
    find_bin(hist, 1024, need, scan, res);
    const uint32_t thr = (pfx << 10) | (uint32_t)res[0];
    const int need_eq = need - res[1];  // >= 1 candidates equal to thr are taken
    emit_selected((int)ncnd, thr, need_eq, [&](int i) { return cand_k[i]; }, [&](int i) { return cand_i[i]; }, out,
                  wsum);
    nsel = kb;
  } else {
    // level 1: the global histogram of the top 11 bits
    const uint32_t* gh = a.hist + (size_t)row * 2048;
    for (int i = t; i < 2048; i += 1024) hist[i] = gh[i];
    __syncthreads();
    find_bin(hist, 2048, kb, scan, res);
    const uint32_t b1 = (uint32_t)res[0];
    int need = kb - res[1];
    // level 2: bits 20..10 inside bin b1
    for (int i = t; i < 2048; i += 1024) hist[i] = 0u;
    __syncthreads();
    for (int i = t; i < ncand; i += 1024) {
      const uint32_t k = keys[i];
      if ((k >> 21) == b1) atomicAdd(&hist[(k >> 10) & 2047u], 1u);
    }
    __syncthreads();
    find_bin(hist, 2048, need, scan, res);
    const uint32_t p2 = (b1 << 11) | (uint32_t)res[0];
    need -= res[1];
    // level 3: bits 9..0
    for (int i = t; i < 1024; i += 1024) hist[i] = 0u;
    __syncthreads();
    for (int i = t; i < ncand; i += 1024) {
      const uint32_t k = keys[i];
      if ((k >> 10) == p2) atomicAdd(&hist[k & 1023u], 1u);
    }
    __syncthreads();
    find_bin(hist, 1024, need, scan, res);
    const uint32_t thr = (p2 << 10) | (uint32_t)res[0];
    const int need_eq = need - res[1];  // >= 1 keys equal to thr are taken
    emit_selected(ncand, thr, need_eq, [&](int i) { return keys[i]; }, [](int i) { return i; }, out, wsum);
    nsel = kb;
  }
  for (int r = t; r < nrec; r += 1024) out[nsel + r] = L - nrec + r;
  for (int r = nsel + nrec + t; r < kb + a.n_recent; r += 1024) out[r] = -1;
}

// ---------------------------------------- token-level top-k from bounds
// The full layer run with token == 2 leaves, per token, z = max_h (logit_h -
// off_h) and, per tile, the offsets off_h.  With the heads' LSEs (log2 units),
// d_h = LSE_h - off_h gives lo = z - max_h d_h <= x <= z - min_h d_h = hi for
// the token's score x = max_h (logit_h - LSE_h).  The k-th largest lo (found
// from a histogram of lo, taken at the lower edge of its bin) is at most the
// k-th largest score, so every token of the top k, ties included, has hi >=
// it: those tokens are the candidates.  Their scores are then computed
// exactly from their key rows, and the exact selection runs on them alone.
// A slack of kBoundSlack (log2 units) on the test covers the rounding of the
// bounds and of the rescoring.

// Fixed-point bins of the lower bounds.  Exact scores are log2 weights, so
// x <= 0 and lo <= x: bin 2047 - j (j < 2047) holds lo in (-(j+1)/64, -j/64],
// bin 0 everything at or below -2047/64.  One histogram then places the k-th
// largest lower bound within 1/64.
constexpr float kZBinScale = 64.f;
__device__ __forceinline__ uint32_t zbin(float lo) {
  const float j = fminf(fmaxf(floorf(-lo * kZBinScale), 0.f), 2047.f);
  return 2047u - (uint32_t)j;
}

// grid (rows, ceil(C / 4096)), 256 threads: per tile, the bound terms of the
// group's heads (d_h = LSE_h - offset_h; lo = z - max_h d_h, hi = z - min_h
// d_h), min_h d_h stored for the candidate pass; the histogram of the
// candidates' lower bounds (plain LDS atomics: the bins of one wave are many)
__global__ __launch_bounds__(256) void token_zhist_kernel(TokenTopkArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ float lse2[16];
  const int row = blockIdx.x;
  const int g = row % a.Hkv, b = row / a.Hkv;
  const int L = ctx_len(a.lens, b, a.C);
  const int ncand = max(0, L - a.n_recent);
  const int G = a.Hq / a.Hkv;
  for (int i = threadIdx.x; i < 2048; i += 256) hist[i] = 0u;
  if (threadIdx.x < G) lse2[threadIdx.x] = a.lse[(size_t)b * a.Hq + g * G + threadIdx.x] * kLog2e;
  __syncthreads();
  const int base = blockIdx.y * 4096;
  const int ntl = a.C / 64;
  const float* zr = a.zb + (size_t)row * a.C;
  const float* ar = a.ab + (size_t)row * ntl * G;
  float* wr = a.wb + (size_t)row * ntl;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int i0 = base + 4 * (threadIdx.x + 256 * n);
    if (i0 < min(L, a.C)) {
      const int tl = i0 >> 6;
      float dmax = -INFINITY, dmin = INFINITY;
      for (int hh = 0; hh < G; ++hh) {
        const float d = lse2[hh] - ar[tl * G + hh];
        dmax = fmaxf(dmax, d);
        dmin = fminf(dmin, d);
      }
      if ((i0 & 63) == 0) wr[tl] = dmin;
      const float4 z = *(const float4*)(zr + i0);
      const float zs[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i0 + e < ncand) atomicAdd(&hist[zbin(zs[e] - dmax)], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = a.hist + (size_t)row * 2048;
  for (int i = threadIdx.x; i < 2048; i += 256)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// grid (rows, ceil(C / kTokSeg)), 1024 threads: the candidates of one row
// segment.  The bin of the k-th largest lower bound gives T, its lower edge
// (at least k scores lie above T); a token is a candidate when its upper
// bound reaches T - kBoundSlack.  The k-th bound in the open bottom bin
// leaves T = -inf: every token is a candidate, more than the candidate
// buffer holds, and the pick takes exact scores of the whole row.
__global__ __launch_bounds__(1024) void token_zcand_kernel(TokenTopkArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scan[1024];
  __shared__ int res[2];
  __shared__ uint32_t base_s;
  const int row = blockIdx.x, t = threadIdx.x;
  const int L = ctx_len(a.lens, row / a.Hkv, a.C);
  const int ncand = max(0, L - a.n_recent);
  const int s0 = blockIdx.y * kTokSeg;
  if (ncand <= a.kb || s0 >= ncand) return;  // uniform
  const size_t rows = (size_t)a.B * a.Hkv;
  for (int i = t; i < 2048; i += 1024) hist[i] = a.hist[(size_t)row * 2048 + i];
  __syncthreads();
  find_bin(hist, 2048, a.kb, scan, res);
  const int bk = res[0];
  const float thr = bk > 0 ? -(float)(2048 - bk) / kZBinScale - kBoundSlack : -INFINITY;
  const float* zr = a.zb + (size_t)row * a.C;
  // thread t takes the PER consecutive tokens s0 + PER*t .. (16-byte loads),
  // so the block's exclusive scan below keeps the candidates in token order
  constexpr int PER = kTokSeg / 1024;
  static_assert(PER % 4 == 0 && 64 % PER == 0, "four z per load; a thread's tokens lie in one tile");
  float zv[PER];
  const int i0 = s0 + PER * t;
#pragma unroll
  for (int n = 0; n < PER; n += 4) {
    // a row holds C values, C a multiple of 64, so a quad never leaves it
    const float4 q = i0 + n < ncand ? *(const float4*)(zr + i0 + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    zv[n] = q.x;
    zv[n + 1] = q.y;
    zv[n + 2] = q.z;
    zv[n + 3] = q.w;
  }
  const float dmin = i0 < ncand ? a.wb[(size_t)row * (a.C / 64) + (i0 >> 6)] : 0.f;
  uint32_t flags = 0u, cnt = 0u;
#pragma unroll
  for (int n = 0; n < PER; ++n) {
    if (i0 + n < ncand && zv[n] - dmin >= thr) {
      flags |= 1u << n;
      ++cnt;
    }
  }
  // block exclusive scan of the per-thread counts
  scan[t] = cnt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const uint32_t x = t >= off ? scan[t - off] : 0u;
    __syncthreads();
    scan[t] += x;
    __syncthreads();
  }
  const uint32_t excl = scan[t] - cnt;
  if (t == 1023) {
    base_s = atomicAdd(a.hist + rows * 2 * 2048 + row, scan[1023]);
    // this segment's run: its candidates in ascending token order
    a.seg[((size_t)row * a.nseg + blockIdx.y) * 2] = base_s;
    a.seg[((size_t)row * a.nseg + blockIdx.y) * 2 + 1] = scan[1023];
  }
  __syncthreads();
  uint32_t pos = base_s + excl;
  int32_t* ci = a.cand_idx + (size_t)row * kTokCap;
#pragma unroll
  for (int n = 0; n < PER; ++n) {
    if ((flags >> n) & 1u) {
      if (pos < (uint32_t)kTokCap) ci[pos] = i0 + n;
      ++pos;
    }
  }
}

// The exact score (log2 units) of token i of row (b, g): max over the group's
// heads of sc2 * k_scale * q_h . k_i - LSE_h, from the fp8 key row; qs holds
// the group's queries (fp32, [G][D]) and lse2 the heads' LSEs (log2 units).
template <int D>
__device__ float exact_token_score(const uint8_t* krow, const float* qs, const float* lse2, int G, float sck) {
  float acc[16];
#pragma unroll
  for (int hh = 0; hh < 16; ++hh) acc[hh] = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const uint4 w = *(const uint4*)(krow + 16 * c);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float kv[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 lo2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[e], false);
      const f32x2 hi2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[e], true);
      kv[4 * e] = lo2[0];
      kv[4 * e + 1] = lo2[1];
      kv[4 * e + 2] = hi2[0];
      kv[4 * e + 3] = hi2[1];
    }
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) {
      if (hh >= G) break;
      const float4* qp = (const float4*)(qs + hh * D + 16 * c);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const float4 qv = qp[f];
        acc[hh] = __builtin_fmaf(qv.x, kv[4 * f], acc[hh]);
        acc[hh] = __builtin_fmaf(qv.y, kv[4 * f + 1], acc[hh]);
        acc[hh] = __builtin_fmaf(qv.z, kv[4 * f + 2], acc[hh]);
        acc[hh] = __builtin_fmaf(qv.w, kv[4 * f + 3], acc[hh]);
      }
    }
  }
  float x = -INFINITY;
#pragma unroll
  for (int hh = 0; hh < 16; ++hh)
    if (hh < G) x = fmaxf(x, acc[hh] * sck - lse2[hh]);
  return x;
}

// Radix select over n keys (in LDS or global memory, read through key_of):
// the key thr of the k-th largest and how many entries equal to thr are
// taken (need_eq >= 1), three levels of 11, 11 and 10 bits.
template <class KF>
__device__ void radix_kth(int n, int k, const KF& key_of, uint32_t* hist, uint32_t* scan, int* res, uint32_t* thr,
                          int* need_eq) {
  const int t = threadIdx.x;
  int need = k;
  uint32_t pfx = 0u;
#pragma unroll 1
  for (int lvl = 0; lvl < 3; ++lvl) {
    const int shift = lvl == 0 ? 21 : (lvl == 1 ? 10 : 0);
    const int nb = lvl == 2 ? 1024 : 2048;
    for (int i = t; i < 2048; i += 1024) hist[i] = 0u;
    __syncthreads();
    for (int i = t; i < n; i += 1024) {
      const uint32_t kk = key_of(i);
      const bool in = lvl == 0 || (lvl == 1 ? (kk >> 21) == pfx : (kk >> 10) == pfx);
      if (in) atomicAdd(&hist[(kk >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    find_bin(hist, nb, need, scan, res);
    pfx = lvl == 0 ? (uint32_t)res[0] : ((pfx << (lvl == 1 ? 11 : 10)) | (uint32_t)res[0]);
    need -= res[1];
  }
  *thr = pfx;
  *need_eq = need;
}

// grid (rows, kTokCap / 256): the exact key of every candidate (in place of
// its lower-bound key), one candidate per thread; rows with more candidates
// than the store holds are left to token_zselect_kernel
template <int D>
__global__ __launch_bounds__(256) void token_rescore_kernel(TokenTopkArgs a) {
  __shared__ __attribute__((aligned(16))) float qs[16 * D];
  __shared__ float lse2[16];
  const int row = blockIdx.x;
  const int b = row / a.Hkv, g = row % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const uint32_t ncnd = a.hist[(size_t)a.B * a.Hkv * 2 * 2048 + row];
  if (ncnd > (uint32_t)kTokCap || blockIdx.y * 256u >= ncnd) return;  // uniform
  const int t = threadIdx.x;
  const uint16_t* qg = (const uint16_t*)a.q + ((size_t)b * a.Hq + g * G) * D;
  for (int i = t; i < G * D; i += 256) qs[i] = __uint_as_float((uint32_t)qg[i] << 16);
  if (t < G) lse2[t] = a.lse[(size_t)b * a.Hq + g * G + t] * kLog2e;
  __syncthreads();
  const uint32_t e = blockIdx.y * 256u + t;
  if (e >= ncnd) return;
  const int id = a.cand_idx[(size_t)row * kTokCap + e];
  const uint8_t* kr = a.k + (((size_t)b * a.Hkv + g) * a.C + id) * D;
  a.cand_key[(size_t)row * kTokCap + e] =
      order_key_f(exact_token_score<D>(kr, qs, lse2, G, a.sc2 * a.kv_scale[g]));
}

// one work group (1024 threads) per (sequence, kv group) row: the exact
// selection among the candidates (rescored by token_rescore_kernel), then the
// newest tokens
template <int D>
__global__ __launch_bounds__(1024) void token_zselect_kernel(TokenTopkArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scan[1024];
  __shared__ int res[2];
  __shared__ uint32_t wsum[32];
  __shared__ uint32_t cand_k[kTokCap];
  __shared__ int32_t cand_i[kTokCap];
  __shared__ __attribute__((aligned(16))) float qs[16 * D];
  __shared__ float lse2[16];
  const int row = blockIdx.x;
  const int b = row / a.Hkv, g = row % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int L = ctx_len(a.lens, b, a.C);
  const int ncand = max(0, L - a.n_recent);
  const int nrec = min(L, a.n_recent);
  const int kb = a.kb;
  const int t = threadIdx.x;
  int32_t* out = a.idx + (size_t)row * (kb + a.n_recent);
  const uint16_t* qg = (const uint16_t*)a.q + ((size_t)b * a.Hq + g * G) * D;
  for (int i = t; i < G * D; i += 1024) qs[i] = __uint_as_float((uint32_t)qg[i] << 16);
  if (t < G) lse2[t] = a.lse[(size_t)b * a.Hq + g * G + t] * kLog2e;
  __syncthreads();
  const float sck = a.sc2 * a.kv_scale[g];
  const uint8_t* kr = a.k + ((size_t)b * a.Hkv + g) * a.C * D;
  int nsel;
  const uint32_t ncnd = a.hist[(size_t)a.B * a.Hkv * 2 * 2048 + row];
  if (ncand <= kb) {
    for (int i = t; i < ncand; i += 1024) out[i] = i;
    nsel = ncand;
  } else if (ncnd <= (uint32_t)kTokCap) {
    // the candidates and their exact keys in ascending token order (each
    // segment's run is in order, and runs follow their segments)
    const int32_t* ci = a.cand_idx + (size_t)row * kTokCap;
    const uint32_t* ck = a.cand_key + (size_t)row * kTokCap;
    const uint32_t* sg = a.seg + (size_t)row * a.nseg * 2;
    const int nsg = (ncand + kTokSeg - 1) / kTokSeg;
    int off = 0;
    for (int q = 0; q < nsg; ++q) {
      const int base = (int)sg[2 * q], cnt = (int)sg[2 * q + 1];
      for (int e = t; e < cnt; e += 1024) {
        cand_i[off + e] = ci[base + e];
        cand_k[off + e] = ck[base + e];
      }
      off += cnt;
    }
    __syncthreads();
    uint32_t thr;
    int need_eq;
    radix_kth((int)ncnd, kb, [&](int i) { return cand_k[i]; }, hist, scan, res, &thr, &need_eq);
    emit_selected((int)ncnd, thr, need_eq, [&](int i) { return cand_k[i]; }, [&](int i) { return cand_i[i]; }, out,
                  wsum);
    nsel = kb;
  } else {
    // too many candidates: exact keys for the whole row, then the same select
    uint32_t* keys = a.keys + (size_t)row * a.C;
    for (int i = t; i < ncand; i += 1024)
      keys[i] = order_key_f(exact_token_score<D>(kr + (size_t)i * D, qs, lse2, G, sck));
    __threadfence_block();
    __syncthreads();
    uint32_t thr;
    int need_eq;
    radix_kth(ncand, kb, [&](int i) { return keys[i]; }, hist, scan, res, &thr, &need_eq);
    emit_selected(ncand, thr, need_eq, [&](int i) { return keys[i]; }, [](int i) { return i; }, out, wsum);
    nsel = kb;
  }
  for (int r = t; r < nrec; r += 1024) out[nsel + r] = L - nrec + r;
  for (int r = nsel + nrec + t; r < kb + a.n_recent; r += 1024) out[r] = -1;
}

// ============================================ token-level sparse layer (fp8)
// One work group (8 waves) per (b, g); work items are tiles of 64 consecutive
// entries of the ascending token list (-1 padding at the end).  Keys and
// values of the selected tokens are gathered straight from the fp8 caches;
// no window branch and no gate (the newest tokens are part of the list).
template <int D>
__global__ __launch_bounds__(512) void decode_sparse_token_kernel(DecodeSparseArgs a) {
  using Tt = Tr<HS_BF16>;
  using Frag = Tt::Frag;
  using Eng = WaveAttn<HS_BF16, D, 1>;
  constexpr int NW = 8;
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ int sm_wtot[NW];
  // canonical selection list (2 x cap words); after the tile loop the same
  // memory holds the waves' partial outputs [NW][G][D] for the merge
  extern __shared__ uint32_t dyn[];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int bg = blockIdx.x;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int L = ctx_len(a.lens, b, a.C);
  const int G = a.Hq / a.Hkv;
  const int col = lane & 15;
  const int h = g * G + col;
  const int r16 = lane & 15, q8 = 8 * (lane >> 4), q4 = (lane >> 4) << 2;
  const float sk = a.kv_scale[g], sv = a.kv_scale[a.Hkv + g];
  const float sc2 = a.sc2 * sk;
  Eng eng;
  eng.reset();
  // the query fragments are requested first, so that their latency overlaps
  // the list canonicalisation; head_dim is taken in the order of fp8_kdim
#pragma unroll
  for (int ks = 0; ks < Eng::NS; ++ks) {
    const Frag f = Tt::ld((const char*)a.q + ((size_t)(b * a.Hq + (col < G ? h : g * G)) * D + fp8_kdim<D>(lane, ks)) * 2);
    eng.qf[0][ks] = col < G ? f : Tt::zero();
  }
  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * a.C * D;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * a.C * D;
  float bmax[1], bsum[1];
  int lo[1], hi[1];

  // A tile's gathered rows are all requested at once, with unconditional
  // loads (lanes past the list repeat a live token; their logits are masked
  // and their values zeroed by selects): a load under a per-lane branch would
  // make the compiler wait for each one in turn.
  struct TileRaw {
    uint4 k[4][Eng::NS / 2];
    Fp8VRow<D> v[2][8];
  };
  auto issue = [&](int tsafe, TileRaw& r) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int tk = __shfl(tsafe, tile_key(c, r16));
#pragma unroll
      for (int j = 0; j < Eng::NS / 2; ++j) r.k[c][j] = *(const uint4*)(kg + (size_t)tk * D + fp8_kdim<D>(lane, 2 * j));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tk = __shfl(tsafe, 32 * u + q8 + e);
        r.v[u][e] = *(const Fp8VRow<D>*)(vg + (size_t)tk * D + (D / 16) * r16);
      }
  };
  // entries s0 .. s0+nvalid-1 of the live list are the tile's keys
  auto compute = [&](int s0, int nvalid, TileRaw& r) {
    lo[0] = col < G ? 0 : kNoKey;
    hi[0] = s0 + nvalid - 1;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool ok = 32 * u + q8 + e < nvalid;
        r.v[u][e] = ok ? r.v[u][e] : Fp8VRow<D>{};
      }
    Frag vc[4];
    auto ldK = [&](int c, int ks) { return fp8x8_frag(half_u4(r.k[c][ks >> 1], ks & 1)); };
    auto ldV = [&](int u, int mc) {
      if ((mc & 3) == 0) fp8_vfrag4_rows<D>(r.v[u], mc >> 2, vc);
      return vc[mc & 3];
    };
    eng.template tile<true, false>(ldK, ldV, s0, lo, hi, sc2, bmax, bsum);
  };

  // Work group blockIdx.y of gridDim.y takes every gridDim.y-th group of
  // eight tiles of the live list; wave w starts at tile it0.  The list's
  // first entries arrive in registers, where this thread's entry of tile it0
  // is v[blockIdx.y]; the wave requests that tile's rows before the list is
  // in LDS.  If the list then proves canonical (live ids ascending, padding
  // at the end, as the selection writes it) those are the tile's rows.
  static_assert(kTokSplitMax <= kSelU, "a work group's first tiles lie in the requested entries");
  const int32_t* il = a.idx + (size_t)(b * a.Hkv + g) * a.nsel;
  uint32_t lv[kSelU];
  sel_list_request<64 * NW>(il, a.nsel, lv);
  const int it0 = blockIdx.y * NW + w;
  uint32_t e = lv[0];
#pragma unroll
  for (int u = 1; u < kSelU; ++u) e = (int)blockIdx.y == u ? lv[u] : e;
  const uint32_t e0 = (uint32_t)__shfl((int)e, 0);
  TileRaw rs;
  issue(e < (uint32_t)L ? (int)e : (e0 < (uint32_t)L ? (int)e0 : 0), rs);

  // live selected tokens: ids i < L, each once, ascending
  const int cap = sel_list_cap(a.nsel);
  const uint32_t* sel = dyn + cap;
  bool canonical;
  const int nlive = canon_sel_list_from<64 * NW>(lv, il, a.nsel, (uint32_t)L, cap, dyn, dyn + cap, sm_wtot, canonical);
  const int ntile = (nlive + 63) / 64;
  int it = it0;
  if (canonical && it0 < ntile) {
    compute(64 * it0, min(64, nlive - 64 * it0), rs);
    it += gridDim.y * NW;
  }
  for (; it < ntile; it += gridDim.y * NW) {
    const int s0 = 64 * it;
    const int nvalid = min(64, nlive - s0);
    TileRaw r;
    issue((int)sel[s0 + min(lane, nvalid - 1)], r);
    compute(s0, nvalid, r);
  }

  const float lt = xlane_sum(eng.l[0]);
  __syncthreads();  // every wave is done with the list: its memory takes sm_o
  // [NW][G][D + 1]: with the odd row stride the 32 stores of each lane below
  // hit 64 distinct banks
  float* sm_o = (float*)dyn;
  if (lane < 16) {
    sm_m[w][col] = eng.m[0];
    sm_l[w][col] = lt;
  }
  if (col < G) {
#pragma unroll
    for (int mc = 0; mc < Eng::NM; ++mc)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[(w * G + col) * (D + 1) + fp8_vrow_dv<D>(mc, q4 + i)] = eng.o[0][mc][i];
  }
  __syncthreads();
  for (int el = threadIdx.x; el < G * D; el += 64 * NW) {
    const int c = el / D, d = el % D;
    // the sparse-branch sink joins here when this group writes o itself; the
    // merge kernel adds it to split partials
    const float sk = a.sinks && gridDim.y == 1 ? a.sinks[g * G + c] * kLog2e : -INFINITY;
    float M = fmaxf(kNegBig, sk);
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww][c]);
    float ls = fast_exp2(sk - M), os = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float wt = fast_exp2(sm_m[ww][c] - M);
      ls += wt * sm_l[ww][c];
      os += wt * sm_o[(ww * G + c) * (D + 1) + d];
    }
    if (gridDim.y == 1) {
      ((uint16_t*)a.o)[((size_t)b * a.Hq + g * G + c) * D + d] =
          (uint16_t)bf16_bits(ls > 0.f ? sv * os / ls : 0.f);
    } else {
      // partial state of this work group: unnormalised o, then m and l
      float* pp = a.part + (((size_t)bg * gridDim.y + blockIdx.y) * G + c) * (D + 2);
      pp[d] = os;
      if (d == 0) {
        pp[D] = M;
        pp[D + 1] = ls;
      }
    }
  }
}

// one work group per (b, g): merges the nsplit partial states of the token
// sparse layer
template <int D>
__global__ __launch_bounds__(1024) void decode_token_combine_kernel(DecodeSparseArgs a) {
  const int bg = blockIdx.x;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int G = a.Hq / a.Hkv;
  const float sv = a.kv_scale[a.Hkv + g];
  for (int el = threadIdx.x; el < G * D; el += 1024) {
    const int c = el / D, d = el % D;
    const float* pp = a.part + ((size_t)bg * a.nsplit * G + c) * (D + 2);
    const size_t st = (size_t)G * (D + 2);
    // all loads of the (at most kTokSplitMax) partials are issued together
    float m[kTokSplitMax], l[kTokSplitMax], x[kTokSplitMax];
#pragma unroll
    for (int sp = 0; sp < kTokSplitMax; ++sp) {
      const bool in = sp < a.nsplit;
      m[sp] = in ? pp[sp * st + D] : kNegBig;
      l[sp] = in ? pp[sp * st + D + 1] : 0.f;
      x[sp] = in ? pp[sp * st + d] : 0.f;
    }
    const float sk = a.sinks ? a.sinks[g * G + c] * kLog2e : -INFINITY;  // sparse-branch sink
    float M = fmaxf(kNegBig, sk);
#pragma unroll
    for (int sp = 0; sp < kTokSplitMax; ++sp) M = fmaxf(M, m[sp]);
    float ls = fast_exp2(sk - M), os = 0.f;
#pragma unroll
    for (int sp = 0; sp < kTokSplitMax; ++sp) {
      const float wt = fast_exp2(m[sp] - M);
      ls += wt * l[sp];
      os += wt * x[sp];
    }
    ((uint16_t*)a.o)[((size_t)b * a.Hq + g * G + c) * D + d] = (uint16_t)bf16_bits(ls > 0.f ? sv * os / ls : 0.f);
  }
}

// ================================================================ launchers
template <int D>
static void decode_full_dispatch(const DecodeFullArgs& a, dim3 grid, hipStream_t s) {
  // token mode (logits or bounds) runs on fp8 caches and block mode on bf16
  // caches; the host has checked the pairing
  if (a.kv_dtype == HS_FP8_E4M3) {
    if (a.token == 2) hipLaunchKernelGGL((decode_full_kernel<D, 2, HS_FP8_E4M3>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((decode_full_kernel<D, 1, HS_FP8_E4M3>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((decode_full_kernel<D, 0, HS_BF16>), grid, dim3(256), 0, s, a);
  }
}

hipError_t launch_decode_full(const DecodeFullArgs& a, int D, hipStream_t s) {
  const long units = (long)a.B * a.Hkv * a.nch;  // upper bound of the live units
  dim3 grid((unsigned)((units + 3) / 4));
  if (D == 128) decode_full_dispatch<128>(a, grid, s);
  else decode_full_dispatch<64>(a, grid, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)((long)a.B * a.Hq));
  if (D == 128) hipLaunchKernelGGL(decode_combine_kernel<128>, g2, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(decode_combine_kernel<64>, g2, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_sparse(const DecodeSparseArgs& a, int D, hipStream_t s) {
  dim3 grid((unsigned)(a.B * a.Hkv));
  const size_t lds = 2 * (size_t)sel_list_cap(a.nsel) * sizeof(uint32_t);
  if (D == 128) hipLaunchKernelGGL(decode_sparse_kernel<128>, grid, dim3(512), lds, s, a);
  else hipLaunchKernelGGL(decode_sparse_kernel<64>, grid, dim3(512), lds, s, a);
  return hipGetLastError();
}

}  // namespace hs

namespace hs {

hipError_t launch_token_topk(const TokenTopkArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.Hkv;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(256), dim3(256), 0, s, a.hist, rows * 2 * 2048 + rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(token_keys_kernel, dim3((unsigned)rows, (unsigned)((a.C + 4095) / 4096)), dim3(256), 0,
                     s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 seg((unsigned)rows, (unsigned)((a.C + kTokSeg - 1) / kTokSeg));
  hipLaunchKernelGGL(token_hist2_kernel, seg, dim3(1024), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(token_cand_kernel, seg, dim3(1024), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(token_select_kernel, dim3((unsigned)rows), dim3(1024), 0, s, a);
  return hipGetLastError();
}

// the histograms and counters were cleared by the full layer's merge kernel
hipError_t launch_token_topk_bounds(const TokenTopkArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.Hkv;
  hipError_t e;
  hipLaunchKernelGGL(token_zhist_kernel, dim3((unsigned)rows, (unsigned)((a.C + 4095) / 4096)), dim3(256), 0,
                     s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 seg((unsigned)rows, (unsigned)((a.C + kTokSeg - 1) / kTokSeg));
  hipLaunchKernelGGL(token_zcand_kernel, seg, dim3(1024), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 rs((unsigned)rows, (unsigned)(kTokCap / 256));
  if (a.D == 128) hipLaunchKernelGGL(token_rescore_kernel<128>, rs, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(token_rescore_kernel<64>, rs, dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.D == 128) hipLaunchKernelGGL(token_zselect_kernel<128>, dim3((unsigned)rows), dim3(1024), 0, s, a);
  else hipLaunchKernelGGL(token_zselect_kernel<64>, dim3((unsigned)rows), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_sparse_token(const DecodeSparseArgs& a, int D, hipStream_t s) {
  dim3 grid((unsigned)(a.B * a.Hkv), (unsigned)a.nsplit);
  // the selection list, or the eight waves' partial outputs after it
  const size_t lds =
      std::max(2 * (size_t)sel_list_cap(a.nsel), (size_t)8 * (a.Hq / a.Hkv) * (D + 1)) * sizeof(uint32_t);
  if (D == 128) hipLaunchKernelGGL(decode_sparse_token_kernel<128>, grid, dim3(512), lds, s, a);
  else hipLaunchKernelGGL(decode_sparse_token_kernel<64>, grid, dim3(512), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  dim3 g2((unsigned)(a.B * a.Hkv));
  if (D == 128) hipLaunchKernelGGL(decode_token_combine_kernel<128>, g2, dim3(1024), 0, s, a);
  else hipLaunchKernelGGL(decode_token_combine_kernel<64>, g2, dim3(1024), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs
