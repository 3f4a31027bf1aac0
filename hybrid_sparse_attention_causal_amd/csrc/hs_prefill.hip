// hs_prefill.hip -- prefill kernels of the hybrid block on gfx950.
//
//  full_prefill_kernel   full causal GQA attention + per-64-block scores in one
//                        pass (HySparse explainer 3.4.1, "Modified
//                        FlashAttention Kernel"; paper 3.2)
//  block_topk_kernel     exp(raw - LSE), GQA group maximum, top-k
//                        (explainer 3.4.1 eq. S_g, 3.4.2; paper 3.2)
//  sparse_prefill_kernel one sparse layer: gathered-block branch over the
//                        shared K/V + sliding window over the layer's own K'/V'
//                        + sigmoid gates (explainer 3.4.3; paper 3.1, 3.3)
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {

__device__ __forceinline__ uint4 keep_u4(uint4 v, int n_keep, int es) {
  // zero the 16-byte chunk's elements with index >= n_keep (es = element bytes)
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const int nb = n_keep * es;  // bytes kept
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b0 = 4 * i;
    if (b0 >= nb) w[i] = 0u;
    else if (b0 + 4 > nb) w[i] &= (1u << (8 * (nb - b0))) - 1u;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ===================================================================== full
// Work group = 4 wavefronts.  With Gw = min(G, 4) query heads of one kv group
// per work group, wave w takes head hb*Gw + w%Gw and 16*NT consecutive query
// positions; all waves of a group share the same K/V tiles, staged through LDS
// (double-buffered, K rows stored in S^T row order, V tiles copied d-major as
// they are in memory).  Grid: x = head blocks (fast, so consecutive groups land
// on the same XCD when Hq/Gw is a multiple of 8), y = position tiles, longest
// (latest) first.
template <int DT, int D, int NT, int SCORE_LSE>
__global__ __launch_bounds__(256, (DT == HS_F32 && D == 128) ? 1 : 2) void full_prefill_kernel(FullPrefillArgs a) {
  using Tt = Tr<DT>;
  using Eng = WaveAttn<DT, D, NT>;
  constexpr int ES = Tt::ES;
  constexpr int KS = D * ES + 16;   // LDS row stride (bytes) of the K tile
  constexpr int VS = 64 * ES + 16;  // LDS row stride of the d-major V tile
  constexpr int KB = 64 * KS, VB = D * VS;
  constexpr int KCH = D * ES / 16, VCH = 64 * ES / 16;  // 16-byte chunks per row
  constexpr int NK = 64 * KCH / 256, NV = D * VCH / 256;
  constexpr int PWAVE = 16 * NT;
  __shared__ __attribute__((aligned(16))) char smem[2 * (KB + VB)];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int G = a.Hq / a.Hkv;
  const int Gw = G < 4 ? G : 4;
  const int PW = 4 / Gw;
  const int nhb = a.Hq / Gw;
  const int hb = blockIdx.x % nhb, b = blockIdx.x / nhb;
  const int pt = gridDim.y - 1 - blockIdx.y;
  const int posw = PW * PWAVE;
  const int h = hb * Gw + (w % Gw);
  const int g = h / G;
  const int wg_p0 = pt * posw;
  const int p0 = wg_p0 + (w / Gw) * PWAVE;
  const int T = a.T;
  const int jmax = (min(T, wg_p0 + posw) - 1) >> 6;
  const int plast = min(T - 1, p0 + PWAVE - 1);

  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * T * D * ES;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * a.nblk * D * 64 * ES;

  uint4 kreg[NK], vreg[NV];
  auto gload = [&](int j) {
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      const int ci = threadIdx.x + 256 * n;
      const int kk = ci / KCH, col = ci % KCH;
      const int key = 64 * j + kk;
      kreg[n] = key < T ? *(const uint4*)(kg + (size_t)key * D * ES + col * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int ci = threadIdx.x + 256 * n;
      const int dd = ci / VCH, col = ci % VCH;
      uint4 x = *(const uint4*)(vg + ((size_t)j * D + dd) * 64 * ES + col * 16);
      const int k0 = 64 * j + col * (16 / ES);
      if (k0 + 16 / ES > T) x = keep_u4(x, T - k0, ES);
      vreg[n] = x;
    }
  };
  auto sstore = [&](int buf) {
    char* ksm = smem + buf * (KB + VB);
    char* vsm = ksm + KB;
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      const int ci = threadIdx.x + 256 * n;
      const int kk = ci / KCH, col = ci % KCH;
      *(uint4*)(ksm + tile_row(kk) * KS + col * 16) = kreg[n];
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int ci = threadIdx.x + 256 * n;
      const int dd = ci / VCH, col = ci % VCH;
      *(uint4*)(vsm + dd * VS + col * 16) = vreg[n];
    }
  };

  Eng eng;
  eng.reset();
  int lo[NT], hi[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int t = p0 + 16 * nt + (lane & 15);
    lo[nt] = 0;
    hi[nt] = t < T ? t : -1;
#pragma unroll
    for (int ks = 0; ks < Eng::NS; ++ks) {
      eng.qf[nt][ks] = t < T ? Tt::ld((const char*)a.q +
                                      (((size_t)(b * T + t) * a.Hq + h) * D + 32 * ks + 8 * (lane >> 4)) * ES)
                             : Tt::zero();
    }
  }

  gload(0);
  sstore(0);
  __syncthreads();
  for (int j = 0; j <= jmax; ++j) {
    const int buf = j & 1;
    if (j < jmax) gload(j + 1);
    if (64 * j <= plast) {
      const char* ksm = smem + buf * (KB + VB);
      const char* vsm = ksm + KB;
      auto ldK = [&](int c, int ks) {
        return Tt::ld(ksm + (16 * c + (lane & 15)) * KS + (32 * ks + 8 * (lane >> 4)) * ES);
      };
      auto ldV = [&](int u, int mc) {
        return Tt::ld(vsm + (16 * mc + (lane & 15)) * VS + (32 * u + 8 * (lane >> 4)) * ES);
      };
      float bmax[NT], bsum[NT];
      if (64 * j + 63 > p0)
        eng.template tile<true, SCORE_LSE != 0>(ldK, ldV, 64 * j, lo, hi, a.sc2, bmax, bsum);
      else
        eng.template tile<false, SCORE_LSE != 0>(ldK, ldV, 64 * j, lo, hi, a.sc2, bmax, bsum);
      if ((lane >> 4) == 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int t = p0 + 16 * nt + lane;
          if (t < T && j <= (t >> 6)) {
            const float r = SCORE_LSE ? eng.m[nt] + fast_log2(bsum[nt]) : bmax[nt];
            a.raw[((size_t)(b * a.Hq + h) * T + t) * a.nblk + j] = r * kLn2;
          }
        }
      }
    }
    if (j < jmax) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float inv, l2;
    eng.finish(nt, inv, l2);
    const int t = p0 + 16 * nt + (lane & 15);
    if (t < T) {
      if ((lane >> 4) == 0) a.lse[(size_t)(b * a.Hq + h) * T + t] = l2 * kLn2;
      char* op = (char*)a.o + (((size_t)(b * T + t) * a.Hq + h) * D + 4 * (lane >> 4)) * ES;
#pragma unroll
      for (int mc = 0; mc < Eng::NM; ++mc) {
        const f32x4 v = eng.o[nt][mc];
        Tt::store4(op + 16 * mc * ES, v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      }
    }
  }
}

// ===================================================================== top-k
// One wavefront per (sequence, kv group, query row).  Candidate j sits in lane
// j % 64, slot j / 64.  The score of a candidate is x = max_h (raw - LSE_h),
// the log of S_g; the k-th largest order key is found by a 32-step bitwise
// search with wave ballots, equal keys are resolved towards smaller j, and the
// selected ids are emitted in ascending order.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int MAXI>
__global__ __launch_bounds__(256) void block_topk_kernel(TopkArgs a) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int R = a.R;
  if (row >= (long)a.B * a.Hkv * R) return;
  const int tr = (int)(row % R);
  const int bg = (int)(row / R);
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int t = a.kv_lens ? a.kv_lens[b] - 1 : tr;
  const int G = a.Hq / a.Hkv;
  const int nvis = (t >> 6) + 1;
  const int ncand = (t >> 6) + (a.diag ? 1 : 0);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  float x[MAXI];
#pragma unroll
  for (int i = 0; i < MAXI; ++i) x[i] = -INFINITY;
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    const float* rp = a.raw + ((size_t)(b * a.Hq + h) * R + tr) * a.raw_stride;
    const float ls = a.lse[(size_t)(b * a.Hq + h) * R + tr];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int j = i * 64 + lane;
      if (j < nvis) x[i] = fmaxf(x[i], rp[j] - ls);
    }
  }
  const size_t orow = (size_t)(b * a.Hkv + g) * R + tr;
  if (a.gs) {
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int j = i * 64 + lane;
      if (j < nvis) a.gs[orow * a.raw_stride + j] = expf(x[i]);
    }
  }
  uint32_t u[MAXI];
#pragma unroll
  for (int i = 0; i < MAXI; ++i) u[i] = (i * 64 + lane < ncand) ? order_key(x[i]) : 0u;

  const int kb = a.kb;
  int32_t* out = a.idx + orow * kb;
  const bool all = ncand <= kb;
  uint32_t thr = 0;
  int need_eq = 0;
  if (!all) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = thr | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < MAXI; ++i) cnt += __popcll(__ballot(u[i] >= c));
      if (cnt >= kb) thr = c;
    }
    int gt = 0;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) gt += __popcll(__ballot(u[i] > thr));
    need_eq = kb - gt;
  }
  int base = 0;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int j = i * 64 + lane;
    bool s;
    if (all) {
      s = j < ncand;
    } else {
      s = u[i] > thr;
      const bool eq = (u[i] == thr) && (j < ncand);
      const uint64_t em = __ballot(eq);
      const int rank = __popcll(em & lt_mask);
      s = s || (eq && rank < need_eq);
      const int ne = __popcll(em);
      need_eq -= ne < need_eq ? ne : need_eq;
    }
    const uint64_t sm = __ballot(s);
    if (s) out[base + __popcll(sm & lt_mask)] = j;
    base += __popcll(sm);
  }
  for (int p = base + lane; p < kb; p += 64) out[p] = -1;
}

// ==================================================================== sparse
// One wavefront per (sequence, kv group, P consecutive query positions) with
// P = 16*NT/G, so its 16*NT MFMA columns are the G heads of P positions.  The
// wave walks the union of its positions' selected blocks in ascending order
// (a bitset in LDS), gathering each 64-key block of the shared K/V straight
// from global memory into MFMA operands; columns whose position did not select
// a block are masked.  The window branch then runs over keys
// [t0-W+1, t0+P-1] of the layer's own K'/V' with per-column masks, and the
// two normalised branches are merged by the sigmoid gates.
template <int DT, int D, int NT>
__global__ __launch_bounds__(256, 2) void sparse_prefill_kernel(SparsePrefillArgs a) {
  using Tt = Tr<DT>;
  using Eng = WaveAttn<DT, D, NT>;
  using Frag = typename Tt::Frag;
  constexpr int ES = Tt::ES;
  extern __shared__ uint32_t shbits[];

  // XCD-aware remap: consecutive ids go round-robin over the 8 XCDs; give each
  // XCD a contiguous range of work groups (same kv group -> shared L2).
  const int per = gridDim.x >> 3;
  const int wgid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const bool live = wgid < a.nwg;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int T = a.T;
  const int G = a.Hq / a.Hkv;
  const int P = 16 * NT / G;
  const int npg = (T + P - 1) / P;
  const int npg4 = (npg + 3) >> 2;
  const int bg = wgid / npg4;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int pg = (wgid % npg4) * 4 + w;
  const int t0 = pg * P;
  const int nw32 = (a.nblk + 31) >> 5;
  uint32_t* U = shbits + w * (1 + P) * nw32;
  uint32_t* S = U + nw32;

  for (int i = lane; i < (1 + P) * nw32; i += 64) U[i] = 0u;
  __syncthreads();
  if (live) {
    for (int e = lane; e < P * a.topk; e += 64) {
      const int p = e / a.topk;
      const int t = t0 + p;
      if (t < T) {
        const int j = a.idx[((size_t)(b * a.Hkv + g) * T + t) * a.topk + (e % a.topk)];
        if (j >= 0 && j < a.nblk) {
          atomicOr(&U[j >> 5], 1u << (j & 31));
          atomicOr(&S[p * nw32 + (j >> 5)], 1u << (j & 31));
        }
      }
    }
  }
  __syncthreads();
  if (!live || t0 >= T) return;

  int tcol[NT], hcol[NT], pcol[NT];
  Eng eng;
  eng.reset();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = 16 * nt + (lane & 15);
    pcol[nt] = col / G;
    tcol[nt] = t0 + pcol[nt];
    hcol[nt] = g * G + col % G;
#pragma unroll
    for (int ks = 0; ks < Eng::NS; ++ks) {
      eng.qf[nt][ks] = tcol[nt] < T
                           ? Tt::ld((const char*)a.q +
                                    (((size_t)(b * T + tcol[nt]) * a.Hq + hcol[nt]) * D + 32 * ks + 8 * (lane >> 4)) * ES)
                           : Tt::zero();
    }
  }

  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * T * D * ES;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * a.nblk * D * 64 * ES;
  const int r16 = lane & 15, q8 = 8 * (lane >> 4);
  int lo[NT], hi[NT];
  float bmax[NT], bsum[NT];

  // ---- branch 1: gathered blocks of the shared K/V
  for (int wi = 0; wi < nw32; ++wi) {
    uint32_t word = __builtin_amdgcn_readfirstlane(U[wi]);
    while (word) {
      const int bit = __builtin_ctz(word);
      word &= word - 1;
      const int j = wi * 32 + bit;
      const int kbase = 64 * j;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bool sel = (S[pcol[nt] * nw32 + wi] >> bit) & 1u;
        lo[nt] = sel ? 0 : kNoKey;
        hi[nt] = tcol[nt] < T ? tcol[nt] : -1;
      }
      const bool full = kbase + 64 <= T;
      auto ldK = [&](int c, int ks) {
        const int key = kbase + tile_key(c, r16);
        return (full || key < T) ? Tt::ld(kg + ((size_t)key * D + 32 * ks + q8) * ES) : Tt::zero();
      };
      auto ldV = [&](int u, int mc) {
        const Frag f = Tt::ld(vg + (((size_t)j * D + 16 * mc + r16) * 64 + 32 * u + q8) * ES);
        if (full) return f;
        const int k0 = kbase + 32 * u + q8;
        return Tt::keep(f, T - k0);
      };
      eng.template tile<true, false>(ldK, ldV, kbase, lo, hi, a.sc2, bmax, bsum);
    }
  }

  // normalise branch 1 and apply its gate
  f32x4 acc[NT][Eng::NM];
  float gw[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float inv, l2;
    eng.finish(nt, inv, l2);
    float g0 = 1.f, g1 = 1.f;
    if (a.gates && tcol[nt] < T) {
      const float2 gl = *(const float2*)(a.gates + ((size_t)(b * T + tcol[nt]) * a.Hq + hcol[nt]) * 2);
      g0 = 1.f / (1.f + expf(-gl.x));
      g1 = 1.f / (1.f + expf(-gl.y));
    }
    gw[nt] = g1;
    const float s0 = inv * g0;
#pragma unroll
    for (int mc = 0; mc < Eng::NM; ++mc) acc[nt][mc] = eng.o[nt][mc] * s0;
  }

  // ---- branch 2: sliding window over the layer's own K'/V'
  if (a.W > 0) {
    eng.reset();
    const char* ksg = (const char*)a.ks + (size_t)(b * a.Hkv + g) * T * D * ES;
    const char* vsg = (const char*)a.vs + (size_t)(b * a.Hkv + g) * a.nblk * D * 64 * ES;
    const int wlo = max(0, t0 - a.W + 1);
    const int whi = min(T - 1, t0 + P - 1);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      lo[nt] = tcol[nt] - a.W + 1;
      hi[nt] = tcol[nt] < T ? tcol[nt] : -1;
    }
    for (int kbase = wlo & ~7; kbase <= whi; kbase += 64) {
      auto ldK = [&](int c, int ks) {
        const int key = kbase + tile_key(c, r16);
        return key < T ? Tt::ld(ksg + ((size_t)key * D + 32 * ks + q8) * ES) : Tt::zero();
      };
      auto ldV = [&](int u, int mc) {
        const int k0 = kbase + 32 * u + q8;
        if (k0 >= T) return Tt::zero();
        const Frag f = Tt::ld(vsg + (((size_t)(k0 >> 6) * D + 16 * mc + r16) * 64 + (k0 & 63)) * ES);
        return k0 + 8 <= T ? f : Tt::keep(f, T - k0);
      };
      eng.template tile<true, false>(ldK, ldV, kbase, lo, hi, a.sc2, bmax, bsum);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float inv, l2;
      eng.finish(nt, inv, l2);
      const float s1 = inv * gw[nt];
#pragma unroll
      for (int mc = 0; mc < Eng::NM; ++mc) acc[nt][mc] += eng.o[nt][mc] * s1;
    }
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (tcol[nt] < T) {
      char* op = (char*)a.o + (((size_t)(b * T + tcol[nt]) * a.Hq + hcol[nt]) * D + 4 * (lane >> 4)) * ES;
#pragma unroll
      for (int mc = 0; mc < Eng::NM; ++mc) {
        const f32x4 v = acc[nt][mc];
        Tt::store4(op + 16 * mc * ES, v[0], v[1], v[2], v[3]);
      }
    }
  }
}

// ================================================================ launchers
template <int DT, int D>
static hipError_t full_dispatch(const FullPrefillArgs& a, int score_lse, hipStream_t s) {
  constexpr int NT = 2;
  const int G = a.Hq / a.Hkv;
  const int Gw = G < 4 ? G : 4;
  const int posw = (4 / Gw) * 16 * NT;
  dim3 grid(a.B * (a.Hq / Gw), (a.T + posw - 1) / posw);
  if (score_lse)
    hipLaunchKernelGGL((full_prefill_kernel<DT, D, NT, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((full_prefill_kernel<DT, D, NT, 0>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_full_prefill(const FullPrefillArgs& a, int dtype, int D, int score_lse,
                               hipStream_t s) {
  if (dtype == HS_BF16) return D == 64 ? full_dispatch<HS_BF16, 64>(a, score_lse, s)
                                       : full_dispatch<HS_BF16, 128>(a, score_lse, s);
  return D == 64 ? full_dispatch<HS_F32, 64>(a, score_lse, s) : full_dispatch<HS_F32, 128>(a, score_lse, s);
}

hipError_t launch_block_topk(const TopkArgs& a, int max_blocks, hipStream_t s) {
  const long rows = (long)a.B * a.Hkv * a.R;
  dim3 grid((unsigned)((rows + 3) / 4));
  if (max_blocks <= 64) hipLaunchKernelGGL(block_topk_kernel<1>, grid, dim3(256), 0, s, a);
  else if (max_blocks <= 128) hipLaunchKernelGGL(block_topk_kernel<2>, grid, dim3(256), 0, s, a);
  else if (max_blocks <= 256) hipLaunchKernelGGL(block_topk_kernel<4>, grid, dim3(256), 0, s, a);
  else if (max_blocks <= 512) hipLaunchKernelGGL(block_topk_kernel<8>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(block_topk_kernel<16>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int D, int NT>
static hipError_t sparse_dispatch(SparsePrefillArgs a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int P = 16 * NT / G;
  const int npg = (a.T + P - 1) / P;
  const int npg4 = (npg + 3) / 4;
  a.nwg = a.B * a.Hkv * npg4;
  const int per = (a.nwg + 7) / 8;
  const size_t lds = (size_t)4 * (1 + P) * ((a.nblk + 31) / 32) * sizeof(uint32_t);
  hipLaunchKernelGGL((sparse_prefill_kernel<DT, D, NT>), dim3(8 * per), dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_prefill(const SparsePrefillArgs& a, int dtype, int D, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (G <= 16) {
    if (dtype == HS_BF16) return D == 64 ? sparse_dispatch<HS_BF16, 64, 1>(a, s) : sparse_dispatch<HS_BF16, 128, 1>(a, s);
    return D == 64 ? sparse_dispatch<HS_F32, 64, 1>(a, s) : sparse_dispatch<HS_F32, 128, 1>(a, s);
  }
  if (dtype == HS_BF16) return D == 64 ? sparse_dispatch<HS_BF16, 64, 2>(a, s) : sparse_dispatch<HS_BF16, 128, 2>(a, s);
  return D == 64 ? sparse_dispatch<HS_F32, 64, 2>(a, s) : sparse_dispatch<HS_F32, 128, 2>(a, s);
}

}  // namespace hs
