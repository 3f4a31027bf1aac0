// hs_prefill_f8.hip -- prefill kernels on fp8 e4m3 queries, keys and values
// (head_dim 128), with fp8 matrix products (hs_device_f8.h).  The pages
// account the KV cache in FP8 (HySparse2 explainer, "What actually
// improved?"); here the full layer and the sparse layers read e4m3 codes with
// one fp32 scale per head and compute S^T and O^T on the fp8 matrix units.
//
//  full_prefill_f8_kernel    full causal layer + block scores, 8 waves,
//                            ping-pong schedule as full_prefill_pp_kernel
//  sparse_prefill_f8_kernel  one sparse layer (selected blocks of the shared
//                            K/V + window over the layer's own K'/V' + gates),
//                            four waves, two work groups per CU, as
//                            sparse_prefill_dual_kernel
#include "hs_device_f8.h"
#include "hs_internal.h"

namespace hs {

constexpr int kF8LA = 2;  // LDS fragment reads kept ahead of the fp8 products

// ===================================================================== full
// Work group: 8 waves, 8*32/G consecutive positions of one kv group; wave w
// holds two column tiles of the G heads of 16/G positions each.  All waves
// read the same K/V tile, staged by direct transfers into three named LDS
// buffers one tile ahead; waves w and w+4 run half a tile out of phase.
// Block scores are staged in LDS and written in runs of SPAN tiles.
template <int SCORE_LSE>
__global__ __launch_bounds__(512, 1) void full_prefill_f8_kernel(FullPrefillArgs a) {
  constexpr int NT = 2;
  constexpr int D = 128;
  using Eng = WaveAttnF8<false>;
  using St = TileStageF8<512>;
  constexpr int NW = 8;
  __shared__ __attribute__((aligned(16))) char tile0[St::BYTES];
  __shared__ __attribute__((aligned(16))) char tile1[St::BYTES];
  __shared__ __attribute__((aligned(16))) char tile2[St::BYTES];
  constexpr int SPAN = 32;
  constexpr int SROW = SPAN + 4;
  __shared__ __attribute__((aligned(16))) float sbuf[8][NT * 16][SROW];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool lag = w >= 4;
  const int T = a.T;
  const int G = a.Hq / a.Hkv;
  const int PT = 16 / G;
  const int PW = NT * PT;
  const int PWG = NW * PW;
  const int nwg_bg = (T + PWG - 1) / PWG;
  const WgSlot ws = wg_slot(a.B * a.Hkv, nwg_bg);
  const bool live = ws.live;
  const int bg = ws.bg;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int t0 = ws.pblk * PWG;
  const int tw0 = t0 + w * PW;
  const int nitems = live ? ((min(T, t0 + PWG) - 1) >> 6) + 1 : 0;

  const int col = lane & 15;
  const int hcol = g * G + col % G;
  int tcol[NT], hicol[NT];
  float sc2[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    tcol[nt] = tw0 + nt * PT + col / G;
    hicol[nt] = (live && tcol[nt] < T) ? tcol[nt] : -1;
  }
  const float qk_scale = a.sc2 * a.q_scale[hcol] * a.kv_scale[g];
  const float v_scale = a.kv_scale[a.Hkv + g];
  Eng eng;
  eng.reset();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    sc2[nt] = qk_scale;
    eng.qf[nt] = hicol[nt] >= 0 ? f8_ld((const char*)a.q + ((size_t)(b * T + tcol[nt]) * a.Hq + hcol) * D +
                                        32 * (lane >> 4))
                                : f8_zero();
  }
  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * T * D;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * a.nblk * D * 64;
  St st;
  st.dma_init();
  auto issue = [&](int j, char* buf) { st.dma(buf, kg + (size_t)64 * j * D, vg + (size_t)j * D * 64, T - 64 * j); };
  if (nitems > 0) issue(0, tile0);
  wait_vmem();
  if (nitems > 0) st.dma_fix(tile0);
  __syncthreads();

  auto act_of = [&](int j) -> unsigned {
    unsigned act = 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) act |= (__ballot(hicol[nt] >= 64 * j) != 0ull ? 1u : 0u) << nt;
    return act;
  };
  int lo[NT], hi[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    lo[nt] = 0;
    hi[nt] = hicol[nt];
  }
  auto scores = [&](int j, const float* bmax, const float* bsum) {
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (hicol[nt] >= 64 * j) {
          const float r = SCORE_LSE ? eng.m[nt] + fast_log2(bsum[nt]) : bmax[nt];
          sbuf[w][nt * 16 + col][j % SPAN] = r * kLn2;
        }
      }
    }
  };
  const bool vec4 = (a.nblk & 3) == 0;
  constexpr int QR = SPAN / 4;
  auto flush = [&](int j) {
    const int j0 = j - j % SPAN;
#pragma unroll
    for (int i = 0; i < NT * 16 * QR / 64; ++i) {
      const int e = lane + 64 * i;
      const int r = e / QR, c = r & 15, nt = r >> 4;
      const int t = tw0 + nt * PT + c / G;
      const int jj = j0 + 4 * (e % QR);
      const int jl = live && t < T ? min(t >> 6, j) : -1;
      if (jj <= jl) {
        const float4 v = *(const float4*)&sbuf[w][r][4 * (e % QR)];
        float* dst = a.raw + ((size_t)(b * a.Hq + g * G + c % G) * T + t) * a.nblk + jj;
        if (vec4 && jj + 3 <= jl) {
          *(float4*)dst = v;
        } else {
          dst[0] = v.x;
          if (jj + 1 <= jl) dst[1] = v.y;
          if (jj + 2 <= jl) dst[2] = v.z;
          if (jj + 3 <= jl) dst[3] = v.w;
        }
      }
    }
  };
  float bmax[NT], bsum[NT];
  f32x4 sreg[NT][4];
  F8x32 pf = f8_zero();
  unsigned p_act = 0;
  auto step = [&](int st_i, const char* prev, const char* cur, char* next) {
    const unsigned c_act = st_i < nitems ? act_of(st_i) : 0u;
    if (st_i + 1 < nitems) issue(st_i + 1, next);
    auto ldV = [&](int mb) { return St::ldV(prev, mb); };
    auto ldK = [&](int c) { return St::ldK(cur, c); };
    if (lag && st_i >= 1 && p_act) {
      eng.template softmax<true, SCORE_LSE != 0>(sreg, 64 * (st_i - 1), lo, hi, sc2, bmax, bsum, pf, p_act);
      scores(st_i - 1, bmax, bsum);
    }
    if (lag && st_i >= 1 && (st_i - 1) % SPAN == SPAN - 1) flush(st_i - 1);
    __builtin_amdgcn_s_setprio(1);
    if (st_i >= 1 && p_act) eng.template pv<kF8LA>(pf, ldV);
    if (c_act) {
      eng.template qk<kF8LA>(ldK, sreg);
      __builtin_amdgcn_s_setprio(0);
      if (!lag) {
        eng.template softmax<true, SCORE_LSE != 0>(sreg, 64 * st_i, lo, hi, sc2, bmax, bsum, pf, c_act);
        scores(st_i, bmax, bsum);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (!lag && st_i < nitems && st_i % SPAN == SPAN - 1) flush(st_i);
    p_act = c_act;
    wait_vmem();
    if (st_i + 1 < nitems) st.dma_fix(next);
    __syncthreads();
  };
  for (int st_i = 0; st_i <= nitems; st_i += 3) {
    step(st_i, tile2, tile0, tile1);
    if (st_i + 1 > nitems) break;
    step(st_i + 1, tile0, tile1, tile2);
    if (st_i + 2 > nitems) break;
    step(st_i + 2, tile1, tile2, tile0);
  }
  if (nitems > 0 && (nitems - 1) % SPAN != SPAN - 1) flush(nitems - 1);

  float inv[NT], l2[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    eng.finish(nt, inv[nt], l2[nt]);
    if (hicol[nt] >= 0 && (lane >> 4) == 0) a.lse[(size_t)(b * a.Hq + hcol) * T + tcol[nt]] = l2[nt] * kLn2;
  }
  // O: the lane's column is column tile (lane/16)%2, column lane%16; value v
  // of block mb is head_dim row 32mb + 8(v/4) + 4(lane/32) + v%4
  const bool t1 = (lane >> 4) & 1;
  const int tl = t1 ? tcol[1] : tcol[0];
  if ((t1 ? hicol[1] : hicol[0]) >= 0) {
    const float sc = (t1 ? inv[1] : inv[0]) * v_scale;
    char* op = (char*)a.o + (((size_t)(b * T + tl) * a.Hq + hcol) * D + 4 * (lane >> 5)) * 2;
#pragma unroll
    for (int mb = 0; mb < Eng::NMB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& v = eng.o[mb];
        Tr<HS_BF16>::store4(op + (32 * mb + 8 * j) * 2, v[4 * j] * sc, v[4 * j + 1] * sc, v[4 * j + 2] * sc,
                            v[4 * j + 3] * sc);
      }
  }
}

// ==================================================================== sparse
// One sparse layer on fp8 inputs: two resident work groups of four waves per
// CU; wave w holds two column tiles, each the G heads of 16/G positions.
// Items are the window blocks of the group's positions, then the union of
// their selected blocks (selection bitsets per position, per wave and per
// group, in LDS).  Each item's K/V tile is transferred into one of two LDS
// buffers one item ahead.  The window branch closes first: its gated output
// is parked in the output rows (bf16) and the sparse branch, run in the same
// registers, adds its own when it closes.
//   window branch: logits scaled by q_scale[h] * swa_scale[0][g], values by
//                  swa_scale[1][g];
//   sparse branch: q_scale[h] * kv_scale[0][g], values kv_scale[1][g].
__global__ __launch_bounds__(256, 2) void sparse_prefill_f8_kernel(SparsePrefillArgs a) {
  constexpr int NT = 2;
  constexpr int D = 128;
  using Eng = WaveAttnF8<true>;
  using St = TileStageF8<256>;
  constexpr int NW = 4;
  __shared__ __attribute__((aligned(16))) char tile0[St::BYTES];
  __shared__ __attribute__((aligned(16))) char tile1[St::BYTES];
  extern __shared__ uint32_t dyn[];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int T = a.T;
  const int G = a.Hq / a.Hkv;
  const int PT = 16 / G;
  const int PW = NT * PT;
  const int PWG = NW * PW;
  const int nwg_bg = (T + PWG - 1) / PWG;
  const WgSlot ws = wg_slot(a.B * a.Hkv, nwg_bg);
  const bool live = ws.live;
  const int bg = ws.bg;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int t0 = ws.pblk * PWG;
  const int tw0 = t0 + w * PW;
  const int nw32 = (a.nblk + 31) >> 5;
  uint32_t* U = dyn;
  uint32_t* Uw = U + nw32;
  uint32_t* S = Uw + NW * nw32;
  int* ulist = (int*)(S + PWG * nw32);
  int* nu_p = ulist + a.nblk;

  int jw0 = 0, nwin = 0;
  if (live && a.W > 0) {
    jw0 = max(0, t0 - a.W + 1) >> 6;
    nwin = (min(T - 1, t0 + PWG - 1) >> 6) - jw0 + 1;
  }

  const int col = lane & 15;
  const int hcol = g * G + col % G;
  int pcol[NT], tcol[NT], hicol[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    pcol[nt] = nt * PT + col / G;
    tcol[nt] = tw0 + pcol[nt];
    hicol[nt] = tcol[nt] < T ? tcol[nt] : -1;
  }
  Eng eng;
  eng.reset();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    eng.qf[nt] = (live && tcol[nt] < T)
                     ? f8_ld((const char*)a.q + ((size_t)(b * T + tcol[nt]) * a.Hq + hcol) * D + 32 * (lane >> 4))
                     : f8_zero();
  float gate0[NT], gate1[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    gate0[nt] = 1.f;
    gate1[nt] = 1.f;
    if (a.gates && live && tcol[nt] < T) {
      const float2 gl = *(const float2*)(a.gates + ((size_t)(b * T + tcol[nt]) * a.Hq + hcol) * 2);
      gate0[nt] = 1.f / (1.f + expf(-gl.x));
      gate1[nt] = 1.f / (1.f + expf(-gl.y));
    }
  }
  float sink0[NT], sink1[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    sink0[nt] = a.sinks ? a.sinks[hcol] * kLog2e : -INFINITY;
    sink1[nt] = a.sinks ? a.sinks[a.Hq + hcol] * kLog2e : -INFINITY;
  }
  // per-branch scales (the caches a branch does not read may be absent)
  const float qs = a.sc2 * a.q_scale[hcol];
  const float sc_sel = a.topk > 0 ? qs * a.kv_scale[g] : 0.f;
  const float vs_sel = a.topk > 0 ? a.kv_scale[a.Hkv + g] : 0.f;
  const float sc_win = a.W > 0 ? qs * a.swa_scale[g] : 0.f;
  const float vs_win = a.W > 0 ? a.swa_scale[a.Hkv + g] : 0.f;
  float sc2w[NT], sc2s[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    sc2w[nt] = sc_win;
    sc2s[nt] = sc_sel;
  }
  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * T * D;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * a.nblk * D * 64;
  const char* ksg = (const char*)a.ks + (size_t)(b * a.Hkv + g) * T * D;
  const char* vsg = (const char*)a.vs + (size_t)(b * a.Hkv + g) * a.nblk * D * 64;
  St st;
  st.dma_init();
  auto issue = [&](int i, char* buf) {
    const bool win = i < nwin;
    const int j = __builtin_amdgcn_readfirstlane(win ? jw0 + i : ulist[max(i - nwin, 0)]);
    st.dma(buf, (win ? ksg : kg) + (size_t)64 * j * D, (win ? vsg : vg) + (size_t)j * D * 64, T - 64 * j);
  };
  if (nwin > 0) issue(0, tile0);

  for (int i = threadIdx.x; i < (1 + NW + PWG) * nw32; i += 64 * NW) U[i] = 0u;
  __syncthreads();
  if (live) {
    for (int e = threadIdx.x; e < PWG * a.topk; e += 64 * NW) {
      const int p = e / a.topk;
      const int t = t0 + p;
      if (t < T) {
        const int j = a.idx[((size_t)(b * a.Hkv + g) * T + t) * a.topk + (e % a.topk)];
        if (j >= 0 && j < a.nblk && 64 * j <= t) atomicOr(&S[p * nw32 + (j >> 5)], 1u << (j & 31));
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NW * nw32; i += 64 * NW) {
    const int ww = i / nw32, k = i % nw32;
    uint32_t v = 0u;
    for (int p = 0; p < PW; ++p) v |= S[(ww * PW + p) * nw32 + k];
    Uw[i] = v;
  }
  __syncthreads();
  for (int k = threadIdx.x; k < nw32; k += 64 * NW) {
    uint32_t v = 0u;
    for (int ww = 0; ww < NW; ++ww) v |= Uw[ww * nw32 + k];
    U[k] = v;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    int base = 0;
    for (int w0 = 0; w0 < nw32; w0 += 64) {
      const uint32_t word = w0 + lane < nw32 ? U[w0 + lane] : 0u;
      const int cnt = __popc(word);
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      int pos = base + incl - cnt;
      uint32_t wd = word;
      while (wd) {
        ulist[pos++] = (w0 + lane) * 32 + __builtin_ctz(wd);
        wd &= wd - 1;
      }
      base += __shfl(incl, 63);
    }
    if (lane == 0) *nu_p = base;
  }
  __syncthreads();
  const int nu = live ? *nu_p : 0;
  const int nitems = nwin + nu;
  if (nwin == 0 && nitems > 0) issue(0, tile0);

  // close a branch: the lane's column is column tile (lane/16)%2; its O^T
  // rows are 32mb + 8j + 4(lane/32) + 0..3
  // the lane's own column: gates and sinks as values (no array indexed by lane)
  const bool t1 = (lane >> 4) & 1;
  const float gate0o = t1 ? gate0[1] : gate0[0], gate1o = t1 ? gate1[1] : gate1[0];
  const float sink0o = t1 ? sink0[1] : sink0[0], sink1o = t1 ? sink1[1] : sink1[0];
  const int tl = t1 ? tcol[1] : tcol[0];
  auto fold = [&](float gate, float sink, float vsc, bool first) {
    const float inv = eng.inv_own(sink);
    if (live && tl < T) {
      const float sc = inv * gate * vsc;
      char* op = (char*)a.o + (((size_t)(b * T + tl) * a.Hq + hcol) * D + 4 * (lane >> 5)) * 2;
#pragma unroll
      for (int mb = 0; mb < Eng::NMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16& o = eng.o[mb];
          f32x4 v = f32x4{o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]} * sc;
          char* dst = op + (32 * mb + 8 * j) * 2;
          if (!first) v += Tr<HS_BF16>::load4(dst);
          Tr<HS_BF16>::store4(dst, v[0], v[1], v[2], v[3]);
        }
    }
  };
  struct Pre {
    int j;
    uint32_t sw[NT];
  };
  auto fetch = [&](int i) {
    Pre p;
    const bool win = i < nwin;
    p.j = __builtin_amdgcn_readfirstlane(win ? jw0 + i : ulist[max(i - nwin, 0)]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) p.sw[nt] = S[(w * PW + pcol[nt]) * nw32 + (win ? 0 : p.j >> 5)];
    return p;
  };
  auto item = [&](int i, const Pre& p, int& kbase, int* lo, int* hi) -> unsigned {
    const bool win = i < nwin;
    kbase = 64 * p.j;
    unsigned act = 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const bool sel = (p.sw[nt] >> (p.j & 31)) & 1u;
      lo[nt] = win ? tcol[nt] - a.W + 1 : (sel ? 0 : kNoKey);
      hi[nt] = hicol[nt];
      const bool live_col = max(lo[nt], kbase) <= min(hi[nt], kbase + 63);
      act |= (__ballot(live_col) != 0ull ? 1u : 0u) << nt;
    }
    return act;
  };

  wait_vmem();
  if (nitems > 0) st.dma_fix(tile0);
  __syncthreads();

  f32x4 sreg[NT][4];
  float bmax[NT], bsum[NT];
  F8x32 pf;
  Pre pre{};
  if (nitems > 0) pre = fetch(0);
  auto step = [&](int st_i, const char* cur, char* next) {
    int kbase = 0, lo[NT], hi[NT];
    const unsigned act = item(st_i, pre, kbase, lo, hi);
    const bool win = st_i < nwin;
    if (st_i + 1 < nitems) {
      pre = fetch(st_i + 1);
      st.dma(next, (st_i + 1 < nwin ? ksg : kg) + (size_t)64 * pre.j * D,
             (st_i + 1 < nwin ? vsg : vg) + (size_t)pre.j * D * 64, T - 64 * pre.j);
    }
    if (st_i == nwin) {  // window branch closed: park it
      fold(gate1o, sink1o, vs_win, true);
      eng.reset();
    }
    if (act) {
      auto ldK = [&](int c) { return St::ldK(cur, c); };
      auto ldV = [&](int mb) { return St::ldV(cur, mb); };
      float sc2c[NT];  // this branch's scales (values, not a chosen pointer: no stack arrays)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sc2c[nt] = win ? sc2w[nt] : sc2s[nt];
      eng.template qk<kF8LA>(ldK, sreg);
      eng.template softmax<true, false>(sreg, kbase, lo, hi, sc2c, bmax, bsum, pf, act);
      eng.template pv<kF8LA>(pf, ldV);
    }
    wait_vmem();
    if (st_i + 1 < nitems) st.dma_fix(next);
    __syncthreads();
  };
  for (int st_i = 0; st_i < nitems; st_i += 2) {
    step(st_i, tile0, tile1);
    if (st_i + 1 >= nitems) break;
    step(st_i + 1, tile1, tile0);
  }
  if (nwin == nitems) {
    fold(gate1o, sink1o, vs_win, true);
  } else {
    fold(gate0o, sink0o, vs_sel, false);
  }
}

// ================================================================ launchers
hipError_t launch_full_prefill_f8(const FullPrefillArgs& a, int score_lse, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int PWG = 8 * (32 / G);
  const unsigned nwg = (unsigned)((long)a.B * a.Hkv * ((a.T + PWG - 1) / PWG));
  if (score_lse)
    hipLaunchKernelGGL(full_prefill_f8_kernel<1>, dim3(nwg), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(full_prefill_f8_kernel<0>, dim3(nwg), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_prefill_f8(const SparsePrefillArgs& a0, hipStream_t s) {
  SparsePrefillArgs a = a0;
  const int G = a.Hq / a.Hkv;
  const int PWG = 4 * (32 / G);
  const int nw32 = (a.nblk + 31) / 32;
  const size_t lds = ((size_t)(1 + 4 + PWG) * nw32 + a.nblk + 1) * sizeof(uint32_t);
  a.nwg = a.B * a.Hkv * ((a.T + PWG - 1) / PWG);
  hipLaunchKernelGGL(sparse_prefill_f8_kernel, dim3(a.nwg), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace hs
