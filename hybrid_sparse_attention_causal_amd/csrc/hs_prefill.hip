// hs_prefill.hip -- prefill kernels of the hybrid block on gfx950.
//
//  full layer: full causal GQA attention + per-64-block scores in one pass
//  (HySparse explainer 3.4.1, "Modified FlashAttention Kernel"; paper 3.2)
//    full_prefill_pp_kernel      8 waves, ping-pong schedule (G <= 16)
//    full_prefill_kernel         4 waves (fp32 with d = 128, or G > 16)
//  block_topk_kernel: exp(raw - LSE), GQA group maximum, top-k
//  (explainer 3.4.1 eq. S_g, 3.4.2; paper 3.2)
//  one sparse layer: gathered-block branch over the shared K/V + sliding
//  window over the layer's own K'/V' + sigmoid gates (explainer 3.4.3; paper
//  3.1, 3.3)
//    sparse_prefill_dual_kernel  4 waves, two work groups per CU (default)
//    sparse_prefill_pp_kernel    8 waves, ping-pong (selection bitsets too
//                                large for two groups per CU)
//    sparse_prefill_kernel       8 waves, one column tile each (fp32, d = 128)
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {


// ===================================================================== full
// Work group = 4 wavefronts.  With Gw = min(G, 4) query heads of one kv group
// per work group, wave w takes head hb*Gw + w%Gw and 16*NT consecutive query
// positions; all waves of a group share the same K/V tiles, staged through LDS
// by direct global-to-LDS transfers (double-buffered, K rows stored in S^T row
// order, V tiles d-major as they are in memory).  Grid: x = head blocks (fast,
// so consecutive groups land on the same XCD when Hq/Gw is a multiple of 8),
// y = position tiles, longest (latest) first.
template <int DT, int D, int NT, int SCORE_LSE>
__global__ __launch_bounds__(256, (DT == HS_F32 && D == 128) ? 1 : 2) void full_prefill_kernel(FullPrefillArgs a) {
  using Tt = Tr<DT>;
  using Eng = WaveAttn<DT, D, NT>;
  using St = TileStage<DT, D, 256>;
  constexpr int ES = Tt::ES;
  constexpr int PWAVE = 16 * NT;
  // two tile buffers as separate arrays, the loop unrolled by two: every
  // access names its buffer, so reads of one are not held up by the transfer
  // in flight into the other
  __shared__ __attribute__((aligned(16))) char buf0[St::BYTES];
  __shared__ __attribute__((aligned(16))) char buf1[St::BYTES];

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
  St st;
  st.dma_init();
  auto issue = [&](int j, char* buf) {
    st.dma(buf, kg + (size_t)64 * j * D * ES, vg + (size_t)j * D * 64 * ES, T - 64 * j);
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

  wait_vmem();
  issue(0, buf0);
  wait_vmem();
  st.dma_fix(buf0);
  __syncthreads();
  auto step = [&](int j, const char* cur, char* next) {
    if (j < jmax) issue(j + 1, next);
    if (64 * j <= plast) {
      auto ldK = [&](int c, int ks) { return St::ldK(cur, c, ks); };
      auto ldV = [&](int u, int mc) { return St::ldV(cur, u, mc); };
      float bmax[NT], bsum[NT];
      f32x4 s[NT][4];
      __builtin_amdgcn_s_setprio(1);
      eng.qk(ldK, s);
      __builtin_amdgcn_s_setprio(0);
      if (64 * j + 63 > p0)
        eng.template softmax<true, SCORE_LSE != 0>(s, 64 * j, lo, hi, a.sc2, bmax, bsum);
      else
        eng.template softmax<false, SCORE_LSE != 0>(s, 64 * j, lo, hi, a.sc2, bmax, bsum);
      __builtin_amdgcn_s_setprio(1);
      eng.pv(s, ldV);
      __builtin_amdgcn_s_setprio(0);
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
    wait_vmem();
    if (j < jmax) st.dma_fix(next);
    __syncthreads();
  };
  for (int j = 0; j <= jmax; j += 2) {
    step(j, buf0, buf1);
    if (j + 1 > jmax) break;
    step(j + 1, buf1, buf0);
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

// Full layer, 8-wavefront ping-pong variant (G <= 16): the work group takes
// 8*32/G consecutive positions of one kv group; wave w holds NT = 2 column
// tiles of the G heads of 16/G positions each (as in the sparse layer), all
// eight waves read the same K/V tile, staged by direct transfers into three
// named LDS buffers one tile ahead, and waves w / w+4 run half a tile out of
// phase (A: P(s-1)V | QK(s) | softmax(s), B: softmax(s-1) | P(s-1)V | QK(s)).
// Block scores are staged in LDS and written in runs of SPAN tiles.
template <int DT, int D, int SCORE_LSE>
__global__ __launch_bounds__(512, 2) void full_prefill_pp_kernel(FullPrefillArgs a) {
  constexpr int NT = 2;
  using Tt = Tr<DT>;
  using Eng = WaveAttn<DT, D, NT>;
  using St = TileStage<DT, D, 512>;
  constexpr int ES = Tt::ES;
  constexpr int NW = 8;
  __shared__ __attribute__((aligned(16))) char tile0[St::BYTES];
  __shared__ __attribute__((aligned(16))) char tile1[St::BYTES];
  __shared__ __attribute__((aligned(16))) char tile2[St::BYTES];
  // block scores of the last SPAN tiles, per wave and column (rows padded by 4
  // floats: the per-tile writes of 16 columns fall in distinct banks); 16
  // tiles with head_dim 64, so that two work groups still fit a CU
  constexpr int SPAN = D >= 128 ? 32 : 16;
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
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    tcol[nt] = tw0 + nt * PT + col / G;
    hicol[nt] = (live && tcol[nt] < T) ? tcol[nt] : -1;
  }
  Eng eng;
  eng.reset();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < Eng::NS; ++ks)
      eng.qf[nt][ks] =
          hicol[nt] >= 0
              ? Tt::ld((const char*)a.q + (((size_t)(b * T + tcol[nt]) * a.Hq + hcol) * D + 32 * ks + 8 * (lane >> 4)) * ES)
              : Tt::zero();
  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * T * D * ES;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * a.nblk * D * 64 * ES;
  St st;
  st.dma_init();
  auto issue = [&](int j, char* buf) {
    st.dma(buf, kg + (size_t)64 * j * D * ES, vg + (size_t)j * D * 64 * ES, T - 64 * j);
  };
  if (nitems > 0) issue(0, tile0);
  wait_vmem();
  if (nitems > 0) st.dma_fix(tile0);
  __syncthreads();

  // tile j for this wave: column tiles with a live key (key <= position)
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
  // Block scores of tile j, once its softmax is done, go to the wave's LDS
  // rows; every SPAN tiles (and after the last) they are written out as whole
  // runs of each score row.  One 4-byte store per tile and column left the
  // rows' lines partly written in L2 for many tiles, and most of them were
  // evicted and written back several times.
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
  // tiles j0 = j - j % SPAN .. j are scored: piece e of the NT*16*SPAN/4
  // float4 pieces takes row e/(SPAN/4) (column tile, column) and tiles
  // j0 + 4(e%(SPAN/4)) .. +3, those up to the row's last visible tile
  const bool vec4 = (a.nblk & 3) == 0;
  constexpr int QR = SPAN / 4;  // float4 pieces per row
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
  unsigned p_act = 0;
  const typename Eng::NoHook nohook;
  auto step = [&](int st_i, const char* prev, const char* cur, char* next) {
    const unsigned c_act = st_i < nitems ? act_of(st_i) : 0u;
    if (st_i + 1 < nitems) issue(st_i + 1, next);
    auto ldV = [&](int u, int mc) { return St::ldV(prev, u, mc); };
    auto ldK = [&](int c, int ks) { return St::ldK(cur, c, ks); };
    if (lag && st_i >= 1 && p_act) {
      eng.template softmax<true, SCORE_LSE != 0>(sreg, 64 * (st_i - 1), lo, hi, a.sc2, bmax, bsum, nohook, p_act);
      scores(st_i - 1, bmax, bsum);
    }
    if (lag && st_i >= 1 && (st_i - 1) % SPAN == SPAN - 1) flush(st_i - 1);
    __builtin_amdgcn_s_setprio(1);
    if (st_i >= 1 && p_act) eng.template pv<kFullLA>(sreg, ldV);
    if (c_act) {
      eng.template qk<kFullLA>(ldK, sreg);
      __builtin_amdgcn_s_setprio(0);
      if (!lag) {
        eng.template softmax<true, SCORE_LSE != 0>(sreg, 64 * st_i, lo, hi, a.sc2, bmax, bsum, nohook, c_act);
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

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float inv, l2;
    eng.finish(nt, inv, l2);
    if (hicol[nt] >= 0) {
      if ((lane >> 4) == 0) a.lse[(size_t)(b * a.Hq + hcol) * T + tcol[nt]] = l2 * kLn2;
      char* op = (char*)a.o + (((size_t)(b * T + tcol[nt]) * a.Hq + hcol) * D + 4 * (lane >> 4)) * ES;
#pragma unroll
      for (int mc = 0; mc < Eng::NM; ++mc) {
        const f32x4 v = eng.o[nt][mc];
        Tt::store4(op + 16 * mc * ES, v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      }
    }
  }
}

// ===================================================================== top-k
// One wavefront per RW consecutive (sequence, kv group, query row) rows.
// Candidate j sits in lane j % 64, slot j / 64.  The score of a candidate is
// x = max_h (raw - LSE_h), the log of S_g; the k-th largest order key is found
// by a bitwise search with wave ballots, equal keys are resolved towards
// smaller j, and the selected ids are emitted in ascending order.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// rows per wavefront: short rows are latency bound (one memory round trip per
// row), so a wave requests two rows' scores together
constexpr int topk_rows_per_wave(int maxi) { return maxi <= 4 ? 2 : 1; }

// selection of one row from its candidates' log scores x (lane's slots)
template <int MAXI>
__device__ __forceinline__ void topk_emit(const TopkArgs& a, const float (&x)[MAXI], int nvis,
                                          int ncand, size_t orow, int lane, uint64_t lt_mask) {
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
      if (cnt >= kb) {
        thr = c;
        // exactly kb keys reach c: they are the selection whatever the lower
        // bits (ties at thr are then all taken)
        if (cnt == kb) break;
      }
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

template <int MAXI>
__global__ __launch_bounds__(256) void block_topk_kernel(TopkArgs a) {
  constexpr int RW = topk_rows_per_wave(MAXI);
  const int lane = threadIdx.x & 63;
  const int R = a.R;
  const long nrows = (long)a.B * a.Hkv * R;
  const long row0 = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * RW;
  if (row0 >= nrows) return;
  const int G = a.Hq / a.Hkv;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // per row: a row past the last one repeats the last row's reads, and its
  // selection is not emitted
  int nvis[RW], ncand[RW], jlast[RW];
  size_t orow[RW], rbase[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const long row = min(row0 + r, nrows - 1);
    const int tr = (int)(row % R);
    const int bg = (int)(row / R);
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    const int t = a.kv_lens ? ctx_len(a.kv_lens, b, 64 * a.raw_stride) - 1 : tr;
    nvis[r] = (t >> 6) + 1;
    ncand[r] = (t >> 6) + (a.diag ? 1 : 0);
    jlast[r] = min(max(nvis[r] - 1, 0), a.raw_stride - 1);
    orow[r] = (size_t)(b * a.Hkv + g) * R + tr;
    rbase[r] = (size_t)(b * a.Hq + g * G) * R + tr;   // (b, head g*G, row tr)
  }

  // every load is unconditional (entries past the visible blocks re-read the
  // last visible one, a line the row fetches anyway, and are dropped by a
  // select): loads under a per-lane branch would be waited for one by one.
  // HB heads' rows of all RW rows are requested together (one memory round
  // trip per HB heads); a batch past the last head re-reads head G-1, which
  // leaves the maximum unchanged
  constexpr int HB = MAXI <= 4 ? 4 : (MAXI == 8 ? 2 : 1);
  float x[RW][MAXI];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int i = 0; i < MAXI; ++i) x[r][i] = -INFINITY;
  for (int hh0 = 0; hh0 < G; hh0 += HB) {
    float v[RW][HB][MAXI], ls[RW][HB];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int e = 0; e < HB; ++e) {
        const size_t hr = rbase[r] + (size_t)min(hh0 + e, G - 1) * R;
        const float* rp = a.raw + hr * a.raw_stride;
        ls[r][e] = a.lse[hr];
#pragma unroll
        for (int i = 0; i < MAXI; ++i) v[r][e][i] = rp[min(i * 64 + lane, jlast[r])];
      }
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int e = 0; e < HB; ++e)
#pragma unroll
        for (int i = 0; i < MAXI; ++i)
          x[r][i] = i * 64 + lane < nvis[r] ? fmaxf(x[r][i], v[r][e][i] - ls[r][e]) : x[r][i];
  }
#pragma unroll
  for (int r = 0; r < RW; ++r)
    if (row0 + r < nrows) topk_emit<MAXI>(a, x[r], nvis[r], ncand[r], orow[r], lane, lt_mask);
}

// ==================================================================== sparse
// One work group of NW wavefronts per (sequence, kv group, NW*PW consecutive
// query positions), PW = 16*NT/G: wave w owns positions t0 + w*PW .. +PW-1,
// and its 16*NT MFMA columns are the G heads of those positions.
// The work group walks, in ascending order, the union of the blocks its
// positions selected (bitsets in LDS), then the 64-key blocks of the layer's
// own K'/V' that cover its windows.  Each block is loaded once per work group
// into a double-buffered LDS tile (the global loads of the next items are in
// flight while the current one is computed); a wave computes a block only if
// one of its positions selected it (window: if it overlaps one of its
// windows), masking the columns that did not.  The two normalised branches are
// merged by the sigmoid gates.
template <int DT, int D, int NT, int NW, int NSTAGE>
__global__ __launch_bounds__(64 * NW, 2) void sparse_prefill_kernel(SparsePrefillArgs a) {
  using Tt = Tr<DT>;
  using Eng = WaveAttn<DT, D, NT>;
  using St = TileStage<DT, D, 64 * NW>;
  constexpr int ES = Tt::ES;
  __shared__ __attribute__((aligned(16))) char tiles[2 * St::BYTES];
  extern __shared__ uint32_t dyn[];

  // XCD-aware remap: consecutive ids go round-robin over the 8 XCDs; give each
  // XCD a contiguous range of work groups (same kv group -> shared L2).

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int T = a.T;
  const int G = a.Hq / a.Hkv;
  const int PW = 16 * NT / G;
  const int PWG = NW * PW;
  const int nwg_bg = (T + PWG - 1) / PWG;
  const WgSlot ws = wg_slot(a.B * a.Hkv, nwg_bg);
  const bool live = ws.live;
  const int bg = ws.bg;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int t0 = ws.pblk * PWG;
  const int tw0 = t0 + w * PW;
  const int nw32 = (a.nblk + 31) >> 5;
  uint32_t* U = dyn;                      // union of the work group
  uint32_t* Uw = U + nw32;                // union of each wave  [NW][nw32]
  uint32_t* S = Uw + NW * nw32;           // selection of each position [PWG][nw32]
  int* ulist = (int*)(S + PWG * nw32);    // ascending union, then its length
  int* nu_p = ulist + a.nblk;

  for (int i = threadIdx.x; i < (1 + NW + PWG) * nw32; i += 64 * NW) U[i] = 0u;
  __syncthreads();
  if (live) {
    for (int e = threadIdx.x; e < PWG * a.topk; e += 64 * NW) {
      const int p = e / a.topk;
      const int t = t0 + p;
      if (t < T) {
        const int j = a.idx[((size_t)(b * a.Hkv + g) * T + t) * a.topk + (e % a.topk)];
        if (j >= 0 && j < a.nblk && 64 * j <= t) {
          const uint32_t bit = 1u << (j & 31);
          atomicOr(&U[j >> 5], bit);
          atomicOr(&Uw[(p / PW) * nw32 + (j >> 5)], bit);
          atomicOr(&S[p * nw32 + (j >> 5)], bit);
        }
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // compact the union: wave 0 scans the words in order with a running count
    int base = 0;
    for (int w0 = 0; w0 < nw32; w0 += 64) {
      const uint32_t word = w0 + lane < nw32 ? U[w0 + lane] : 0u;
      int cnt = __popc(word);
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
  int jw0 = 0, nwin = 0;
  if (live && a.W > 0) {
    jw0 = max(0, t0 - a.W + 1) >> 6;
    nwin = (min(T - 1, t0 + PWG - 1) >> 6) - jw0 + 1;
  }
  const int nitems = nu + nwin;

  // per-lane columns: position tcol (of this wave), head hcol
  int tcol[NT], hcol[NT], pcol[NT], hicol[NT];
  Eng eng;
  eng.reset();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = 16 * nt + (lane & 15);
    pcol[nt] = col / G;
    tcol[nt] = tw0 + pcol[nt];
    hcol[nt] = g * G + col % G;
    hicol[nt] = tcol[nt] < T ? tcol[nt] : -1;
#pragma unroll
    for (int ks = 0; ks < Eng::NS; ++ks)
      eng.qf[nt][ks] = (live && tcol[nt] < T)
                           ? Tt::ld((const char*)a.q +
                                    (((size_t)(b * T + tcol[nt]) * a.Hq + hcol[nt]) * D + 32 * ks + 8 * (lane >> 4)) * ES)
                           : Tt::zero();
  }

  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * T * D * ES;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * a.nblk * D * 64 * ES;
  const char* ksg = (const char*)a.ks + (size_t)(b * a.Hkv + g) * T * D * ES;
  const char* vsg = (const char*)a.vs + (size_t)(b * a.Hkv + g) * a.nblk * D * 64 * ES;
  auto issue = [&](St& st, int i) {
    const bool win = i >= nu;
    const int j = win ? jw0 + (i - nu) : ulist[min(i, a.nblk - 1)];
    st.gload((win ? ksg : kg) + (size_t)64 * j * D * ES, (win ? vsg : vg) + (size_t)j * D * 64 * ES,
             T - 64 * j);
  };

  f32x4 acc[NT][Eng::NM];
  float gate0[NT], gate1[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    gate0[nt] = 1.f;
    gate1[nt] = 1.f;
    if (a.gates && live && tcol[nt] < T) {
      const float2 gl = *(const float2*)(a.gates + ((size_t)(b * T + tcol[nt]) * a.Hq + hcol[nt]) * 2);
      gate0[nt] = 1.f / (1.f + expf(-gl.x));
      gate1[nt] = 1.f / (1.f + expf(-gl.y));
    }
  }
  // per-head sink logits of the sparse (0) and window (1) branch, log2
  // units; -inf without sinks
  float sink0[NT], sink1[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    sink0[nt] = a.sinks ? a.sinks[hcol[nt]] * kLog2e : -INFINITY;
    sink1[nt] = a.sinks ? a.sinks[a.Hq + hcol[nt]] * kLog2e : -INFINITY;
  }
  auto fold = [&](const float* gate, const float* sink, bool first) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float inv, l2;
      eng.finish(nt, inv, l2, sink[nt]);
      const float sc = inv * gate[nt];
#pragma unroll
      for (int mc = 0; mc < Eng::NM; ++mc)
        acc[nt][mc] = first ? eng.o[nt][mc] * sc : acc[nt][mc] + eng.o[nt][mc] * sc;
    }
  };

  float bmax[NT], bsum[NT];
  int lo[NT], hi[NT];
  auto compute = [&](int i) {
    const char* buf = tiles + (i & 1) * St::BYTES;
    auto ldK = [&](int c, int ks) { return St::ldK(buf, c, ks); };
    auto ldV = [&](int u, int mc) { return St::ldV(buf, u, mc); };
    if (i < nu) {
      const int j = ulist[i];
      const bool mine = (__builtin_amdgcn_readfirstlane(Uw[w * nw32 + (j >> 5)]) >> (j & 31)) & 1u;
      if (mine) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bool sel = (S[(w * PW + pcol[nt]) * nw32 + (j >> 5)] >> (j & 31)) & 1u;
          lo[nt] = sel ? 0 : kNoKey;
          hi[nt] = hicol[nt];
        }
        eng.template tile<true, false>(ldK, ldV, 64 * j, lo, hi, a.sc2, bmax, bsum);
      }
    } else {
      const int j = jw0 + (i - nu);
      const bool mine = tw0 < T && 64 * j <= tw0 + PW - 1 && 64 * j + 63 >= tw0 - a.W + 1;
      if (mine) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          lo[nt] = tcol[nt] - a.W + 1;
          hi[nt] = hicol[nt];
        }
        eng.template tile<true, false>(ldK, ldV, 64 * j, lo, hi, a.sc2, bmax, bsum);
      }
    }
  };

  if (NSTAGE == 2) {
    // two register stages: the global loads of item i+2 are in flight while
    // item i is computed and item i+1 is written to LDS
    St st0, st1;
    if (nitems > 0) {
      issue(st0, 0);
      st0.sstore(tiles);
    }
    if (nitems > 1) issue(st1, 1);
    __syncthreads();
    auto step = [&](int i, St& ld_into, St& store_from) {
      if (i == nu) {
        fold(gate0, sink0, true);
        eng.reset();
      }
      if (i + 2 < nitems) issue(ld_into, i + 2);
      compute(i);
      if (i + 1 < nitems) store_from.sstore(tiles + ((i + 1) & 1) * St::BYTES);
      __syncthreads();
    };
    for (int i = 0; i < nitems; i += 2) {
      step(i, st0, st1);
      if (i + 1 < nitems) step(i + 1, st1, st0);
    }
  } else {
    St st;
    if (nitems > 0) {
      issue(st, 0);
      st.sstore(tiles);
    }
    __syncthreads();
    for (int i = 0; i < nitems; ++i) {
      if (i == nu) {
        fold(gate0, sink0, true);
        eng.reset();
      }
      if (i + 1 < nitems) issue(st, i + 1);
      compute(i);
      if (i + 1 < nitems) st.sstore(tiles + ((i + 1) & 1) * St::BYTES);
      __syncthreads();
    }
  }
  if (nu == nitems) {  // no window tiles: the sparse branch is still open
    fold(gate0, sink0, true);
  } else {
    fold(gate1, sink1, false);
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (live && tcol[nt] < T) {
      char* op = (char*)a.o + (((size_t)(b * T + tcol[nt]) * a.Hq + hcol[nt]) * D + 4 * (lane >> 4)) * ES;
#pragma unroll
      for (int mc = 0; mc < Eng::NM; ++mc) {
        const f32x4 v = acc[nt][mc];
        Tt::store4(op + 16 * mc * ES, v[0], v[1], v[2], v[3]);
      }
    }
  }
}

// Ping-pong variant of the sparse kernel (8 wavefronts, NT column tiles of
// 16 columns per wavefront).  The two wavefronts that share a SIMD (w and w+4)
// work one half-tile out of phase: waves 0-3 run QK^T -> softmax -> PV on item
// s, waves 4-7 run softmax -> PV on item s-1 and then QK^T on item s, so one
// wave's exponentials overlap the other's matrix instructions.  Three LDS tile
// buffers hold items s-1, s and s+1; the loads of item s+2 are in flight during
// step s.  Work assignment, masking and the two branches are as in
// sparse_prefill_kernel; column tile nt of wave w holds the G heads of the
// 16/G positions tw0 + nt*16/G + col/G.
template <int DT, int D, int NT>
__global__ __launch_bounds__(512, 2) void sparse_prefill_pp_kernel(SparsePrefillArgs a) {
  using Tt = Tr<DT>;
  using Eng = WaveAttn<DT, D, NT, true>;
  using St = TileStage<DT, D, 512>;
  constexpr int ES = Tt::ES;
  constexpr int NW = 8;
  // three tile buffers as separate arrays: with the step loop unrolled by
  // three every access names its buffer, so the compiler can tell the
  // in-flight transfer into one buffer from the reads of the other two
  __shared__ __attribute__((aligned(16))) char tile0[St::BYTES];
  __shared__ __attribute__((aligned(16))) char tile1[St::BYTES];
  __shared__ __attribute__((aligned(16))) char tile2[St::BYTES];
  extern __shared__ uint32_t dyn[];


  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool lag = w >= 4;  // waves 4-7 run half a tile behind
  const int T = a.T;
  const int G = a.Hq / a.Hkv;
  const int PT = 16 / G;  // positions per column tile
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

  // Items: first the window blocks of the group's positions (known at once),
  // then the union of their selected blocks.
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
  // query fragments, gates and the first window tile are in flight while the
  // selection bitsets are built
  Eng eng;
  eng.reset();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < Eng::NS; ++ks)
      eng.qf[nt][ks] =
          (live && tcol[nt] < T)
              ? Tt::ld((const char*)a.q +
                       (((size_t)(b * T + tcol[nt]) * a.Hq + hcol) * D + 32 * ks + 8 * (lane >> 4)) * ES)
              : Tt::zero();
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
  // per-head sink logits of the sparse (0) and window (1) branch, log2
  // units; -inf without sinks
  float sink0[NT], sink1[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    sink0[nt] = a.sinks ? a.sinks[hcol] * kLog2e : -INFINITY;
    sink1[nt] = a.sinks ? a.sinks[a.Hq + hcol] * kLog2e : -INFINITY;
  }
  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * T * D * ES;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * a.nblk * D * 64 * ES;
  const char* ksg = (const char*)a.ks + (size_t)(b * a.Hkv + g) * T * D * ES;
  const char* vsg = (const char*)a.vs + (size_t)(b * a.Hkv + g) * a.nblk * D * 64 * ES;
  St st;
  st.dma_init();
  auto issue = [&](int i, char* buf) {  // item i -> buf (tile i % 3), in flight until wait_vmem
    const bool win = i < nwin;
    const int j = __builtin_amdgcn_readfirstlane(win ? jw0 + i : ulist[max(i - nwin, 0)]);
    st.dma(buf, (win ? ksg : kg) + (size_t)64 * j * D * ES, (win ? vsg : vg) + (size_t)j * D * 64 * ES,
           T - 64 * j);
  };
  if (nwin > 0) issue(0, tile0);

  // selection bitsets: per position (S), per wave (Uw) and per group (U);
  // positions own their words, the unions are OR-reductions (no contended
  // atomics)
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

  // Close a branch.  The first branch's gated output is parked in the output
  // rows themselves (in the output dtype) while the second branch runs and is
  // added back when that one closes: no registers hold it in between.
  auto fold = [&](const float* gate, const float* sink, bool first) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float inv, l2;
      eng.finish(nt, inv, l2, sink[nt]);
      const float sc = inv * gate[nt];
      if (live && tcol[nt] < T) {
        char* op = (char*)a.o + (((size_t)(b * T + tcol[nt]) * a.Hq + hcol) * D + 4 * (lane >> 4)) * ES;
#pragma unroll
        for (int mc = 0; mc < Eng::NM; ++mc) {
          f32x4 v = eng.o[nt][mc] * sc;
          if (!first) v += Tt::load4(op + 16 * mc * ES);
          Tt::store4(op + 16 * mc * ES, v[0], v[1], v[2], v[3]);
        }
      }
    }
  };
  // item i: first key, per-column-tile key range, and the column tiles of
  // this wave that have a live key in it (0: the wave skips the item)
  auto item = [&](int i, int& kbase, int* lo, int* hi) -> unsigned {
    const bool win = i < nwin;
    const int j = win ? jw0 + i : ulist[max(i - nwin, 0)];
    kbase = 64 * j;
    unsigned act = 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (win) {
        lo[nt] = tcol[nt] - a.W + 1;
      } else {
        const bool sel = (S[(w * PW + pcol[nt]) * nw32 + (j >> 5)] >> (j & 31)) & 1u;
        lo[nt] = sel ? 0 : kNoKey;
      }
      hi[nt] = hicol[nt];
      const bool live_col = max(lo[nt], kbase) <= min(hi[nt], kbase + 63);
      act |= (__ballot(live_col) != 0ull ? 1u : 0u) << nt;
    }
    return act;
  };

  wait_vmem();
  if (nitems > 0) st.dma_fix(tile0);
  __syncthreads();

  // Per step s, wave A (0-3) runs  P(s-1)V | QK(s) | softmax(s)  and wave B
  // (4-7) runs  softmax(s-1) | P(s-1)V | QK(s): one wave's matrix block
  // (PV + QK, 64 MFMAs) overlaps its partner's exponentials.  A wave raises
  // its issue priority for its matrix block, so the partner's vector work
  // fills the gaps between MFMAs instead of delaying them.  Across the
  // barrier A carries the packed P of item s, B its logits, both in sreg.
  float bmax[NT], bsum[NT];
  f32x4 sreg[NT][4];
  int p_kbase = 0, p_lo[NT], p_hi[NT];
  unsigned p_act = 0;
  const typename Eng::NoHook nohook;
  // step st_i: item st_i - 1 in `prev`, item st_i in `cur`, item st_i + 1
  // is transferred into `next` (the buffer of item st_i - 2, last read before
  // the barrier that ended the previous step)
  // All reads of the item lists and bitsets come before the step's transfer
  // is issued (the compiler cannot tell them apart from it and would wait).
  auto step = [&](int st_i, const char* prev, const char* cur, char* next) {
    unsigned c_act = 0;
    int c_kbase = 0, c_lo[NT], c_hi[NT];
    if (st_i < nitems) c_act = item(st_i, c_kbase, c_lo, c_hi);
    if (st_i + 1 < nitems) issue(st_i + 1, next);
    auto ldV = [&](int u, int mc) { return St::ldV(prev, u, mc); };
    auto ldK = [&](int c, int ks) { return St::ldK(cur, c, ks); };
    if (lag && st_i >= 1 && p_act)
      eng.template softmax<true, false>(sreg, p_kbase, p_lo, p_hi, a.sc2, bmax, bsum, nohook, p_act);
    __builtin_amdgcn_s_setprio(1);
    if (st_i >= 1 && p_act) eng.pv(sreg, ldV);
    if (st_i < nitems) {
      if (st_i == nwin) {  // window branch closed: park it
        fold(gate1, sink1, true);
        eng.reset();
      }
      if (c_act) {
        eng.qk(ldK, sreg);
        __builtin_amdgcn_s_setprio(0);
        if (!lag)
          eng.template softmax<true, false>(sreg, c_kbase, c_lo, c_hi, a.sc2, bmax, bsum, nohook, c_act);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    p_act = c_act;
    p_kbase = c_kbase;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      p_lo[nt] = c_lo[nt];
      p_hi[nt] = c_hi[nt];
    }
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
  if (nwin == nitems) {
    fold(gate1, sink1, true);
  } else {
    fold(gate0, sink0, false);
  }
}

// Sparse kernel for two resident work groups per CU (4 wavefronts each, NT
// column tiles of 16 columns per wavefront).  Each wavefront runs QK^T ->
// softmax -> PV on item s while item s+1 is transferred into the second of
// two LDS tile buffers.  With two groups on a CU, one group's barrier waits,
// selection set-up and closing writes overlap the other group's tiles.  Work
// assignment, masking and the two branches are as in sparse_prefill_kernel;
// column tile nt of wave w holds the G heads of the 16/G positions
// tw0 + nt*16/G + col/G.
template <int DT, int D, int NT, bool TRAIN>
__global__ __launch_bounds__(256, 2) void sparse_prefill_dual_kernel(SparsePrefillArgs a) {
  using Tt = Tr<DT>;
  using Eng = WaveAttn<DT, D, NT, true>;
  using St = TileStage<DT, D, 256>;
  constexpr int ES = Tt::ES;
  constexpr int NW = 4;
  // two tile buffers as separate arrays: with the step loop unrolled by two
  // every access names its buffer, so the compiler can tell the in-flight
  // transfer into one buffer from the reads of the other
  __shared__ __attribute__((aligned(16))) char tile0[St::BYTES];
  __shared__ __attribute__((aligned(16))) char tile1[St::BYTES];
  extern __shared__ uint32_t dyn[];


  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int T = a.T;
  const int G = a.Hq / a.Hkv;
  const int PT = 16 / G;  // positions per column tile
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

  // Items: first the window blocks of the group's positions (known at once),
  // then the union of their selected blocks.
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
  // query fragments, gates and the first window tile are in flight while the
  // selection bitsets are built
  Eng eng;
  eng.reset();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < Eng::NS; ++ks)
      eng.qf[nt][ks] =
          (live && tcol[nt] < T)
              ? Tt::ld((const char*)a.q +
                       (((size_t)(b * T + tcol[nt]) * a.Hq + hcol) * D + 32 * ks + 8 * (lane >> 4)) * ES)
              : Tt::zero();
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
  // per-head sink logits of the sparse (0) and window (1) branch, log2
  // units; -inf without sinks
  float sink0[NT], sink1[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    sink0[nt] = a.sinks ? a.sinks[hcol] * kLog2e : -INFINITY;
    sink1[nt] = a.sinks ? a.sinks[a.Hq + hcol] * kLog2e : -INFINITY;
  }
  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * T * D * ES;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * a.nblk * D * 64 * ES;
  const char* ksg = (const char*)a.ks + (size_t)(b * a.Hkv + g) * T * D * ES;
  const char* vsg = (const char*)a.vs + (size_t)(b * a.Hkv + g) * a.nblk * D * 64 * ES;
  St st;
  st.dma_init();
  auto issue = [&](int i, char* buf) {  // item i -> buf (tile i % 2), in flight until wait_vmem
    const bool win = i < nwin;
    const int j = __builtin_amdgcn_readfirstlane(win ? jw0 + i : ulist[max(i - nwin, 0)]);
    st.dma(buf, (win ? ksg : kg) + (size_t)64 * j * D * ES, (win ? vsg : vg) + (size_t)j * D * 64 * ES,
           T - 64 * j);
  };
  if (nwin > 0) issue(0, tile0);

  // selection bitsets: per position (S), per wave (Uw) and per group (U);
  // positions own their words, the unions are OR-reductions (no contended
  // atomics)
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

  // Close a branch.  The first branch's gated output is parked in the output
  // rows themselves (in the output dtype) while the second branch runs and is
  // added back when that one closes: no registers hold it in between.  The
  // training forward also writes the branch's own (ungated) output and LSE.
  auto fold = [&](const float* gate, const float* sink, bool first) __attribute__((always_inline)) {
    const int br = first ? 1 : 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float inv, l2;
      eng.finish(nt, inv, l2, sink[nt]);
      const float sc = inv * gate[nt];
      if (live && tcol[nt] < T) {
        const size_t row = (size_t)(b * T + tcol[nt]) * a.Hq + hcol;
        char* op = (char*)a.o + (row * D + 4 * (lane >> 4)) * ES;
#pragma unroll
        for (int mc = 0; mc < Eng::NM; ++mc) {
          f32x4 v = eng.o[nt][mc] * sc;
          if (!first) v += Tt::load4(op + 16 * mc * ES);
          Tt::store4(op + 16 * mc * ES, v[0], v[1], v[2], v[3]);
        }
        if constexpr (TRAIN) {
          char* bp = (char*)a.o_br + (((size_t)br * a.B * T * a.Hq + row) * D + 4 * (lane >> 4)) * ES;
#pragma unroll
          for (int mc = 0; mc < Eng::NM; ++mc) {
            const f32x4 v = eng.o[nt][mc] * inv;
            Tt::store4(bp + 16 * mc * ES, v[0], v[1], v[2], v[3]);
          }
          if ((lane >> 4) == 0) a.lse_br[((size_t)br * a.B * a.Hq + b * a.Hq + hcol) * T + tcol[nt]] = l2 * kLn2;
        }
      }
    }
  };
  // Item i's block and the selection-bitset word of each column tile's
  // position for it, read one step ahead (the reads are in flight while the
  // step before computes; window items read an unused word)
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
  // item i: first key, per-column-tile key range, and the column tiles of
  // this wave that have a live key in it (0: the wave skips the item)
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

  // Step s: item s is in `cur`; item s+1 goes into `next`, the buffer of
  // item s-1, whose last reads came before the barrier that ended the
  // previous step.  All reads of the item lists and bitsets come before the
  // step's transfer is issued (the compiler cannot tell them apart from it
  // and would wait).
  f32x4 sreg[NT][4];
  float bmax[NT], bsum[NT];
  const typename Eng::NoHook nohook;
  Pre pre{};
  if (nitems > 0) pre = fetch(0);
  auto step = [&](int st_i, const char* cur, char* next) {
    int kbase = 0, lo[NT], hi[NT];
    const unsigned act = item(st_i, pre, kbase, lo, hi);
    if (st_i + 1 < nitems) {
      pre = fetch(st_i + 1);
      st.dma(next, (st_i + 1 < nwin ? ksg : kg) + (size_t)64 * pre.j * D * ES,
             (st_i + 1 < nwin ? vsg : vg) + (size_t)pre.j * D * 64 * ES, T - 64 * pre.j);
    }
    if (st_i == nwin) {  // window branch closed: park it
      fold(gate1, sink1, true);
      eng.reset();
    }
    if (act) {
      auto ldK = [&](int c, int ks) { return St::ldK(cur, c, ks); };
      auto ldV = [&](int u, int mc) { return St::ldV(cur, u, mc); };
      eng.template qk<kSparseLA>(ldK, sreg);
      eng.template softmax<true, false>(sreg, kbase, lo, hi, a.sc2, bmax, bsum, nohook, act);
      eng.template pv<kSparseLA>(sreg, ldV);
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
    fold(gate1, sink1, true);
    if constexpr (TRAIN) {  // no selected block: the sparse branch is empty (its sink alone)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (live && tcol[nt] < T) {
          const float l2 = sink0[nt] > -INFINITY ? sink0[nt] : -INFINITY;  // log2 of the sink's weight alone
          const size_t row = (size_t)(b * T + tcol[nt]) * a.Hq + hcol;
          char* bp = (char*)a.o_br + (row * D + 4 * (lane >> 4)) * ES;
#pragma unroll
          for (int mc = 0; mc < Eng::NM; ++mc) Tt::store4(bp + 16 * mc * ES, 0.f, 0.f, 0.f, 0.f);
          if ((lane >> 4) == 0) a.lse_br[((size_t)b * a.Hq + hcol) * T + tcol[nt]] = l2 * kLn2;
        }
      }
    }
  } else {
    fold(gate0, sink0, false);
  }
}

// ================================================================ launchers
template <int DT, int D>
static hipError_t full_dispatch(const FullPrefillArgs& a, int score_lse, hipStream_t s) {
  constexpr int NT = 2;
  const int G = a.Hq / a.Hkv;
  // the ping-pong kernel needs G <= 16 and three tile buffers in LDS
  constexpr bool pingpong = 3 * TileStage<DT, D, 512>::BYTES <= 100 * 1024;
  if constexpr (pingpong) {
    if (G <= 16) {
      const int PWG = 8 * (16 * NT / G);
      const unsigned nwg = (unsigned)((long)a.B * a.Hkv * ((a.T + PWG - 1) / PWG));
      if (score_lse)
        hipLaunchKernelGGL((full_prefill_pp_kernel<DT, D, 1>), dim3(nwg), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((full_prefill_pp_kernel<DT, D, 0>), dim3(nwg), dim3(512), 0, s, a);
      return hipGetLastError();
    }
  }
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

// four waves per work group, topk_rows_per_wave(MAXI) rows per wave
template <int MAXI>
static void topk_launch(const TopkArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.Hkv * a.R;
  const long per_wg = 4L * topk_rows_per_wave(MAXI);
  hipLaunchKernelGGL(block_topk_kernel<MAXI>, dim3((unsigned)((rows + per_wg - 1) / per_wg)),
                     dim3(256), 0, s, a);
}

hipError_t launch_block_topk(const TopkArgs& a, int max_blocks, hipStream_t s) {
  if (max_blocks <= 64) topk_launch<1>(a, s);
  else if (max_blocks <= 128) topk_launch<2>(a, s);
  else if (max_blocks <= 256) topk_launch<4>(a, s);
  else if (max_blocks <= 512) topk_launch<8>(a, s);
  else if (max_blocks <= 1024) topk_launch<16>(a, s);
  else if (max_blocks <= 2048) topk_launch<32>(a, s);
  else topk_launch<64>(a, s);
  return hipGetLastError();
}

// sparse prefill launch shape: waves per work group, column tiles per wave,
// register prefetch stages
constexpr int kSparseWaves = 8;
constexpr int kSparseNT = 2;
constexpr int kSparseStages = 2;

template <int DT, int D>
static hipError_t sparse_dispatch(SparsePrefillArgs a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  // two resident work groups of four waves per CU when two of them fit in LDS
  constexpr bool dual = 2 * TileStage<DT, D, 256>::BYTES <= 64 * 1024;
  if constexpr (dual) {
    constexpr int NT = kSparseNT;
    const int PWG = 4 * (16 * NT / G);
    const int nw32 = (a.nblk + 31) / 32;
    const size_t lds = ((size_t)(1 + 4 + PWG) * nw32 + a.nblk + 1) * sizeof(uint32_t);
    if (lds <= 16 * 1024) {
      a.nwg = a.B * a.Hkv * ((a.T + PWG - 1) / PWG);
      if (a.o_br)
        hipLaunchKernelGGL((sparse_prefill_dual_kernel<DT, D, NT, true>), dim3(a.nwg), dim3(256), lds, s, a);
      else
        hipLaunchKernelGGL((sparse_prefill_dual_kernel<DT, D, NT, false>), dim3(a.nwg), dim3(256), lds, s, a);
      return hipGetLastError();
    }
  }
  constexpr int NW = kSparseWaves;
  // the ping-pong kernel needs three tile buffers in LDS (f32 with d = 128
  // does not fit and takes the one-column-tile kernel)
  constexpr bool pingpong = NW == 8 && 3 * TileStage<DT, D, 512>::BYTES <= 100 * 1024;
  constexpr int NT = pingpong ? kSparseNT : 1;
  const int PWG = NW * (16 * NT / G);
  a.nwg = a.B * a.Hkv * ((a.T + PWG - 1) / PWG);
  const int nw32 = (a.nblk + 31) / 32;
  const size_t lds = ((size_t)(1 + NW + PWG) * nw32 + a.nblk + 1) * sizeof(uint32_t);
  if constexpr (pingpong)
    hipLaunchKernelGGL((sparse_prefill_pp_kernel<DT, D, NT>), dim3(a.nwg), dim3(512), lds, s, a);
  else
    hipLaunchKernelGGL((sparse_prefill_kernel<DT, D, NT, NW, kSparseStages>), dim3(a.nwg), dim3(64 * NW), lds,
                       s, a);
  return hipGetLastError();
}

bool sparse_prefill_dual_ok(const SparsePrefillArgs& a, int dtype, int D) {
  if (dtype == HS_F32 && D == 128) return false;
  const int G = a.Hq / a.Hkv;
  const int PWG = 4 * (16 * kSparseNT / G);
  const int nw32 = (a.nblk + 31) / 32;
  return ((size_t)(1 + 4 + PWG) * nw32 + a.nblk + 1) * sizeof(uint32_t) <= 16 * 1024;
}

// dynamic LDS of the widest sparse launch shape (an upper bound for all)
size_t sparse_prefill_lds_bytes(int T, int G) {
  const int nblk = (T + 63) / 64, nw32 = (nblk + 31) / 32, PWG = kSparseWaves * (16 * kSparseNT / G);
  return ((size_t)(1 + kSparseWaves + PWG) * nw32 + nblk + 1) * sizeof(uint32_t);
}

hipError_t launch_sparse_prefill(const SparsePrefillArgs& a, int dtype, int D, hipStream_t s) {
  if (dtype == HS_BF16) return D == 64 ? sparse_dispatch<HS_BF16, 64>(a, s) : sparse_dispatch<HS_BF16, 128>(a, s);
  return D == 64 ? sparse_dispatch<HS_F32, 64>(a, s) : sparse_dispatch<HS_F32, 128>(a, s);
}

}  // namespace hs
