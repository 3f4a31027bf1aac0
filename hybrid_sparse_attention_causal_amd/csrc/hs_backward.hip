// hs_backward.hip -- backward pass of the hybrid block (bf16 inputs, fp32
// gradients).  The models of the pages are trained with this architecture
// (HySparse paper 4.1 "Experiments Setup"); the sparse layers' gradients
// reach the shared K/V (explainer 3.4 "Training Pipeline").  The selection is
// a discrete choice of the forward pass: indices are inputs, block scores
// get no gradient.
//
// For one attention branch with p = softmax(tau q.k) and o = p v, given dO:
//   dV = p^T dO~,  dP = dO~ . v,  dS = p (dP - dO~ . o),
//   dQ = tau dS K,  dK = tau dS^T Q,  with dO~ = sigma(gate) dO
// (sigma = 1 for the full layer and ungated layers).
//
// Every matrix product reads its operands in the order the MFMA wants, from
// a layout copy made first (a memory-bound transpose) or from transposing
// LDS reads (queries, output gradients, and K^T for dQ^T = K^T dS^T):
//   Vp  values position-major [..][T][D]     (dP = dO V^T, both orientations)
//
//  bwd_kv_kernel  key side: one work group per (sequence, kv group, 64-key
//                 block), wave w owning keys 16w..16w+15 (K and V rows in
//                 registers).  It walks the positions that attend the block
//                 in tiles of 32 columns (32/Gp positions x Gp heads): the
//                 tile's Q and dO rows, its Q^T and dO^T columns and its
//                 per-column statistics are staged in LDS by direct
//                 transfers, one tile ahead, and shared by the four waves.
//                 S = Q K^T and dP = dO V^T take the queries as M rows (lane
//                 = key, 8 consecutive columns), so P and dS are directly the
//                 B operands of dV^T += dO^T P and dK^T += Q^T dS.  Positions:
//                 full layer t >= 64j (causal), window branch t in
//                 [64j, 64j + 63 + W - 1], sparse branch the ascending list of
//                 the positions that selected the block (built from the
//                 indices first, so no tile without a selecting position is
//                 visited).
//  bwd_q_kernel   query side: work groups of 4*16/G positions as in the
//                 forward; per item (key tile) S^T = K Q^T and dP^T = V dO^T
//                 (K rows and V rows staged in LDS), dS^T elementwise, then
//                 dQ^T += K^T dS^T reading K^T from the staged K rows by
//                 transposing LDS reads, as the forward's P V.  Sparse layers: window items (branch 1)
//                 then the union of the selected blocks (branch 0), each
//                 with its own LSE, dO.o and gate.
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;

// ================================================== layout conversions
// V [B*Hkv][nblk][D][64] -> Vp [B*Hkv][nblk*64][D], zero past T (the tail of
// the last value tile may hold anything)
template <int D>
__global__ __launch_bounds__(256) void v_to_posmajor_kernel(const uint16_t* v, uint16_t* vp, int T, int nblk) {
  __shared__ uint16_t tl[D][64 + 2];
  const int j = blockIdx.x % nblk;
  const size_t bg = blockIdx.x / nblk;
  for (int e = threadIdx.x; e < D * 8; e += 256) {
    const int dd = e / 8, c = e % 8;
    const uint4 x = *(const uint4*)(v + ((bg * nblk + j) * D + dd) * 64 + 8 * c);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tl[dd][8 * c + 2 * i] = (uint16_t)(w[i] & 0xffffu);
      tl[dd][8 * c + 2 * i + 1] = (uint16_t)(w[i] >> 16);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * D / 8; e += 256) {
    const int r = e / (D / 8), c = e % (D / 8);
    const bool in = 64 * j + r < T;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = in ? ((uint32_t)tl[8 * c + 2 * i][r] | ((uint32_t)tl[8 * c + 2 * i + 1][r] << 16)) : 0u;
    *(uint4*)(vp + (bg * nblk * 64 + 64 * j + r) * D + 8 * c) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ===================================================== per-row preparation
// One row per 16 lanes: delta[br] = dO . o_br (bf16 rows), and for gated
// layers dG_br = s (1 - s) delta_br; with sinks the row's sink term
// -exp(b - lse_br) s delta_br (summed per head by bwd_sink_reduce_kernel).
__global__ __launch_bounds__(256) void bwd_rows_kernel(BwdRowArgs a) {
  const int lane = threadIdx.x & 63;
  const long row = ((long)blockIdx.x * 256 + threadIdx.x) / 16;  // (b, t, h)
  const int sub = lane & 15;
  const long nrows = (long)a.B * a.T * a.Hq;
  const bool in = row < nrows;
  const long rr = in ? row : 0;
  const int h = (int)(rr % a.Hq);
  const long bt = rr / a.Hq;
  const int t = (int)(bt % a.T), b = (int)(bt / a.T);
  // a lane's D/16 elements (8 or 4 bf16) of a row in one vector load
  auto ld = [&](const void* base, float* x) {
    const char* p = (const char*)base + (rr * a.D + sub * (a.D / 16)) * 2;
    uint32_t u[4];
    if (a.D == 128) {
      const uint4 v = *(const uint4*)p;
      u[0] = v.x, u[1] = v.y, u[2] = v.z, u[3] = v.w;
    } else {
      const uint2 v = *(const uint2*)p;
      u[0] = v.x, u[1] = v.y, u[2] = 0u, u[3] = 0u;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  };
  float dx[8];
  ld(a.dout, dx);
  for (int br = 0; br < a.nbr; ++br) {
    float ox[8];
    ld(a.o[br], ox);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += ox[i] * dx[i];
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (in && sub == 0) {
      const size_t ri = ((size_t)b * a.Hq + h) * a.T + t;
      a.delta[br][ri] = acc;
      const float s = a.gates ? 1.f / (1.f + expf(-a.gates[(size_t)rr * 2 + br])) : 1.f;
      if (a.dgates) a.dgates[(size_t)rr * 2 + br] = s * (1.f - s) * acc;
      if (a.sinks) a.sterm[br][ri] = -expf(a.sinks[br * a.Hq + h] - a.lse[br][ri]) * s * acc;
      if (a.cstat[br]) {  // the key side's per-column copy (column t*Gp + hh of the kv group)
        const int G = a.Hq / a.Hkv;
        float* cs = a.cstat[br] + ((size_t)b * a.Hkv + h / G) * 3 * a.NC + (size_t)t * a.Gp + h % G;
        cs[0] = a.lse_col[br][ri] * kLog2e;
        cs[a.NC] = acc;
        cs[2 * (size_t)a.NC] = s;
      }
    }
  }
}

// dsinks[br][h] = sum over (b, t) of the sink terms; one work group per (br, h)
__global__ __launch_bounds__(256) void bwd_sink_reduce_kernel(BwdRowArgs a) {
  __shared__ float part[4];
  const int br = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  float acc = 0.f;
  for (long i = threadIdx.x; i < (long)a.B * a.T; i += 256) {
    const int b = (int)(i / a.T), t = (int)(i % a.T);
    acc += a.sterm[br][((size_t)b * a.Hq + h) * a.T + t];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) a.dsinks[br * a.Hq + h] = part[0] + part[1] + part[2] + part[3];
}

// Position lists of the sparse branch.  colbits [B*Hkv][nblk][nwt] (nwt =
// ceil(T/32)): bit t of block j's row is set when position t's list holds j
// with 0 <= j < nblk and 64 j <= t (the forward's rule; duplicates count
// once).
// One work group per (kv group, run of nword words of positions): the
// group's bits are gathered in LDS ([nblk][nword] words, atomics in LDS only)
// and every word of the run is written, zero or not.
__global__ __launch_bounds__(256) void colbits_kernel(const int32_t* idx, uint32_t* bits, int T, int topk, int nblk,
                                                      int nwt, int nword) {
  extern __shared__ uint32_t sb[];
  const int bg = blockIdx.y;
  const int w0 = blockIdx.x * nword;
  const int nw = min(nword, nwt - w0);
  for (int i = threadIdx.x; i < nblk * nword; i += 256) sb[i] = 0u;
  __syncthreads();
  const int t0 = 32 * w0, tn = min(T, t0 + 32 * nw);
  const int32_t* ir = idx + ((size_t)bg * T + t0) * topk;
  for (int e = threadIdx.x; e < (tn - t0) * topk; e += 256) {
    const int t = t0 + e / topk;
    const int j = ir[e];
    if (j >= 0 && j < nblk && 64 * j <= t) atomicOr(&sb[j * nword + ((t - t0) >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nblk * nw; i += 256) {
    const int j = i / nw, w = i % nw;
    bits[((size_t)bg * nblk + j) * nwt + w0 + w] = sb[j * nword + w];
  }
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
// one wave per (kv group, block): list length
__global__ __launch_bounds__(256) void pos_count_kernel(const uint32_t* bits, int32_t* pcnt, int nbj, int nblk,
                                                        int nwt) {
  const int wv = (int)(((long)blockIdx.x * 256 + threadIdx.x) >> 6), lane = threadIdx.x & 63;
  if (wv >= nbj) return;  // wave-uniform
  const uint32_t* row = bits + (size_t)wv * nwt;
  int c = 0;
  for (int w = 2 * (wv % nblk) + lane; w < nwt; w += 64) c += __popc(row[w]);
  c = wave_sum(c);
  if (lane == 0) pcnt[wv] = c;
}
// one wave per (kv group, block): its offset (the lengths of the group's
// earlier blocks) and its positions, ascending
__global__ __launch_bounds__(256) void pos_write_kernel(const uint32_t* bits, const int32_t* pcnt, int32_t* poff,
                                                        int32_t* plist, int nbj, int nblk, int nwt, long cap) {
  const int wv = (int)(((long)blockIdx.x * 256 + threadIdx.x) >> 6), lane = threadIdx.x & 63;
  if (wv >= nbj) return;  // wave-uniform
  const int bg = wv / nblk, j = wv % nblk;
  int off = 0;
  for (int jj = lane; jj < j; jj += 64) off += pcnt[bg * nblk + jj];
  off = wave_sum(off);
  if (lane == 0) poff[wv] = off;
  int32_t* out = plist + bg * cap + off;
  const uint32_t* row = bits + (size_t)wv * nwt;
  int base = 0;
  for (int w0 = 2 * j; w0 < nwt; w0 += 64) {
    const int w = w0 + lane;
    uint32_t word = w < nwt ? row[w] : 0u;
    const int cnt = __popc(word);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int pos = base + incl - cnt;
    while (word) {
      out[pos++] = 32 * w + __builtin_ctz(word);
      word &= word - 1u;
    }
    base += __shfl(incl, 63);
  }
}

// ============================================================ key side
// LDS layout of one staged query tile (32 columns) of the key side.  Column c
// of the tile is (position slot c / Gp, head c % Gp); row c of the row tiles
// holds column c's Q (or dO) row, its 16-byte chunk p at p ^ swz(c).  The
// swizzle keeps both readers free of bank conflicts: the A fragments of S
// (rows 8(r/4) + 4e + r%4, r = 0..15, one chunk) and the transposing reads
// that build the A fragments of dO^T and Q^T (4 rows x 2 chunks per 16
// lanes).  The statistics (lse*log2(e), dO.o, sigma(gate) of the 32 columns)
// follow, transferred with padding to 1 KiB.
template <int D>
struct KvStage {
  static constexpr int KS = D * 2;
  static constexpr int KCH = KS / 16;
  static constexpr int QB = 32 * KS;
  static constexpr int OQ = 0, OD = QB, OS = 2 * QB;
  static constexpr int BYTES = OS + 1024;
  static constexpr int NQI = QB / 1024;   // row-tile transfers of 16 bytes per lane
  static constexpr int NDMA = NQI / 2 + 1;  // transfers per wave and tile (Q, dO rows; statistics)
  static_assert(NQI % 4 == 0 || NQI == 4, "row tiles do not split over four waves");
  // D = 128 (16 chunks per row, one bank sweep): the S reads of 16 lanes take
  // rows 8a + 4e + b (a, b = 0..3) and get chunks 4b + (2 (a&1) + a/2) ^ ...,
  // all distinct; the transposing reads of 32 lanes (row groups q = 0, 1 or
  // 2, 3; 4 rows and 2 chunks each) get 16 distinct chunks as well
  __device__ __forceinline__ static int swz(int c) {
    return KCH >= 16 ? (((c & 3) << 2) | (((c >> 3) & 1) << 1) | ((c >> 4) & 1))
                     : ((((c & 3) << 1) | ((c >> 3) & 1)) & (KCH - 1));
  }
};
constexpr int kPosChunk = 512;  // positions staged in LDS at a time
constexpr int kKvBufs = 4;      // tile buffers per work group (three tiles in flight)

// s_waitcnt with vmcnt = n (n < 64), the other counters not waited on
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void bwd_kv_kernel(BwdKVArgs a) {
  using Tt = Tr<HS_BF16>;
  using Frag = Tt::Frag;
  using KS_ = KvStage<D>;
  constexpr int NS = D / 32, NM = D / 16;
  constexpr int ND = KS_::NDMA;
  __shared__ __attribute__((aligned(16))) char buf0[KS_::BYTES];
  __shared__ __attribute__((aligned(16))) char buf1[KS_::BYTES];
  __shared__ __attribute__((aligned(16))) char buf2[KS_::BYTES];
  __shared__ __attribute__((aligned(16))) char buf3[KS_::BYTES];
  __shared__ int posl[kPosChunk];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int nbg = a.B * a.Hkv;
  const int bg = blockIdx.x % nbg;
  int j = blockIdx.x / nbg, part = 0, nparts = 1;  // early (long) blocks first
  if (MODE == 2) {  // work unit u of the kv group: part `part` of block j's list
    const int u = blockIdx.x / nbg;
    if (u >= a.ucount[bg]) return;
    const int code = a.utab[(size_t)bg * a.umax + u];
    j = code >> 16;
    part = code & 0xffff;
  }
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int G = a.Hq / a.Hkv, Gp = a.Gp;
  const int lgGp = 31 - __clz(Gp);
  const int PQ = 32 >> lgGp;  // positions per tile
  const int T = a.T;
  const int key = 64 * j + 16 * w + r16;

  int npos, pbase = 64 * j;
  if (MODE == 2) {
    const int cnt = a.pcnt[bg * a.nblk + j];
    nparts = max(1, (cnt + kUnitPos - 1) / kUnitPos);
    npos = min(kUnitPos, cnt - part * kUnitPos);
    pbase = a.poff[bg * a.nblk + j] + part * kUnitPos;
  } else if (MODE == 1) {
    npos = min(T - 1, 64 * j + 63 + a.W - 1) - 64 * j + 1;
  } else {
    npos = T - 64 * j;
  }
  // a block split over several units writes each part's share to its own
  // slot; kv_part_sum_kernel adds them up in part order
  const bool split = MODE == 2 && nparts > 1;
  const bool accumulate = a.accumulate && !split;
  float* dkp = a.dk + ((size_t)bg * T + key) * D + 4 * q4;
  float* dvp = a.dv + ((size_t)bg * T + key) * D + 4 * q4;
  if (split) {
    dkp = a.pbuf + ((size_t)bg * a.smax + a.soff[bg * a.nblk + j] + part) * 2 * 64 * D + (16 * w + r16) * D + 4 * q4;
    dvp = dkp + 64 * D;
  }
  if (npos <= 0) {  // nothing attends the block (sparse branch): its share is 0
    if (!accumulate && key < T) {
#pragma unroll
      for (int mc = 0; mc < NM; ++mc) {
        *(float4*)(dkp + 16 * mc) = make_float4(0.f, 0.f, 0.f, 0.f);
        *(float4*)(dvp + 16 * mc) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }

  // the wave's 16 keys and values as B operands (lane: key r16, 8 dims)
  Frag kf[NS], vf[NS];
  {
    const int keyc = min(key, T - 1);
    const char* krow = (const char*)a.k + ((size_t)bg * T + keyc) * D * 2;
    const char* vrow = (const char*)a.vp + ((size_t)bg * a.nblk * 64 + key) * D * 2;
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) {
      kf[ks] = Tt::ld(krow + (32 * ks + 8 * q4) * 2);
      vf[ks] = Tt::ld(vrow + (32 * ks + 8 * q4) * 2);
    }
  }
  f32x4 dkT[NM], dvT[NM];
#pragma unroll
  for (int mc = 0; mc < NM; ++mc) {
    dkT[mc] = f32x4{0.f, 0.f, 0.f, 0.f};
    dvT[mc] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const char* qg = (const char*)a.q + (size_t)b * T * a.Hq * D * 2;
  const char* dg = (const char*)a.dout + (size_t)b * T * a.Hq * D * 2;
  const float* csg = a.cstat + (size_t)bg * 3 * a.NC;

  int nc = 0;  // positions in the current chunk
  // tile `it` of the chunk (positions posl[it*PQ ..]) -> buf: every wave
  // issues ND transfers (its share of the two row tiles, one of the four
  // 256-byte pieces of the statistics)
  auto issue = [&](int it, char* buf) {
    const int pb = it * PQ;
#pragma unroll
    for (int k = 0; k < KS_::NQI / 4; ++k) {
      const int n = w + 4 * k;
      const int o = 1024 * n + 16 * lane;
      const int c = o / KS_::KS, lc = ((o % KS_::KS) >> 4) ^ KS_::swz(c);
      const int t = posl[pb + (c >> lgGp)];
      const int hh = min(c & (Gp - 1), G - 1);
      const uint32_t ro = (uint32_t)((t * a.Hq + g * G + hh) * D) * 2u + 16u * lc;
      const char* s1 = qg + ro;
      const char* s2 = dg + ro;
      __builtin_amdgcn_global_load_lds(s1, (__attribute__((address_space(3))) void*)(buf + KS_::OQ + 1024 * n), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds(s2, (__attribute__((address_space(3))) void*)(buf + KS_::OD + 1024 * n), 16,
                                       0, 0);
    }
    {  // statistics: 96 floats; lanes past them reload the last array into the padding
      const int ix = 64 * w + lane;
      const int arr = min(ix >> 5, 2), c = ix & 31;
      const int t = posl[pb + (c >> lgGp)];
      const float* s1 = csg + (uint32_t)(arr * a.NC + t * Gp + (c & (Gp - 1)));
      __builtin_amdgcn_global_load_lds(s1, (__attribute__((address_space(3))) void*)(buf + KS_::OS + 256 * w), 4, 0,
                                       0);
    }
  };

  auto compute = [&](int it, const char* cur) {
    f32x4 S[2], dP[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      S[e] = f32x4{0.f, 0.f, 0.f, 0.f};
      dP[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // S = Q K^T, dP = dO V^T: chunk e's A row r16 is column 8(r16/4) + 4e + r16%4,
    // so that a lane of the result holds columns 8 q4 .. 8 q4 + 7
#pragma unroll
    for (int ks = 0; ks < NS; ++ks)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = 8 * (r16 >> 2) + 4 * e + (r16 & 3);
        const int off = c * KS_::KS + 16 * ((4 * ks + q4) ^ KS_::swz(c));
        Tt::mma(S[e], Tt::ld(cur + KS_::OQ + off), kf[ks]);
        Tt::mma(dP[e], Tt::ld(cur + KS_::OD + off), vf[ks]);
      }
    const float* st = (const float*)(cur + KS_::OS) + 8 * q4;
    float ps[8], ds[8];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float4 l4 = *(const float4*)(st + 4 * e);
      const float4 d4 = *(const float4*)(st + 32 + 4 * e);
      const float4 g4 = *(const float4*)(st + 64 + 4 * e);
      const float lse2[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
      const float sg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // the column's position; none past the chunk's positions or for a padding head
        const int c = 8 * q4 + 4 * e + i, slot = it * PQ + (c >> lgGp);
        const int tp = posl[slot];
        bool valid = slot < nc && (c & (Gp - 1)) < G && key <= tp && key < T;
        if (MODE == 1) valid = valid && key > tp - a.W;
        const float p = fast_exp2(S[e][i] * a.sc2 - lse2[i]) * sg[i];
        ps[4 * e + i] = valid ? p : 0.f;
        ds[4 * e + i] = valid ? p * (dP[e][i] - dl[i]) : 0.f;
      }
    }
    const Frag pf = Tt::pack(ps), dsf = Tt::pack(ds);
    // dV^T += dO^T P and dK^T += Q^T dS.  The A fragment (head_dim rows
    // 16 mc + r16, columns 8 q4 .. 8 q4 + 7) is two transposing reads: lane L
    // points at 4 dims (16 mc + 4 (L%4) ..) of row 8 (L/16) + 4 h + (L%16)/4
    // and receives one dim of 4 rows.
    const int tr_c = 8 * q4 + (r16 >> 2);
#pragma unroll
    for (int mc = 0; mc < NM; ++mc) {
      uint2 hq[2], hd[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = tr_c + 4 * h;
        const int byte = 32 * mc + 8 * (r16 & 3);
        const int off = c * KS_::KS + (((byte >> 4) ^ KS_::swz(c)) << 4) + (byte & 15);
        hd[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                             (__attribute__((address_space(3))) bf16x4_t*)(cur + KS_::OD + off)));
        hq[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                             (__attribute__((address_space(3))) bf16x4_t*)(cur + KS_::OQ + off)));
      }
      Frag fd, fq;
      fd.u = make_uint4(hd[0].x, hd[0].y, hd[1].x, hd[1].y);
      fq.u = make_uint4(hq[0].x, hq[0].y, hq[1].x, hq[1].y);
      Tt::mma(dvT[mc], fd, pf);
      Tt::mma(dkT[mc], fq, dsf);
    }
  };

  // Tiles are visited from the latest positions down: the work groups that
  // start together (one kv group per XCD, successive blocks) then read the
  // same query tiles at about the same time, so most of their transfers hit
  // in L2.  Step k computes tile nit-1-k from buffer k % 4 and issues tile
  // nit-4-k into the buffer of tile nit-k, read in the previous step.
  int nit = 0;
  auto step = [&](int k, const char* cur, char* ahead) {
    if (k + 3 < nit) issue(nit - 4 - k, ahead);
    compute(nit - 1 - k, cur);
    // the next tile has landed (this wave's transfers: in order); up to two
    // more may stay in flight
    const int later = min(2, nit - 2 - k);
    if (later >= 2) wait_vmcnt<2 * ND>();
    else if (later == 1) wait_vmcnt<ND>();
    else wait_vmem();
    __syncthreads();
  };
  const int nch = (npos + kPosChunk - 1) / kPosChunk;
  for (int ci = nch - 1; ci >= 0; --ci) {
    const int c0 = ci * kPosChunk;
    nc = min(kPosChunk, npos - c0);
    __syncthreads();  // the previous chunk's tiles and positions are no longer read
    for (int i = threadIdx.x; i < kPosChunk; i += 256) {
      const int ii = min(i, nc - 1);
      posl[i] = MODE == 2 ? a.plist[(size_t)bg * T * a.topk + pbase + c0 + ii] : pbase + c0 + ii;
    }
    __syncthreads();
    nit = (nc + PQ - 1) / PQ;
    issue(nit - 1, buf0);
    if (nit > 1) issue(nit - 2, buf1);
    if (nit > 2) issue(nit - 3, buf2);
    if (nit > 2) wait_vmcnt<2 * ND>();
    else if (nit > 1) wait_vmcnt<ND>();
    else wait_vmem();
    __syncthreads();
    for (int k = 0; k < nit; k += 4) {
      step(k, buf0, buf3);
      if (k + 1 >= nit) break;
      step(k + 1, buf1, buf0);
      if (k + 2 >= nit) break;
      step(k + 2, buf2, buf1);
      if (k + 3 >= nit) break;
      step(k + 3, buf3, buf2);
    }
  }
  if (key < T) {
#pragma unroll
    for (int mc = 0; mc < NM; ++mc) {
      float4 x = make_float4(a.tau * dkT[mc][0], a.tau * dkT[mc][1], a.tau * dkT[mc][2], a.tau * dkT[mc][3]);
      float4 y = make_float4(dvT[mc][0], dvT[mc][1], dvT[mc][2], dvT[mc][3]);
      if (accumulate) {
        const float4 x0 = *(const float4*)(dkp + 16 * mc), y0 = *(const float4*)(dvp + 16 * mc);
        x = make_float4(x.x + x0.x, x.y + x0.y, x.z + x0.z, x.w + x0.w);
        y = make_float4(y.x + y0.x, y.y + y0.y, y.z + y0.z, y.w + y0.w);
      }
      *(float4*)(dkp + 16 * mc) = x;
      *(float4*)(dvp + 16 * mc) = y;
    }
  }
}

// ========================================================== query side
// Rows-only LDS staging (K or V rows of a 64-key tile, in S^T row order,
// chunk-swizzled as TileStage's key rows), direct global -> LDS.
template <int D, int NTHR>
struct RowStage {
  static constexpr int KS = D * 2;
  static constexpr int KCH = KS / 16;
  static constexpr int KSW = (KCH < 16 ? KCH : 16) - 1;
  static constexpr int BYTES = 64 * KS;
  static constexpr int NWV = NTHR / 64;
  static constexpr int NDMA = BYTES / 1024 / NWV;
  static_assert(NDMA * NWV * 1024 == BYTES, "tile does not split into wave chunks");
  int dkey[NDMA];
  uint32_t doff[NDMA];
  __device__ __forceinline__ static int k_lds(int row, int chunk) { return row * KS + ((chunk ^ (row & KSW)) << 4); }
  __device__ __forceinline__ void dma_init() {
    const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int off = (w + NWV * n) * 1024 + 16 * lane;
      const int r = off / KS, c = ((off % KS) >> 4) ^ (r & KSW);
      dkey[n] = tile_key(r >> 4, r & 15);
      doff[n] = dkey[n] * KS + c * 16;
    }
  }
  // rows: row 0 of the tile; rows past nk read row nk-1
  __device__ __forceinline__ void dma(char* buf, const char* rows, int nk) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int kk = dkey[n];
      const char* src = rows + (doff[n] - (uint32_t)((kk - min(kk, nk - 1)) * KS));
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(buf + (w + NWV * n) * 1024), 16,
                                       0, 0);
    }
  }
  __device__ __forceinline__ static Tr<HS_BF16>::Frag ldK(const char* buf, int c, int ks) {
    const int lane = lane_id();
    const int row = 16 * c + (lane & 15);
    const int ch = (32 * ks + 8 * (lane >> 4)) * 2 / 16;
    return Tr<HS_BF16>::ld(buf + k_lds(row, ch));
  }
  // The transposed tile as an A fragment: head_dim rows 16 mc + r16, keys
  // 32 u + 8 q .. +7 (the P.V key order).  Two transposing reads: lane L of
  // each 16-lane group points at 4 dims (16 mc + 4 (L%4) ..) of the row of
  // key 32 u + 8 q + 4 h + (L%16)/4 and receives one dim of 4 keys.
  __device__ __forceinline__ static Tr<HS_BF16>::Frag ldKT(const char* buf, int u, int mc) {
    const int lane = lane_id(), r16 = lane & 15;
    const int byte = 32 * mc + 8 * (r16 & 3);
    uint2 hh[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = tile_row(32 * u + 8 * (lane >> 4) + 4 * h + (r16 >> 2));
      const int off = k_lds(row, byte >> 4) + (byte & 15);
      hh[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                           (__attribute__((address_space(3))) bf16x4_t*)(buf + off)));
    }
    Tr<HS_BF16>::Frag f;
    f.u = make_uint4(hh[0].x, hh[0].y, hh[1].x, hh[1].y);
    return f;
  }
};

template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void bwd_q_kernel(BwdQArgs a) {
  using Tt = Tr<HS_BF16>;
  using Eng = WaveAttn<HS_BF16, D, 1>;
  // K rows (S^T = K Q^T reads them as they are, dQ^T += K^T dS^T through
  // transposing reads) and V rows: 64 KiB of tiles, two work groups per CU
  using StK = RowStage<D, 256>;
  using StV = RowStage<D, 256>;
  constexpr int NW = 4;
  __shared__ __attribute__((aligned(16))) char kt0[StK::BYTES];
  __shared__ __attribute__((aligned(16))) char kt1[StK::BYTES];
  __shared__ __attribute__((aligned(16))) char vt0[StV::BYTES];
  __shared__ __attribute__((aligned(16))) char vt1[StV::BYTES];
  extern __shared__ uint32_t dyn[];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int T = a.T;
  const int G = a.Hq / a.Hkv;
  const int PT = 16 / G;
  const int PWG = NW * PT;
  const int nwg_bg = (T + PWG - 1) / PWG;
  const WgSlot ws = wg_slot(a.B * a.Hkv, nwg_bg);
  const bool live = ws.live;
  const int bg = ws.bg;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int t0 = ws.pblk * PWG;
  const int col = lane & 15;
  const int h = g * G + col % G;
  const int tcol = t0 + w * PT + col / G;
  const int hicol = live && tcol < T ? tcol : -1;
  const int tc = min(tcol, T - 1);

  Eng eq, ed;  // eq: Q fragments and the dQ^T accumulators; ed: dO fragments
  eq.reset();
#pragma unroll
  for (int ks = 0; ks < Eng::NS; ++ks) {
    const size_t off = ((((size_t)b * T + tc) * a.Hq + h) * D + 32 * ks + 8 * (lane >> 4)) * 2;
    eq.qf[0][ks] = Tt::ld((const char*)a.q + off);
    ed.qf[0][ks] = Tt::ld((const char*)a.dout + off);
  }
  // per-branch column statistics (log2-unit LSE, dO.o, gate)
  const size_t ri = ((size_t)b * a.Hq + h) * T + tc;
  float lse2[2], dl[2], sg[2];
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    const float* L = br ? a.lse1 : a.lse0;
    const float* Dl = br ? a.delta1 : a.delta0;
    lse2[br] = L ? L[ri] * kLog2e : 0.f;
    dl[br] = Dl ? Dl[ri] : 0.f;
    sg[br] = a.gates ? 1.f / (1.f + expf(-a.gates[(((size_t)b * T + tc) * a.Hq + h) * 2 + br])) : 1.f;
  }

  // items: MODE 0 the causal tiles 0 .. of the group's last position; MODE 1
  // the window tiles (branch 1, the layer's own cache) then the union of the
  // positions' selected blocks (branch 0, the shared cache)
  const int nw32 = (a.nblk + 31) >> 5;
  uint32_t* S = dyn;                 // [PWG][nw32] per position
  uint32_t* U = S + PWG * nw32;      // [nw32] union
  int* ulist = (int*)(U + nw32);     // [nblk]
  int* nu_p = ulist + a.nblk;
  int jw0 = 0, nwin = 0, nu = 0;
  if (MODE == 0) {
    nu = live ? ((min(T, t0 + PWG) - 1) >> 6) + 1 : 0;
  } else {
    if (live && a.W > 0) {
      jw0 = max(0, t0 - a.W + 1) >> 6;
      nwin = (min(T - 1, t0 + PWG - 1) >> 6) - jw0 + 1;
    }
    for (int i = threadIdx.x; i < (PWG + 1) * nw32; i += 64 * NW) S[i] = 0u;
    __syncthreads();
    if (live) {
      for (int e = threadIdx.x; e < PWG * a.topk; e += 64 * NW) {
        const int p = e / a.topk, t = t0 + p;
        if (t < T) {
          const int j = a.idx[((size_t)bg * T + t) * a.topk + (e % a.topk)];
          if (j >= 0 && j < a.nblk && 64 * j <= t) atomicOr(&S[p * nw32 + (j >> 5)], 1u << (j & 31));
        }
      }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < nw32; k += 64 * NW) {
      uint32_t v = 0u;
      for (int p = 0; p < PWG; ++p) v |= S[p * nw32 + k];
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
    nu = live ? *nu_p : 0;
  }
  const int nitems = nwin + nu;

  StK sk;
  StV sv;
  sk.dma_init();
  sv.dma_init();
  auto blk = [&](int i) {
    return __builtin_amdgcn_readfirstlane(MODE == 0 ? i : (i < nwin ? jw0 + i : ulist[max(i - nwin, 0)]));
  };
  auto issue = [&](int i, char* kb, char* vb) {
    const bool win = MODE == 1 && i < nwin;
    const int j = blk(i);
    const char* kr = (const char*)(win ? a.k1 : a.k0) + ((size_t)bg * T + 64 * j) * D * 2;
    const char* vr = (const char*)(win ? a.vp1 : a.vp0) + ((size_t)bg * a.nblk * 64 + 64 * j) * D * 2;
    sk.dma(kb, kr, T - 64 * j);
    sv.dma(vb, vr, T - 64 * j);
  };
  if (nitems > 0) issue(0, kt0, vt0);
  wait_vmem();
  __syncthreads();

  auto step = [&](int i, const char* kc, const char* vc, char* kn, char* vn) {
    const bool win = MODE == 1 && i < nwin;
    const int j = blk(i);
    if (i + 1 < nitems) issue(i + 1, kn, vn);
    const int kbase = 64 * j;
    int lo, hi = hicol;
    if (MODE == 0) {
      lo = 0;
    } else if (win) {
      lo = tcol - a.W + 1;
    } else {
      const bool sel = hicol >= 0 && ((S[(w * PT + col / G) * nw32 + (j >> 5)] >> (j & 31)) & 1u);
      lo = sel ? 0 : kNoKey;
    }
    const bool livecol = hicol >= 0 && lo != kNoKey && max(lo, kbase) <= min(hi, kbase + 63);
    if (__ballot(livecol) != 0ull) {
      f32x4 s[1][4], dp[1][4];
      eq.qk([&](int c, int ks) { return StK::ldK(kc, c, ks); }, s);
      ed.qk([&](int c, int ks) { return StV::ldK(vc, c, ks); }, dp);
      const int br = win ? 1 : 0;
      const float l2 = br ? lse2[1] : lse2[0], d0 = br ? dl[1] : dl[0], s0 = br ? sg[1] : sg[0];
      const int kb8 = kbase + 8 * (lane >> 4);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int k = kb8 + 32 * (c >> 1) + 4 * (c & 1) + i2;
          const bool valid = livecol && k >= lo && k <= hi;
          const float p = valid ? fast_exp2(s[0][c][i2] * a.sc2 - l2) : 0.f;
          s[0][c][i2] = p * s0 * (dp[0][c][i2] - d0);
        }
      Tt::pack_p(s[0]);
      eq.pv(s, [&](int u, int mc) { return StK::ldKT(kc, u, mc); });
    }
    wait_vmem();
    __syncthreads();
  };
  for (int i = 0; i < nitems; i += 2) {
    step(i, kt0, vt0, kt1, vt1);
    if (i + 1 >= nitems) break;
    step(i + 1, kt1, vt1, kt0, vt0);
  }
  if (hicol >= 0) {
    float* op = a.dq + (((size_t)b * T + tcol) * a.Hq + h) * D + 4 * (lane >> 4);
#pragma unroll
    for (int mc = 0; mc < Eng::NM; ++mc) {
      const f32x4 v = eq.o[0][mc];
      *(float4*)(op + 16 * mc) = make_float4(a.tau * v[0], a.tau * v[1], a.tau * v[2], a.tau * v[3]);
    }
  }
}

// ============================================================= launchers
template <int D>
static hipError_t layouts(const BwdLayoutArgs& l, hipStream_t s) {
  const unsigned nkb = (unsigned)((long)l.B * l.Hkv * l.nblk);
  for (int i = 0; i < 2; ++i) {
    if (l.v[i]) hipLaunchKernelGGL(v_to_posmajor_kernel<D>, dim3(nkb), dim3(256), 0, s, (const uint16_t*)l.v[i],
                                   (uint16_t*)l.vp[i], l.T, l.nblk);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_layouts(const BwdLayoutArgs& l, int D, hipStream_t s) {
  return D == 128 ? layouts<128>(l, s) : layouts<64>(l, s);
}

hipError_t launch_bwd_rows(const BwdRowArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.T * a.Hq;
  hipLaunchKernelGGL(bwd_rows_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.sinks) return e;
  hipLaunchKernelGGL(bwd_sink_reduce_kernel, dim3((unsigned)(a.nbr * a.Hq)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pos_lists(const int32_t* idx, uint32_t* colbits, int32_t* plist, int32_t* pcnt, int32_t* poff,
                            int B, int Hkv, int T, int topk, int nblk, hipStream_t s) {
  const int nwt = (T + 31) / 32;
  const int nbj = B * Hkv * nblk;
  // 8 words (256 positions) per work group, fewer when nblk x 8 words would
  // pass 32 KiB of LDS
  const int nword = std::max(1, std::min(8, 8192 / nblk));
  hipLaunchKernelGGL(colbits_kernel, dim3((unsigned)((nwt + nword - 1) / nword), (unsigned)(B * Hkv)), dim3(256),
                     (size_t)nblk * nword * sizeof(uint32_t), s, idx, colbits, T, topk, nblk, nwt, nword);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nwg = (unsigned)((nbj + 3) / 4);
  hipLaunchKernelGGL(pos_count_kernel, dim3(nwg), dim3(256), 0, s, colbits, pcnt, nbj, nblk, nwt);
  hipLaunchKernelGGL(pos_write_kernel, dim3(nwg), dim3(256), 0, s, colbits, pcnt, poff, plist, nbj, nblk, nwt,
                     (long)T * topk);
  return hipGetLastError();
}

// Work units of the sparse branch's key side, one work group per kv group:
// block j gets max(1, ceil(n_j / kUnitPos)) units (n_j: its list length),
// numbered in block order; a block of several parts gets as many partial slots.
__global__ __launch_bounds__(256) void kv_units_kernel(const int32_t* pcnt, int32_t* utab, int32_t* ucount,
                                                       int32_t* soff, int nblk, int umax) {
  __shared__ int wsum[2][4];
  const int bg = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int ubase = 0, sbase = 0;
  for (int j0 = 0; j0 < nblk; j0 += 256) {
    const int jj = j0 + (int)threadIdx.x;
    const int cnt = jj < nblk ? pcnt[(size_t)bg * nblk + jj] : 0;
    const int np = jj < nblk ? max(1, (cnt + kUnitPos - 1) / kUnitPos) : 0;
    const int ns = np > 1 ? np : 0;
    int iu = np, is = ns;  // inclusive wave scans
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int vu = __shfl_up(iu, off), vs = __shfl_up(is, off);
      if (lane >= off) {
        iu += vu;
        is += vs;
      }
    }
    if (lane == 63) {
      wsum[0][w] = iu;
      wsum[1][w] = is;
    }
    __syncthreads();
    int pu = 0, ps = 0, tu = 0, ts = 0;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      if (ww < w) {
        pu += wsum[0][ww];
        ps += wsum[1][ww];
      }
      tu += wsum[0][ww];
      ts += wsum[1][ww];
    }
    __syncthreads();  // wsum is rewritten by the next round
    if (jj < nblk) {
      const int uo = ubase + pu + iu - np;
      soff[(size_t)bg * nblk + jj] = sbase + ps + is - ns;
      for (int p = 0; p < np; ++p) utab[(size_t)bg * umax + uo + p] = (jj << 16) | p;
    }
    ubase += tu;
    sbase += ts;
  }
  if (threadIdx.x == 0) ucount[bg] = ubase;
}

// dK and dV of the blocks split over several units: the parts' shares summed
// in part order, then added to (or written as) the gradient; kPartSlices work
// groups per (block, kv group), each a slice of the 2 x 64 x D entries
constexpr int kPartSlices = 16;
template <int D>
__global__ __launch_bounds__(256) void kv_part_sum_kernel(BwdKVArgs a) {
  const int j = blockIdx.x, bg = blockIdx.y;
  const int np = (a.pcnt[(size_t)bg * a.nblk + j] + kUnitPos - 1) / kUnitPos;
  if (np <= 1) return;
  const float* pp = a.pbuf + ((size_t)bg * a.smax + a.soff[(size_t)bg * a.nblk + j]) * 2 * 64 * D;
  const int nk = min(64, a.T - 64 * j);
  const int per = nk * D / 4;  // float4 pieces of one gradient
  for (int e = blockIdx.z * 256 + threadIdx.x; e < 2 * per; e += kPartSlices * 256) {
    const int kv = e / per, r = e % per;
    const float* src = pp + (size_t)kv * 64 * D + 4 * r;
    float4 x = *(const float4*)src;
    for (int p = 1; p < np; ++p) {
      const float4 y = *(const float4*)(src + (size_t)p * 2 * 64 * D);
      x = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
    }
    float* dst = (kv ? a.dv : a.dk) + ((size_t)bg * a.T + 64 * j) * D + 4 * r;
    if (a.accumulate) {
      const float4 y = *(const float4*)dst;
      x = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
    }
    *(float4*)dst = x;
  }
}

hipError_t launch_kv_units(const int32_t* pcnt, int32_t* utab, int32_t* ucount, int32_t* soff, int nbg, int nblk,
                           int umax, hipStream_t s) {
  hipLaunchKernelGGL(kv_units_kernel, dim3((unsigned)nbg), dim3(256), 0, s, pcnt, utab, ucount, soff, nblk, umax);
  return hipGetLastError();
}

template <int D>
static void kv_dispatch(const BwdKVArgs& a, int mode, hipStream_t s) {
  const long nbg = (long)a.B * a.Hkv;
  const dim3 grid((unsigned)(nbg * a.nblk));
  if (mode == 0) hipLaunchKernelGGL((bwd_kv_kernel<D, 0>), grid, dim3(256), 0, s, a);
  else if (mode == 1) hipLaunchKernelGGL((bwd_kv_kernel<D, 1>), grid, dim3(256), 0, s, a);
  else {
    hipLaunchKernelGGL((bwd_kv_kernel<D, 2>), dim3((unsigned)(nbg * a.umax)), dim3(256), 0, s, a);
    hipLaunchKernelGGL((kv_part_sum_kernel<D>), dim3((unsigned)a.nblk, (unsigned)nbg, kPartSlices), dim3(256), 0, s,
                       a);
  }
}
hipError_t launch_bwd_kv(const BwdKVArgs& a, int mode, int D, hipStream_t s) {
  if (D == 128) kv_dispatch<128>(a, mode, s);
  else kv_dispatch<64>(a, mode, s);
  return hipGetLastError();
}

size_t bwd_q_lds_bytes(int T, int G) {
  const int nblk = (T + 63) / 64, nw32 = (nblk + 31) / 32, PWG = 4 * (16 / G);
  return ((size_t)(PWG + 1) * nw32 + nblk + 1) * sizeof(uint32_t);
}

template <int D>
static void q_dispatch(const BwdQArgs& a, int mode, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int PWG = 4 * (16 / G);
  const dim3 grid((unsigned)((long)a.B * a.Hkv * ((a.T + PWG - 1) / PWG)));
  const size_t lds = bwd_q_lds_bytes(a.T, G);
  if (mode == 0) hipLaunchKernelGGL((bwd_q_kernel<D, 0>), grid, dim3(256), lds, s, a);
  else hipLaunchKernelGGL((bwd_q_kernel<D, 1>), grid, dim3(256), lds, s, a);
}
hipError_t launch_bwd_q(const BwdQArgs& a, int mode, int D, hipStream_t s) {
  if (D == 128) q_dispatch<128>(a, mode, s);
  else q_dispatch<64>(a, mode, s);
  return hipGetLastError();
}

}  // namespace hs
