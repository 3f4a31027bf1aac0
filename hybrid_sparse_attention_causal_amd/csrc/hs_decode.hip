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
//  decode_sparse_kernel   one sparse layer: the selected blocks of the shared
//                         cache plus the layer's own window ring, merged by the
//                         sigmoid gates (explainer 3.4.3)
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {

// ======================================================== split-K full layer
// Unit (b, g, ch) covers keys [ch*CH*64, min(L, (ch+1)*CH*64)).  MFMA columns
// 0..G-1 are the G query heads of kv group g (G <= 16).
template <int D, int TOKEN>
__global__ __launch_bounds__(256) void decode_full_kernel(DecodeFullArgs a) {
  using Tt = Tr<HS_BF16>;
  using Eng = WaveAttn<HS_BF16, D, 1>;
  constexpr int ES = 2;
  const int lane = threadIdx.x & 63;
  const long unit = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= (long)a.B * a.Hkv * a.nch) return;
  const int ch = (int)(unit % a.nch);
  const int bg = (int)(unit / a.nch);
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int L = a.lens[b];
  const int span = a.ch_blocks * 64;
  const int kstart = ch * span;
  if (kstart >= L) return;
  const int kend = min(L, kstart + span);
  const int G = a.Hq / a.Hkv;
  const int col = lane & 15;
  const int h = g * G + col;
  const int r16 = lane & 15, q8 = 8 * (lane >> 4);

  Eng eng;
  eng.reset();
  int lo[1], hi[1];
  lo[0] = col < G ? 0 : kNoKey;
  hi[0] = L - 1;
#pragma unroll
  for (int ks = 0; ks < Eng::NS; ++ks)
    eng.qf[0][ks] = col < G ? Tt::ld((const char*)a.q + ((size_t)(b * a.Hq + h) * D + 32 * ks + q8) * ES)
                            : Tt::zero();
  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * a.C * D * ES;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * (a.C / 64) * D * 64 * ES;
  float* rawrow = a.raw + (size_t)(b * a.Hq + h) * (TOKEN ? a.C : a.C / 64);
  const int q4 = (lane >> 4) << 2;

  for (int kb0 = kstart; kb0 < kend; kb0 += 64) {
    const bool partial = kb0 + 64 > L;
    const int j = kb0 >> 6;
    auto ldK = [&](int c, int ks) {
      const int key = kb0 + tile_key(c, r16);
      return (!partial || key < L) ? Tt::ld(kg + ((size_t)key * D + 32 * ks + q8) * ES) : Tt::zero();
    };
    auto ldV = [&](int u, int mc) {
      const auto f = Tt::ld(vg + (((size_t)j * D + 16 * mc + r16) * 64 + 32 * u + q8) * ES);
      return partial ? Tt::keep(f, L - (kb0 + 32 * u + q8)) : f;
    };
    float bmax[1], bsum[1];
    if (TOKEN) {
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
      eng.template tile<true, false>(ldK, ldV, kb0, lo, hi, a.sc2, bmax, bsum, hook);
    } else {
      eng.template tile<true, false>(ldK, ldV, kb0, lo, hi, a.sc2, bmax, bsum);
      if (lane < 16 && col < G) rawrow[j] = bmax[0] * kLn2;
    }
  }

  // partial state: unnormalised o (head_dim floats), m (log2 units), l
  float lt = eng.l[0] + __shfl_xor(eng.l[0], 16);
  lt += __shfl_xor(lt, 32);
  if (col < G) {
    float* pp = a.part + ((size_t)(b * a.Hq + h) * a.nch + ch) * (D + 2);
#pragma unroll
    for (int mc = 0; mc < Eng::NM; ++mc) *(float4*)(pp + 16 * mc + q4) = *(const float4*)&eng.o[0][mc];
    if (lane < 16) {
      pp[D] = eng.m[0];
      pp[D + 1] = lt;
    }
  }
}

// One wave per (b, h): merge the nchb = ceil(L / (CH*64)) partials.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeFullArgs a) {
  const int lane = threadIdx.x & 63;
  const long bh = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= (long)a.B * a.Hq) return;
  const int b = (int)(bh / a.Hq);
  const int L = a.lens[b];
  const int span = a.ch_blocks * 64;
  const int nchb = L > 0 ? (L + span - 1) / span : 0;
  const float* pp = a.part + (size_t)bh * a.nch * (D + 2);
  float M = kNegBig;
  for (int c = lane; c < nchb; c += 64) M = fmaxf(M, pp[(size_t)c * (D + 2) + D]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float lsum = 0.f;
  for (int c = lane; c < nchb; c += 64) {
    const float* p = pp + (size_t)c * (D + 2);
    lsum += p[D + 1] * fast_exp2(p[D] - M);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int c = 0; c < nchb; ++c) {
    const float* p = pp + (size_t)c * (D + 2);
    const float w = fast_exp2(p[D] - M);
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] += w * p[lane + 64 * i];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* o = (uint16_t*)a.o + (size_t)bh * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[lane + 64 * i] = (uint16_t)bf16_bits(acc[i] * inv);
  if (lane == 0) a.lse[bh] = lsum > 0.f ? (M + fast_log2(lsum)) * kLn2 : -INFINITY;
}

// ============================================================ sparse layer
// One work group (8 waves) per (b, g).  Work items: the n_sel selected blocks
// of the shared cache, then the ceil(min(L, W)/64) tiles of the window ring;
// item i goes to wave i % 8.  Each wave keeps one online-softmax state per
// branch; the 8 partial states are merged through LDS and the two branches
// combined with the gates.
template <int D>
__global__ __launch_bounds__(512) void decode_sparse_kernel(DecodeSparseArgs a) {
  using Tt = Tr<HS_BF16>;
  using Eng = WaveAttn<HS_BF16, D, 1>;
  constexpr int ES = 2;
  constexpr int NW = 8;
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ __attribute__((aligned(16))) float sm_o[NW][16][D];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int bg = blockIdx.x;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int L = a.lens[b];
  const int G = a.Hq / a.Hkv;
  const int col = lane & 15;
  const int h = g * G + col;
  const int r16 = lane & 15, q8 = 8 * (lane >> 4), q4 = (lane >> 4) << 2;
  const int nring = a.W > 0 ? (min(L, a.W) + 63) / 64 : 0;
  const int nslots = min(L, a.W);

  Eng sp, sw;
  sp.reset();
  sw.reset();
#pragma unroll
  for (int ks = 0; ks < Eng::NS; ++ks) {
    sp.qf[0][ks] = col < G ? Tt::ld((const char*)a.q + ((size_t)(b * a.Hq + h) * D + 32 * ks + q8) * ES)
                           : Tt::zero();
    sw.qf[0][ks] = sp.qf[0][ks];
  }
  const char* kg = (const char*)a.k + (size_t)(b * a.Hkv + g) * a.C * D * ES;
  const char* vg = (const char*)a.v + (size_t)(b * a.Hkv + g) * (a.C / 64) * D * 64 * ES;
  const int32_t* il = a.idx + (size_t)(b * a.Hkv + g) * a.nsel;
  float bmax[1], bsum[1];
  int lo[1], hi[1];

  for (int it = w; it < a.nsel + nring; it += NW) {
    if (it < a.nsel) {
      const int j = il[it];
      if (j < 0 || 64 * j >= L) continue;
      const int kb0 = 64 * j;
      const bool partial = kb0 + 64 > L;
      lo[0] = col < G ? 0 : kNoKey;
      hi[0] = L - 1;
      auto ldK = [&](int c, int ks) {
        const int key = kb0 + tile_key(c, r16);
        return (!partial || key < L) ? Tt::ld(kg + ((size_t)key * D + 32 * ks + q8) * ES) : Tt::zero();
      };
      auto ldV = [&](int u, int mc) {
        const auto f = Tt::ld(vg + (((size_t)j * D + 16 * mc + r16) * 64 + 32 * u + q8) * ES);
        return partial ? Tt::keep(f, L - (kb0 + 32 * u + q8)) : f;
      };
      sp.template tile<true, false>(ldK, ldV, kb0, lo, hi, a.sc2, bmax, bsum);
    } else {
      const int r = it - a.nsel;
      const int s0 = 64 * r;
      const char* krg = (const char*)a.kr + (size_t)(b * a.Hkv + g) * a.W * D * ES;
      const char* vrg = (const char*)a.vr + (size_t)(b * a.Hkv + g) * ((a.W + 63) / 64) * D * 64 * ES;
      lo[0] = col < G ? 0 : kNoKey;
      hi[0] = nslots - 1;
      auto ldK = [&](int c, int ks) {
        const int s = s0 + tile_key(c, r16);
        return s < nslots ? Tt::ld(krg + ((size_t)s * D + 32 * ks + q8) * ES) : Tt::zero();
      };
      auto ldV = [&](int u, int mc) {
        const int s = s0 + 32 * u + q8;
        if (s >= nslots) return Tt::zero();
        const auto f = Tt::ld(vrg + (((size_t)r * D + 16 * mc + r16) * 64 + 32 * u + q8) * ES);
        return s + 8 <= nslots ? f : Tt::keep(f, nslots - s);
      };
      sw.template tile<true, false>(ldK, ldV, s0, lo, hi, a.sc2, bmax, bsum);
    }
  }

  // merge the 8 partial states of each branch through LDS, one branch at a
  // time; thread -> (head column, d) outputs
  constexpr int PER = (16 * D + 64 * NW - 1) / (64 * NW);
  float out[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) out[i] = 0.f;
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    Eng& e = br ? sw : sp;
    float lt = e.l[0] + __shfl_xor(e.l[0], 16);
    lt += __shfl_xor(lt, 32);
    if (lane < 16) {
      sm_m[w][col] = e.m[0];
      sm_l[w][col] = lt;
    }
#pragma unroll
    for (int mc = 0; mc < Eng::NM; ++mc) *(float4*)&sm_o[w][col][16 * mc + q4] = *(const float4*)&e.o[0][mc];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int el = threadIdx.x + 64 * NW * i;
      const int c = el / D, d = el % D;
      if (c < G) {
        float M = kNegBig;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww][c]);
        float ls = 0.f, os = 0.f;
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
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int el = threadIdx.x + 64 * NW * i;
    const int c = el / D, d = el % D;
    if (c < G) ((uint16_t*)a.o)[((size_t)b * a.Hq + g * G + c) * D + d] = (uint16_t)bf16_bits(out[i]);
  }
}

// ================================================================ launchers
hipError_t launch_decode_full(const DecodeFullArgs& a, int D, hipStream_t s) {
  const long units = (long)a.B * a.Hkv * a.nch;
  dim3 grid((unsigned)((units + 3) / 4));
  if (D == 128) {
    if (a.token) hipLaunchKernelGGL((decode_full_kernel<128, 1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((decode_full_kernel<128, 0>), grid, dim3(256), 0, s, a);
  } else {
    if (a.token) hipLaunchKernelGGL((decode_full_kernel<64, 1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((decode_full_kernel<64, 0>), grid, dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)(((long)a.B * a.Hq + 3) / 4));
  if (D == 128) hipLaunchKernelGGL(decode_combine_kernel<128>, g2, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(decode_combine_kernel<64>, g2, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_sparse(const DecodeSparseArgs& a, int D, hipStream_t s) {
  dim3 grid((unsigned)(a.B * a.Hkv));
  if (D == 128) hipLaunchKernelGGL(decode_sparse_kernel<128>, grid, dim3(512), 0, s, a);
  else hipLaunchKernelGGL(decode_sparse_kernel<64>, grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs
