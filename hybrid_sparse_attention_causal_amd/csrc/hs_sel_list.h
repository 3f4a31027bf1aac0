// hs_sel_list.h -- a selection list (block or token ids) as a set, in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

// ================================================= selection list as a set
// The sparse branch attends the union of the selected blocks or tokens
// (explainer 3.4.3 eq. K~,V~): the list is a set.  Every decode sparse work
// group first copies its (sequence, kv head) list into LDS in a canonical
// form: ids that are negative or not below `limit` are dropped, an id listed
// twice counts once, and the input order does not matter.  The live ids end
// up ascending in out[0 .. n), and n is returned to every thread.
// The selection kernels write their lists ascending and duplicate-free with
// the padding at the end; such a list is taken as it is after one check pass
// (two barriers).  Anything else is sorted (bitonic, in LDS) and compacted.
// buf and out hold `cap` words each, cap = the power of two >= nsel (at
// least 64).  NTHR threads, all of which must call this.
//
// The work comes in two parts.  sel_list_request requests entries
// u * NTHR + tid (u < kSelU) of the list into registers; canon_sel_list_from
// stores them and the rest of the list into LDS and makes it canonical.  A
// caller can use the requested entries in between (thread tid of wave w holds
// entry 64 (NTHR/64 u + w) + lane in v[u]), and learns through `canonical`
// whether the list was taken as it was.
constexpr int kSelU = 8;
constexpr uint32_t kSelEmpty = 0xFFFFFFFFu;
template <int NTHR>
__device__ __forceinline__ void sel_list_request(const int32_t* il, int nsel, uint32_t (&v)[kSelU]) {
#pragma unroll
  for (int u = 0; u < kSelU; ++u) {
    const int p = u * NTHR + (int)threadIdx.x;
    v[u] = p < nsel ? (uint32_t)il[p] : kSelEmpty;
  }
}

template <int NTHR>
__device__ int canon_sel_list_from(const uint32_t (&v0)[kSelU], const int32_t* il, int nsel, uint32_t limit,
                                   int cap, uint32_t* buf, uint32_t* out, int* sm_wtot, bool& canonical) {
  constexpr int NWV = NTHR / 64;
  constexpr int U = kSelU;
  constexpr uint32_t kEmpty = kSelEmpty;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // copy into out (ids out of range become kEmpty); past the requested part,
  // a thread's U loads are all requested before the first store
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = u * NTHR + tid;
    if (p < cap) out[p] = v0[u] < limit ? v0[u] : kEmpty;
  }
  for (int p0 = U * NTHR; p0 < cap; p0 += U * NTHR) {
    uint32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * NTHR + tid;
      v[u] = p < nsel ? (uint32_t)il[p] : kEmpty;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * NTHR + tid;
      if (p < cap) out[p] = v[u] < limit ? v[u] : kEmpty;
    }
  }
  __syncthreads();
  // canonical already: every live id below its successor, and nothing but
  // kEmpty after the first kEmpty?  The live ids are then out[0 .. n).
  int cnt = 0;
  bool bad = false;
  for (int p0 = 0; p0 < cap; p0 += U * NTHR) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * NTHR + tid;
      if (p < cap) {
        const uint32_t x = out[p], nx = p + 1 < cap ? out[p + 1] : kEmpty;
        bad |= !(x < nx || nx == kEmpty);
        cnt += x != kEmpty;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  const bool wbad = __ballot(bad) != 0;
  if (lane == 0) sm_wtot[w] = cnt | (wbad ? 1 << 30 : 0);
  __syncthreads();
  int n = 0, anybad = 0;
#pragma unroll
  for (int ww = 0; ww < NWV; ++ww) {
    n += sm_wtot[ww] & ((1 << 30) - 1);
    anybad |= sm_wtot[ww] >> 30;
  }
  canonical = !anybad;
  if (!anybad) return n;

  // general case: sort a copy if it is out of order, then keep the first of
  // each run of equal ids
  bool unsorted = false;
  for (int p = tid; p < cap; p += NTHR) buf[p] = out[p];
  __syncthreads();  // also: every thread has read sm_wtot
  for (int p = tid; p + 1 < cap; p += NTHR) unsorted |= buf[p] > buf[p + 1];
  if (__syncthreads_or(unsorted)) {
    for (int k = 2; k <= cap; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < cap; i += NTHR) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint32_t x = buf[i], y = buf[ixj];
            if ((x > y) == ((i & k) == 0)) {
              buf[i] = y;
              buf[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
  }
  // compaction: thread tid owns entries [tid*per, tid*per + per)
  const int per = (cap + NTHR - 1) / NTHR;
  cnt = 0;
  for (int i = 0; i < per; ++i) {
    const int p = tid * per + i;
    if (p < cap) {
      const uint32_t x = buf[p];
      cnt += x != kEmpty && (p == 0 || x != buf[p - 1]);
    }
  }
  int inc = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sm_wtot[w] = inc;
  __syncthreads();
  int off = inc - cnt;
  n = 0;
#pragma unroll
  for (int ww = 0; ww < NWV; ++ww) {
    off += ww < w ? sm_wtot[ww] : 0;
    n += sm_wtot[ww];
  }
  for (int i = 0; i < per; ++i) {
    const int p = tid * per + i;
    if (p < cap) {
      const uint32_t x = buf[p];
      if (x != kEmpty && (p == 0 || x != buf[p - 1])) out[off++] = x;
    }
  }
  __syncthreads();
  return n;
}

template <int NTHR>
__device__ int canon_sel_list(const int32_t* il, int nsel, uint32_t limit, int cap, uint32_t* buf,
                              uint32_t* out, int* sm_wtot) {
  uint32_t v[kSelU];
  sel_list_request<NTHR>(il, nsel, v);
  bool canonical;
  return canon_sel_list_from<NTHR>(v, il, nsel, limit, cap, buf, out, sm_wtot, canonical);
}

__host__ __device__ inline int sel_list_cap(int nsel) {
  int c = 64;
  while (c < nsel) c <<= 1;
  return c;
}

}  // namespace hs
