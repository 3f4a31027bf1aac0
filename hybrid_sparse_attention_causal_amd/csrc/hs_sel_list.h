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
// hs_block_topk writes its lists ascending and duplicate-free; such a list
// is only checked, anything else is sorted first (bitonic, in LDS).
// buf and out hold `cap` words each, cap = the power of two >= nsel (at
// least 64).  NTHR threads, all of which must call this.
template <int NTHR>
__device__ int canon_sel_list(const int32_t* il, int nsel, uint32_t limit, int cap, uint32_t* buf,
                              uint32_t* out, int* sm_wtot) {
  constexpr int NWV = NTHR / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  bool unsorted = false;
  for (int p = tid; p < cap; p += NTHR) {
    uint32_t v = p < nsel ? (uint32_t)il[p] : 0xFFFFFFFFu;
    buf[p] = v < limit ? v : 0xFFFFFFFFu;
  }
  __syncthreads();
  for (int p = tid; p + 1 < nsel; p += NTHR) unsorted |= buf[p] > buf[p + 1];
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
  int cnt = 0;
  for (int i = 0; i < per; ++i) {
    const int p = tid * per + i;
    if (p < cap) {
      const uint32_t x = buf[p];
      cnt += x != 0xFFFFFFFFu && (p == 0 || x != buf[p - 1]);
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
  int off = inc - cnt, n = 0;
#pragma unroll
  for (int ww = 0; ww < NWV; ++ww) {
    off += ww < w ? sm_wtot[ww] : 0;
    n += sm_wtot[ww];
  }
  for (int i = 0; i < per; ++i) {
    const int p = tid * per + i;
    if (p < cap) {
      const uint32_t x = buf[p];
      if (x != 0xFFFFFFFFu && (p == 0 || x != buf[p - 1])) out[off++] = x;
    }
  }
  __syncthreads();
  return n;
}

__host__ __device__ inline int sel_list_cap(int nsel) {
  int c = 64;
  while (c < nsel) c <<= 1;
  return c;
}

}  // namespace hs
