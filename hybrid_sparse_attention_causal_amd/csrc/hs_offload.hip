// hs_offload.hip -- the full layer's KV cache held in host memory (HySparse
// paper, section 5 "Discussion & Future Works": offload the full attention
// layer's cache to external memory and prefetch it before the computation,
// keeping only the selected blocks on the GPU for the sparse layers).
//
//  gather_blocks_kernel  copies each (sequence, kv head)'s selected 64-token
//                        blocks of a block-mode cache into a compact cache:
//                        the concatenation K~, V~ of explainer 3.4.3
//  offload_pipeline      one decode step's full layer over a host cache:
//                        double-buffered chunk prefetch on a copy stream,
//                        then the split-K full layer, the block top-k and
//                        the gather of each chunk on the compute stream
#include <mutex>

#include "hs_internal.h"
#include "hs_sel_list.h"

namespace hs {

// grid (B*Hkv, ceil(nsel / kGatherSlots)), 256 threads; each work group
// canonicalises the row (the list is a set of fully-past blocks) and copies
// up to kGatherSlots of its live blocks.  Slot p < n receives live block sel[p]; idx_sel[p] = p,
// and -1 for p >= n (those slots are not written).
constexpr int kGatherSlots = 8;

__global__ __launch_bounds__(256) void gather_blocks_kernel(GatherArgs a) {
  __shared__ int sm_wtot[4];
  extern __shared__ uint32_t dyn[];
  const int bg = blockIdx.x;
  const int b = bg / a.Hkv;
  const int L = min(max(a.lens[b], 0), a.C);
  const int cap = sel_list_cap(a.nsel);
  const uint32_t* sel = dyn + cap;
  // fully-past blocks only (j < floor((L-1)/64)): a gathered block is whole
  const int n = canon_sel_list<256>(a.idx + (size_t)bg * a.nsel, a.nsel, (uint32_t)(L > 0 ? (L - 1) / 64 : 0),
                                    cap, dyn, dyn + cap, sm_wtot);
  const size_t blk_bytes = (size_t)64 * a.D * a.es;  // one block of keys, or of values
  const int p0 = blockIdx.y * kGatherSlots;
  for (int p = p0 + (threadIdx.x >> 6); p < min(p0 + kGatherSlots, a.nsel); p += 4) {
    if (threadIdx.x % 64 == 0) a.idx_sel[(size_t)bg * a.nsel + p] = p < n ? p : -1;
  }
  const int nblk = blk_bytes / 16;  // 16-byte words per block
  for (int p = p0; p < min(p0 + kGatherSlots, n); ++p) {
    const size_t j = sel[p];
    const uint4* ks = (const uint4*)((const char*)a.k + ((size_t)bg * a.C + 64 * j) * a.D * a.es);
    const uint4* vs = (const uint4*)((const char*)a.v + ((size_t)bg * (a.C / 64) + j) * blk_bytes);
    uint4* kd = (uint4*)((char*)a.k_sel + ((size_t)bg * a.nsel + p) * blk_bytes);
    uint4* vd = (uint4*)((char*)a.v_sel + ((size_t)bg * a.nsel + p) * blk_bytes);
    for (int i = threadIdx.x; i < nblk; i += 256) {
      const uint4 x = ks[i], y = vs[i];
      kd[i] = x;
      vd[i] = y;
    }
  }
}

hipError_t launch_gather_blocks(const GatherArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.B * a.Hkv), (unsigned)((a.nsel + kGatherSlots - 1) / kGatherSlots));
  const size_t lds = 2 * (size_t)sel_list_cap(a.nsel) * sizeof(uint32_t);
  hipLaunchKernelGGL(gather_blocks_kernel, grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

size_t offload_stage_bytes(int chunk, int Hkv, int C, int D, int es) {
  return 2 * (size_t)chunk * Hkv * C * D * es;
}

namespace {

// events of the pipeline, created once per device and reused.  A stream's
// wait on an event binds to the event's latest record at the time the wait
// is enqueued, so calls that enqueue one after another may share them; the
// pipeline holds g_ev_mu while it enqueues, so calls from several host
// threads do not interleave their records and waits.
struct PipeEvents {
  hipEvent_t entry, ready[2], free_[2];
  bool made = false;
};
std::mutex g_ev_mu;
PipeEvents g_ev[256];

// called with g_ev_mu held
hipError_t pipe_events(PipeEvents** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 256) return hipErrorInvalidDevice;
  PipeEvents& p = g_ev[dev];
  if (!p.made) {
    hipEvent_t* all[5] = {&p.entry, &p.ready[0], &p.ready[1], &p.free_[0], &p.free_[1]};
    for (hipEvent_t* ev : all) {
      e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
    p.made = true;
  }
  *out = &p;
  return hipSuccess;
}

#define HS_TRY(x)                          \
  do {                                     \
    hipError_t e_ = (x);                   \
    if (e_ != hipSuccess) return e_;       \
  } while (0)

}  // namespace

hipError_t offload_pipeline(const OffloadArgs& a, int D, hipStream_t s, hipStream_t cs) {
  std::lock_guard<std::mutex> lock(g_ev_mu);
  PipeEvents* ev = nullptr;
  HS_TRY(pipe_events(&ev));
  const int B = a.full.B, Hkv = a.full.Hkv, Hq = a.full.Hq, C = a.full.C, es = a.gather.es;
  const size_t krow = (size_t)D * es;             // bytes of one key row
  const size_t vblk = (size_t)64 * D * es;        // bytes of one value block
  const size_t kseq = (size_t)C * krow;           // one (sequence, kv head) key slab
  const size_t vseq = (size_t)(C / 64) * vblk;
  const size_t stage_k = (size_t)a.chunk * Hkv * kseq;  // keys first, then values
  // the staging buffers may still be read by earlier work on the compute stream
  HS_TRY(hipEventRecord(ev->entry, s));
  HS_TRY(hipStreamWaitEvent(cs, ev->entry, 0));
  const int nchunk = (B + a.chunk - 1) / a.chunk;
  for (int c = 0; c < nchunk; ++c) {
    const int b0 = c * a.chunk, nb = min(a.chunk, B - b0), sl = c & 1;
    char* sk = (char*)a.stage[sl];
    char* sv = sk + stage_k;
    // prefetch: the live key rows and value blocks of every (sequence, kv head)
    if (c >= 2) HS_TRY(hipStreamWaitEvent(cs, ev->free_[sl], 0));
    for (int i = 0; i < nb; ++i) {
      const int L = min(max(a.lens_host[b0 + i], 0), C);
      for (int g = 0; g < Hkv; ++g) {
        const size_t src = (size_t)(b0 + i) * Hkv + g, dst = (size_t)i * Hkv + g;
        if (L > 0) {
          HS_TRY(hipMemcpyAsync(sk + dst * kseq, (const char*)a.full.k + src * kseq, L * krow,
                                hipMemcpyHostToDevice, cs));
          HS_TRY(hipMemcpyAsync(sv + dst * vseq, (const char*)a.full.v + src * vseq, ((L + 63) / 64) * vblk,
                                hipMemcpyHostToDevice, cs));
        }
      }
    }
    HS_TRY(hipEventRecord(ev->ready[sl], cs));
    HS_TRY(hipStreamWaitEvent(s, ev->ready[sl], 0));
    // full layer, selection and gather of this chunk, on the staged caches
    DecodeFullArgs f = a.full;
    f.k = sk;
    f.v = sv;
    f.B = nb;
    f.q = (const char*)a.full.q + (size_t)b0 * Hq * D * 2;
    f.o = (char*)a.full.o + (size_t)b0 * Hq * D * 2;
    f.lse = a.full.lse + (size_t)b0 * Hq;
    f.raw = a.full.raw + (size_t)b0 * Hq * (C / 64);
    f.lens = a.full.lens + b0;
    HS_TRY(launch_decode_full(f, D, s));
    TopkArgs t = a.topk;
    t.B = nb;
    t.raw = f.raw;
    t.lse = f.lse;
    t.gs = a.topk.gs ? a.topk.gs + (size_t)b0 * Hkv * (C / 64) : nullptr;
    t.idx = a.topk.idx + (size_t)b0 * Hkv * a.topk.kb;
    t.kv_lens = f.lens;
    HS_TRY(launch_block_topk(t, t.raw_stride, s));
    GatherArgs gth = a.gather;
    gth.k = sk;
    gth.v = sv;
    gth.idx = t.idx;
    gth.lens = f.lens;
    gth.B = nb;
    gth.k_sel = (char*)a.gather.k_sel + (size_t)b0 * Hkv * a.gather.nsel * vblk;
    gth.v_sel = (char*)a.gather.v_sel + (size_t)b0 * Hkv * a.gather.nsel * vblk;
    gth.idx_sel = a.gather.idx_sel + (size_t)b0 * Hkv * a.gather.nsel;
    HS_TRY(launch_gather_blocks(gth, s));
    HS_TRY(hipEventRecord(ev->free_[sl], s));
  }
  return hipSuccess;
}

}  // namespace hs
