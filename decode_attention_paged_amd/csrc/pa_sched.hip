// Work order of the grouped-query kernel over a ragged batch (gfx950).
//
// Flash-Decoding's split-KV step gives each (sequence, KV head, split) its own
// workgroup (the "flash decoding ++" entry, its "three steps" snippet: the
// chunks are processed in parallel, each keeping its log-sum-exp).  With
// ragged lengths those units differ in size: every split holds c pages but a
// sequence's last split holds the remainder, and short sequences have a single
// small one.  The hardware dispatches workgroups in grid order as slots free
// up, so a long unit dispatched late leaves the other CUs idle at the end of
// the launch.  This kernel writes, into the workspace, the order in which the
// grid takes the units: every full split first, then the last splits by
// decreasing size (the longest-processing-time-first rule, sizes bucketed),
// then one "no unit" entry for every grid slot left over.  The partial kernel
// reads its (sequence, split) from this table; what each unit computes is
// unchanged, so the outputs do not depend on the order.
//
// One workgroup: a count pass and a placement pass over the B context lengths
// (read once for batches up to 1024 sequences) around a scan of a
// 1024-bucket histogram in LDS.

#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSchedBuckets = 1024;   // one per thread in the scan
static_assert(kSchedBuckets == kSchedThreads, "one bucket per thread");

// The units of one sequence: `full` splits of c pages, then (if `part`) one
// last split of `last` < c pages, in bucket `bucket` (larger splits in lower
// buckets).  A sequence with no pages still has one unit (it writes the
// empty result), of size 0.
struct SeqUnits {
  int full;
  bool part;
  int bucket;
};

__device__ __forceinline__ SeqUnits seq_units(int ctx, int max_ctx, int bs, int c) {
  const int n = min(max(ctx, 0), max_ctx);
  const int pages = (n + bs - 1) / bs;
  const int ns = pages > 0 ? (pages + c - 1) / c : 1;
  const int last = pages - (ns - 1) * c;               // pages of the last split, 0 .. c
  SeqUnits u;
  u.part = last < c;
  u.full = u.part ? ns - 1 : ns;
  // c - last in 1 .. c maps onto buckets 0 .. kSchedBuckets - 1 in order
  u.bucket = (int)(((long long)(c - last) * (kSchedBuckets - 1)) / c);
  return u;
}

__global__ __launch_bounds__(kSchedThreads) void unit_schedule(const int32_t* __restrict__ ctx,
                                                              int B, int max_ctx, int bs, int c,
                                                              int entries,
                                                              uint32_t* __restrict__ table) {
  __shared__ int hist[kSchedBuckets];
  __shared__ int wave_sum[kSchedThreads / 64];
  __shared__ int n_full, full_pos, n_real;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  // this thread's first sequence stays in registers between the passes (one
  // read of the lengths for batches up to kSchedThreads); further ones are
  // read again in the second pass
  const SeqUnits u0 = t < B ? seq_units(ctx[t], max_ctx, bs, c) : SeqUnits{0, false, 0};
  hist[t] = 0;
  if (t == 0) {
    n_full = 0;
    full_pos = 0;
  }
  __syncthreads();
  auto count = [&](const SeqUnits& u) {
    if (u.full) atomicAdd(&n_full, u.full);
    if (u.part) atomicAdd(&hist[u.bucket], 1);
  };
  count(u0);
  for (int b = t + kSchedThreads; b < B; b += kSchedThreads)
    count(seq_units(ctx[b], max_ctx, bs, c));
  __syncthreads();
  // exclusive scan of the histogram, after the full splits
  const int h = hist[t];
  int v = h;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) wave_sum[wave] = v;
  __syncthreads();
  int before = n_full;
  for (int i = 0; i < wave; ++i) before += wave_sum[i];
  hist[t] = before + v - h;
  if (t == kSchedThreads - 1) n_real = before + v;
  __syncthreads();
  auto place = [&](int b, const SeqUnits& u) {
    if (u.full) {
      const int base = atomicAdd(&full_pos, u.full);
      for (int s = 0; s < u.full; ++s) table[base + s] = (uint32_t)b | ((uint32_t)s << 16);
    }
    if (u.part) {
      const int pos = atomicAdd(&hist[u.bucket], 1);
      table[pos] = (uint32_t)b | ((uint32_t)u.full << 16);
    }
  };
  if (t < B) place(t, u0);
  for (int b = t + kSchedThreads; b < B; b += kSchedThreads)
    place(b, seq_units(ctx[b], max_ctx, bs, c));
  for (int i = n_real + t; i < entries; i += kSchedThreads) table[i] = kNoUnit;
}

}  // namespace

hipError_t launch_unit_schedule(const Params& p, hipStream_t st) {
  hipLaunchKernelGGL(unit_schedule, dim3(1), dim3(kSchedThreads), 0, st, p.context_lens, p.B,
                     p.max_ctx, p.bs, p.c, p.B * p.S, p.sched);
  return hipGetLastError();
}

}  // namespace pa
