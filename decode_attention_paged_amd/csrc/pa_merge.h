// Split results: writing a split's (o_s, lse_s), and the fused reduction run
// by the last workgroup of a (sequence, head unit) to finish.
//
// The reduction is Flash-Decoding's third step (the "flash decoding ++" entry,
// its three-steps snippet): rescale each split
// output by exp(lse_s - max lse) and sum, normalised by the sum of weights;
// lse = max + ln(sum of weights).
#pragma once

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// How a workgroup's split result leaves the kernel.
//   direct: the split is the whole sequence (S == 1, or a fused call whose
//           sequence needs one split): write out/lse.
//   else:   write o_part/lse_part; in a fused call the last workgroup of the
//           unit then merges.
__device__ __forceinline__ bool split_is_direct(const Params& p, int nsplit) {
  return p.final_write || (p.fused && nsplit <= 1);
}

// Split partials cross workgroups (and XCDs, whose L2 caches are not coherent
// with each other) only through device-scope coherent accesses: agent-scope
// atomic stores and loads (global_store/global_load with sc1), which complete
// at the device-coherent level.  arrive_last orders them before the arrival
// (each thread waits for its own stores) and after it (the last workgroup
// acquires before it reads), without writing back whole L2 caches.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One value of a split partial.  Read back in this launch (the fused merge):
// a coherent store.  Read by a separate reduction launch: a plain store, made
// visible by the kernel boundary; the coherent store writes through to memory
// and measured 2.5-4.5 % slower on the MHA partial kernel.
__device__ __forceinline__ void store_partial(const Params& p, float* dst, float v) {
  if (p.fused)
    store_coherent(dst, v);
  else
    *dst = v;
}

template <bool BF16>
__device__ __forceinline__ void store_out(const Params& p, size_t row, int d, float o) {
  if constexpr (BF16)
    static_cast<uint16_t*>(p.out)[row * p.Dv + d] = to_bf16(o);
  else
    static_cast<float*>(p.out)[row * p.Dv + d] = o;
}

// Arrive at the unit's counter after this workgroup's partials are written
// (with store_coherent).  Returns true (in every thread) when this workgroup
// is the last of the unit's `nsplit` splits.
//
// Release: a barrier alone does not wait for outstanding vector-memory
// stores, so every thread first waits until its own partial stores have
// completed (vmcnt(0)); they are coherent stores, so completed means visible
// to every CU.  Only then does the barrier let thread 0 bump the counter.
// Acquire: the workgroup that takes the last arrival invalidates its
// non-coherent cached lines (an agent-scope acquire fence, once per unit)
// before the barrier that releases its threads to read the partials.
// The last workgroup resets the counter, leaving the workspace ready for the
// next call.
__device__ __forceinline__ bool arrive_last(const Params& p, int unit, int nsplit, int* sm_flag) {
  wait_stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old =
        __hip_atomic_fetch_add(p.counters + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (old == nsplit - 1) ? 1 : 0;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *sm_flag = last;
  }
  __syncthreads();
  return *sm_flag != 0;
}

__device__ __forceinline__ void reset_counter(const Params& p, int unit) {
  if (threadIdx.x == 0)
    __hip_atomic_store(p.counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the `nsplit` partials of heads [h0, h0 + nh) of sequence b and write
// out/lse.  All NT threads take part: thread t owns a float4 column of one
// head and a residue class of splits; residue classes are summed in `scratch`
// (>= NT * 4 floats of LDS).
template <bool BF16, int NT>
__device__ __forceinline__ void merge_unit(const Params& p, int b, int h0, int nh, int nsplit,
                                           float* scratch) {
  const int cols = p.Dv / 4;
  const int items = nh * cols;
  const int groups = items >= NT ? 1 : NT / items;
  const int t = threadIdx.x;
  for (int base = 0; base < items; base += NT) {
    const int item = base + (groups == 1 ? t : t % items);
    const int grp = groups == 1 ? 0 : t / items;
    const bool active = item < items && grp < groups;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float M = kNegInf, L = 0.f;
    size_t row = 0;
    int c4 = 0;
    if (active) {
      const int hn = item / cols;
      c4 = item % cols;
      row = (size_t)b * p.Hq + h0 + hn;
      const float* lp = p.lse_part + row * p.S;
      for (int s = 0; s < nsplit; ++s) M = fmaxf(M, load_coherent(lp + s));
      if (M != kNegInf) {
        for (int s = 0; s < nsplit; ++s) L += fast_exp2((load_coherent(lp + s) - M) * kLog2e);
        const float* op = p.o_part + row * p.S * p.Dv + c4 * 4;
#pragma unroll 4
        for (int s = grp; s < nsplit; s += groups) {
          const float wt = fast_exp2((load_coherent(lp + s) - M) * kLog2e);
          const float* os = op + (size_t)s * p.Dv;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = fmaf(wt, load_coherent(os + r), acc[r]);
        }
      }
    }
    if (groups > 1) {
      __syncthreads();
      if (active) *reinterpret_cast<f32x4*>(scratch + t * 4) = acc;
      __syncthreads();
      if (active && grp == 0) {
        for (int g2 = 1; g2 < groups; ++g2) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(scratch + (g2 * items + item) * 4);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] += v[r];
        }
      }
    }
    if (active && grp == 0) {
      const bool empty = (M == kNegInf);
      const float inv = empty ? 0.f : 1.f / L;
#pragma unroll
      for (int r = 0; r < 4; ++r) store_out<BF16>(p, row, c4 * 4 + r, acc[r] * inv);
      if (c4 == 0 && p.lse) p.lse[row] = empty ? kNegInf : M + fast_log2(L) * kLn2;
    }
  }
}

}  // namespace pa
