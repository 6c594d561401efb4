// Paged KV append: the new token of every sequence goes to the page and slot
// its position selects (the wenku.it search page for "paged attention", its
// vLLM README snippets: the KV cache lives in fixed-size pages named by a
// per-sequence block table), right before the decode step
// reads it.  Position n = context_lens[b] (the length before the append):
//   page = block_table[b][n / bs], slot = n % bs.
// A sequence whose position is outside its block table, or whose page id is
// outside the pool, writes nothing.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

__device__ __forceinline__ bool append_slot(const AppendParams& a, int b, int& page, int& slot) {
  const int n = a.context_lens[b];
  if (n < 0 || (int64_t)n >= (int64_t)a.maxb * a.bs) return false;
  page = a.block_table[(size_t)b * a.maxb + n / a.bs];
  slot = n % a.bs;
  return page >= 0 && page < a.nblocks;
}

// One workgroup per (KV head, sequence); threads stride over the head dims.
// K rows are contiguous; a V column is strided by the page size (V is stored
// [dim][token] per page).
template <typename T>
__global__ __launch_bounds__(256) void append_kv_kernel(AppendParams a) {
  const int g = blockIdx.x, b = blockIdx.y;
  int page, slot;
  if (!append_slot(a, b, page, slot)) return;
  const T* kn = static_cast<const T*>(a.k_new) + ((size_t)b * a.Hkv + g) * a.D;
  const T* vn = static_cast<const T*>(a.v_new) + ((size_t)b * a.Hkv + g) * a.Dv;
  T* kc = static_cast<T*>(a.k_cache) + (((size_t)page * a.Hkv + g) * a.bs + slot) * a.D;
  T* vc = static_cast<T*>(a.v_cache) + ((size_t)page * a.Hkv + g) * (size_t)a.Dv * a.bs + slot;
  for (int d = threadIdx.x; d < a.D; d += blockDim.x) kc[d] = kn[d];
  for (int d = threadIdx.x; d < a.Dv; d += blockDim.x) vc[(size_t)d * a.bs] = vn[d];
}

// MLA: one latent row per token, one workgroup per sequence.
template <typename T>
__global__ __launch_bounds__(256) void append_latent_kernel(AppendParams a) {
  const int b = blockIdx.x;
  int page, slot;
  if (!append_slot(a, b, page, slot)) return;
  const T* cn = static_cast<const T*>(a.k_new) + (size_t)b * a.D;
  T* cc = static_cast<T*>(a.k_cache) + ((size_t)page * a.bs + slot) * a.D;
  for (int d = threadIdx.x; d < a.D; d += blockDim.x) cc[d] = cn[d];
}

template <typename T>
hipError_t launch_typed(const AppendParams& a, bool mla, hipStream_t st) {
  if (mla)
    hipLaunchKernelGGL(append_latent_kernel<T>, dim3(a.B), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(append_kv_kernel<T>, dim3(a.Hkv, a.B), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendParams& a, int esize, bool mla, hipStream_t st) {
  switch (esize) {
    case 1: return launch_typed<uint8_t>(a, mla, st);    // FP8 codes
    case 2: return launch_typed<uint16_t>(a, mla, st);   // bfloat16
    case 4: return launch_typed<uint32_t>(a, mla, st);   // float32
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
