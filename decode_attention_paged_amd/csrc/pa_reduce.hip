// Log-sum-exp weighted reduction of split partials (Flash-Decoding's third
// step, page 4: rescale each split's output by its log-sum-exp and combine).
//
//   M = max_s lse_s,  w_s = exp(lse_s - M),
//   out = sum_s w_s o_s / sum_s w_s,  lse = M + ln(sum_s w_s).
//
// One workgroup per (query head, sequence, block of 64 output dims); its four
// waves each sum a quarter of the splits for the same 64 dims and the
// quarters are added in LDS.  Only the splits the sequence actually used are
// read (ragged batches use fewer splits for shorter sequences).
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kRedWaves = 4;

__device__ __forceinline__ float block_max(float x, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  if (lane == 0) red[w] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kRedWaves; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

template <bool BF16>
__global__ __launch_bounds__(kRedWaves * 64) void split_reduce(Params p) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = blockIdx.z * 64 + lane;
  const int ctx = clampi(p.context_lens[b], 0, p.max_ctx);
  const int pages = (ctx + p.bs - 1) / p.bs;
  int nsp = splits_of(pages, p.c);
  nsp = nsp > 0 ? nsp : 1;
  const size_t row = (size_t)b * p.Hq + h;
  const float* lp = p.lse_part + row * p.S;
  const float* op = p.o_part + row * p.S * p.Dv;

  __shared__ float red[kRedWaves];
  __shared__ float part[kRedWaves][64];
  __shared__ float lsum[kRedWaves];

  float mx = kNegInf;
  for (int i = threadIdx.x; i < nsp; i += kRedWaves * 64) mx = fmaxf(mx, lp[i]);
  const float M = block_max(mx, red);
  const bool empty = (M == kNegInf);

  float acc = 0.f, L = 0.f;
  if (!empty) {
    for (int i = w; i < nsp; i += kRedWaves) {
      const float wt = fast_exp2((lp[i] - M) * kLog2e);
      L += wt;
      if (d < p.Dv) acc = fmaf(wt, op[(size_t)i * p.Dv + d], acc);
    }
  }
  part[w][lane] = acc;
  if (lane == 0) lsum[w] = L;
  __syncthreads();
  if (w == 0) {
    float o = 0.f, lt = 0.f;
#pragma unroll
    for (int i = 0; i < kRedWaves; ++i) {
      o += part[i][lane];
      lt += lsum[i];
    }
    o = empty ? 0.f : o / lt;
    if (d < p.Dv) {
      if constexpr (BF16)
        static_cast<uint16_t*>(p.out)[row * p.Dv + d] = to_bf16(o);
      else
        static_cast<float*>(p.out)[row * p.Dv + d] = o;
    }
    if (blockIdx.z == 0 && lane == 0 && p.lse)
      p.lse[row] = empty ? kNegInf : M + fast_log2(lt) * kLn2;
  }
}

__global__ void zero_i32(int32_t* dst, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = 0;
}

}  // namespace

hipError_t launch_zero_i32(int32_t* dst, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(zero_i32, dim3(blocks), dim3(256), 0, st, dst, n);
  return hipGetLastError();
}

hipError_t launch_reduce(const Params& p, bool bf16, hipStream_t st) {
  dim3 grid(p.Hq, p.B, (p.Dv + 63) / 64);
  if (bf16)
    hipLaunchKernelGGL(split_reduce<true>, grid, dim3(kRedWaves * 64), 0, st, p);
  else
    hipLaunchKernelGGL(split_reduce<false>, grid, dim3(kRedWaves * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace pa
