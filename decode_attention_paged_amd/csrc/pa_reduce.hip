// Log-sum-exp weighted reduction of split partials (Flash-Decoding's third
// step in the "flash decoding ++" entry, its three-steps snippet: rescale
// each split's output by its log-sum-exp and combine).
//
//   M = max_s lse_s,  w_s = exp(lse_s - M),
//   out = sum_s w_s o_s / sum_s w_s,  lse = M + ln(sum_s w_s).
//
// One wave per (sequence, query row, head) row, four rows per workgroup.  The
// row's split weights come from its lse values (uniform across the wave);
// each lane owns float4 columns of the output (8 columns when the partials
// are bfloat16) and sums the splits it needs with 16-byte loads, several
// splits in flight at once.  Only the splits the sequence actually used are
// read (ragged batches use fewer splits for shorter sequences).
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kRedWaves = 4;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <bool BF16>
__global__ __launch_bounds__(kRedWaves * 64) void split_reduce(Params p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRedWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= p.B * p.ql * p.Hq) return;
  const int b = row / (p.ql * p.Hq);                 // rows are (sequence, query row, head)
  const int ctx = clampi(p.context_lens[b], 0, p.max_ctx);
  const int pages = (ctx + p.bs - 1) / p.bs;
  int nsp = splits_of(pages, p.c);
  nsp = nsp > 0 ? nsp : 1;
  const float* lp = p.lse_part + (size_t)row * p.S;
  const float* op = p.o_part + (size_t)row * p.S * p.Dv;

  float m = kNegInf;
  for (int i = lane; i < nsp; i += 64) m = fmaxf(m, lp[i]);
  const float M = wave_max(m);
  const bool empty = (M == kNegInf);
  float l = 0.f;
  if (!empty)
    for (int i = lane; i < nsp; i += 64) l += fast_exp2((lp[i] - M) * kLog2e);
  const float L = wave_sum(l);
  const float inv = empty ? 0.f : 1.f / L;

  const int cols = p.Dv / 4;
  for (int c = lane; c < cols; c += 64) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (!empty) {
#pragma unroll 8
      for (int s = 0; s < nsp; ++s) {
        const float wt = fast_exp2((lp[s] - M) * kLog2e);
        const f32x4 v = *reinterpret_cast<const f32x4*>(op + (size_t)s * p.Dv + c * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(wt, v[r], acc[r]);
      }
    }
    if constexpr (BF16) {
      u32x2 pk;
      pk[0] = pack_bf16(acc[0] * inv, acc[1] * inv);
      pk[1] = pack_bf16(acc[2] * inv, acc[3] * inv);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + (size_t)row * p.Dv + c * 4) = pk;
    } else {
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = acc[r] * inv;
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + (size_t)row * p.Dv + c * 4) = o;
    }
  }
  // dims past the last full float4 column (head dims not a multiple of 4)
  for (int d = cols * 4 + lane; d < p.Dv; d += 64) {
    float acc = 0.f;
    if (!empty)
      for (int s = 0; s < nsp; ++s)
        acc = fmaf(fast_exp2((lp[s] - M) * kLog2e), op[(size_t)s * p.Dv + d], acc);
    if constexpr (BF16)
      static_cast<uint16_t*>(p.out)[(size_t)row * p.Dv + d] = to_bf16(acc * inv);
    else
      static_cast<float*>(p.out)[(size_t)row * p.Dv + d] = acc * inv;
  }
  if (lane == 0 && p.lse) p.lse[row] = empty ? kNegInf : M + fast_log2(L) * kLn2;
}

// Partials stored as bfloat16 (the MLA matrix-core path; head_dim_v a
// multiple of 8, output bfloat16): the same merge, 8 columns per lane.
__global__ __launch_bounds__(kRedWaves * 64) void split_reduce_p16(Params p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRedWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= p.B * p.ql * p.Hq) return;
  const int b = row / (p.ql * p.Hq);
  const int ctx = clampi(p.context_lens[b], 0, p.max_ctx);
  const int pages = (ctx + p.bs - 1) / p.bs;
  int nsp = splits_of(pages, p.c);
  nsp = nsp > 0 ? nsp : 1;
  const float* lp = p.lse_part + (size_t)row * p.S;
  const uint16_t* op = p.o_part16 + (size_t)row * p.S * p.Dv;

  float m = kNegInf;
  for (int i = lane; i < nsp; i += 64) m = fmaxf(m, lp[i]);
  const float M = wave_max(m);
  const bool empty = (M == kNegInf);
  float l = 0.f;
  if (!empty)
    for (int i = lane; i < nsp; i += 64) l += fast_exp2((lp[i] - M) * kLog2e);
  const float L = wave_sum(l);
  const float inv = empty ? 0.f : 1.f / L;

  for (int c = lane; c < p.Dv / 8; c += 64) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (!empty) {
#pragma unroll 8
      for (int s = 0; s < nsp; ++s) {
        const float wt = fast_exp2((lp[s] - M) * kLog2e);
        const u32x4 v = *reinterpret_cast<const u32x4*>(op + (size_t)s * p.Dv + c * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] = fmaf(wt, bf16lo(v[j]), acc[2 * j]);
          acc[2 * j + 1] = fmaf(wt, bf16hi(v[j]), acc[2 * j + 1]);
        }
      }
    }
    u32x4 pk;
#pragma unroll
    for (int j = 0; j < 4; ++j) pk[j] = pack_bf16(acc[2 * j] * inv, acc[2 * j + 1] * inv);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + (size_t)row * p.Dv + c * 8) = pk;
  }
  if (lane == 0 && p.lse) p.lse[row] = empty ? kNegInf : M + fast_log2(L) * kLn2;
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
  const int rows = p.B * p.ql * p.Hq;
  dim3 grid((rows + kRedWaves - 1) / kRedWaves);
  if (p.o_part16 != nullptr)   // bfloat16 partials: bfloat16 output, head_dim_v % 8 == 0
    hipLaunchKernelGGL(split_reduce_p16, grid, dim3(kRedWaves * 64), 0, st, p);
  else if (bf16)
    hipLaunchKernelGGL(split_reduce<true>, grid, dim3(kRedWaves * 64), 0, st, p);
  else
    hipLaunchKernelGGL(split_reduce<false>, grid, dim3(kRedWaves * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace pa
