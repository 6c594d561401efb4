// Split-KV partial kernel for MLA latent decode on the matrix cores.
//
// All query heads attend to one latent row per token (keys: the whole
// 576-wide row; values: its first 512 entries, the same memory).  Every
// latent page is a dense contraction shared by all heads: scores
// S^T[64 tok x 16 heads] = C[64 x 576] Q^T and values
// O^T[512 x 16] += V^T[512 x 64] P^T, per wave of 16 heads, on
// v_mfma_f32_16x16x32_bf16.  A workgroup (NW waves, 16*NW heads) stages one
// page of the latent pool in LDS and all its waves read it; each wave keeps
// the online-softmax state of its own heads over the split's pages and
// writes the split's (o_s, lse_s) (page 4, Flash-Decoding's second step).
//
// LDS tile: 64 token rows of 1152 bytes, padded to 1168 so that rows start
// in different banks.  Score A operands are 16-byte reads of token rows.
// Value A operands need 8 consecutive tokens of one dim per lane from this
// token-major tile; ds_read_b64_tr_b16 provides them: within each 16-lane
// group, lane i receives element i%4 of the 8-byte chunks read by lanes
// i/4 + 4r (r = 0..3), so lane i pointing at row t0 + i/4, column
// c0 + 4*(i%4) returns V[t0 + r][c0 + i] for r = 0..3.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kBS = 64;
constexpr int kRowB = kDqk * 2;           // 1152 bytes per latent row
constexpr int kLdsRow = kRowB + 16;       // padded LDS row
constexpr int kKSteps = kDqk / 32;        // 18 score k-steps
constexpr int kNB = kDv / 16;             // 32 value dim blocks
constexpr int kChunks = kBS * kRowB / 16; // 4608 16-byte chunks per page
constexpr int kChunksPerRow = kRowB / 16; // 72

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x2 lds_tr16(const lds_char* p) {
  short4v t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)p);
  return __builtin_bit_cast(u32x2, t);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void mla_mfma_partial(Params p) {
  __shared__ __attribute__((aligned(16))) char tile_g[kBS * kLdsRow];
  lds_char* tile = (lds_char*)tile_g;

  const int hb = blockIdx.x, b = blockIdx.z;
  const int s = split_of_block(blockIdx.y, b, p.S);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int quad = lane >> 4, n = lane & 15;
  const int h0 = (hb * NW + w) * 16;
  const int ctx = clampi(p.context_lens[b], 0, p.max_ctx);
  const int pages = (ctx + kBS - 1) / kBS;
  const int nsplit = splits_of(pages, p.c);
  if (s >= (nsplit > 0 ? nsplit : 1)) return;
  const int p0 = s * p.c;
  const int p1 = min(pages, p0 + p.c);

  // Q^T as B operands: head h0 + n, dims kb*32 + quad*8 .. +8
  u32x4 qf[kKSteps];
  {
    const char* qr = static_cast<const char*>(p.q) + ((size_t)b * p.Hq + h0 + n) * kRowB;
#pragma unroll
    for (int kb = 0; kb < kKSteps; ++kb) qf[kb] = ld128(qr + kb * 64 + quad * 16);
  }

  f32x4 acc[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.f;

  const int* bt = p.block_table + (size_t)b * p.maxb;
  const char* cbase = static_cast<const char*>(p.k);
  const size_t pstride = (size_t)kBS * kRowB;

  // score A-operand rows: chain (ks, c), row n <-> token ks*32 + (n/4)*8 + 4c + n%4
  int srow[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      srow[ks][c] = (ks * 32 + (n >> 2) * 8 + c * 4 + (n & 3)) * kLdsRow + quad * 16;
  // value A-operand addresses: read h, k-step ks, dim block nb
  const int vrow = (quad * 8 + (n >> 2)) * kLdsRow + (n & 3) * 8;

  for (int pg = p0; pg < p1; ++pg) {
    const int id = clampi(bt[pg], 0, p.nblocks - 1);
    const char* src = cbase + id * pstride;
    const int nvalid = min(kBS, ctx - pg * kBS);
    __syncthreads();   // every wave is done with the previous tile
    for (int c = threadIdx.x; c < kChunks; c += NW * 64) {
      const int tok = c / kChunksPerRow, cc = c % kChunksPerRow;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (tok < nvalid) v = ld128_stream(src + (size_t)c * 16);
      *(__attribute__((address_space(3))) u32x4*)(tile + tok * kLdsRow + cc * 16) = v;
    }
    __syncthreads();

    f32x4 sacc[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int c = 0; c < 2; ++c) sacc[ks][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < kKSteps; ++kb) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4 a = *(const __attribute__((address_space(3))) u32x4*)(tile + srow[ks][c] + kb * 64);
          sacc[ks][c] = mfma(a, qf[kb], sacc[ks][c]);
        }
    }
    // this lane's scores: token ks*32 + quad*8 + c*4 + r of the page, head n
    float sc[2][8];
    float mx = kNegInf;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = ks * 32 + quad * 8 + c * 4 + r;
          float x = sacc[ks][c][r] * p.scale_log2;
          x = (tok < nvalid) ? x : kNegInf;
          sc[ks][c * 4 + r] = x;
          mx = fmaxf(mx, x);
        }
    mx = max_xor32(max_xor16(mx));
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    u32x4 pb[2];
    float ls = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pr[j] = fast_exp2(sc[ks][j] - mn);
        ls += pr[j];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) pb[ks][e] = pack_bf16(pr[2 * e], pr[2 * e + 1]);
    }
    l = fmaf(l, alpha, ls);
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      f32x4 a = acc[nb];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const lds_char* base = tile + vrow + ks * 32 * kLdsRow + nb * 32;
        const u32x2 lo = lds_tr16(base);
        const u32x2 hi = lds_tr16(base + 4 * kLdsRow);
        const u32x4 va = u32x4{lo[0], lo[1], hi[0], hi[1]};
        a = mfma(va, pb[ks], a);
      }
      acc[nb] = a;
    }
  }
  const float ltot = sum_xor32(sum_xor16(l));
  const bool empty = (m == kNegInf);
  const float inv = empty ? 0.f : 1.f / ltot;
  const float lse = empty ? kNegInf : (m + fast_log2(ltot)) * kLn2;
  const size_t row = (size_t)b * p.Hq + h0 + n;
  if (p.final_write) {
    uint16_t* o = static_cast<uint16_t*>(p.out) + row * kDv;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      u32x2 pk;
      pk[0] = pack_bf16(acc[nb][0] * inv, acc[nb][1] * inv);
      pk[1] = pack_bf16(acc[nb][2] * inv, acc[nb][3] * inv);
      *reinterpret_cast<u32x2*>(o + nb * 16 + quad * 4) = pk;
    }
    if (quad == 0 && p.lse) p.lse[row] = lse;
  } else {
    float* o = p.o_part + (row * p.S + s) * kDv;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      f32x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[nb][r] * inv;
      *reinterpret_cast<f32x4*>(o + nb * 16 + quad * 4) = v;
    }
    if (quad == 0) p.lse_part[row * p.S + s] = lse;
  }
}

template <int NW>
hipError_t launch_nw(const Params& p, hipStream_t st) {
  dim3 grid(p.Hq / (16 * NW), p.S, p.B);
  hipLaunchKernelGGL(mla_mfma_partial<NW>, grid, dim3(NW * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace

bool mla_mfma_supported(bool bf16, int Dqk, int Dv, int bs, int Hq) {
  return bf16 && Dqk == kDqk && Dv == kDv && bs == kBS && Hq % 16 == 0;
}

hipError_t launch_mla_mfma(const Params& p, hipStream_t st) {
  const int hblocks = p.Hq / 16;
  if (hblocks % 8 == 0) return launch_nw<8>(p, st);
  if (hblocks % 4 == 0) return launch_nw<4>(p, st);
  if (hblocks % 2 == 0) return launch_nw<2>(p, st);
  return launch_nw<1>(p, st);
}

}  // namespace pa
