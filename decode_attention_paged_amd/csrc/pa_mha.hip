// Split-KV partial kernel for plain multi-head decode, on the vector ALUs.
//
// One workgroup per (split, query head, sequence); its NW waves take the
// split's pages round-robin and each keeps its own running (max, sum, acc)
// state, merged in LDS at the end (the per-chunk step of Flash-Decoding in
// the "flash decoding ++" entry, its three-steps snippet: attention of the
// query with each chunk, recording its log-sum-exp).  A single query row per KV head gives no operand reuse, so
// the dot products run on the VALU (v_dot2_f32_bf16 for bf16) rather than
// on MFMA.
//
// Lane mapping for one (page, head) tile:
//   K rows are D*esize bytes; LPR lanes cover a row with 16-byte loads and a
//   wave loads RPI = 64/LPR rows per instruction.  The score of token
//   i*RPI + r ends up in every lane of row group r after a DPP reduction.
//   V is stored [D][bs] (a row of bs tokens per dim).  Each V load reads 1 KiB
//   of the tile contiguously: lane l takes 16 bytes, TPL tokens of one dim,
//   so LPD lanes share a dim and each keeps a partial sum over its tokens;
//   the LPD partials are added once, after the loop.  Token weights are
//   read into SGPRs (v_readlane) and each lane selects its TPL of them.
//   (Loads that each cover a full 1 KiB run measurably faster than loads
//   of 16 bytes at a 32-byte stride, which read every cache line twice.)
#include "pa_device.h"
#include "pa_launch.h"
#include "pa_merge.h"

namespace pa {
namespace {

// F8: the caches hold FP8 E4M3 codes (BF16 queries); ES is the cache
// element size, QES the query's.
template <bool BF16, int D, int BS, bool F8 = false>
struct MhaCfg {
  static constexpr int ES = F8 ? 1 : (BF16 ? 2 : 4);
  static constexpr int QES = BF16 ? 2 : 4;
  static constexpr int ROWB = D * ES;      // bytes per K row
  static constexpr int QROWB = D * QES;    // bytes per query row
  static constexpr int QPL = 16 / ES;      // dims of a K row per lane (one 16-byte load)
  static constexpr int QV = QPL * QES / 16;   // 16-byte query loads per lane
  static constexpr int LPR = ROWB / 16;    // lanes per K row
  static constexpr int RPI = 64 / LPR;     // K rows per load instruction
  static constexpr int KI = BS / RPI;      // K loads per page
  static constexpr int VROWB = BS * ES;    // bytes per V row (one dim's bs tokens)
  static constexpr int LPD = VROWB / 16;   // lanes per V row in a load
  static constexpr int DPI = 64 / LPD;     // dims per V load (1 KiB)
  static constexpr int VI = D / DPI;       // V loads per page = partial sums per lane
  static constexpr int TPL = BS / LPD;     // tokens per lane in a V load (16 / ES)
  static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32, "row width");
  static_assert(!F8 || BF16, "FP8 caches take bf16 queries");
  static_assert(BS % RPI == 0 && VROWB % 16 == 0 && LPD <= 8 && D % DPI == 0, "tile shape");
  static_assert(TPL == 16 / ES, "a V load holds whole tokens");
};

// Sum over the LPR lanes of one K row.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (LPR == 4) {
    x += dpp<kDppQuadXor2>(x);
    return x + dpp<kDppQuadXor1>(x);
  } else if constexpr (LPR == 8) {
    return group_sum<8>(x);
  } else if constexpr (LPR == 16) {
    return group_sum<16>(x);
  } else {
    return sum_xor16(group_sum<16>(x));
  }
}

// Max / sum across the RPI row groups of a wave.
// (rows of 4 lanes: the four row groups of a 16-lane DPP row are lanes 4
// apart, combined by rotations of 4 and 8)
template <int LPR>
__device__ __forceinline__ float across_rows_max(float x) {
  if constexpr (LPR == 4) x = fmaxf(x, dpp<kDppRowRor4>(x));
  if constexpr (LPR <= 8) x = fmaxf(x, dpp<kDppRowRor8>(x));
  if constexpr (LPR <= 16) x = max_xor16(x);
  return max_xor32(x);
}
template <int LPR>
__device__ __forceinline__ float across_rows_sum(float x) {
  if constexpr (LPR == 4) x += dpp<kDppRowRor4>(x);
  if constexpr (LPR <= 8) x += dpp<kDppRowRor8>(x);
  if constexpr (LPR <= 16) x = sum_xor16(x);
  return sum_xor32(x);
}

template <bool BF16, int D, int BS, bool F8>
struct MhaTile {
  u32x4 k[MhaCfg<BF16, D, BS, F8>::KI];
  u32x4 v[MhaCfg<BF16, D, BS, F8>::VI];
};

template <bool BF16, int D, int BS, bool F8>
__device__ __forceinline__ void load_tile(MhaTile<BF16, D, BS, F8>& t, const char* kp,
                                          const char* vp, int lane) {
  using C = MhaCfg<BF16, D, BS, F8>;
  const char* kl = kp + (lane / C::LPR) * C::ROWB + (lane % C::LPR) * 16;
#pragma unroll
  for (int i = 0; i < C::KI; ++i) t.k[i] = ld128_stream(kl + i * C::RPI * C::ROWB);
#pragma unroll
  for (int k = 0; k < C::VI; ++k) t.v[k] = ld128_stream(vp + k * 1024 + lane * 16);
}

// Running state of one wave: max (log2 domain, wave-uniform), this lane's
// row-group share of the sum, and the lane's partial sums of VI output dims
// (dim k*DPI + lane/LPD over its TPL tokens of each page).
template <int VI>
struct MhaState {
  float m;
  float l;
  float acc[VI];
};

template <bool BF16, int D, int BS, bool F8, bool PARTIAL>
__device__ __forceinline__ void consume_tile(const MhaTile<BF16, D, BS, F8>& t,
                                             MhaState<MhaCfg<BF16, D, BS, F8>::VI>& st,
                                             const u32x4 (&qv)[MhaCfg<BF16, D, BS, F8>::QV],
                                             const float (&qf)[4], float scale_log2, int lane,
                                             int nvalid) {
  using C = MhaCfg<BF16, D, BS, F8>;
  const int row = lane / C::LPR;
  float sc[C::KI];
#pragma unroll
  for (int i = 0; i < C::KI; ++i) {
    float d = 0.f;
    if constexpr (F8) {
      // 16 dims: word e holds dims 4e .. 4e+3, matched by query words 2e, 2e+1
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = t.k[i][e];
        d = dot2_bf16(qv[e >> 1][(2 * e) & 3], fp8x2_to_bf16x2<false>(w), d);
        d = dot2_bf16(qv[e >> 1][(2 * e + 1) & 3], fp8x2_to_bf16x2<true>(w), d);
      }
    } else if constexpr (BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) d = dot2_bf16(qv[0][e], t.k[i][e], d);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) d = fmaf(qf[e], as_f32(t.k[i][e]), d);
    }
    d = row_sum<C::LPR>(d) * scale_log2;
    if constexpr (PARTIAL) d = (i * C::RPI + row < nvalid) ? d : kNegInf;
    sc[i] = d;
  }
  float mx = sc[0];
#pragma unroll
  for (int i = 1; i < C::KI; ++i) mx = fmaxf(mx, sc[i]);
  mx = across_rows_max<C::LPR>(mx);
  const float mn = fmaxf(st.m, mx);          // finite: the tile has a valid token
  const float alpha = fast_exp2(st.m - mn);  // 0 on the first tile (m = -inf)
  st.m = mn;
  float pr[C::KI];
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < C::KI; ++i) {
    pr[i] = fast_exp2(sc[i] - mn);
    lsum += pr[i];
  }
  st.l = fmaf(st.l, alpha, lsum);
  // token weights as wave-uniform scalars: token i*RPI + r lives in row group r
  float ps[BS];
#pragma unroll
  for (int t2 = 0; t2 < BS; ++t2) ps[t2] = readlane(pr[t2 / C::RPI], (t2 % C::RPI) * C::LPR);
  // this lane's tokens in every V load: tb .. tb + TPL - 1
  const int sub = lane % C::LPD;
  const int tb = sub * C::TPL;
  float wt[C::TPL];
#pragma unroll
  for (int e = 0; e < C::TPL; ++e) {
    float x = ps[e];
#pragma unroll
    for (int g = 1; g < C::LPD; ++g) x = (sub == g) ? ps[g * C::TPL + e] : x;
    wt[e] = x;
  }
#pragma unroll
  for (int k = 0; k < C::VI; ++k) {
    float a = st.acc[k] * alpha;
    const u32x4 vv = t.v[k];
    if constexpr (F8) {
      // 16 tokens: word e holds tokens 4e .. 4e+3
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(vv[e], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(vv[e], true);
        const float v4[4] = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int te = 4 * e + j;
          const float v0 = (PARTIAL && tb + te >= nvalid) ? 0.f : v4[j];
          a = fmaf(wt[te], v0, a);
        }
      }
    } else if constexpr (BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int te = 2 * e;
        float v0 = bf16lo(vv[e]), v1 = bf16hi(vv[e]);
        if constexpr (PARTIAL) {
          v0 = (tb + te < nvalid) ? v0 : 0.f;
          v1 = (tb + te + 1 < nvalid) ? v1 : 0.f;
        }
        a = fmaf(wt[te], v0, a);
        a = fmaf(wt[te + 1], v1, a);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v0 = as_f32(vv[e]);
        if constexpr (PARTIAL) v0 = (tb + e < nvalid) ? v0 : 0.f;
        a = fmaf(wt[e], v0, a);
      }
    }
    st.acc[k] = a;
  }
}

// Add the LPD partial sums of each dim (lanes l ^ 1, l ^ 2, l ^ 4 within a row).
template <int LPD>
__device__ __forceinline__ float dim_sum(float x) {
  if constexpr (LPD >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (LPD >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (LPD >= 8) x += dpp<kDppRowHalfMirror>(x);
  return x;
}

template <bool BF16, int D, int BS, bool F8, int NW>
__global__ __launch_bounds__(NW * 64) void mha_valu_partial(Params p) {
  using C = MhaCfg<BF16, D, BS, F8>;
  // head fastest: consecutive workgroups land on different XCDs with equal work
  const int h = blockIdx.x, b = blockIdx.z;
  const int s = split_of_block(blockIdx.y, b, p.S);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int ctx = clampi(p.context_lens[b], 0, p.max_ctx);
  const int pages = (ctx + BS - 1) / BS;
  const int nsplit = splits_of(pages, p.c);
  if (s >= (nsplit > 0 ? nsplit : 1)) return;
  const int g = h / (p.Hq / p.Hkv);
  const int p0 = s * p.c;
  const int p1 = min(pages, p0 + p.c);

  // the query dims matching this lane's part of a K row
  const char* qrow = static_cast<const char*>(p.q) + ((size_t)b * p.Hq + h) * C::QROWB;
  u32x4 qv[C::QV];
#pragma unroll
  for (int i = 0; i < C::QV; ++i) qv[i] = ld128(qrow + (lane % C::LPR) * C::QV * 16 + i * 16);
  float qf[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) qf[e] = as_f32(qv[0][e]);

  const int* bt = p.block_table + (size_t)b * p.maxb;
  const size_t kstride = (size_t)p.Hkv * BS * C::ROWB;      // bytes per K page
  const size_t vstride = (size_t)p.Hkv * D * BS * C::ES;    // bytes per V page
  const char* kbase = static_cast<const char*>(p.k) + (size_t)g * BS * C::ROWB;
  const char* vbase = static_cast<const char*>(p.v) + (size_t)g * D * BS * C::ES;

  MhaState<C::VI> st;
  st.m = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int k = 0; k < C::VI; ++k) st.acc[k] = 0.f;

  auto issue = [&](MhaTile<BF16, D, BS, F8>& t, int pg) {
    if (pg >= p1) {                                  // past the split: read zeros (L2)
      const char* z = reinterpret_cast<const char*>(g_zero_tile);
      load_tile(t, z, z, lane);
      return;
    }
    const int id = clampi(bt[pg], 0, p.nblocks - 1);
    load_tile(t, kbase + id * kstride, vbase + id * vstride, lane);
  };
  auto consume = [&](MhaTile<BF16, D, BS, F8>& t, int pg) {
    const int nvalid = ctx - pg * BS;
    if (nvalid >= BS)
      consume_tile<BF16, D, BS, F8, false>(t, st, qv, qf, p.scale_log2, lane, BS);
    else
      consume_tile<BF16, D, BS, F8, true>(t, st, qv, qf, p.scale_log2, lane, nvalid);
  };
  // Two register tiles in turn (see the grouped-query kernel): each consume
  // waits only for its own tile's loads; tiles past the split read zeros.
  int pg = p0 + w;
  MhaTile<BF16, D, BS, F8> t0, t1;
  issue(t0, pg);
  issue(t1, pg + NW);
  for (; pg < p1; pg += 2 * NW) {
    consume(t0, pg);
    issue(t0, pg + 2 * NW);
    if (pg + NW >= p1) break;
    consume(t1, pg + NW);
    issue(t1, pg + 3 * NW);
  }
  const float ltot = across_rows_sum<C::LPR>(st.l);

  // ---- merge the NW wave states and write the split result
  __shared__ float sm_m[NW], sm_l[NW];
  __shared__ float sm_acc[NW][D];
  if (lane == 0) {
    sm_m[w] = st.m;
    sm_l[w] = ltot;
  }
#pragma unroll
  for (int k = 0; k < C::VI; ++k) {
    const float a = dim_sum<C::LPD>(st.acc[k]);
    if (lane % C::LPD == 0) sm_acc[w][k * C::DPI + lane / C::LPD] = a;
  }
  __syncthreads();

  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < NW; ++i) M = fmaxf(M, sm_m[i]);
  float f[NW];
  float L = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    f[i] = (M == kNegInf) ? 0.f : fast_exp2(sm_m[i] - M);
    L = fmaf(f[i], sm_l[i], L);
  }
  const bool empty = (M == kNegInf);
  // FP8 caches: every value carries v_scale, applied once here
  const float inv = empty ? 0.f : (F8 ? p.v_scale : 1.f) / L;
  const float lse = empty ? kNegInf : (M + fast_log2(L)) * kLn2;
  const size_t row = (size_t)b * p.Hq + h;
  const bool direct = split_is_direct(p, nsplit);
  for (int d = threadIdx.x; d < D; d += NW * 64) {
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) o = fmaf(f[i], sm_acc[i][d], o);
    o *= inv;
    if (direct)
      store_out<BF16>(p, row, d, o);
    else
      store_partial(p, p.o_part + (row * p.S + s) * D + d, o);
  }
  if (threadIdx.x == 0) {
    if (direct) {
      if (p.lse) p.lse[row] = lse;
    } else {
      store_partial(p, p.lse_part + row * p.S + s, lse);
    }
  }
  if (!direct && p.fused) {
    __shared__ int sm_flag;
    __shared__ __attribute__((aligned(16))) float scratch[NW * 64 * 4];
    const int unit = b * p.Hq + h;
    if (arrive_last(p, unit, nsplit, &sm_flag)) {
      merge_unit<BF16, NW * 64>(p, b, h, 1, nsplit, scratch);
      reset_counter(p, unit);
    }
  }
}

constexpr int kMhaWaves = 4;

template <bool BF16, int D, int BS, bool F8 = false>
hipError_t launch_one(const Params& p, hipStream_t st) {
  dim3 grid(p.Hq, p.S, p.B);
  hipLaunchKernelGGL((mha_valu_partial<BF16, D, BS, F8, kMhaWaves>), grid, dim3(kMhaWaves * 64), 0,
                     st, p);
  return hipGetLastError();
}

}  // namespace

// 256-dim heads: bfloat16 only (a float32 K row would need 64 lanes of 16 bytes)
bool mha_valu_supported(bool bf16, int D, int bs) {
  return (D == 64 || D == 128 || (bf16 && D == 256)) && (bs == 16 || bs == 32);
}

bool mha_valu_fp8_supported(int D, int bs) {
  return (D == 64 || D == 128 || D == 256) && (bs == 16 || bs == 32);
}

hipError_t launch_mha_valu(const Params& p, bool bf16, bool fp8kv, hipStream_t st) {
  const int D = p.D, bs = p.bs;
  if (fp8kv) {
    if (!bf16) return hipErrorInvalidValue;
    if (D == 64 && bs == 16) return launch_one<true, 64, 16, true>(p, st);
    if (D == 64 && bs == 32) return launch_one<true, 64, 32, true>(p, st);
    if (D == 256 && bs == 16) return launch_one<true, 256, 16, true>(p, st);
    if (D == 256 && bs == 32) return launch_one<true, 256, 32, true>(p, st);
    if (D == 128 && bs == 16) return launch_one<true, 128, 16, true>(p, st);
    if (D == 128 && bs == 32) return launch_one<true, 128, 32, true>(p, st);
    return hipErrorInvalidValue;
  }
  if (bf16) {
    if (D == 256 && bs == 16) return launch_one<true, 256, 16>(p, st);
    if (D == 256 && bs == 32) return launch_one<true, 256, 32>(p, st);
    if (D == 128 && bs == 16) return launch_one<true, 128, 16>(p, st);
    if (D == 128 && bs == 32) return launch_one<true, 128, 32>(p, st);
    if (D == 64 && bs == 16) return launch_one<true, 64, 16>(p, st);
    if (D == 64 && bs == 32) return launch_one<true, 64, 32>(p, st);
  } else {
    if (D == 128 && bs == 16) return launch_one<false, 128, 16>(p, st);
    if (D == 128 && bs == 32) return launch_one<false, 128, 32>(p, st);
    if (D == 64 && bs == 16) return launch_one<false, 64, 16>(p, st);
    if (D == 64 && bs == 32) return launch_one<false, 64, 32>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
