// Split-KV partial kernel for grouped-query decode on the matrix cores.
//
// When G = Hq / Hkv query heads share one KV head, each K/V tile is a real
// dense contraction with G columns, so the scores S^T = K Q^T and the value
// product O^T = V^T P^T run on v_mfma_f32_16x16x32_bf16 (heads padded to
// 16 columns).  One workgroup handles one (split, KV head, sequence): the
// tile of a page is read from HBM once for all G heads.  Its NW waves take
// 32-token steps round-robin (the MFMA contraction depth of the value
// product: a pair of 16-token pages, or one 32-token page) and merge their
// running states in LDS at the
// end, which yields the split's (o_s, lse_s) of Flash-Decoding's second step
// (the "flash decoding ++" entry, its three-steps snippet).  NW is 4 (two
// workgroups per CU), or 8 when the grid holds one workgroup per CU: a
// batch too small to fill the CUs, split so that every CU gets one.
//
// Operand layouts (MFMA 16x16x32 bf16: A[i][k] in lane i + 16*(k/8), element
// k%8; B[k][j] in lane j + 16*(k/8); D[i][j] in lane j + 16*(i/4), reg i%4):
//   K is [bs][D] per (page, head): lane (quad, n) loads 16 bytes of one token
//   row, so K is the A operand as stored.  Row n of score chain c is the
//   token (n/8 selects the page of the pair) ((n/4)%2)*8 + 4c + n%4; with this
//   assignment the 8 scores a lane receives (both chains) are tokens
//   (quad%2)*8 + 0..7 of page quad/2, exactly the 8 contraction entries its
//   B operand of the value product needs.  So P^T comes from the lane's own
//   registers, without shuffles.
//   V is stored [D][bs]: 16 contiguous bytes are 8 consecutive tokens of one
//   dim, i.e. the A operand of O^T = V^T P^T as stored.
//   Both outputs put head n in lane column n, so the running max, the
//   rescale factor and the accumulator of a head live in the same lanes.
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"
#include "pa_merge.h"

namespace pa {
namespace {

// D: head dim, 64 or 128 (D / 32 score k-steps, D / 16 value dim blocks).
template <int D>
struct PairTile {
  u32x4 k[2][D / 32];   // [chain][k-step]
  u32x4 v[D / 16];      // [dim block]
};

// The same pair of pages with FP8 E4M3 caches (rows of D bytes), as
// loaded.  The contraction order over dims is free as long as K and Q use
// the same one, so a lane loads 16 contiguous dims of its K row at once:
// k[c][kb2] holds dims (kb2*4 + quad)*16 .. +15, which become the A operands
// of k-steps 2*kb2 (first 8) and 2*kb2 + 1; the query operands follow the
// same order.
// A V row of one dim is 16 bytes (16 tokens; on 32-token pages each
// 16-token half of the 32-byte row).  Lane (n, quad) loads whole rows:
// v[j] holds dim 16*(2j + (quad & 1)) + n, all 16 tokens of page (or half)
// quad / 2.  The value operand needs tokens 8*(quad & 1) .. +7 of dims
// 16*nb + n for every nb, so lanes l and l ^ 16 (rows quad and quad ^ 1 of
// the same page) each hold half of what the other needs; widen() trades
// those halves with v_permlane16_swap.
template <int D>
struct PairTile8 {
  u32x4 k[2][D / 64];
  u32x4 v[D / 32];
};

template <int BS, int D>
__device__ __forceinline__ void load_pair(PairTile8<D>& t, const char* ka, const char* kb_,
                                          const char* va, const char* vb, int koff, int voff,
                                          bool ksel, bool vsel) {
  const char* kp = (ksel ? kb_ : ka) + koff;
  const char* vp = (vsel ? vb : va) + voff;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int kb2 = 0; kb2 < D / 64; ++kb2) t.k[c][kb2] = ld128_stream(kp + c * 4 * D + kb2 * 64);
#pragma unroll
  for (int j = 0; j < D / 32; ++j) t.v[j] = ld128_stream(vp + j * 32 * BS);
}

// Trade words between lanes l and l ^ 16: odd rows of `a` take the even
// rows' `b`, even rows of `b` take the odd rows' `a` (v_permlane16_swap).
__device__ __forceinline__ void swap_rows16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// Widen an FP8 pair tile to the bf16 operands consume_pair takes (exact).
template <int D>
__device__ __forceinline__ void widen(const PairTile8<D>& f, PairTile<D>& t) {
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      const u32x4& w = f.k[c][kb >> 1];
      t.k[c][kb] = (kb & 1) ? fp8x8_to_bf16x8(w[2], w[3]) : fp8x8_to_bf16x8(w[0], w[1]);
    }
  // v[j] of an even row holds dim block 2j (its own tokens 0-7, then the
  // partner's 8-15); of an odd row, dim block 2j + 1 (the partner's tokens
  // 0-7, then its own 8-15).  After the swap every lane has its 8 tokens of
  // both blocks: lo = block 2j, hi = block 2j + 1.
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    uint32_t lo0 = f.v[j][0], lo1 = f.v[j][1], hi0 = f.v[j][2], hi1 = f.v[j][3];
    swap_rows16(lo0, hi0);
    swap_rows16(lo1, hi1);
    t.v[2 * j] = fp8x8_to_bf16x8(lo0, lo1);
    t.v[2 * j + 1] = fp8x8_to_bf16x8(hi0, hi1);
  }
}

template <int BS, int D>
__device__ __forceinline__ void load_pair(PairTile<D>& t, const char* ka, const char* kb_,
                                          const char* va, const char* vb, int koff, int voff,
                                          bool ksel, bool vsel) {
  const char* kp = (ksel ? kb_ : ka) + koff;
  const char* vp = (vsel ? vb : va) + voff;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) t.k[c][kb] = ld128_stream(kp + c * 4 * (2 * D) + kb * 64);
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) t.v[nb] = ld128_stream(vp + nb * 16 * (2 * BS));
}

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <bool PARTIAL, int D>
__device__ __forceinline__ void consume_pair(PairTile<D>& t, const u32x4 (&qf)[D / 32],
                                             f32x4 (&acc)[D / 16],
                                             float& m, float& l, float scale_log2, int tok0,
                                             int ctx_col, int ctx) {
  // tok0: logical index of this lane's first score token; the lane's tokens
  // are tok0 .. tok0+7 (tok0 < 0 marks a page missing from the pair).  The
  // lane's column sees tokens below ctx_col (ctx, or less for an earlier
  // query row); V rows at or past ctx are zeroed.
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb) {
    s0 = mfma(t.k[0][kb], qf[kb], s0);
    s1 = mfma(t.k[1][kb], qf[kb], s1);
  }
  float sc[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sc[r] = s0[r] * scale_log2;
    sc[4 + r] = s1[r] * scale_log2;
  }
  if constexpr (PARTIAL) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sc[j] = (tok0 >= 0 && tok0 + j < ctx_col) ? sc[j] : kNegInf;
  }
  float mx = sc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
  mx = max_xor32(max_xor16(mx));
  const float mn = fmaxf(m, mx);
  // a column that has seen no token yet (an early query row) keeps m = -inf
  // and takes weights of 0 instead of exp2(-inf - -inf)
  const float mref = (PARTIAL && mn == kNegInf) ? 0.f : mn;
  const float alpha = fast_exp2(m - mref);
  m = mn;
  float pr[8];
  float ls = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pr[j] = fast_exp2(sc[j] - mref);
    ls += pr[j];
  }
  l = fmaf(l, alpha, ls);
  u32x4 pb;
#pragma unroll
  for (int e = 0; e < 4; ++e) pb[e] = pack_bf16(pr[2 * e], pr[2 * e + 1]);
  if constexpr (PARTIAL) {
    // tokens past the context may hold anything (NaN): zero them in V
    u32x4 keep;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool v0 = tok0 >= 0 && tok0 + 2 * e < ctx;
      const bool v1 = tok0 >= 0 && tok0 + 2 * e + 1 < ctx;
      keep[e] = (v0 ? 0x0000ffffu : 0u) | (v1 ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) t.v[nb][e] &= keep[e];
  }
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    f32x4 a = acc[nb];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] *= alpha;
    acc[nb] = mfma(t.v[nb], pb, a);
  }
}

// The bf16 operands of a loaded tile: the tile itself, or its FP8 codes widened into tw.
template <bool F8, int D, typename Tile>
__device__ __forceinline__ PairTile<D>& bf16_tile(Tile& tin, PairTile<D>& tw) {
  if constexpr (F8) {
    widen(tin, tw);
    return tw;
  } else {
    return tin;
  }
}

// BS: tokens per page, 16 or 32.  A step consumes 32 tokens: two 16-token
// pages, or one 32-token page as two halves of 16 (K rows 16 apart, V
// tokens 16 apart within each dim's row), so the lane layouts are the same.
template <int NW, bool F8, int BS, int D>
__global__ __launch_bounds__(NW * 64) void gqa_mfma_partial(Params p) {
  using Tile = typename std::conditional<F8, PairTile8<D>, PairTile<D>>::type;
  constexpr int kKS = D / 32;                           // score k-steps
  constexpr int kNB = D / 16;                           // value dim blocks
  constexpr int kR = F8 ? D : 2 * D;                    // bytes per K row
  constexpr int kT = BS * kR;                           // bytes per (page, head) tile
  constexpr int kVR = F8 ? BS : 2 * BS;                 // bytes per V row (one dim)
  const int kvh = blockIdx.x;
  int b, s;
  if (p.sched) {
    // the unit order of a ragged batch (longest first; see pa_sched.hip)
    const uint32_t e = p.sched[blockIdx.z * p.S + blockIdx.y];
    if (e == kNoUnit) return;
    b = (int)(e & 0xffffu);
    s = (int)(e >> 16);
  } else {
    b = blockIdx.z;
    s = split_of_block(blockIdx.y, b, p.S);
  }
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int quad = lane >> 4, n = lane & 15;
  const int G = p.Hq / p.Hkv;
  const int ql = p.ql;
  const int NC = G * ql;                             // MFMA columns in use (<= 16)
  const int ctx = clampi(p.context_lens[b], 0, p.max_ctx);
  // column n is query row cj = n / G of head cg = n % G; row j sees the first
  // ctx - ql + 1 + j tokens (causal over the last ql positions)
  const int cj = n / G, cg = n - cj * G;
  const int ctx_col = ctx - ql + 1 + cj;
  const int ctx_lo = ctx - ql + 1;                   // the shortest any column sees
  const int pages = (ctx + BS - 1) / BS;
  const int nsplit = splits_of(pages, p.c);
  if (s >= (nsplit > 0 ? nsplit : 1)) return;
  const int p0 = s * p.c;
  const int p1 = min(pages, p0 + p.c);

  // Q^T as the B operand of the score MFMA: column n = (row cj, head kvh*G + cg)
  u32x4 qf[kKS];
  if (n < NC) {
    const char* qr =
        static_cast<const char*>(p.q) + (((size_t)b * ql + cj) * p.Hq + kvh * G + cg) * (2 * D);
#pragma unroll
    for (int kb = 0; kb < kKS; ++kb) {
      // k-step kb: dims kb*32 + quad*8 (bf16 caches), or, in the FP8 tile's
      // order, (kb/2*4 + quad)*16 + (kb%2)*8
      const int qo = F8 ? (kb >> 1) * 128 + quad * 32 + (kb & 1) * 16 : kb * 64 + quad * 16;
      qf[kb] = ld128(qr + qo);
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < kKS; ++kb) qf[kb] = u32x4{0u, 0u, 0u, 0u};
  }

  const int* bt = p.block_table + (size_t)b * p.maxb;
  const size_t pstride = (size_t)p.Hkv * kT;      // bytes per page, K and V pools alike
  const char* kbase = static_cast<const char*>(p.k) + (size_t)kvh * kT;
  const char* vbase = static_cast<const char*>(p.v) + (size_t)kvh * kT;
  const bool ksel = (n >> 3) != 0;
  const int koff = (((n >> 2) & 1) * 8 + (n & 3)) * kR + quad * 16;
  const bool vsel = (quad >> 1) != 0;
  // the V bytes of the lane's 16-token page, or of its half of a 32-token one
  const int vhalf = BS == 32 && vsel ? kVR / 2 : 0;
  const int voff = (F8 ? (16 * (quad & 1) + n) * kVR : n * kVR + (quad & 1) * 16) + vhalf;

  f32x4 acc[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.f;

  // 32-token steps: page pairs, or single 32-token pages
  const int npairs = BS == 32 ? p1 - p0 : (p1 - p0 + 1) >> 1;
  int k = w;
  auto issue = [&](Tile& t, int kk) {
    if (kk >= npairs) {                              // past the split: read zeros (L2)
      const char* z = reinterpret_cast<const char*>(g_zero_tile);
      load_pair<BS>(t, z, z, z, z, koff, voff, ksel, vsel);
      return;
    }
    if constexpr (BS == 32) {
      const size_t off = (size_t)clampi(bt[p0 + kk], 0, p.nblocks - 1) * pstride;
      load_pair<BS>(t, kbase + off, kbase + off + 16 * kR, vbase + off, vbase + off, koff, voff,
                    ksel, vsel);
    } else {
      const int pa_ = p0 + 2 * kk;
      const bool hasb = pa_ + 1 < p1;
      const int ida = clampi(bt[pa_], 0, p.nblocks - 1);
      const int idb = hasb ? clampi(bt[pa_ + 1], 0, p.nblocks - 1) : ida;
      load_pair<BS>(t, kbase + ida * pstride, kbase + idb * pstride, vbase + ida * pstride,
                    vbase + idb * pstride, koff, voff, ksel, vsel);
    }
  };
  auto consume = [&](Tile& tin, int kk) {
    // the step's first token and whether its second 16 tokens exist
    const int tok_step = BS == 32 ? (p0 + kk) * 32 : (p0 + 2 * kk) * 16;
    const bool hasb = BS == 32 || p0 + 2 * kk + 1 < p1;
    const bool partial = !hasb || tok_step + 32 > ctx_lo;
    const int tok0 = (vsel && !hasb) ? -1 : tok_step + (vsel ? 16 : 0) + (quad & 1) * 8;
    PairTile<D> tw;
    PairTile<D>& t = bf16_tile<F8, D>(tin, tw);
    if (partial)
      consume_pair<true>(t, qf, acc, m, l, p.scale_log2, tok0, ctx_col, ctx);
    else
      consume_pair<false>(t, qf, acc, m, l, p.scale_log2, tok0, ctx_col, ctx);
  };
  // Two register tiles in turn: while one pair is consumed the next one's
  // loads are in flight, and each consume waits only for its own loads (a
  // copy between tiles at the loop edge would wait for all of them).  Every
  // step issues its loads, past the split's end from the zero tile, so the
  // wait counts are the same on every path.
  Tile t0, t1;
  issue(t0, k);
  issue(t1, k + NW);
  for (; k < npairs; k += 2 * NW) {
    consume(t0, k);
    issue(t0, k + 2 * NW);
    if (k + NW >= npairs) break;
    consume(t1, k + NW);
    issue(t1, k + 3 * NW);
  }
  const float ltot = sum_xor32(sum_xor16(l));

  // ---- merge the NW wave states per head and write the split result
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  constexpr int kOPad = D + 4;                          // LDS row stride of the merge buffer
  __shared__ float sm_o[NW][16][kOPad];
  if (quad == 0) {
    sm_m[w][n] = m;
    sm_l[w][n] = ltot;
  }
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[w][n][nb * 16 + quad * 4 + r] = acc[nb][r];
  __syncthreads();

  const bool direct = split_is_direct(p, nsplit);
  for (int idx = threadIdx.x; idx < NC * D; idx += NW * 64) {
    const int hn = idx / D, d = idx % D;
    const int rj = hn / G, rg = hn - rj * G;
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < NW; ++i) M = fmaxf(M, sm_m[i][hn]);
    const bool empty = (M == kNegInf);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const float f = empty ? 0.f : fast_exp2(sm_m[i][hn] - M);
      L = fmaf(f, sm_l[i][hn], L);
      o = fmaf(f, sm_o[i][hn][d], o);
    }
    o = empty ? 0.f : o * (F8 ? p.v_scale : 1.f) / L;   // FP8 caches: values carry v_scale
    const float lse = empty ? kNegInf : (M + fast_log2(L)) * kLn2;
    const size_t row = ((size_t)b * ql + rj) * p.Hq + kvh * G + rg;
    if (direct) {
      store_out<true>(p, row, d, o);
      if (d == 0 && p.lse) p.lse[row] = lse;
    } else {
      store_partial(p, p.o_part + (row * p.S + s) * D + d, o);
      if (d == 0) store_partial(p, p.lse_part + row * p.S + s, lse);
    }
  }
  if (!direct && p.fused) {
    __shared__ int sm_flag;
    const int unit = b * p.Hkv + kvh;
    if (arrive_last(p, unit, nsplit, &sm_flag)) {
      merge_unit<true, NW * 64>(p, b, kvh * G, G, nsplit, &sm_o[0][0][0]);
      reset_counter(p, unit);
    }
  }
}

template <int NW, int BS, int D>
void launch_shape(const Params& p, bool fp8kv, hipStream_t st) {
  dim3 grid(p.Hkv, p.S, p.B);
  if (fp8kv)
    hipLaunchKernelGGL((gqa_mfma_partial<NW, true, BS, D>), grid, dim3(NW * 64), 0, st, p);
  else
    hipLaunchKernelGGL((gqa_mfma_partial<NW, false, BS, D>), grid, dim3(NW * 64), 0, st, p);
}
template <int NW, int BS>
void launch_dim(const Params& p, bool fp8kv, hipStream_t st) {
  if (p.D == 64)
    launch_shape<NW, BS, 64>(p, fp8kv, st);
  else
    launch_shape<NW, BS, 128>(p, fp8kv, st);
}
template <int NW>
void launch_waves(const Params& p, bool fp8kv, hipStream_t st) {
  if (p.bs == 32)
    launch_dim<NW, 32>(p, fp8kv, st);
  else
    launch_dim<NW, 16>(p, fp8kv, st);
}

}  // namespace

bool gqa_mfma_fp8_supported(int D, int bs, int G, int ql) {
  const int cols = G * ql;
  return (D == 64 || D == 128) && (bs == 16 || bs == 32) && G >= 1 && cols >= 2 && cols <= 16;
}

bool gqa_mfma_supported(bool bf16, int D, int Dv, int bs, int G, int ql) {
  const int cols = G * ql;
  return bf16 && (D == 64 || D == 128) && Dv == D && (bs == 16 || bs == 32) && G >= 1 &&
         cols >= 2 && cols <= 16;
}

hipError_t launch_gqa_mfma(const Params& p, bool fp8kv, hipStream_t st) {
  if (p.wg_waves == 8)
    launch_waves<8>(p, fp8kv, st);
  else if (p.wg_waves == 4)
    launch_waves<4>(p, fp8kv, st);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
