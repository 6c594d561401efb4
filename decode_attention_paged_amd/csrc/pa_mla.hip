// Split-KV partial kernel for MLA latent decode on the matrix cores.
//
// All query heads attend to one latent row per token (keys: the whole
// 576-wide row; values: its first 512 entries, the same memory).  A
// workgroup of NW waves (one per SIMD) handles NH = 16*HB*NW heads of one
// (sequence, split) and walks the split in chunks of 32 tokens (half a
// 64-token page):
//
//   scores  S^T[32 tok x 16*HB heads] = C[32 x 576] Q_w^T   wave w: its 16*HB heads
//   values  O_w^T[DW dims x NH heads] += V^T[DW x 32] P^T     wave w: dims DW*w..DW*w+DW-1
//
// on v_mfma_f32_16x16x32_bf16.  Scores are split by heads (each wave keeps its
// heads' queries in registers) and the value product by output dims (each
// wave keeps DW = 512/NW dims of every head, the accumulators live in AGPRs),
// so the transposed value reads (ds_read_b64_tr_b16, the slowest LDS read)
// touch each latent element once per workgroup and each score A operand feeds
// HB MFMAs.  The probabilities P move between the two phases through LDS as
// [head][token] rows, read back as 16-byte B operands.  This is
// Flash-Decoding's per-chunk attention with a running max and sum (page 4,
// the second of its three steps); the split's (o_s, lse_s) go to the
// workspace for the reduction.
//
// The reference max of each head is fixed for a pass over the split: the
// first chunk's max.  Every later chunk's weights 2^(s - m) stay below
// 2^kHeadroom unless its max exceeds m by more than kHeadroom (log2 units);
// then the workgroup starts the split over with m raised to the largest max
// seen so far.  Sum and accumulators use the same m, so the result is the exact
// softmax of the online-softmax recurrence with its rescaling steps left out,
// and the hot loop never touches the accumulators outside the MFMAs.  Every
// restart is triggered by a later chunk than the one before, so a split is
// passed over at most once per chunk; scores that climb by 2^kHeadroom chunk
// after chunk are the only inputs that pay for it.
//
// Chunks stream HBM -> LDS with direct-to-LDS loads (global_load_lds_dwordx4,
// no registers), AHEAD chunks in flight while one is consumed.  Barriers are
// raw s_barrier with explicit waits: __syncthreads() would also wait for every
// chunk in flight.  Each ring slot is its own LDS array and the chunk loop is
// unrolled over the ring, so the compiler can tell the slots apart.
//
// LDS chunk rows are 1152 bytes (72 chunks of 16 bytes); chunk c of token row
// t sits at position c ^ (t & 7), which spreads both the score reads (16 rows,
// same chunk) and the transposed value reads over the banks.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kBS = 64;                    // tokens per page
constexpr int kRowB = kDqk * 2;            // 1152 bytes per latent row
constexpr int kCT = 32;                    // tokens per chunk
constexpr int kChunkB = kCT * kRowB;       // 36864 bytes per chunk
constexpr int kDmaInst = kChunkB / 1024;   // 36 wave-wide 1 KiB loads per chunk
constexpr int kKSteps = kDqk / 32;         // 18 score k-steps

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) float lds_float;

// 16 zero bytes in global memory: the load source for token slots past the
// context, so no NaN or stale data reaches the value product.
__device__ __attribute__((aligned(16))) uint32_t g_zero16[4] = {0u, 0u, 0u, 0u};

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Score products in the VGPR form of the MFMA, written as asm because the
// compiler gives all MFMAs of a kernel one form and the value accumulators of
// this kernel fill the AGPRs.  The compiler's hazard pass does not see into
// asm, so each statement carries its own padding (CDNA3/CDNA4 ISA dependency
// tables): two wait states in front cover a VALU write of an operand;
// accumulating into the same registers back to back needs none; reading the
// result with any other instruction needs 16, supplied by mfma_v_drain.
__device__ __forceinline__ void mfma_v_first(f32x4& d, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x4& d, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
template <int HB>
__device__ __forceinline__ void mfma_v_drain(f32x4 (&d)[HB][2]) {
  if constexpr (HB == 1)
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(d[0][0]), "+v"(d[0][1]));
  else
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(d[0][0]), "+v"(d[0][1]), "+v"(d[1][0]), "+v"(d[1][1]));
}

// Direct-to-LDS load of 16 bytes per lane (lane L writes wave_base + 16 L),
// non-temporal.  Written as asm so the compiler's wait-count pass does not see
// an LDS write through the vector memory path: it cannot tell the ring slots
// apart and would make every later LDS access wait for all loads in flight,
// draining the ring each chunk.  Completion is awaited explicitly (wait_vm
// before the barrier that opens each chunk).  M0 takes the LDS base; an SALU
// write of M0 needs one wait state before the load that uses it.
__device__ __forceinline__ void dma16(const void* g, lds_char* wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "s"((uint32_t)(uintptr_t)wave_base)
               : "memory", "m0");
}

// LDS stores that the compiler's wait-count pass cannot see as LDS accesses.
// It makes every LDS store wait for all direct-to-LDS loads in flight (it
// cannot tell the ring buffers from the rest of LDS), which would drain the
// load ring each chunk; these stores never touch the ring.  Their completion
// is awaited by the lgkmcnt(0) of the next lds_barrier.
__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) {
  return (uint32_t)(uintptr_t)p;
}
__device__ __forceinline__ void ds_store_b64(lds_char* p, u32x2 v) {
  asm volatile("ds_write_b64 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void ds_store_b32(lds_char* p, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

__device__ __forceinline__ u32x2 lds_tr16(const lds_char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)p));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
constexpr int vm_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }
constexpr int kLgkm0 = 0xC07F;   // lgkmcnt(0), others unlimited

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(vm_imm(N));
}

// Wait until at most n vector-memory ops of this wave are outstanding.  n is
// wave-uniform and every value a launch can produce has a case; anything else
// waits for all.
__device__ __forceinline__ void wait_vm_dyn(int n) {
  switch (n) {
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 8: wait_vm<8>(); break;
    case 9: wait_vm<9>(); break;
    case 10: wait_vm<10>(); break;
    case 18: wait_vm<18>(); break;
    case 27: wait_vm<27>(); break;
    case 36: wait_vm<36>(); break;
    default: wait_vm<0>(); break;
  }
}

// Barrier that makes this wave's LDS writes visible but leaves its
// direct-to-LDS loads in flight.  The signal fences keep the compiler from
// moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Byte offset of 16-byte chunk c of token row t inside a chunk buffer.
__device__ __forceinline__ int swz(int t, int c) { return t * kRowB + ((c ^ (t & 7)) << 4); }

constexpr float kHeadroom = 16.0f;   // log2 units a chunk's max may exceed the reference max

template <int NW, int HB>
struct MlaCfg {
  static constexpr int NH = 16 * HB * NW;            // heads per workgroup
  static constexpr int NB = NH / 16;                 // head blocks (value N-blocks)
  static constexpr int DW = kDv / NW;                // value dims per wave
  static constexpr int MB = DW / 16;                 // value M-blocks per wave
  static constexpr int NWI = kDmaInst / NW;          // direct-to-LDS loads per wave per chunk, at least
  static constexpr int AHEAD = NW >= 4 ? 2 : 1;      // chunks in flight beyond the current one
  static constexpr int RING = AHEAD + 2;             // 4, or 3
  static_assert(AHEAD * NWI <= 63, "vmcnt range");
};

template <int NW, int HB>
struct MlaLds {
  uint16_t p[MlaCfg<NW, HB>::NH * kCT];   // probabilities, [head][token] bf16
  int restart[2];                         // per chunk parity: a head's max overflowed the headroom
  float stat_m[MlaCfg<NW, HB>::NH];
  float stat_l[MlaCfg<NW, HB>::NH];
};

// Physical page ids of the split, one per lane for a window of 64 logical
// pages, so the chunk loop reads them with v_readlane instead of a memory load
// (a vector load there would have to wait for every chunk in flight).
struct PageIds {
  int v;      // lane L: id of logical page base + L
  int base;   // first logical page of the window (wave-uniform)
};

__device__ __forceinline__ void load_ids(PageIds& ids, const int* bt, int base, int p1, int nblocks,
                                         int lane) {
  const int pg = base + lane;
  ids.v = pg < p1 ? clampi(bt[pg], 0, nblocks - 1) : 0;
  ids.base = base;
}

// Page id of chunk ci; reloads the id window when the chunk leaves it (every
// 128 chunks at most; that reload waits for the loads in flight).
__device__ __forceinline__ int chunk_page_id(PageIds& ids, const int* bt, int t0, int ci, int p1,
                                             int nblocks, int lane) {
  const int pg = (t0 + ci * kCT) / kBS;
  if (pg >= ids.base + 64) load_ids(ids, bt, pg, p1, nblocks, lane);
  return __builtin_amdgcn_readlane(ids.v, pg - ids.base);
}

// Issue this wave's share (NWI 1 KiB loads) of chunk `ci` into `dst`.
template <int NW>
__device__ __forceinline__ void issue_chunk(lds_char* dst, const char* cbase, int id, int t0,
                                            int ci, int ctx, int w, int lane) {
  const int tok0 = t0 + ci * kCT;
  const char* src = cbase + (size_t)id * (kBS * kRowB) + (tok0 % kBS) * kRowB;
  const int lim = (ctx - tok0) * kRowB;              // bytes of the chunk that hold context tokens
#pragma unroll
  for (int k = 0; k < (kDmaInst + NW - 1) / NW; ++k) {
    const int j = w + NW * k;
    if (kDmaInst % NW != 0 && j >= kDmaInst) break;
    const int slot = j * 64 + lane;                  // 16-byte slot of the chunk buffer
    const int t = slot / (kRowB / 16);
    const int c = (slot % (kRowB / 16)) ^ (t & 7);
    const int off = t * kRowB + c * 16;
    const void* g = off < lim ? (const void*)(src + off) : (const void*)g_zero16;
    dma16(g, dst + j * 1024);
  }
}

// The ring slots, addressed by compile-time slot index.
struct Ring {
  lds_char* s0;
  lds_char* s1;
  lds_char* s2;
  lds_char* s3;
  template <int K>
  __device__ __forceinline__ lds_char* at() const {
    if constexpr (K == 0) return s0;
    else if constexpr (K == 1) return s1;
    else if constexpr (K == 2) return s2;
    else return s3;
  }
};

template <int NW, int HB>
struct MlaState {
  u32x4 qf[HB][kKSteps];                              // Q^T B operands
  f32x4 acc[MlaCfg<NW, HB>::MB][MlaCfg<NW, HB>::NB];  // O^T, dims x heads
  float m[HB];                                        // reference max per score head (log2)
  float mtop[HB];                                     // largest chunk max seen (log2)
  float l[HB];                                        // this lane's share of the sum
};

// One chunk of the split.  Returns true (uniformly over the workgroup) when a
// head's max overflowed the headroom: the chunk's value product is skipped and
// the caller starts the split over.
template <int NW, int HB, int SLOT>
__device__ __forceinline__ bool mla_chunk(const Params& p, MlaLds<NW, HB>& sm, const Ring& ring,
                                          MlaState<NW, HB>& st, int ci, int nchunks, int t0,
                                          int ctx, const char* cbase, const int* bt, PageIds& ids,
                                          int p1, int w, int lane) {
  using C = MlaCfg<NW, HB>;
  const int quad = lane >> 4, n = lane & 15;
  // wait for this wave's loads of chunk ci, then (barrier) for every wave's;
  // the barrier also means every wave is done with the slot refilled below
  const int ahead = min(C::AHEAD, nchunks - 1 - ci);
  wait_vm_dyn(ahead * C::NWI);
  lds_barrier();
  if (ci + C::AHEAD + 1 < nchunks) {
    const int cn = ci + C::AHEAD + 1;
    const int id = chunk_page_id(ids, bt, t0, cn, p1, p.nblocks, lane);
    issue_chunk<NW>(ring.template at<(SLOT + C::AHEAD + 1) % C::RING>(), cbase, id, t0, cn, ctx,
                    w, lane);
  }
  const lds_char* buf = ring.template at<SLOT>();

  // ---- scores.  Row n (and 16 + n), 16-byte chunk kb*4 + quad: with the
  // swizzle its byte offset is n*kRowB + 16*(quad ^ (n & 3)) + 64*(kb ^ ((n>>2)&1)),
  // i.e. one per-lane base for even and one for odd k-steps plus 64*kb.
  const int xb = (n >> 2) & 1;
  const int sbase = n * kRowB + 16 * (quad ^ (n & 3));
  const lds_char* se = buf + sbase + 64 * xb;
  const lds_char* so = buf + sbase - 64 * xb;
  f32x4 sa[HB][2];
  // A operands one k-step ahead of the MFMAs that use them
  u32x4 an0 = *(const lds_u32x4*)se;
  u32x4 an1 = *(const lds_u32x4*)(se + 16 * kRowB);          // row 16 + n: same swizzle
#pragma unroll
  for (int kb = 0; kb < kKSteps; ++kb) {
    const u32x4 a0 = an0, a1 = an1;
    if (kb + 1 < kKSteps) {
      const lds_char* rp = (((kb + 1) & 1) ? so : se) + 64 * (kb + 1);
      an0 = *(const lds_u32x4*)rp;
      an1 = *(const lds_u32x4*)(rp + 16 * kRowB);
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      if (kb == 0) {
        mfma_v_first(sa[hb][0], a0, st.qf[hb][kb]);
        mfma_v_first(sa[hb][1], a1, st.qf[hb][kb]);
      } else {
        mfma_v(sa[hb][0], a0, st.qf[hb][kb]);
        mfma_v(sa[hb][1], a1, st.qf[hb][kb]);
      }
    }
  }
  mfma_v_drain<HB>(sa);
  const int tbase = t0 + ci * kCT;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    float sc[8];
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = (tbase + quad * 4 + r < ctx) ? sa[hb][0][r] * p.scale_log2 : kNegInf;
      sc[4 + r] = (tbase + 16 + quad * 4 + r < ctx) ? sa[hb][1][r] * p.scale_log2 : kNegInf;
      mx = fmaxf(mx, fmaxf(sc[r], sc[4 + r]));
    }
    mx = max_xor32(max_xor16(mx));                  // same in the 4 quads of a head
    st.mtop[hb] = fmaxf(st.mtop[hb], mx);
    if (st.m[hb] == kNegInf) st.m[hb] = mx;          // first chunk of the pass
    if (mx > st.m[hb] + kHeadroom) ds_store_b32((lds_char*)&sm.restart[ci & 1], 1u);
    const float mn = st.m[hb];
    float pr[8];
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pr[j] = fast_exp2(sc[j] - mn);
      ls += pr[j];
    }
    st.l[hb] += ls;
    const int head = 16 * (HB * w + hb) + n;
    lds_char* prow = (lds_char*)sm.p + head * (kCT * 2);
    u32x2 v0, v1;
    v0[0] = pack_bf16(pr[0], pr[1]);
    v0[1] = pack_bf16(pr[2], pr[3]);
    v1[0] = pack_bf16(pr[4], pr[5]);
    v1[1] = pack_bf16(pr[6], pr[7]);
    ds_store_b64(prow + quad * 8, v0);               // tokens quad*4 .. +3
    ds_store_b64(prow + 32 + quad * 8, v1);          // tokens 16 + quad*4 .. +3
  }
  lds_barrier();
  // every wave has read the other parity's flag (last chunk's) before the
  // barrier above, and it is next written after the next chunk's first barrier
  if (w == 0 && lane == 0) ds_store_b32((lds_char*)&sm.restart[(ci + 1) & 1], 0u);
  if (__builtin_amdgcn_readfirstlane(sm.restart[ci & 1]) != 0) return true;

  // ---- values for dims DW*w .. DW*w + DW - 1 of every head
  // A operand (V^T): tokens quad*8 .. +7 of dim DW*w + mb*16 + n, two transposed reads
  auto load_va = [&](int mb) {
    const int bc = (C::DW * w + mb * 16) * 2 + (n & 3) * 8;    // byte column this lane reads
    const int r0 = quad * 8 + (n >> 2), r1 = r0 + 4;
    const lds_char* lo = buf + r0 * kRowB + (((bc >> 4) ^ (r0 & 7)) << 4) + (bc & 15);
    const lds_char* hi = buf + r1 * kRowB + (((bc >> 4) ^ (r1 & 7)) << 4) + (bc & 15);
    const u32x2 vlo = lds_tr16(lo), vhi = lds_tr16(hi);
    return u32x4{vlo[0], vlo[1], vhi[0], vhi[1]};
  };
  // B operand (P^T): tokens quad*8 .. +7 of head nb*16 + n
  auto load_pb = [&](int nb) {
    return *(const lds_u32x4*)((const lds_char*)sm.p + (nb * 16 + n) * (kCT * 2) + quad * 16);
  };
  if constexpr (C::MB < C::NB) {
    u32x4 va[C::MB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) va[mb] = load_va(mb);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      const u32x4 pb = load_pb(nb);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) st.acc[mb][nb] = mfma(va[mb], pb, st.acc[mb][nb]);
    }
  } else {
    u32x4 pb[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) pb[nb] = load_pb(nb);
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const u32x4 va = load_va(mb);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) st.acc[mb][nb] = mfma(va, pb[nb], st.acc[mb][nb]);
    }
  }
  return false;
}

template <int NW, int HB>
__global__ __launch_bounds__(NW * 64) void mla_mfma_partial(Params p) {
  using C = MlaCfg<NW, HB>;
  __shared__ __attribute__((aligned(16))) char ring0[kChunkB];
  __shared__ __attribute__((aligned(16))) char ring1[kChunkB];
  __shared__ __attribute__((aligned(16))) char ring2[kChunkB];
  __shared__ __attribute__((aligned(16))) char ring3[C::RING > 3 ? kChunkB : 16];
  __shared__ __attribute__((aligned(16))) MlaLds<NW, HB> sm;
  const Ring ring{(lds_char*)ring0, (lds_char*)ring1, (lds_char*)ring2, (lds_char*)ring3};

  const int hg = blockIdx.x, b = blockIdx.z;
  const int s = split_of_block(blockIdx.y, b, p.S);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quad = lane >> 4, n = lane & 15;
  const int head0 = hg * C::NH;
  const int ctx = clampi(p.context_lens[b], 0, p.max_ctx);
  const int pages = (ctx + kBS - 1) / kBS;
  const int nsplit = splits_of(pages, p.c);
  if (s >= (nsplit > 0 ? nsplit : 1)) return;
  const int t0 = s * p.c * kBS;
  const int t1 = min(ctx, (s * p.c + p.c) * kBS);
  const int p1 = min(pages, s * p.c + p.c);
  const int nchunks = t1 > t0 ? (t1 - t0 + kCT - 1) / kCT : 0;

  MlaState<NW, HB> st;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    // Q^T B operands: head head0 + 16*(HB*w + hb) + n, dims kb*32 + quad*8 .. +8
    const char* qr = static_cast<const char*>(p.q) +
                     ((size_t)b * p.Hq + head0 + 16 * (HB * w + hb) + n) * kRowB;
#pragma unroll
    for (int kb = 0; kb < kKSteps; ++kb) st.qf[hb][kb] = ld128(qr + kb * 64 + quad * 16);
    st.m[hb] = kNegInf;
    st.mtop[hb] = kNegInf;
  }
  if (w == 0 && lane == 0) sm.restart[0] = sm.restart[1] = 0;

  const int* bt = p.block_table + (size_t)b * p.maxb;
  const char* cbase = static_cast<const char*>(p.k);
  PageIds ids;
  for (;;) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) st.l[hb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) st.acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    load_ids(ids, bt, s * p.c, p1, p.nblocks, lane);
    // The first AHEAD + 1 chunks are issued even past the split's end (those
    // loads read the zero block), so the count in flight is known here and
    // one wait retires the query loads, which are older: no wait inside the
    // loop has to allow for them.
    issue_chunk<NW>(ring.at<0>(), cbase, chunk_page_id(ids, bt, t0, 0, p1, p.nblocks, lane), t0, 0,
                    ctx, w, lane);
    issue_chunk<NW>(ring.at<1>(), cbase, chunk_page_id(ids, bt, t0, 1, p1, p.nblocks, lane), t0, 1,
                    ctx, w, lane);
    if constexpr (C::AHEAD >= 2)
      issue_chunk<NW>(ring.at<2>(), cbase, chunk_page_id(ids, bt, t0, 2, p1, p.nblocks, lane), t0,
                      2, ctx, w, lane);
    constexpr int kInit = (C::AHEAD + 1) * C::NWI;
    wait_vm<kInit <= 63 ? kInit : 0>();

    bool again = false;
    for (int c0 = 0; c0 < nchunks; c0 += C::RING) {
      again = mla_chunk<NW, HB, 0>(p, sm, ring, st, c0, nchunks, t0, ctx, cbase, bt, ids, p1, w,
                                   lane);
      if (again) break;
      if (c0 + 1 < nchunks) {
        again = mla_chunk<NW, HB, 1>(p, sm, ring, st, c0 + 1, nchunks, t0, ctx, cbase, bt, ids, p1,
                                     w, lane);
        if (again) break;
      }
      if (c0 + 2 < nchunks) {
        again = mla_chunk<NW, HB, 2>(p, sm, ring, st, c0 + 2, nchunks, t0, ctx, cbase, bt, ids, p1,
                                     w, lane);
        if (again) break;
      }
      if constexpr (C::RING > 3) {
        if (c0 + 3 < nchunks) {
          again = mla_chunk<NW, HB, 3>(p, sm, ring, st, c0 + 3, nchunks, t0, ctx, cbase, bt, ids,
                                       p1, w, lane);
          if (again) break;
        }
      }
    }
    if (!again) break;
    // Start over with the raised reference max: drain this wave's loads, wait
    // for every wave (all have read the flag and finished their loads), then
    // clear the flags before the next pass's first barrier.
    wait_vm<0>();
    lds_barrier();
    if (w == 0 && lane == 0) sm.restart[0] = sm.restart[1] = 0;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) st.m[hb] = st.mtop[hb];
  }
  wait_vm<0>();   // loads issued past the end of a short split

  // ---- finish: per-head statistics to every wave, normalise, write
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const float lt = sum_xor32(sum_xor16(st.l[hb]));
    if (quad == 0) {
      const int head = 16 * (HB * w + hb) + n;
      *((lds_float*)sm.stat_m + head) = st.m[hb];
      *((lds_float*)sm.stat_l + head) = lt;
    }
  }
  lds_barrier();
  const size_t row0 = (size_t)b * p.Hq + head0;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    const float mm = *((const lds_float*)sm.stat_m + nb * 16 + n);
    const float lt = *((const lds_float*)sm.stat_l + nb * 16 + n);
    const float inv = (mm == kNegInf) ? 0.f : 1.f / lt;
    const size_t row = row0 + nb * 16 + n;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const int d = C::DW * w + mb * 16 + quad * 4;
      if (p.final_write) {
        u32x2 pk;
        pk[0] = pack_bf16(st.acc[mb][nb][0] * inv, st.acc[mb][nb][1] * inv);
        pk[1] = pack_bf16(st.acc[mb][nb][2] * inv, st.acc[mb][nb][3] * inv);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + row * kDv + d) = pk;
      } else {
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = st.acc[mb][nb][r] * inv;
        *reinterpret_cast<f32x4*>(p.o_part + (row * p.S + s) * kDv + d) = v;
      }
    }
  }
  if (quad == 0) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = 16 * (HB * w + hb) + n;
      const float mm = *((const lds_float*)sm.stat_m + head);
      const float lt = *((const lds_float*)sm.stat_l + head);
      const float lse = (mm == kNegInf) ? kNegInf : (mm + fast_log2(lt)) * kLn2;
      const size_t row = row0 + head;
      if (p.final_write) {
        if (p.lse) p.lse[row] = lse;
      } else {
        p.lse_part[row * p.S + s] = lse;
      }
    }
  }
}

template <int NW, int HB>
hipError_t launch_cfg(const Params& p, hipStream_t st) {
  dim3 grid(p.Hq / MlaCfg<NW, HB>::NH, p.S, p.B);
  hipLaunchKernelGGL((mla_mfma_partial<NW, HB>), grid, dim3(NW * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace

bool mla_mfma_supported(bool bf16, int Dqk, int Dv, int bs, int Hq) {
  return bf16 && Dqk == kDqk && Dv == kDv && bs == kBS &&
         (Hq % 128 == 0 || Hq == 64 || Hq == 32 || Hq == 16);
}

hipError_t launch_mla_mfma(const Params& p, hipStream_t st) {
  if (p.Hq % 128 == 0) return launch_cfg<4, 2>(p, st);
  if (p.Hq == 64) return launch_cfg<4, 1>(p, st);
  if (p.Hq == 32) return launch_cfg<2, 1>(p, st);
  if (p.Hq == 16) return launch_cfg<1, 1>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
