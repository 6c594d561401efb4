// Split-KV partial kernels for MLA latent decode on the matrix cores.
//
// All query heads attend to one latent row per token (keys: the whole
// 576-wide row; values: its first 512 entries, the same memory).  A workgroup
// handles the heads of one head group for one (sequence, split) and walks
// the split in chunks of 32 tokens (half a 64-token page):
//
//   scores  S^T[32 tok x 16 heads] = C[32 x 576] Q^T        per 16-head block
//   values  O^T[512 dims x heads] += V^T[512 x 32] P^T      split by dims over waves
//
// on v_mfma_f32_16x16x32_bf16.  Queries stay in registers as score B
// operands; the value product is split by output dims, so the transposed
// value reads (ds_read_b64_tr_b16, the slowest LDS read) touch each latent
// element once per workgroup.  The probabilities P move from the score to the
// value product through LDS.  This is Flash-Decoding's attention of the query
// with one block of keys and values plus the block's log-sum-exp (the
// "flash decoding ++" entry, its three-steps snippet, second step); the
// split's (o_s, lse_s) go to the workspace for the reduction.
//
// Two workgroup shapes, both with two waves per SIMD (at most 256 registers
// a wave):
//   * wide (128 heads, 64-token pages): 8 alike waves.  Wave w scores head
//     block w and accumulates dims 64w .. 64w+63 of all 128 heads; each CU
//     streams every latent row of its split once.
//   * role-split (16, 32 or 64 heads; also one-token pages, whose token ids
//     take 8 KiB of LDS): score waves hold the queries, value waves hold the
//     accumulators and issue the chunk loads.  With 128 heads the grid has
//     two such workgroups per (sequence, split), 8 apart in dispatch order:
//     the same XCD (workgroups go round-robin to the 8 XCDs), so the second
//     reads the rows from that XCD's L2.
//
// The reference max of each head is fixed for a pass over the split: the
// first chunk's max.  Every later chunk's weights 2^(s - m) stay below
// 2^kHeadroom unless its max exceeds m by more than kHeadroom (log2 units);
// then, at the end of the pass, the workgroup starts the split over with m
// raised to the largest chunk max of the pass, which no chunk can exceed.  Sum
// and accumulators use the same m, so the result is the exact softmax of the
// online-softmax recurrence with its rescaling steps left out, the hot loop
// never touches the accumulators outside the MFMAs, and a split is passed
// over at most twice; only scores that climb by 2^kHeadroom within a split
// pay for the second pass.
//
// Chunks stream HBM -> LDS with direct-to-LDS loads (global_load_lds_dwordx4,
// no registers), two chunks in flight while one is scored and the one before
// goes through the value product.  Barriers are raw s_barrier with explicit
// waits: __syncthreads() would also wait for every chunk in flight.
//
// LDS chunk rows are 1152 bytes (72 chunks of 16 bytes).  Chunk c of token
// row t sits at position c ^ (t & 7); with it the score reads (16 rows, one
// chunk each) and the transposed value reads run at the conflict-free rate
// (measured against a linear read of the same size).  The probabilities are
// stored so that the value product's B-operand read is linear: for head block
// nb, the 16-byte slot q*16 + n holds tokens 8q .. 8q+7 of head 16 nb + n.

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowB = kDqk * 2;            // 1152 bytes per latent row
constexpr int kCT = 32;                    // tokens per chunk
constexpr int kChunkB = kCT * kRowB;       // 36864 bytes per chunk
constexpr int kDmaInst = kChunkB / 1024;   // 36 wave-wide 1 KiB loads per chunk
constexpr int kKSteps = kDqk / 32;         // 18 score k-steps

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// 16 zero bytes in global memory: the load source for token slots past the
// context, so no NaN or stale data reaches the value product.
__device__ __attribute__((aligned(16))) uint32_t g_zero16[4] = {0u, 0u, 0u, 0u};


// MFMAs with VGPR accumulators, written as asm so that the accumulators stay
// in VGPRs whatever the compiler would choose (two waves per SIMD leave no
// room for a second register file's worth).  The compiler's hazard pass does
// not see into asm, so each statement carries its own padding (CDNA3/CDNA4
// ISA dependency tables): two wait states in front cover a VALU write of an
// operand; accumulating into the same registers back to back needs none;
// reading the result with any other instruction needs 16, supplied by
// drain_scores or an explicit run of s_nop.
__device__ __forceinline__ void mfma_v_first(f32x4& d, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x4& d, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// Drain before VALU reads score accumulators.
template <int N>
__device__ __forceinline__ void drain_scores(f32x4 (&sa)[N]) {
  if constexpr (N == 1)
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(sa[0]));
  else
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(sa[0]), "+v"(sa[1]));
}

// Direct-to-LDS load of 16 bytes per lane (lane L writes wave_base + 16 L),
// non-temporal.  Written as asm so the compiler's wait-count pass does not see
// an LDS write through the vector memory path: it cannot tell the ring slots
// apart and would make every later LDS access wait for all loads in flight,
// draining the ring each chunk.  Completion is awaited explicitly (wait_vm
// before the barrier that opens each chunk).  The compiler sets M0 (the LDS
// base) for the asm; an SALU write of M0 needs one wait state before the load
// that uses it.
__device__ __forceinline__ void dma16(const void* g, lds_char* wave_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "{m0}"((uint32_t)(uintptr_t)wave_base)
               : "memory");
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
__device__ __forceinline__ int row_key(int t) { return t & 7; }

constexpr float kHeadroom = 16.0f;   // log2 units a chunk's max may exceed the reference max
constexpr int kRing = 4;             // chunk slots: value product, scores, two loads in flight
constexpr int kMaxIdsBS1 = 2048;     // token ids of one split held in LDS (one-token pages)

// Where the rows of chunk ci come from, for 64-token pages (one page id per
// chunk) and for one-token pages (a per-sequence token-index list: every row
// has its own id).  Rows at or past the split's end t1 are read from the
// zero block, so no NaN or stale data reaches the value product and no token
// is counted by two splits.
template <int NW, int BS>
struct ChunkSource;

template <int NW>
struct ChunkSource<NW, 64> {
  // Physical page ids of the split, one per lane for a window of 64 logical
  // pages, read in the chunk loop with v_readlane (a vector load there would
  // have to wait for every chunk in flight).
  const int* bt;
  const char* cbase;
  int t0, t1, p1, nblocks, w, lane;
  int v;      // lane L: id of logical page base + L
  int base;   // first logical page of the window (wave-uniform)

  __device__ __forceinline__ void load_window(int first) {
    const int pg = first + lane;
    v = pg < p1 ? clampi(bt[pg], 0, nblocks - 1) : 0;
    base = first;
  }
  __device__ __forceinline__ void begin(int first_page) { load_window(first_page); }
  // Page id of chunk ci (chunks are visited in order); reloads the id window
  // when the chunk leaves it (every 128 chunks at most; that reload waits for
  // the loads in flight).
  __device__ __forceinline__ int page_of(int ci) {
    const int pg = (t0 + ci * kCT) / 64;
    if (pg >= base + 64) load_window(pg);
    return __builtin_amdgcn_readlane(v, pg - base);
  }
  // This wave's share of a chunk: load j of the chunk's kDmaInst loads of
  // 1 KiB goes to wave j % NW, as its load k = j / NW.
  static constexpr int kPer = (kDmaInst + NW - 1) / NW;
  struct Prep {
    const char* src;   // the chunk's first row
    int lim;           // bytes of the chunk inside the split
  };
  __device__ __forceinline__ Prep prepare(int ci) {
    const int tok0 = t0 + ci * kCT;
    return Prep{cbase + (size_t)page_of(ci) * (64 * kRowB) + (tok0 % 64) * kRowB,
                (t1 - tok0) * kRowB};
  }
  __device__ __forceinline__ void issue_k(const Prep& pr, lds_char* dst, int k) {
    const int j = w + NW * k;
    if (kDmaInst % NW != 0 && j >= kDmaInst) return;
    int ln = lane;
    // recompute the per-lane offsets at every issue rather than keep them in
    // registers across the loop (a few VALU ops against ~18 VGPRs)
    asm volatile("" : "+v"(ln));
    const int slot = j * 64 + ln;                    // 16-byte slot of the chunk buffer
    const int t = slot / (kRowB / 16);
    const int c = (slot % (kRowB / 16)) ^ row_key(t);
    const int off = t * kRowB + c * 16;
    const void* g = off < pr.lim ? (const void*)(pr.src + off) : (const void*)g_zero16;
    dma16(g, dst + j * 1024);
  }
  // Issue this wave's whole share of chunk ci into dst.
  __device__ __forceinline__ void issue(lds_char* dst, int ci) {
    const Prep pr = prepare(ci);
#pragma unroll
    for (int k = 0; k < kPer; ++k) issue_k(pr, dst, k);
  }
};

template <int NW>
struct ChunkSource<NW, 1> {
  static_assert(kDmaInst % NW == 0, "uniform load share");
  // The split's token ids (at most kMaxIdsBS1, checked by the host) are
  // copied into LDS once per pass; each 1 KiB load of a chunk spans at most
  // two token rows (64 slots of 16 bytes, rows of 72), whose ids are read
  // from LDS by every lane.
  const int* bt;
  const char* cbase;
  int t0, t1, p1, nblocks, w, lane;
  int* ids;   // LDS, kMaxIdsBS1 entries: id of token t0 + i

  __device__ __forceinline__ void begin(int /*first_page*/) {
    // no loads are in flight here (start of a pass), so the full barrier is free
    const int n = t1 - t0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) ids[i] = clampi(bt[t0 + i], 0, nblocks - 1);
    __syncthreads();
  }
  __device__ __forceinline__ void issue(lds_char* dst, int ci) {
    const int tok0 = t0 + ci * kCT;
    const int nrows = t1 - tok0;                     // rows of the chunk inside the split
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // ids of the two rows each load touches, all read before the first load
    int id0[kDmaInst / NW], id1[kDmaInst / NW];
#pragma unroll
    for (int k = 0; k < kDmaInst / NW; ++k) {
      const int T = ((w + NW * k) * 64) / (kRowB / 16);   // first row load k touches
      const int i0 = tok0 - t0 + T;                  // rows past the split never use their id
      id0[k] = ids[min(i0, kMaxIdsBS1 - 1)];
      id1[k] = ids[min(i0 + 1, kMaxIdsBS1 - 1)];
    }
#pragma unroll
    for (int k = 0; k < kDmaInst / NW; ++k) {
      const int j = w + NW * k;
      const int T = (j * 64) / (kRowB / 16);
      const int slot = j * 64 + ln;
      const int t = slot / (kRowB / 16);
      const int c = (slot % (kRowB / 16)) ^ row_key(t);
      const int id = t == T ? id0[k] : id1[k];
      const void* g = t < nrows ? (const void*)(cbase + (size_t)id * kRowB + c * 16)
                                : (const void*)g_zero16;
      dma16(g, dst + j * 1024);
    }
  }
};

// Operands of the value product for dims DW*w .. DW*w + DW - 1 of every
// head.  A operand (V^T): tokens quad*8 .. +7 of one dim per lane, two
// transposed reads; B operand (P^T): one 16-byte slot.
template <int DW>
struct ValueOps {
  const lds_char* buf;
  const lds_char* pbuf;
  int w, n, quad;
  __device__ __forceinline__ u32x4 va(int mb) const {
    const int bc = (DW * w + mb * 16) * 2 + (n & 3) * 8;   // byte column
    const int r0 = quad * 8 + (n >> 2), r1 = r0 + 4;
    const lds_char* lo = buf + r0 * kRowB + (((bc >> 4) ^ row_key(r0)) << 4) + (bc & 15);
    const lds_char* hi = buf + r1 * kRowB + (((bc >> 4) ^ row_key(r1)) << 4) + (bc & 15);
    const u32x2 vlo = lds_tr16(lo), vhi = lds_tr16(hi);
    return u32x4{vlo[0], vlo[1], vhi[0], vhi[1]};
  }
  __device__ __forceinline__ u32x4 pb(int nb) const {
    return *(const lds_u32x4*)(pbuf + nb * (16 * kCT * 2) + 16 * (quad * 16 + n));
  }
};

// Head group hg and (sequence, split) unit u of workgroup L, for HG head
// groups per unit and U units.  The HG workgroups of a unit are 8 apart in
// dispatch order: workgroups go round-robin to the 8 XCDs, so they run on the
// same XCD at about the same time and all but the first read the latent rows
// from its L2.  Head groups are groups of query heads, or of query rows when
// a sequence has several.
__device__ __forceinline__ void group_and_unit(int L, int HG, int U, int& hg, int& u) {
  const int full = (U / 8) * 8 * HG;                  // workgroups in whole groups of 8 units
  if (L < full) {
    const int g = L / (8 * HG), r = L - g * 8 * HG;
    hg = r >> 3;
    u = g * 8 + (r & 7);
  } else {
    const int r = L - full;
    hg = r % HG;
    u = (U / 8) * 8 + r / HG;
  }
}

// Causal end of the query row that head group head0 (of Hq * ql row-heads)
// belongs to: row j sees ctx - ql + 1 + j tokens.
__device__ __forceinline__ int row_end(int ctx, int head0, const Params& p) {
  return ctx - p.ql + 1 + head0 / p.Hq;
}

// ---------------------------------------------------------------------------
// Role-split workgroup: two waves per SIMD, one scoring and one accumulating.
//
// A workgroup of NS + 4 waves holds NH = 16*HBW*HH heads.  Score wave (th, hp)
// computes S^T for the 16 tokens th*16 .. th*16+15 of each chunk and the
// 16*HBW heads of head part hp (so every A operand read from LDS feeds HBW
// MFMAs), turns them into weights and writes those to LDS.  Value wave v
// accumulates O^T for dims 128v .. 128v+127 of every head one chunk behind
// and issues the chunk loads.  The two roles keep disjoint state (queries in
// the score waves, accumulators in the value waves), each role runs its own
// copy of the pass loop, so the register allocator places both in the same
// 256 registers; and a SIMD always has a second wave to issue from while one
// waits on LDS, a barrier or the load pipeline.
//
// The two token halves of a head share its reference max: after the first
// chunk's scores the score waves swap their half maxima through LDS and both
// take the larger.  Overflow checks and sums stay per half; the sums are
// added at the end.  Both loops run the same barrier sequence (one template,
// role_loop, instantiated per role).

template <int HH, int HBW>
struct RoleCfg {
  static constexpr int NH = 16 * HBW * HH;   // heads per workgroup
  static constexpr int NB = NH / 16;         // head blocks
  static constexpr int NS = 2 * HH;          // score waves: token half x head part
  static constexpr int NP = 4;               // value waves
  static constexpr int NW = NS + NP;
  static constexpr int DW = kDv / NP;        // value dims per value wave
  static constexpr int MB = DW / 16;         // value M-blocks per value wave
  static constexpr int NWI = kDmaInst / NP;  // direct-to-LDS loads per value wave per chunk
  static constexpr int LOOK = 4;             // score operand loads ahead of their MFMAs
  static_assert(HBW == 1 || HBW == 2, "head blocks per score wave");
};

// LDS shared by both roles.  Region offsets inside the ring, used only when
// no chunk is in flight (end of a pass).
constexpr int kVoteOff = 0;        // int votes[NS]
constexpr int kMtopOff = 64;       // float mtop[2][NH]: largest chunk max per token half
constexpr int kStatOff = 2048;     // float stat_m[NH], stat_l[2][NH]
static_assert(kMtopOff + 2 * 64 * 4 <= kStatOff && kStatOff + 3 * 64 * 4 <= kChunkB,
              "end-of-pass regions fit the ring's first slot for up to 64 heads");

template <int HH, int HBW>
struct RoleShared {
  lds_char* ring;
  lds_char* pl;                    // probabilities, two buffers of NH*kCT bf16
  int nchunks;
  __device__ __forceinline__ lds_char* slot(int ci) const { return ring + (ci % kRing) * kChunkB; }
  __device__ __forceinline__ lds_char* pbuf(int ci) const {
    return pl + (ci & 1) * (RoleCfg<HH, HBW>::NH * kCT * 2);
  }
};

template <int HH, int HBW, int BS>
struct ScoreRole {
  using C = RoleCfg<HH, HBW>;
  const RoleShared<HH, HBW>& sh;
  int th, hp, lane, t0, t1;
  float cs;
  u32x4 qf[HBW][kKSteps];   // Q^T B operands of this wave's heads
  float m[HBW];             // reference max (log2), shared by both token halves
  float mtop[HBW];          // largest chunk max of this half (log2)
  float l[HBW];             // this lane's share of the half's sum
  bool bad;                 // a chunk max of this half overflowed the headroom
  f32x4 sa[HBW];            // scores of the current chunk
  float mx[HBW];            // their max per head (log2)

  __device__ __forceinline__ int head(int hb) const { return 16 * (HBW * hp + hb) + (lane & 15); }

  __device__ __forceinline__ void load_q(const char* qrow0) {
    const int quad = lane >> 4;
#pragma unroll
    for (int hb = 0; hb < HBW; ++hb) {
      const char* qr = qrow0 + (size_t)head(hb) * kRowB;
#pragma unroll
      for (int kb = 0; kb < kKSteps; ++kb) qf[hb][kb] = ld128(qr + kb * 64 + quad * 16);
      m[hb] = kNegInf;
      mtop[hb] = kNegInf;
    }
  }

  // S^T of this wave's token half and heads, then the mask and the max.
  __device__ __forceinline__ void scores(int ci) {
    const lds_char* buf = sh.slot(ci);
    const int quad = lane >> 4, n = lane & 15;
    // Row th*16 + n, 16-byte chunk kb*4 + quad, stored at chunk (kb*4 + quad) ^ (n & 7):
    // byte offset 16*(quad ^ (n & 3)) + 64*(kb ^ ((n >> 2) & 1)).
    const int xb = (n >> 2) & 1;
    const int sbase = (th * 16 + n) * kRowB + 16 * (quad ^ (n & 3));
    const lds_char* se = buf + sbase + 64 * xb;
    const lds_char* so = buf + sbase - 64 * xb;
    auto load_a = [&](int kb) { return *(const lds_u32x4*)(((kb & 1) ? so : se) + 64 * kb); };
    constexpr int L = C::LOOK;
    u32x4 ab[L + 1];
#pragma unroll
    for (int kb = 0; kb < L; ++kb) ab[kb] = load_a(kb);
#pragma unroll
    for (int kb = 0; kb < kKSteps; ++kb) {
      if (kb + L < kKSteps) ab[(kb + L) % (L + 1)] = load_a(kb + L);
      const u32x4 a = ab[kb % (L + 1)];
#pragma unroll
      for (int hb = 0; hb < HBW; ++hb) {
        if (kb == 0) mfma_v_first(sa[hb], a, qf[hb][kb]);
        else mfma_v(sa[hb], a, qf[hb][kb]);
      }
    }
    drain_scores<HBW>(sa);
    const int tok = t0 + ci * kCT + th * 16 + quad * 4;   // this lane's first token
#pragma unroll
    for (int hb = 0; hb < HBW; ++hb) {
      if (tok + 4 > t1) {                                // only a split's last chunk runs past t1
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (tok + j >= t1) sa[hb][j] = kNegInf;
      }
      const float x = fmaxf(fmaxf(sa[hb][0], sa[hb][1]), fmaxf(sa[hb][2], sa[hb][3]));
      mx[hb] = max_xor32(max_xor16(x)) * cs;             // same in the 4 quads
    }
  }

  // Overflow bookkeeping, weights, their sum and the probabilities to LDS.
  __device__ __forceinline__ void weights(int ci) {
    const int quad = lane >> 4, n = lane & 15;
    lds_char* pb = sh.pbuf(ci);
#pragma unroll
    for (int hb = 0; hb < HBW; ++hb) {
      mtop[hb] = fmaxf(mtop[hb], mx[hb]);
      bad |= mx[hb] > m[hb] + kHeadroom;
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) e[j] = fast_exp2(fmaf(sa[hb][j], cs, -m[hb]));
      l[hb] += (e[0] + e[1]) + (e[2] + e[3]);
      u32x2 v;
      v[0] = pack_bf16(e[0], e[1]);
      v[1] = pack_bf16(e[2], e[3]);
      // tokens th*16 + quad*4 .. +3 of head block HBW*hp + hb: 16-byte slot
      // (2*th + quad/2)*16 + n, half quad & 1
      ds_store_b64(pb + (HBW * hp + hb) * (16 * kCT * 2) + ((2 * th + (quad >> 1)) * 16 + n) * 16 +
                       8 * (quad & 1),
                   v);
    }
  }

  __device__ __forceinline__ void pass_begin() {
#pragma unroll
    for (int hb = 0; hb < HBW; ++hb) l[hb] = 0.f;
    bad = false;
  }
  __device__ __forceinline__ void prologue() { wait_vm<0>(); }   // the queries
  // First chunk: scores, then this half's maxima to the partner through the
  // second probability buffer (unused until chunk 1).
  __device__ __forceinline__ void step0a() {
    if (sh.nchunks == 0) return;
    scores(0);
    float* xm = (float*)sh.pbuf(1);
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int hb = 0; hb < HBW; ++hb) xm[th * C::NH + head(hb)] = mx[hb];
    }
  }
  __device__ __forceinline__ void step0b() {
    if (sh.nchunks == 0) return;
    const float* xm = (const float*)sh.pbuf(1);
#pragma unroll
    for (int hb = 0; hb < HBW; ++hb) {
      const float other = xm[(1 - th) * C::NH + head(hb)];
      if (m[hb] == kNegInf) m[hb] = fmaxf(mx[hb], other);   // first pass
    }
    weights(0);
  }
  __device__ __forceinline__ void before_barrier(int) {}
  __device__ __forceinline__ void step(int ci) {
    if (ci < sh.nchunks) {
      scores(ci);
      weights(ci);
    }
  }
  __device__ __forceinline__ void pass_end() {}
  __device__ __forceinline__ void vote(int w) {
    int* votes = (int*)(sh.ring + kVoteOff);
    float* mt = (float*)(sh.ring + kMtopOff);
    const bool any = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (lane == 0) votes[w] = any;
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int hb = 0; hb < HBW; ++hb) mt[th * C::NH + head(hb)] = mtop[hb];
    }
  }
  // Start over with the reference max raised to the largest chunk max of
  // either half: no chunk can overflow then.
  __device__ __forceinline__ void after_vote(bool restart) {
    if (!restart) return;
    const float* mt = (const float*)(sh.ring + kMtopOff);
#pragma unroll
    for (int hb = 0; hb < HBW; ++hb) m[hb] = fmaxf(mt[head(hb)], mt[C::NH + head(hb)]);
  }
  __device__ __forceinline__ void finish_a() {
    float* stat_m = (float*)(sh.ring + kStatOff);
    float* stat_l = stat_m + C::NH;
#pragma unroll
    for (int hb = 0; hb < HBW; ++hb) {
      const float lt = sum_xor32(sum_xor16(l[hb]));
      if ((lane >> 4) == 0) {
        if (th == 0) stat_m[head(hb)] = m[hb];
        stat_l[th * C::NH + head(hb)] = lt;
      }
    }
  }
  __device__ __forceinline__ void finish_b() {}
};

template <int HH, int HBW, int BS>
struct ValueRole {
  using C = RoleCfg<HH, HBW>;
  const RoleShared<HH, HBW>& sh;
  ChunkSource<C::NP, BS>& src;
  int v, lane;
  f32x4 acc[C::MB][C::NB];   // O^T: dims DW*v + 16*mb .., heads 16*nb ..

  __device__ __forceinline__ void pv(int ci) {
    const int quad = lane >> 4, n = lane & 15;
    const ValueOps<C::DW> vo{sh.slot(ci), sh.pbuf(ci), v, n, quad};
    u32x4 pb[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) pb[nb] = vo.pb(nb);
    u32x4 va[2];
    va[0] = vo.va(0);
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      if (mb + 1 < C::MB) va[(mb + 1) & 1] = vo.va(mb + 1);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) mfma_v(acc[mb][nb], va[mb & 1], pb[nb]);
    }
  }

  __device__ __forceinline__ void pass_begin() {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Chunks 0 and 1 are issued even past the split's end (those loads read
  // the zero block), so the count in flight is known: chunk 0 has landed once
  // at most one chunk's loads are outstanding.
  __device__ __forceinline__ void prologue() {
    src.issue(sh.slot(0), 0);
    src.issue(sh.slot(1), 1);
    wait_vm<C::NWI>();
  }
  __device__ __forceinline__ void step0a() {
    if (2 < sh.nchunks) src.issue(sh.slot(2), 2);
  }
  __device__ __forceinline__ void step0b() {}
  // Before the barrier that opens step ci: chunk ci has landed.
  __device__ __forceinline__ void before_barrier(int ci) {
    if (ci + 1 < sh.nchunks) wait_vm<C::NWI>(); else wait_vm<0>();
  }
  // Step ci: refill the slot of chunk ci - 2 with chunk ci + 2, then the value
  // product of chunk ci - 1.
  __device__ __forceinline__ void step(int ci) {
    if (ci + 2 < sh.nchunks) src.issue(sh.slot(ci + 2), ci + 2);
    pv(ci - 1);
  }
  __device__ __forceinline__ void pass_end() { wait_vm<0>(); }
  __device__ __forceinline__ void vote(int) {}
  __device__ __forceinline__ void after_vote(bool) {}
  __device__ __forceinline__ void finish_a() {}
};

// The pass loop both roles run; every barrier of the workgroup is here, so
// both roles meet the same barriers in the same order.
template <typename Role, typename Begin>
__device__ __forceinline__ void role_loop(Role& r, int nchunks, const lds_char* ring, int ns, int w,
                                          const Begin& begin_pass) {
  for (;;) {
    r.pass_begin();
    begin_pass();                   // may hold a full barrier (token-id staging)
    r.prologue();
    lds_barrier();                  // chunk 0 in LDS
    r.step0a();
    lds_barrier();                  // first-chunk maxima exchanged
    r.step0b();
    for (int ci = 1; ci <= nchunks; ++ci) {
      r.before_barrier(ci);
      lds_barrier();                // chunk ci in LDS, probabilities of ci - 1 written,
                                    // value product of ci - 2 done
      r.step(ci);
    }
    r.pass_end();
    lds_barrier();                  // every read of the ring done, every load landed
    r.vote(w);
    lds_barrier();
    const int* votes = (const int*)(ring + kVoteOff);
    int any = 0;
    for (int i = 0; i < ns; ++i) any |= votes[i];
    any = __builtin_amdgcn_readfirstlane(any);
    r.after_vote(any != 0);
    lds_barrier();                  // votes read before the ring is refilled
    if (any == 0) return;
  }
}

template <int HH, int HBW, int BS>
__global__ __launch_bounds__((RoleCfg<HH, HBW>::NW * 64)) void mla_roles_partial(Params p) {
  using C = RoleCfg<HH, HBW>;
  __shared__ __attribute__((aligned(16))) char ring_lds[kRing * kChunkB];
  __shared__ __attribute__((aligned(16))) uint16_t pl_lds[2 * C::NH * kCT];
  __shared__ int ids_lds[BS == 1 ? kMaxIdsBS1 : 1];

  // 1-D grid of HG x S x B workgroups, HG = ql * Hq / NH head groups
  const int HG = p.ql * p.Hq / C::NH;
  int hg, u;
  group_and_unit(blockIdx.x, HG, p.S * p.B, hg, u);
  const int b = u / p.S;
  const int s = split_of_block(u % p.S, b, p.S);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int head0 = hg * C::NH;                       // of the ql * Hq row-heads
  const int ctx = clampi(p.context_lens[b], 0, p.max_ctx);
  const int pages = (ctx + BS - 1) / BS;
  const int nsplit = splits_of(pages, p.c);
  if (s >= (nsplit > 0 ? nsplit : 1)) return;
  const int t0 = s * p.c * BS;
  const int t1 = min(row_end(ctx, head0, p), (s * p.c + p.c) * BS);
  const int p1 = min(pages, s * p.c + p.c);
  const int nchunks = t1 > t0 ? (t1 - t0 + kCT - 1) / kCT : 0;

  RoleShared<HH, HBW> sh{(lds_char*)ring_lds, (lds_char*)pl_lds, nchunks};
  ChunkSource<C::NP, BS> src;
  src.bt = p.block_table + (size_t)b * p.maxb;
  src.cbase = static_cast<const char*>(p.k);
  src.t0 = t0;
  src.t1 = t1;
  src.p1 = p1;
  src.nblocks = p.nblocks;
  src.w = w < C::NS ? 0 : w - C::NS;
  src.lane = lane;
  if constexpr (BS == 1) src.ids = ids_lds;
  auto begin_pass = [&]() { src.begin(s * p.c); };
  const size_t row0 = (size_t)b * p.ql * p.Hq + head0;

  if (w < C::NS) {
    ScoreRole<HH, HBW, BS> r{sh, w & 1, w >> 1, lane, t0, t1, p.scale_log2};
    r.load_q(static_cast<const char*>(p.q) + row0 * kRowB);
    role_loop(r, nchunks, (const lds_char*)ring_lds, C::NS, w, begin_pass);
    r.finish_a();
    lds_barrier();                                    // statistics visible
  } else {
    ValueRole<HH, HBW, BS> r{sh, src, w - C::NS, lane};
    role_loop(r, nchunks, (const lds_char*)ring_lds, C::NS, w, begin_pass);
    lds_barrier();                                    // statistics visible
    // the accumulators are read by VALU below: cover the last MFMA's latency
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const float* stat_m = (const float*)(ring_lds + kStatOff);
    const float* stat_l = stat_m + C::NH;
    const int quad = lane >> 4, n = lane & 15;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      const int h = nb * 16 + n;
      const float mm = stat_m[h];
      const float lt = stat_l[h] + stat_l[C::NH + h];
      const float inv = (mm == kNegInf) ? 0.f : 1.f / lt;
      const size_t row = row0 + h;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int d = C::DW * r.v + mb * 16 + quad * 4;
        if (p.final_write) {
          u32x2 pk;
          pk[0] = pack_bf16(r.acc[mb][nb][0] * inv, r.acc[mb][nb][1] * inv);
          pk[1] = pack_bf16(r.acc[mb][nb][2] * inv, r.acc[mb][nb][3] * inv);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + row * kDv + d) = pk;
        } else {
          f32x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = r.acc[mb][nb][j] * inv;
          *reinterpret_cast<f32x4*>(p.o_part + (row * p.S + s) * kDv + d) = o;
        }
      }
    }
    if (r.v == 0 && lane < C::NH) {
      const float mm = stat_m[lane];
      const float lt = stat_l[lane] + stat_l[C::NH + lane];
      const float lse = (mm == kNegInf) ? kNegInf : (mm + fast_log2(lt)) * kLn2;
      const size_t row = row0 + lane;
      if (p.final_write) {
        if (p.lse) p.lse[row] = lse;
      } else {
        p.lse_part[row * p.S + s] = lse;
      }
    }
  }
}

template <int HH, int HBW>
hipError_t launch_roles(const Params& p, hipStream_t st) {
  using C = RoleCfg<HH, HBW>;
  const long blocks = (long)(p.ql * p.Hq / C::NH) * p.S * p.B;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  if (p.bs == 1)
    hipLaunchKernelGGL((mla_roles_partial<HH, HBW, 1>), dim3((unsigned)blocks), dim3(C::NW * 64), 0,
                       st, p);
  else
    hipLaunchKernelGGL((mla_roles_partial<HH, HBW, 64>), dim3((unsigned)blocks), dim3(C::NW * 64),
                       0, st, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Wide workgroup: all 128 heads of a (sequence, split) in one workgroup of 8
// waves, two per SIMD, so every CU streams each latent row of its split once.
// Wave w scores head block w (16 heads, both token halves of a chunk: S^T
// 32 x 16, queries in 72 registers) and accumulates O^T for dims 64w ..
// 64w+63 of all 128 heads (accumulators in 128 registers): 200 of the 256
// registers a wave has at two waves per SIMD.  Each step scores chunk i and
// then runs the value product of chunk i - 1.  Every wave issues its
// share of the chunk loads (4 or 5 of the 36 per chunk).  Softmax bookkeeping
// is per wave as its heads are its own: reference max fixed per pass, restart
// on overflow, sums per lane.
constexpr int kWideNW = 8;
constexpr int kWideNH = 128;
constexpr int kWideDW = kDv / kWideNW;   // 64 value dims per wave
constexpr int kWideMB = kWideDW / 16;    // 4 M-blocks
constexpr int kWideNB = kWideNH / 16;    // 8 head blocks

struct WideOps {
  const lds_char* ring;
  const lds_char* pl;
  int w, lane;
  __device__ __forceinline__ const lds_char* slot(int ci) const { return ring + (ci % kRing) * kChunkB; }
  __device__ __forceinline__ const lds_char* pbuf(int ci) const {
    return pl + (ci & 1) * (kWideNH * kCT * 2);
  }
  // V^T A operand of M-block mb: dims 64w + 16mb + (lane & 15), tokens
  // 8*quad .. +7, two transposed reads.
  __device__ __forceinline__ u32x4 va(const lds_char* buf, int mb) const {
    const int quad = lane >> 4, n = lane & 15;
    const int bc = (kWideDW * w + mb * 16) * 2 + (n & 3) * 8;   // byte column
    const int r0 = quad * 8 + (n >> 2), r1 = r0 + 4;
    const lds_char* lo = buf + r0 * kRowB + (((bc >> 4) ^ row_key(r0)) << 4) + (bc & 15);
    const lds_char* hi = buf + r1 * kRowB + (((bc >> 4) ^ row_key(r1)) << 4) + (bc & 15);
    const u32x2 vlo = lds_tr16(lo), vhi = lds_tr16(hi);
    return u32x4{vlo[0], vlo[1], vhi[0], vhi[1]};
  }
  // P^T B operand of head block nb: tokens 8*quad .. +7 of head 16nb + (lane & 15).
  __device__ __forceinline__ u32x4 pb(const lds_char* pbuf, int nb) const {
    const int quad = lane >> 4, n = lane & 15;
    return *(const lds_u32x4*)(pbuf + nb * (16 * kCT * 2) + 16 * (quad * 16 + n));
  }
};

struct WideState {
  u32x4 qf[kKSteps];                  // Q^T B operands of head block w
  f32x4 acc[kWideMB][kWideNB];        // O^T: dims 64w + 16mb .., heads 16nb ..
  float m, mtop, l;                   // reference max, largest chunk max (log2), lane's sum
  bool bad;
};

// Scores of chunk ci for head block w, softmax weights, probabilities to LDS.
__device__ __forceinline__ void wide_scores(WideState& st, const WideOps& op, int ci, int t0, int t1,
                                            float cs) {
  const lds_char* buf = op.slot(ci);
  const int lane = op.lane, quad = lane >> 4, n = lane & 15;
  // Row n (and 16 + n), 16-byte chunk kb*4 + quad, stored at chunk (kb*4 + quad) ^ (n & 7).
  const int xb = (n >> 2) & 1;
  const int sbase = n * kRowB + 16 * (quad ^ (n & 3));
  const lds_char* se = buf + sbase + 64 * xb;
  const lds_char* so = buf + sbase - 64 * xb;
  auto load_a = [&](int kb, u32x4& x0, u32x4& x1) {
    const lds_char* rp = ((kb & 1) ? so : se) + 64 * kb;
    x0 = *(const lds_u32x4*)rp;
    x1 = *(const lds_u32x4*)(rp + 16 * kRowB);
  };
  constexpr int L = 1;
  u32x4 ab[L + 1][2];
  f32x4 sa[2];
#pragma unroll
  for (int kb = 0; kb < L; ++kb) load_a(kb, ab[kb][0], ab[kb][1]);
#pragma unroll
  for (int kb = 0; kb < kKSteps; ++kb) {
    if (kb + L < kKSteps) load_a(kb + L, ab[(kb + L) % (L + 1)][0], ab[(kb + L) % (L + 1)][1]);
    if (kb == 0) {
      mfma_v_first(sa[0], ab[0][0], st.qf[0]);
      mfma_v_first(sa[1], ab[0][1], st.qf[0]);
    } else {
      mfma_v(sa[0], ab[kb % (L + 1)][0], st.qf[kb]);
      mfma_v(sa[1], ab[kb % (L + 1)][1], st.qf[kb]);
    }
  }
  drain_scores<2>(sa);
  // lane: tokens quad*4 + j (sa[0]) and 16 + quad*4 + j (sa[1]) of head 16w + n
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = sa[0][j];
    v[4 + j] = sa[1][j];
  }
  const int tb = t0 + ci * kCT + quad * 4;
  if (tb + 16 + 4 > t1) {                            // only a split's last chunk runs past t1
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (tb + j >= t1) v[j] = kNegInf;
      if (tb + 16 + j >= t1) v[4 + j] = kNegInf;
    }
  }
  float mx = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])),
                   fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
  mx = max_xor32(max_xor16(mx)) * cs;                // log2 units, same in the 4 quads
  st.mtop = fmaxf(st.mtop, mx);
  if (st.m == kNegInf) st.m = mx;                    // first chunk of the first pass
  st.bad |= mx > st.m + kHeadroom;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = fast_exp2(fmaf(v[j], cs, -st.m));
  st.l += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
  // head block w, 16-byte slot q*16 + n holds tokens 8q .. 8q+7
  lds_char* prow = (lds_char*)op.pbuf(ci) + op.w * (16 * kCT * 2) + n * 16;
  u32x2 p0, p1;
  p0[0] = pack_bf16(v[0], v[1]);
  p0[1] = pack_bf16(v[2], v[3]);
  p1[0] = pack_bf16(v[4], v[5]);
  p1[1] = pack_bf16(v[6], v[7]);
  ds_store_b64(prow + 256 * (quad >> 1) + 8 * (quad & 1), p0);
  ds_store_b64(prow + 256 * (2 + (quad >> 1)) + 8 * (quad & 1), p1);
}

// Value product of chunk ci: dims 64w .. 64w+63 of all 128 heads.
__device__ __forceinline__ void wide_values(WideState& st, const WideOps& op, int ci) {
  const lds_char* buf = op.slot(ci);
  const lds_char* pb = op.pbuf(ci);
  u32x4 va[kWideMB];
#pragma unroll
  for (int mb = 0; mb < kWideMB; ++mb) va[mb] = op.va(buf, mb);
  u32x4 b[2];
  b[0] = op.pb(pb, 0);
#pragma unroll
  for (int nb = 0; nb < kWideNB; ++nb) {
    if (nb + 1 < kWideNB) b[(nb + 1) & 1] = op.pb(pb, nb + 1);
#pragma unroll
    for (int mb = 0; mb < kWideMB; ++mb) mfma_v(st.acc[mb][nb], va[mb], b[nb & 1]);
  }
}

__global__ __launch_bounds__(kWideNW * 64) void mla_wide_partial(Params p) {
  __shared__ __attribute__((aligned(16))) char ring_lds[kRing * kChunkB];
  __shared__ __attribute__((aligned(16))) uint16_t pl_lds[2 * kWideNH * kCT];

  const int HG = p.ql * p.Hq / kWideNH;               // head groups (of query rows too)
  int hg, u;
  group_and_unit(blockIdx.x, HG, p.S * p.B, hg, u);
  // split-major: the splits of sequence b are B workgroups apart, so with B a
  // multiple of 8 they share an XCD (workgroups go round-robin to the 8
  // XCDs) and its L2 serves the queries to all but the first
  const int b = u % p.B;
  const int s = u / p.B;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quad = lane >> 4, n = lane & 15;
  const int head0 = hg * kWideNH;
  const int ctx = clampi(p.context_lens[b], 0, p.max_ctx);
  const int pages = (ctx + 63) / 64;
  const int nsplit = splits_of(pages, p.c);
  if (s >= (nsplit > 0 ? nsplit : 1)) return;
  const int t0 = s * p.c * 64;
  const int t1 = min(row_end(ctx, head0, p), (s * p.c + p.c) * 64);
  const int p1 = min(pages, s * p.c + p.c);
  const int nchunks = t1 > t0 ? (t1 - t0 + kCT - 1) / kCT : 0;
  const float cs = p.scale_log2;                      // > 0, checked by the host
  const int nwi = (kDmaInst - w + kWideNW - 1) / kWideNW;   // this wave's loads per chunk

  WideState st;
  const size_t row0 = (size_t)b * p.ql * p.Hq + head0;
  {
    const char* qr = static_cast<const char*>(p.q) + (row0 + 16 * w + n) * kRowB;
#pragma unroll
    for (int kb = 0; kb < kKSteps; ++kb) st.qf[kb] = ld128(qr + kb * 64 + quad * 16);
  }
  st.m = kNegInf;
  st.mtop = kNegInf;

  const WideOps op{(const lds_char*)ring_lds, (const lds_char*)pl_lds, w, lane};
  lds_char* const ring = (lds_char*)ring_lds;
  auto slot = [&](int ci) { return ring + (ci % kRing) * kChunkB; };
  ChunkSource<kWideNW, 64> src;
  src.bt = p.block_table + (size_t)b * p.maxb;
  src.cbase = static_cast<const char*>(p.k);
  src.t0 = t0;
  src.t1 = t1;
  src.p1 = p1;
  src.nblocks = p.nblocks;
  src.w = w;
  src.lane = lane;
  for (;;) {
    st.l = 0.f;
#pragma unroll
    for (int mb = 0; mb < kWideMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kWideNB; ++nb) st.acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.bad = false;
    src.begin(s * p.c);
    // Chunks 0 and 1 are issued even past the split's end (those loads read
    // the zero block), so the count in flight is known here: one wait retires
    // the query loads (older) and chunk 0.
    src.issue(slot(0), 0);
    src.issue(slot(1), 1);
    wait_vm_dyn(nwi);
    lds_barrier();
    if (nchunks > 0) {
      if (2 < nchunks) src.issue(slot(2), 2);
      wide_scores(st, op, 0, t0, t1, cs);
    }
    for (int ci = 1; ci < nchunks; ++ci) {
      // chunk ci has landed (this wave's loads, then, after the barrier,
      // every wave's); the probabilities of ci - 1 are complete; the value
      // product of ci - 2 is done, so its slot can be refilled
      if (ci + 1 < nchunks) wait_vm_dyn(nwi); else wait_vm<0>();
      lds_barrier();
      if (ci + 2 < nchunks) src.issue(slot(ci + 2), ci + 2);
      wide_scores(st, op, ci, t0, t1, cs);
      wide_values(st, op, ci - 1);
    }
    if (nchunks > 0) {
      lds_barrier();                                  // the last chunk's probabilities
      wide_values(st, op, nchunks - 1);
    }
    // Did any head's chunk max overflow the headroom over its reference max?
    wait_vm<0>();                                     // loads issued past the end of a short split
    lds_barrier();
    int* votes = (int*)ring_lds;
    if (lane == 0) votes[w] = __builtin_amdgcn_ballot_w64(st.bad) != 0;
    lds_barrier();
    int any = 0;
#pragma unroll
    for (int i = 0; i < kWideNW; ++i) any |= votes[i];
    lds_barrier();                                    // votes read before the ring is refilled
    if (__builtin_amdgcn_readfirstlane(any) == 0) break;
    // Start over with the reference max raised to the largest chunk max: no
    // chunk can overflow then, so this happens at most once.
    st.m = st.mtop;
  }
  // the accumulators are read by VALU below: cover the last MFMA's latency
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  float* stat_m = (float*)ring_lds;
  float* stat_l = stat_m + kWideNH;
  {
    const float lt = sum_xor32(sum_xor16(st.l));
    if (quad == 0) {
      stat_m[16 * w + n] = st.m;
      stat_l[16 * w + n] = lt;
    }
  }
  lds_barrier();
#pragma unroll
  for (int nb = 0; nb < kWideNB; ++nb) {
    const float mm = stat_m[nb * 16 + n];
    const float lt = stat_l[nb * 16 + n];
    const float inv = (mm == kNegInf) ? 0.f : 1.f / lt;
    const size_t row = row0 + nb * 16 + n;
#pragma unroll
    for (int mb = 0; mb < kWideMB; ++mb) {
      const int d = kWideDW * w + mb * 16 + quad * 4;
      if (p.final_write) {
        u32x2 pk;
        pk[0] = pack_bf16(st.acc[mb][nb][0] * inv, st.acc[mb][nb][1] * inv);
        pk[1] = pack_bf16(st.acc[mb][nb][2] * inv, st.acc[mb][nb][3] * inv);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + row * kDv + d) = pk;
      } else {
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = st.acc[mb][nb][j] * inv;
        *reinterpret_cast<f32x4*>(p.o_part + (row * p.S + s) * kDv + d) = o;
      }
    }
  }
  if (quad == 0) {
    const int h = 16 * w + n;
    const float mm = stat_m[h];
    const float lt = stat_l[h];
    const float lse = (mm == kNegInf) ? kNegInf : (mm + fast_log2(lt)) * kLn2;
    const size_t row = row0 + h;
    if (p.final_write) {
      if (p.lse) p.lse[row] = lse;
    } else {
      p.lse_part[row * p.S + s] = lse;
    }
  }
}

hipError_t launch_wide(const Params& p, hipStream_t st) {
  const long blocks = (long)(p.ql * p.Hq / kWideNH) * p.S * p.B;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_wide_partial, dim3((unsigned)blocks), dim3(kWideNW * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace

bool mla_mfma_supported(bool bf16, int Dqk, int Dv, int bs, int Hq) {
  return bf16 && Dqk == kDqk && Dv == kDv && (bs == 64 || bs == 1) &&
         (Hq % 64 == 0 || Hq == 32 || Hq == 16);
}

int mla_heads_per_workgroup(int Hq, int bs) {
  if (bs == 64 && Hq % kWideNH == 0) return kWideNH;
  return Hq % 64 == 0 ? 64 : Hq;
}

int mla_max_split_tokens(int bs) { return bs == 1 ? kMaxIdsBS1 : 0x7fffffff; }

hipError_t launch_mla_mfma(const Params& p, hipStream_t st) {
  if (p.bs == 64 && p.Hq % kWideNH == 0) return launch_wide(p, st);
  if (p.Hq % 64 == 0) return launch_roles<2, 2>(p, st);
  if (p.Hq == 32) return launch_roles<2, 1>(p, st);
  if (p.Hq == 16) return launch_roles<1, 1>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
