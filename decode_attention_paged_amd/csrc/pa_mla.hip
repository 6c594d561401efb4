// Split-KV partial kernels for MLA latent decode on the matrix cores.
//
// All query heads attend to one latent row per token (keys: the whole
// 576-wide row; values: its first 512 entries, the same memory).  A workgroup
// handles the heads of one head group for one (sequence, split) and walks
// the split in chunks of 32 tokens (half a 64-token page):
//
//   scores  S^T[32 tok x heads] = C[32 x 576] Q^T
//   values  O^T[512 dims x heads] += V^T[512 x 32] P^T      split by dims over waves
//
// on the matrix cores.  Queries stay in registers as score B operands; the
// value product is split by output dims, so the transposed value reads
// (ds_read_b64_tr_b16, the slowest LDS read) touch each latent element once
// per workgroup.  The probabilities P move from the score to the value
// product through LDS.  This is Flash-Decoding's attention of the query with
// one block of keys and values plus the block's log-sum-exp (the "flash
// decoding ++" entry, its three-steps snippet, second step); the split's
// (o_s, lse_s) go to the workspace for the reduction, o_s in bfloat16 (the
// output's type), lse_s in float32.
//
// Two workgroup shapes:
//   * wide (128 heads, 64-token pages): 4 waves, one per SIMD, on
//     v_mfma_f32_32x32x16_bf16; wave w scores heads 32w .. 32w+31 and
//     accumulates dims 128w .. 128w+127 of all 128 heads; each CU streams
//     every latent row of its split once (details at mla_wide_partial).
//   * role-split (16, 32 or 64 heads; also one-token pages, whose token ids
//     take 8 KiB of LDS): two waves per SIMD on v_mfma_f32_16x16x32_bf16;
//     score waves hold the queries, value waves hold the accumulators and
//     issue the chunk loads.  With 128 heads the grid has two such
//     workgroups per (sequence, split), 8 apart in dispatch order: the same
//     XCD (workgroups go round-robin to the 8 XCDs), so the second reads the
//     rows from that XCD's L2.
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
// Chunks stream HBM -> LDS with direct-to-LDS loads (no registers), two
// chunks in flight while one is scored and the one before goes through the
// value product.  Barriers are raw s_barrier with explicit waits:
// __syncthreads() would also wait for every chunk in flight.
//
// LDS chunk rows are 1152 bytes (72 chunks of 16 bytes).  Chunk c of token
// row t sits at position c ^ (t & 7); with it the score reads (rows of one
// chunk each) and the transposed value reads run at the conflict-free rate
// (measured against a linear read of the same size).  The probabilities are
// stored so that the value product's B-operand read is linear.

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

// The same through a buffer resource: lane L reads record bytes voff .. +15
// of the resource and writes them to wave_base + 16 L.  A lane whose bytes
// lie past the resource's record count reads zeros (the buffer range check),
// so the resource bounds what is read without per-lane selects.  The wave
// offset operand stays 0 (on gfx950 the direct-to-LDS forms take the whole
// global offset from voff).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma16_buf(const i32x4& rsrc, int voff, lds_char* wave_base) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"((uint32_t)(uintptr_t)wave_base)
               : "memory");
}
// Raw buffer resource over `bytes` bytes from `base` (stride 0, 32-bit
// data format: byte-addressed records), held in SGPRs.
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
               __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
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
__device__ __forceinline__ void ds_store_b128(lds_char* p, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
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

// FP8 latent rows (one E4M3 code per element, 576 bytes) for the role-split
// workgroup: a 32-token chunk is 18 KiB of codes, staged linearly (row t at
// 576 t) by 20 loads of 1 KiB, 5 per loading wave (the last two read the
// zero block into the slot's padding), and widened into the bf16 chunk
// layout in LDS before its scores (widen_rows8).
constexpr int kRow8 = kDqk;                     // 576 bytes per FP8 row
constexpr int kChunk8 = kCT * kRow8;            // 18432 bytes of codes per chunk
constexpr int kLoads8 = 20;                     // loads per FP8 chunk (18 + 2 of padding)
constexpr int kStage8 = kLoads8 * 1024;         // bytes per FP8 staging slot

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
  // FP8 rows: this wave's share of chunk ci's codes (half a page, contiguous)
  // into a staging slot, linearly; bytes past the split's end read zeros.
  __device__ __forceinline__ void issue8(lds_char* dst, int ci) {
    static_assert(kLoads8 % NW == 0, "uniform FP8 load share");
    const int tok0 = t0 + ci * kCT;
    const char* src = cbase + (size_t)page_of(ci) * (64 * kRow8) + (tok0 % 64) * kRow8;
    const int lim = min((t1 - tok0) * kRow8, kChunk8);
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < kLoads8 / NW; ++k) {
      const int j = w + NW * k;
      const int off = 1024 * j + 16 * ln;
      dma16(off < lim ? (const void*)(src + off) : (const void*)g_zero16, dst + 1024 * j);
    }
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
  // FP8 rows: this wave's share of chunk ci's codes into a staging slot,
  // linearly (row t at 576 t); a 1 KiB load spans up to three rows, each
  // lane reads the id of its own row.  Rows past the split's end, and the
  // padding, read zeros.
  __device__ __forceinline__ void issue8(lds_char* dst, int ci) {
    static_assert(kLoads8 % NW == 0, "uniform FP8 load share");
    const int tok0 = t0 + ci * kCT;
    const int nrows = min(t1 - tok0, kCT);
    int ln = lane;
    asm volatile("" : "+v"(ln));
    int id[kLoads8 / NW];
#pragma unroll
    for (int k = 0; k < kLoads8 / NW; ++k) {
      const int t = (1024 * (w + NW * k) + 16 * ln) / kRow8;
      id[k] = ids[min(max(tok0 - t0 + t, 0), kMaxIdsBS1 - 1)];
    }
#pragma unroll
    for (int k = 0; k < kLoads8 / NW; ++k) {
      const int j = w + NW * k;
      const int off = 1024 * j + 16 * ln;
      const int t = off / kRow8;
      const void* g = t < nrows ? (const void*)(cbase + (size_t)id[k] * kRow8 + (off - t * kRow8))
                                : (const void*)g_zero16;
      dma16(g, dst + 1024 * j);
    }
  }
};

// Operands of the value product for dims DW*w .. DW*w + DW - 1 of every
// head.  A operand (V^T): tokens quad*8 .. +7 of one dim per lane, two
// transposed reads; B operand (P^T): one 16-byte slot.  The probabilities of
// head block nb are stored so that this read is linear: 16-byte slot
// q*16 + n holds tokens 8q .. 8q+7 of head 16 nb + n.
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
static_assert(2 * kChunkB + 3 * kStage8 <= kRing * kChunkB, "FP8 staging fits the ring");

// Widen the 32 staged FP8 rows of a chunk into a bf16 chunk buffer (the
// role-split layout: 16-byte piece c of row t at c ^ row_key(t)); thread i of
// NT takes pieces i, i + NT, ...  Piece m is codes 8 m .. 8 m + 7 of the
// stage, i.e. elements 8 (m % 72) .. +7 of row m / 72.
template <int NT>
__device__ __forceinline__ void widen_rows8(const lds_char* stg, lds_char* dst) {
  int i0 = threadIdx.x;
  asm volatile("" : "+v"(i0));
#pragma unroll
  for (int k = 0; k < (kCT * (kRowB / 16) + NT - 1) / NT; ++k) {
    const int m = i0 + NT * k;
    if (m < kCT * (kRowB / 16)) {
      const u32x2 c8 = *(const __attribute__((address_space(3))) u32x2*)(stg + 8 * m);
      const int t = m / (kRowB / 16), c = m - t * (kRowB / 16);
      ds_store_b128(dst + t * kRowB + 16 * (c ^ row_key(t)), fp8x8_to_bf16x8(c8[0], c8[1]));
    }
  }
}

template <int HH, int HBW>
struct RoleShared {
  lds_char* ring;
  lds_char* pl;                    // probabilities, two buffers of NH*kCT bf16
  int nchunks;
  int nslots;                      // bf16 chunk slots: 4, or 2 with FP8 staging after them
  __device__ __forceinline__ lds_char* slot(int ci) const {
    return ring + (ci & (nslots - 1)) * kChunkB;
  }
  // FP8 codes of chunk ci (three staging slots after the two bf16 ones)
  __device__ __forceinline__ lds_char* stg8(int ci) const {
    return ring + 2 * kChunkB + (ci % 3) * kStage8;
  }
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

template <int HH, int HBW, int BS, bool F8>
struct ValueRole {
  using C = RoleCfg<HH, HBW>;
  static constexpr int kNwi = F8 ? kLoads8 / C::NP : C::NWI;   // loads per chunk and wave
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
  // chunk ci into its bf16 slot, or its codes into its FP8 staging slot
  __device__ __forceinline__ void load(int ci) {
    if constexpr (F8) src.issue8(sh.stg8(ci), ci);
    else src.issue(sh.slot(ci), ci);
  }
  __device__ __forceinline__ void prologue() {
    load(0);
    load(1);
    wait_vm<kNwi>();
  }
  __device__ __forceinline__ void step0a() {
    if (2 < sh.nchunks) load(2);
  }
  __device__ __forceinline__ void step0b() {}
  // Before the barrier that opens step ci: chunk ci has landed.
  __device__ __forceinline__ void before_barrier(int ci) {
    if (ci + 1 < sh.nchunks) wait_vm<kNwi>(); else wait_vm<0>();
  }
  // Step ci: refill the slot of chunk ci - 2 with chunk ci + 2 (FP8: the
  // staging slot of chunk ci - 1, widened in the step before), then the value
  // product of chunk ci - 1.
  __device__ __forceinline__ void step(int ci) {
    if (ci + 2 < sh.nchunks) load(ci + 2);
    pv(ci - 1);
  }
  __device__ __forceinline__ void pass_end() { wait_vm<0>(); }
  __device__ __forceinline__ void vote(int) {}
  __device__ __forceinline__ void after_vote(bool) {}
  __device__ __forceinline__ void finish_a() {}
};

// The pass loop both roles run; every barrier of the workgroup is here, so
// both roles meet the same barriers in the same order.
// With FP8 rows, each chunk is widened by every wave between two barriers
// (the first: its codes have landed; the second: its bf16 rows are in place).
template <bool F8, typename Role, typename Begin, typename Widen>
__device__ __forceinline__ void role_loop(Role& r, int nchunks, const lds_char* ring, int ns, int w,
                                          const Begin& begin_pass, const Widen& widen) {
  for (;;) {
    r.pass_begin();
    begin_pass();                   // may hold a full barrier (token-id staging)
    r.prologue();
    lds_barrier();                  // chunk 0 in LDS
    if constexpr (F8) {
      if (nchunks > 0) {
        widen(0);
        lds_barrier();
      }
    }
    r.step0a();
    lds_barrier();                  // first-chunk maxima exchanged
    r.step0b();
    for (int ci = 1; ci <= nchunks; ++ci) {
      r.before_barrier(ci);
      lds_barrier();                // chunk ci in LDS, probabilities of ci - 1 written,
                                    // value product of ci - 2 done
      if constexpr (F8) {
        if (ci < nchunks) {
          widen(ci);
          lds_barrier();
        }
      }
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

template <int HH, int HBW, int BS, bool F8>
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

  RoleShared<HH, HBW> sh{(lds_char*)ring_lds, (lds_char*)pl_lds, nchunks, F8 ? 2 : kRing};
  auto widen = [&](int ci) { widen_rows8<C::NW * 64>(sh.stg8(ci), sh.slot(ci)); };
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
    role_loop<F8>(r, nchunks, (const lds_char*)ring_lds, C::NS, w, begin_pass, widen);
    r.finish_a();
    lds_barrier();                                    // statistics visible
  } else {
    ValueRole<HH, HBW, BS, F8> r{sh, src, w - C::NS, lane};
    role_loop<F8>(r, nchunks, (const lds_char*)ring_lds, C::NS, w, begin_pass, widen);
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
      // (v_scale: the factor of every FP8 value, 1 for bf16 caches)
      const float inv = (mm == kNegInf) ? 0.f : p.v_scale / lt;
      const size_t row = row0 + h;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int d = C::DW * r.v + mb * 16 + quad * 4;
        // the output, or this split's partial (bfloat16 either way)
        uint16_t* dst = p.final_write ? static_cast<uint16_t*>(p.out) + row * kDv + d
                                      : p.o_part16 + (row * p.S + s) * kDv + d;
        u32x2 pk;
        pk[0] = pack_bf16(r.acc[mb][nb][0] * inv, r.acc[mb][nb][1] * inv);
        pk[1] = pack_bf16(r.acc[mb][nb][2] * inv, r.acc[mb][nb][3] * inv);
        *reinterpret_cast<u32x2*>(dst) = pk;
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

template <int HH, int HBW, int BS, bool F8>
void launch_roles_as(const Params& p, long blocks, hipStream_t st) {
  hipLaunchKernelGGL((mla_roles_partial<HH, HBW, BS, F8>), dim3((unsigned)blocks),
                     dim3(RoleCfg<HH, HBW>::NW * 64), 0, st, p);
}

template <int HH, int HBW>
hipError_t launch_roles(const Params& p, bool fp8kv, hipStream_t st) {
  using C = RoleCfg<HH, HBW>;
  const long blocks = (long)(p.ql * p.Hq / C::NH) * p.S * p.B;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  if (p.bs == 1) {
    if (fp8kv) launch_roles_as<HH, HBW, 1, true>(p, blocks, st);
    else launch_roles_as<HH, HBW, 1, false>(p, blocks, st);
  } else {
    if (fp8kv) launch_roles_as<HH, HBW, 64, true>(p, blocks, st);
    else launch_roles_as<HH, HBW, 64, false>(p, blocks, st);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Wide workgroup: all 128 heads of a (sequence, split) in one workgroup of 4
// waves, one per SIMD, so every CU streams each latent row of its split once.
//
// One wave per SIMD gives each wave the whole register file (256 VGPRs and
// 256 AGPRs), which lets the larger MFMA shape v_mfma_f32_32x32x16_bf16 serve
// both products:
//   scores  wave w: S^T[32 tokens x 32 heads] = C[32 x 576] Q^T for heads
//           32w .. 32w+31; the queries stay in 144 VGPRs as B operands, and
//           each latent row is read from LDS once per 32 heads (4 times per
//           chunk and workgroup, where 16-head blocks read it 8 times);
//   values  wave w: O^T[128 dims x 128 heads] += V^T[128 x 32] P^T for dims
//           128w .. 128w+127; the accumulators fill the 256 AGPRs.
// Each step scores chunk i and then runs the value product of chunk i - 1;
// every wave issues 9 of the chunk's 36 direct-to-LDS loads.  Softmax
// bookkeeping is per wave, as its score heads are its own: reference max
// fixed per pass, restart on overflow, sums per lane.
//
// 32x32 MFMA operand layouts (K = 16: A[i][k] in lane i + 32*(k/8), element
// k%8; B[k][j] in lane j + 32*(k/8); D[i][j] in lane j + 32*((i/4)%2),
// register 4*(i/8) + i%4):
//   score A: token (lane & 31), 16-byte chunk 2*kb + (lane >> 5) of its row;
//   score D: lane holds head (lane & 31), tokens 8g + 4*(lane >> 5) + r in
//            register 4g + r;
//   value A: dim (lane & 31) of an M-block, tokens 8*(lane >> 5) .. +7 of a
//            16-token k-step (two transposed reads);
//   value B: the 8 weights of those tokens for head (lane & 31) of a head
//            block: one 16-byte slot, stored so that the read is linear.
constexpr int kWideNW = 4;
constexpr int kWideNH = 128;
constexpr int kWideHW = kWideNH / kWideNW;   // 32 score heads per wave
constexpr int kWideDW = kDv / kWideNW;       // 128 value dims per wave
constexpr int kWideMB = kWideDW / 32;        // 4 M-blocks of 32 dims
constexpr int kWideNB = kWideNH / 32;        // 4 head blocks of 32
constexpr int kWideKS = kDqk / 16;           // 36 score k-steps
// Score operand reads in flight ahead of their MFMAs.  With one wave per
// SIMD an LDS read's latency is covered only by the reads issued before it:
// eight 1 KiB reads in flight (one accumulation chain leaves the registers
// for them) measured 2-4 % faster than four with two chains.
constexpr int kWideLook = 8;
constexpr int kWidePB = kWideNH * kCT * 2;   // bytes of one probability buffer
static_assert(kDmaInst % kWideNW == 0, "uniform load share");
constexpr int kWideOutRowB = 2 * kDv + 16;   // staged output row (bytes), padded against bank conflicts
static_assert(kWideNH * kWideOutRowB <= kRing * kChunkB, "output tile fits the ring");
static_assert(2 * kWideNH * 4 <= 2 * kWidePB, "statistics fit the probability buffers");
static_assert(kDv == 64 * 8, "one 16-byte store per lane covers an output row");

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Score MFMAs as asm, so their accumulators stay in VGPRs (see the 16x16
// forms above for the padding); the drain covers an 8-pass result before
// VALU reads it.
__device__ __forceinline__ void mfma32_v_first(f32x16& d, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_v(f32x16& d, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void drain_scores32(f32x16& s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
}
// Value MFMA (accumulators in AGPRs: the compiler places them there, as
// the VGPRs hold the queries).
__device__ __forceinline__ void mfma32_a(f32x16& d, const u32x4& a, const u32x4& b) {
  d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                              __builtin_bit_cast(bf16x8, b), d, 0, 0, 0);
}

// Swizzle key of the wide workgroup's chunk rows: 16-byte chunk c of row t
// sits at c ^ wide_key(t), with key bits (t1 ^ t2, t3, t1) of the row's bits
// t1..t3.  A 16-byte read instruction is served 16 lanes at a time across
// 64 banks; for the score and query reads (16 consecutive rows at one chunk)
// the key spreads the 8 even and the 8 odd rows over distinct bank groups,
// and for the transposed value reads (rows r, r + 1, r + 2, r + 3 at four
// chunks, r a multiple of 4) it separates rows r and r + 2, which a key of
// t & 7 maps to the same banks (measured: 62 % fewer bank-conflict cycles).
// Rows r and r + 4 (r & 4 == 0) differ in key bit 2 only.
__device__ __forceinline__ int wide_key(int t) {
  return ((((t >> 2) ^ (t >> 1)) & 1) << 2) | (((t >> 3) & 1) << 1) | ((t >> 1) & 1);
}

// Chunk loads of the wide workgroup.  A chunk is 36 loads of 1 KiB: load
// j = 9q + r covers 16-byte slots 64r .. 64r + 63 of token rows 8q .. 8q + 7
// (8 rows of 72 slots); the swizzle key repeats every 16 rows, so its lanes
// read the bytes of load r's lanes in a row group of q's parity plus 16 rows
// (18432 bytes) times q / 2.  Wave w issues loads r = 2w and 2w + 1 of every
// row group q and load r = 8 of group w, so it needs the lane offsets of
// five loads only, computed once; a load is then one add and the buffer load
// (its chunk's resource bounds it: rows past the split's end read zeros).
struct WideLoads {
  int pa0, pb0, pa1, pb1;   // lane offsets of loads r = 2w, 2w + 1 in row groups 0 and 1
  int p8;                   // of load r = 8 in row group w % 2
  int w;
  __device__ __forceinline__ static int lane_off(int r, int parity, int lane) {
    const int slot = 64 * r + lane;
    const int t = 8 * parity + slot / (kRowB / 16);
    const int c = (slot % (kRowB / 16)) ^ wide_key(t);
    return t * kRowB + c * 16;
  }
  __device__ __forceinline__ void init(int w_, int lane) {
    w = w_;
    pa0 = lane_off(2 * w, 0, lane);
    pb0 = lane_off(2 * w + 1, 0, lane);
    pa1 = lane_off(2 * w, 1, lane);
    pb1 = lane_off(2 * w + 1, 1, lane);
    p8 = lane_off(8, w & 1, lane);
  }
  // A fresh definition of the offsets for each chunk, so the compiler does
  // not hoist all nine sums out of the chunk loop (nine live registers).
  __device__ __forceinline__ void refresh() {
    asm volatile("" : "+v"(pa0), "+v"(pb0), "+v"(pa1), "+v"(pb1), "+v"(p8));
  }
  // Load i (0 .. 8) of this wave's share of a chunk into chunk buffer dst.
  __device__ __forceinline__ void issue(const i32x4& rsrc, lds_char* dst, int i) const {
    const int q = i < 8 ? i >> 1 : w;
    const int r = i < 8 ? 2 * w + (i & 1) : 8;
    const int lo = i < 8 ? ((i & 1) ? ((q & 1) ? pb1 : pb0) : ((q & 1) ? pa1 : pa0)) : p8;
    dma16_buf(rsrc, lo + 16 * kRowB * (q >> 1), dst + (9 * q + r) * 1024);
  }
  __device__ __forceinline__ void issue_all(const i32x4& rsrc, lds_char* dst) const {
#pragma unroll
    for (int i = 0; i < 9; ++i) issue(rsrc, dst, i);
  }
};
static_assert(kDmaInst == 36 && kWideNW == 4 && kRowB == 1152, "wide load plan");
static_assert(kWideNH == kRing * kCT, "the queries of a head group fill the ring");

// Resource of chunk ci: its rows in the cache, the record count the bytes of
// the chunk inside the split (0 for a chunk past its end).
__device__ __forceinline__ i32x4 wide_rsrc(ChunkSource<kWideNW, 64>& src, int ci) {
  const int tok0 = src.t0 + ci * kCT;
  if (tok0 >= src.t1) return raw_rsrc(src.cbase, 0);
  const char* base = src.cbase + (size_t)src.page_of(ci) * (64 * kRowB) + (tok0 % 64) * kRowB;
  return raw_rsrc(base, min(src.t1 - tok0, kCT) * kRowB);
}

// FP8 latent caches (one E4M3 code per element: a 64-token page is 36864
// bytes, the size of a bf16 chunk).  Whole pages stream linearly into two
// staging slots (load j of a page: bytes 1024 j .. +1023, wave w issues
// j = w + 4i), two pages ahead; each step widens the 32 rows of its chunk
// (half a page) into the bf16 chunk layout above, so the score and value
// products run unchanged.  The page's record count bounds it: rows past the
// split's end read zeros.
constexpr int kPageB8 = 64 * kDqk;                   // 36864 bytes per FP8 page
static_assert(kPageB8 == kChunkB, "an FP8 page fills a chunk slot");
__device__ __forceinline__ i32x4 page8_rsrc(ChunkSource<kWideNW, 64>& src, int g) {
  const int tok0 = src.t0 + 64 * g;
  if (tok0 >= src.t1) return raw_rsrc(src.cbase, 0);
  const char* base = src.cbase + (size_t)src.page_of(2 * g) * kPageB8;
  return raw_rsrc(base, min(src.t1 - tok0, 64) * kDqk);
}
// Load k (0 .. 8) of this wave's share of a page into staging slot dst.
__device__ __forceinline__ void page8_issue(const i32x4& rsrc, lds_char* dst, int w, int lane,
                                            int k) {
  const int j = w + kWideNW * k;
  dma16_buf(rsrc, 1024 * j + 16 * lane, dst + 1024 * j);
}
__device__ __forceinline__ void page8_issue_all(const i32x4& rsrc, lds_char* dst, int w, int lane) {
#pragma unroll
  for (int k = 0; k < kDmaInst / kWideNW; ++k) page8_issue(rsrc, dst, w, lane, k);
}
// Widen rows 32h .. 32h+31 of a staged page into a bf16 chunk buffer: wave w
// takes the 8-byte pieces m = 64 j + lane (j = w + 4i) of the half, piece m
// being elements 8 (m % 72) .. +7 of row m / 72, i.e. 16-byte chunk m % 72
// of that bf16 row (stored at chunk ^ wide_key(row)).
__device__ __forceinline__ void widen_half(const lds_char* stg, int h, lds_char* dst, int w,
                                           int lane) {
  // addresses derived afresh each call (an opaque copy of the lane id), not
  // kept in registers across the chunk loop
  asm volatile("" : "+v"(lane));
#pragma unroll
  for (int i = 0; i < kDmaInst / kWideNW; ++i) {
    const int m = 64 * (w + kWideNW * i) + lane;
    const u32x2 c8 = *(const __attribute__((address_space(3))) u32x2*)(stg + 18432 * h + 8 * m);
    const int t = m / (kRowB / 16), c = m - t * (kRowB / 16);
    ds_store_b128(dst + t * kRowB + 16 * (c ^ wide_key(t)), fp8x8_to_bf16x8(c8[0], c8[1]));
  }
}

struct WideState {
  u32x4 qf[kWideKS];                  // Q^T B operands of heads 32w .. 32w+31
  f32x16 acc[kWideMB][kWideNB];       // O^T: dims 128w + 32mb .., heads 32nb ..
  float m, mtop, l;                   // reference max, largest chunk max (log2), lane's sum
  bool bad;
};

// Score MFMAs of chunk `buf` for heads 32w .. 32w+31 (S^T, 32 tokens x 32
// heads, one accumulation chain: a dependent MFMA with the same accumulator
// issues back to back).  issue(k) runs
// before k-step 4k (k < 9): this wave's loads of a later chunk go out between
// the MFMAs, so the matrix core stays busy while the load path accepts them.
// Lane pointers of the 16-byte operand reads of a buffer in the chunk layout:
// k-step kb of lane (r, hsel) is chunk 2kb + hsel of row r, which sits at
// chunk (2kb + hsel) ^ k (k = wide_key(r)), byte 16*(hsel ^ (k & 1)) +
// 32*((kb & 3) ^ (k >> 1)) + 128*(kb >> 2) of the row.  As a score A
// operand the row is a token; as a query B operand it is a head.
struct WideRowReads {
  const lds_char* pr[4];
  __device__ __forceinline__ WideRowReads(const lds_char* buf, int lane) {
    const int r = lane & 31, hsel = lane >> 5, k = wide_key(r);
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4)
      pr[m4] = buf + r * kRowB + 16 * (hsel ^ (k & 1)) + 32 * (m4 ^ (k >> 1));
  }
  __device__ __forceinline__ u32x4 operator()(int kb) const {
    return *(const lds_u32x4*)(pr[kb & 3] + 128 * (kb >> 2));
  }
};

template <typename Issue>
__device__ __forceinline__ void wide_score_mfma(const WideState& st, const lds_char* buf, int lane,
                                                f32x16& sc, const Issue& issue) {
  const WideRowReads load_a(buf, lane);
  constexpr int L = kWideLook;
  u32x4 ab[L + 1];
#pragma unroll
  for (int kb = 0; kb < L; ++kb) ab[kb] = load_a(kb);
#pragma unroll
  for (int kb = 0; kb < kWideKS; ++kb) {
    if ((kb & 3) == 0 && kb / 4 < kDmaInst / kWideNW) issue(kb / 4);
    // the buffer refilled here was consumed one step earlier
    if (kb + L < kWideKS) ab[(kb + L) % (L + 1)] = load_a(kb + L);
    const u32x4 a = ab[kb % (L + 1)];
    if (kb == 0) mfma32_v_first(sc, a, st.qf[kb]);
    else mfma32_v(sc, a, st.qf[kb]);
  }
  drain_scores32(sc);
}

// Softmax of one chunk, first part: the scores, masked past the split's end
// t1, and their max per head, with the overflow bookkeeping.  tok0: the
// chunk's first token.
__device__ __forceinline__ void wide_scores_max(WideState& st, const f32x16& sc,
                                                float (&v)[16], int lane, int tok0, int t1,
                                                float cs) {
  const int hsel = lane >> 5;
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = sc[i];
  // lane: head 32w + (lane & 31), tokens tok0 + 8g + 4*hsel + j in v[4g + j]
  const int tb = tok0 + 4 * hsel;
  if (tok0 + kCT > t1) {                             // only a split's last chunk runs past t1
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (tb + 8 * (i >> 2) + (i & 3) >= t1) v[i] = kNegInf;
  }
  float mx = v[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, v[i]);
  mx = max_xor32(mx) * cs;                           // log2 units, same in both lane halves
  st.mtop = fmaxf(st.mtop, mx);
  if (st.m == kNegInf) st.m = mx;                    // first chunk of the first pass
  st.bad |= mx > st.m + kHeadroom;
}

// Second part: the weights, their sum, and the probabilities to `pbuf`.
__device__ __forceinline__ void wide_weights(WideState& st, float (&v)[16], lds_char* pbuf, int w,
                                             int lane, float cs) {
  const int r = lane & 31, hsel = lane >> 5;
  float ls = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = fast_exp2(fmaf(v[i], cs, -st.m));
    ls += v[i];
  }
  st.l += ls;
  // tokens 8g + 4*hsel .. +3 of head 32w + r: 16-byte slot (4w + g)*32 + r
  // (head block w, k-step g/2, half g%2), bytes 8*hsel .. +7
  lds_char* pw = pbuf + (4 * w * 32 + r) * 16 + 8 * hsel;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    u32x2 pk;
    pk[0] = pack_bf16(v[4 * g], v[4 * g + 1]);
    pk[1] = pack_bf16(v[4 * g + 2], v[4 * g + 3]);
    ds_store_b64(pw + g * 32 * 16, pk);
  }
}

// Per-lane LDS byte offsets of the transposed V^T reads, relative to a
// chunk buffer.  The A operand of M-block mb (dims 128w + 32mb + (lane & 31))
// and k-step kb (tokens 16kb + 8*(lane >> 5) .. +7) is two reads, rows r0
// and r0 + 4 (r0 = 16kb + 8*(lane >> 5) + (lane & 15) / 4), each of a
// 4-token x 16-dim block per 16 lanes.  Its 16-byte chunk index within the
// row is 16w + 4mb + b2 (b2 in 0..3: dim half and lane), stored at that index
// XOR wide_key(row).  Bit 2 of the index is mb & 1 and rows r0 and r0 + 4 differ
// in bit 2 of the key, so every read address is one of two bases plus an
// immediate: 128*(mb >> 1) + 18432*kb (+ 4608 for the second row).
struct WideVaBase {
  int even, odd;   // bytes: chunk pattern (b2 ^ key) and (b2 ^ key ^ 4) on row r0
};
__device__ __forceinline__ WideVaBase wide_va_base(int w, int lane) {
  const int gq = lane >> 4, n = lane & 15;
  const int r0 = 8 * (gq >> 1) + (n >> 2);           // k-step 0
  const int bc = 2 * (16 * (gq & 1)) + (n & 3) * 8;  // byte column within the 64-byte M-block
  const int b2 = bc >> 4, lo = bc & 15;
  const int row = r0 * kRowB + 16 * 16 * w + lo;
  return WideVaBase{row + 16 * (b2 ^ wide_key(r0)), row + 16 * ((b2 ^ wide_key(r0)) ^ 4)};
}
__device__ __forceinline__ u32x4 wide_va(const lds_char* buf, const WideVaBase& vb, int mb, int kb) {
  const int imm = 128 * (mb >> 1) + 16 * kRowB * kb;
  const lds_char* lo = buf + ((mb & 1) ? vb.odd : vb.even) + imm;
  const lds_char* hi = buf + ((mb & 1) ? vb.even : vb.odd) + imm + 4 * kRowB;
  const u32x2 vlo = lds_tr16(lo), vhi = lds_tr16(hi);
  return u32x4{vlo[0], vlo[1], vhi[0], vhi[1]};
}

// Value product of one chunk: dims 128w .. 128w+127 of all 128 heads.
__device__ __forceinline__ void wide_values(WideState& st, const lds_char* buf, const lds_char* pbuf,
                                            const WideVaBase& vb, int lane) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    u32x4 b[kWideNB];
#pragma unroll
    for (int nb = 0; nb < kWideNB; ++nb)
      b[nb] = *(const lds_u32x4*)(pbuf + (nb * 4 + kb * 2) * 512 + lane * 16);
    u32x4 a[2];
    a[0] = wide_va(buf, vb, 0, kb);
#pragma unroll
    for (int mb = 0; mb < kWideMB; ++mb) {
      if (mb + 1 < kWideMB) a[(mb + 1) & 1] = wide_va(buf, vb, mb + 1, kb);
#pragma unroll
      for (int nb = 0; nb < kWideNB; ++nb) mfma32_a(st.acc[mb][nb], a[mb & 1], b[nb]);
    }
  }
}

// F8: FP8 E4M3 latent cache (two bf16 chunk slots plus two FP8 page slots in
// the same LDS; see page8_issue and widen_half).
template <bool F8>
__global__ __launch_bounds__(kWideNW * 64) void mla_wide_partial(Params p) {
  __shared__ __attribute__((aligned(16))) char ring_lds[kRing * kChunkB];
  __shared__ __attribute__((aligned(16))) char pl_lds[2 * kWidePB];

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
  constexpr int kNwi = kDmaInst / kWideNW;            // this wave's loads per chunk

  lds_char* const ring = (lds_char*)ring_lds;
  lds_char* const pl = (lds_char*)pl_lds;
  constexpr int kSlots = F8 ? 2 : kRing;              // bf16 chunk slots
  auto slot = [&](int ci) { return ring + (ci % kSlots) * kChunkB; };
  auto stg = [&](int g) { return ring + (2 + (g & 1)) * kChunkB; };   // FP8 page slots
  auto pbuf = [&](int ci) { return pl + (ci & 1) * kWidePB; };
  ChunkSource<kWideNW, 64> src;
  src.bt = p.block_table + (size_t)b * p.maxb;
  src.cbase = static_cast<const char*>(p.k);
  src.t0 = t0;
  src.t1 = t1;
  src.p1 = p1;
  src.nblocks = p.nblocks;
  src.w = w;
  src.lane = lane;
  WideLoads ld;
  ld.init(w, lane);
  WideState st;
  const WideVaBase vb = wide_va_base(w, lane);
  const size_t row0 = (size_t)b * p.ql * p.Hq + head0;
  {
    // The queries of the 128 heads (rows of 1152 bytes, like latent rows)
    // come through the ring, 32 heads to a slot in the chunk layout, with the
    // chunk loads (contiguous 1 KiB per load); wave w then reads the B
    // operands of heads 32w .. 32w+31 from slot w: k-step kb of lane
    // (r, hsel) is dims 16kb + 8*hsel .. +7 of head 32w + r.  Loaded from
    // global memory straight into these registers, every load would touch
    // 32 rows with 32 bytes each.
    const char* qb = static_cast<const char*>(p.q) + row0 * kRowB;
#pragma unroll
    for (int i = 0; i < kRing; ++i)
      ld.issue_all(raw_rsrc(qb + i * kChunkB, kChunkB), ring + i * kChunkB);
    wait_vm<0>();
    lds_barrier();
    const WideRowReads load_q(ring + w * kChunkB, lane);
#pragma unroll
    for (int kb = 0; kb < kWideKS; ++kb) st.qf[kb] = load_q(kb);
    lds_barrier();                                    // every wave holds its queries
  }
  // Every chunk is loaded, also past the split's end (those loads write
  // zeros), so the count in flight is the same at every step.
  auto issue_first_two = [&]() {
    src.begin(s * p.c);
    if constexpr (F8) {
      page8_issue_all(page8_rsrc(src, 0), stg(0), w, lane);
      page8_issue_all(page8_rsrc(src, 1), stg(1), w, lane);
    } else {
      ld.issue_all(wide_rsrc(src, 0), slot(0));
      ld.issue_all(wide_rsrc(src, 1), slot(1));
    }
  };
  issue_first_two();
  st.m = kNegInf;
  st.mtop = kNegInf;
  for (bool first = true;; first = false) {
    st.l = 0.f;
#pragma unroll
    for (int mb = 0; mb < kWideMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kWideNB; ++nb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) st.acc[mb][nb][i] = 0.f;
      }
    st.bad = false;
    if (!first) issue_first_two();
    if constexpr (F8) {
      // Page g (chunks 2g, 2g+1) is issued at step 2g - 3 into FP8 slot
      // g % 2, freed when step 2g - 1 has widened its second half; step ci
      // widens its chunk into bf16 slot ci % 2, whose last reader was the
      // value product of ci - 2 (step ci - 1), between two barriers.
      auto widen = [&](int ci) {
        if ((ci & 1) == 0) wait_vm<kNwi>();           // page ci / 2 (the next one may be in flight)
        lds_barrier();
        widen_half(stg(ci >> 1), ci & 1, slot(ci), w, lane);
        lds_barrier();
        if (ci & 1) page8_issue_all(page8_rsrc(src, (ci + 3) >> 1), stg((ci + 3) >> 1), w, lane);
      };
      if (nchunks > 0) {
        widen(0);
        f32x16 sc;
        wide_score_mfma(st, slot(0), lane, sc, [&](int) {});
        float v[16];
        wide_scores_max(st, sc, v, lane, t0, t1, cs);
        wide_weights(st, v, pbuf(0), w, lane, cs);
      }
      for (int ci = 1; ci < nchunks; ++ci) {
        widen(ci);
        f32x16 sc;
        wide_score_mfma(st, slot(ci), lane, sc, [&](int) {});
        float v[16];
        wide_scores_max(st, sc, v, lane, t0 + ci * kCT, t1, cs);
        wide_values(st, slot(ci - 1), pbuf(ci - 1), vb, lane);
        wide_weights(st, v, pbuf(ci), w, lane, cs);
      }
    } else {
    wait_vm<kNwi>();                                  // chunk 0 (chunk 1 may be in flight)
    lds_barrier();
    if (nchunks > 0) {
      ld.refresh();
      const i32x4 rs = wide_rsrc(src, 2);
      f32x16 sc;
      wide_score_mfma(st, slot(0), lane, sc, [&](int k) { ld.issue(rs, slot(2), k); });
      float v[16];
      wide_scores_max(st, sc, v, lane, t0, t1, cs);
      wide_weights(st, v, pbuf(0), w, lane, cs);
    }
    for (int ci = 1; ci < nchunks; ++ci) {
      // chunk ci has landed (this wave's loads, then, after the barrier,
      // every wave's); the probabilities of ci - 1 are complete; the value
      // product of ci - 2 is done, so its slot and probability buffer are free
      wait_vm<kNwi>();
      lds_barrier();
      // scores of ci (with the loads of ci + 2 between them) and their max,
      // the value product of ci - 1 (independent of them), then the weights
      // of ci, which the compiler can interleave with that value product
      // (chunks past the split's end are loaded too, as zeros: every step
      // issues the same loads, so the wait counts above hold)
      ld.refresh();
      const i32x4 rs = wide_rsrc(src, ci + 2);
      f32x16 sc;
      wide_score_mfma(st, slot(ci), lane, sc, [&](int k) { ld.issue(rs, slot(ci + 2), k); });
      float v[16];
      wide_scores_max(st, sc, v, lane, t0 + ci * kCT, t1, cs);
      wide_values(st, slot(ci - 1), pbuf(ci - 1), vb, lane);
      wide_weights(st, v, pbuf(ci), w, lane, cs);
    }
    }
    if (nchunks > 0) {
      lds_barrier();                                  // the last chunk's probabilities
      wide_values(st, slot(nchunks - 1), pbuf(nchunks - 1), vb, lane);
    }
    // Did any head's chunk max overflow the headroom over its reference max?
    wait_vm<0>();                                     // the loads past the split's end
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

  // Per-head statistics go to the probability buffers (free now); the
  // normalised outputs of all 128 heads are staged in the ring as bfloat16
  // rows and then written with contiguous 16-byte stores, one 1 KiB row per
  // store instruction.  Written from the accumulators directly, every store
  // instruction would scatter 16-byte pieces over 32 rows.
  float* stat_m = (float*)pl_lds;
  float* stat_l = stat_m + kWideNH;
  // The epilogue derives its lane values afresh (an opaque copy of the lane
  // id), so the compiler keeps nothing from the prologue alive across the
  // loop for them.
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));
  const int re = lane_e & 31, he = lane_e >> 5;
  {
    const float lt = st.l + __shfl_xor(st.l, 32, 64);
    if (he == 0) {
      stat_m[kWideHW * w + re] = st.m;
      stat_l[kWideHW * w + re] = lt;
    }
  }
  lds_barrier();
  char* const tile = ring_lds;
#pragma unroll
  for (int nb = 0; nb < kWideNB; ++nb) {
    const int h = 32 * nb + re;
    const float mm = stat_m[h];
    // (v_scale: the factor of every FP8 value, 1 for bf16 caches)
    const float inv = (mm == kNegInf) ? 0.f : p.v_scale / stat_l[h];
#pragma unroll
    for (int mb = 0; mb < kWideMB; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // dims 128w + 32mb + 8g + 4*hsel .. +3 of head h
        const int d = kWideDW * w + 32 * mb + 8 * g + 4 * he;
        const f32x16& a = st.acc[mb][nb];
        u32x2 pk;
        pk[0] = pack_bf16(a[4 * g] * inv, a[4 * g + 1] * inv);
        pk[1] = pack_bf16(a[4 * g + 2] * inv, a[4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(tile + h * kWideOutRowB + 2 * d) = pk;
      }
    }
  }
  lds_barrier();
  // wave w writes the rows of heads 32w .. 32w+31: the output, or this
  // split's partial (bfloat16 either way)
#pragma unroll
  for (int i = 0; i < kWideHW; i += 8) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = *reinterpret_cast<const u32x4*>(tile + (kWideHW * w + i + j) * kWideOutRowB +
                                             16 * lane_e);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t row = row0 + kWideHW * w + i + j;
      uint16_t* dst = p.final_write ? static_cast<uint16_t*>(p.out) + row * kDv
                                    : p.o_part16 + (row * p.S + s) * kDv;
      *reinterpret_cast<u32x4*>(dst + 8 * lane_e) = v[j];
    }
  }
  if (he == 0) {
    const int h = kWideHW * w + re;
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

template <bool F8>
hipError_t launch_wide(const Params& p, hipStream_t st) {
  const long blocks = (long)(p.ql * p.Hq / kWideNH) * p.S * p.B;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_wide_partial<F8>, dim3((unsigned)blocks), dim3(kWideNW * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace

bool mla_mfma_supported(bool bf16, int Dqk, int Dv, int bs, int Hq) {
  return bf16 && Dqk == kDqk && Dv == kDv && (bs == 64 || bs == 1) &&
         (Hq % 64 == 0 || Hq == 32 || Hq == 16);
}

bool mla_mfma_fp8_supported(int Dqk, int Dv, int bs, int Hq) {
  return mla_mfma_supported(true, Dqk, Dv, bs, Hq);
}

int mla_heads_per_workgroup(int Hq, int bs) {
  if (bs == 64 && Hq % kWideNH == 0) return kWideNH;
  return Hq % 64 == 0 ? 64 : Hq;
}

int mla_max_split_tokens(int bs) { return bs == 1 ? kMaxIdsBS1 : 0x7fffffff; }

hipError_t launch_mla_mfma(const Params& p, bool fp8kv, hipStream_t st) {
  if (p.bs == 64 && p.Hq % kWideNH == 0)
    return fp8kv ? launch_wide<true>(p, st) : launch_wide<false>(p, st);
  if (p.Hq % 64 == 0) return launch_roles<2, 2>(p, fp8kv, st);
  if (p.Hq == 32) return launch_roles<2, 1>(p, fp8kv, st);
  if (p.Hq == 16) return launch_roles<1, 1>(p, fp8kv, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
