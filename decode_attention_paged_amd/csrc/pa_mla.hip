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
// LDS chunk rows are 1152 bytes (72 chunks of 16 bytes).  Chunk c of token
// row t sits at position c ^ (t & 7); with it the score reads (16 rows, one
// chunk each) and the transposed value reads run at the conflict-free rate
// (measured against a linear read of the same size).  The probabilities are
// stored so that the value product's B-operand read is linear: for head block
// nb, the 16-byte slot q*16 + n holds tokens 8q .. 8q+7 of head 16 nb + n.
#include <type_traits>

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
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) float lds_float;

// 16 zero bytes in global memory: the load source for token slots past the
// context, so no NaN or stale data reaches the value product.
__device__ __attribute__((aligned(16))) uint32_t g_zero16[4] = {0u, 0u, 0u, 0u};


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
// Value products accumulate in AGPRs (asm too, so the accumulators are
// pinned there whatever the wave's register budget).  Same padding rules.
__device__ __forceinline__ void mfma_a(f32x4& d, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
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
__device__ __forceinline__ int row_key(int t) { return t & 7; }

constexpr float kHeadroom = 16.0f;   // log2 units a chunk's max may exceed the reference max
constexpr int kRing = 4;             // chunk slots: value product, scores, two loads in flight

template <int NW, int HB>
struct MlaCfg {
  static constexpr int NH = 16 * HB * NW;            // heads per workgroup
  static constexpr int NB = NH / 16;                 // head blocks (value N-blocks)
  static constexpr int DW = kDv / NW;                // value dims per wave
  static constexpr int MB = DW / 16;                 // value M-blocks per wave
  static constexpr int NWI = kDmaInst / NW;          // direct-to-LDS loads per wave per chunk
  static constexpr int LOOK = 2;                     // score operand loads ahead of their MFMAs
  static_assert(kDmaInst % NW == 0, "uniform load share");
  static_assert(HB == 1 || HB == 2, "head blocks per wave");
};

// Probabilities of two consecutive chunks (written for chunk i while the
// value product of chunk i - 1 reads the other buffer).
template <int NW, int HB>
struct MlaLds {
  uint16_t p[2][MlaCfg<NW, HB>::NH * kCT];
};

constexpr int kMaxIdsBS1 = 2048;   // token ids of one split held in LDS (one-token pages)

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
  // Page id of chunk ci; reloads the id window when the chunk leaves it
  // (every 128 chunks at most; that reload waits for the loads in flight).
  __device__ __forceinline__ int page_of(int ci) {
    const int pg = (t0 + ci * kCT) / 64;
    if (pg >= base + 64) load_window(pg);
    return __builtin_amdgcn_readlane(v, pg - base);
  }
  // Issue this wave's share (kDmaInst / NW loads of 1 KiB) of chunk ci into dst.
  __device__ __forceinline__ void issue(lds_char* dst, int ci) {
    const int tok0 = t0 + ci * kCT;
    const char* src = cbase + (size_t)page_of(ci) * (64 * kRowB) + (tok0 % 64) * kRowB;
    const int lim = (t1 - tok0) * kRowB;             // bytes of the chunk inside the split
    int ln = lane;
    // recompute the per-lane offsets at every issue rather than keep them in
    // registers across the loop (a few VALU ops against ~18 VGPRs)
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < kDmaInst / NW; ++k) {
      const int j = w + NW * k;
      const int slot = j * 64 + ln;                  // 16-byte slot of the chunk buffer
      const int t = slot / (kRowB / 16);
      const int c = (slot % (kRowB / 16)) ^ row_key(t);
      const int off = t * kRowB + c * 16;
      const void* g = off < lim ? (const void*)(src + off) : (const void*)g_zero16;
      dma16(g, dst + j * 1024);
    }
  }
};

template <int NW>
struct ChunkSource<NW, 1> {
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
    for (int i = threadIdx.x; i < n; i += NW * 64) ids[i] = clampi(bt[t0 + i], 0, nblocks - 1);
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

template <int NW, int HB>
struct MlaState {
  u32x4 qf[HB][kKSteps];                              // Q^T B operands
  f32x4 acc[MlaCfg<NW, HB>::MB][MlaCfg<NW, HB>::NB];  // O^T, dims x heads
  float m[HB];                                        // reference max per score head (log2)
  float mtop[HB];                                     // largest chunk max seen (log2)
  float l[HB];                                        // this lane's share of the sum
  bool bad;                                           // a chunk max overflowed the headroom
};

// Scores of one chunk: S^T for this wave's 16*HB heads, 32 tokens.
template <int NW, int HB>
__device__ __forceinline__ void chunk_scores(const lds_char* buf, const MlaState<NW, HB>& st,
                                             f32x4 (&sa)[HB][2], int lane) {
  using C = MlaCfg<NW, HB>;
  const int quad = lane >> 4, n = lane & 15;
  // Row n (and 16 + n), 16-byte chunk kb*4 + quad: with the swizzle its byte
  // offset is n*kRowB + 16*(quad ^ (n & 3)) + 64*(kb ^ ((n >> 2) & 1)), i.e.
  // one per-lane base for even and one for odd k-steps plus 64*kb.
  const int xb = (n >> 2) & 1;
  const int sbase = n * kRowB + 16 * (quad ^ (n & 3));
  const lds_char* se = buf + sbase + 64 * xb;
  const lds_char* so = buf + sbase - 64 * xb;
  auto load_a = [&](int kb, u32x4& x0, u32x4& x1) {
    const lds_char* rp = ((kb & 1) ? so : se) + 64 * kb;
    x0 = *(const lds_u32x4*)rp;
    x1 = *(const lds_u32x4*)(rp + 16 * kRowB);               // row 16 + n: same swizzle
  };
  constexpr int L = C::LOOK;
  u32x4 ab[L + 1][2];
#pragma unroll
  for (int kb = 0; kb < L; ++kb) load_a(kb, ab[kb][0], ab[kb][1]);
#pragma unroll
  for (int kb = 0; kb < kKSteps; ++kb) {
    if (kb + L < kKSteps) load_a(kb + L, ab[(kb + L) % (L + 1)][0], ab[(kb + L) % (L + 1)][1]);
    const u32x4 a0 = ab[kb % (L + 1)][0], a1 = ab[kb % (L + 1)][1];
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
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E - 1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Softmax of one head block of a chunk, in four stages so that the caller can
// spread them between value-product MFMAs.  Stage 0: mask and the lane's max;
// 1: the head's max, reference max and overflow check; 2: weights and sum (in
// place); 3: probabilities to LDS ([head block][token / 8][head % 16] 16-byte
// slots, which the value product reads linearly).
struct SoftmaxRow {
  float v[8];   // scores, then weights
  float mx;
};

template <int NW, int HB, int STAGE>
__device__ __forceinline__ void softmax_stage(SoftmaxRow& r, const f32x4 (&sa)[2],
                                              MlaState<NW, HB>& st, int hb, int tbase, int tend,
                                              float cs, lds_char* pbuf, int w, int lane) {
  const int quad = lane >> 4, n = lane & 15;
  if constexpr (STAGE == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.v[j] = sa[0][j];
      r.v[4 + j] = sa[1][j];
    }
    if (tbase + kCT > tend) {                         // only a split's last chunk runs past its end
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (tbase + quad * 4 + j >= tend) r.v[j] = kNegInf;
        if (tbase + 16 + quad * 4 + j >= tend) r.v[4 + j] = kNegInf;
      }
    }
    r.mx = fmaxf(fmaxf(fmaxf(r.v[0], r.v[1]), fmaxf(r.v[2], r.v[3])),
                 fmaxf(fmaxf(r.v[4], r.v[5]), fmaxf(r.v[6], r.v[7])));
  } else if constexpr (STAGE == 1) {
    const float mx = max_xor32(max_xor16(r.mx)) * cs;    // same in the 4 quads; log2 units
    st.mtop[hb] = fmaxf(st.mtop[hb], mx);
    if (st.m[hb] == kNegInf) st.m[hb] = mx;          // first chunk of the first pass
    st.bad |= mx > st.m[hb] + kHeadroom;
  } else if constexpr (STAGE == 2) {
    const float mn = st.m[hb];
#pragma unroll
    for (int j = 0; j < 8; ++j) r.v[j] = fast_exp2(fmaf(r.v[j], cs, -mn));
    st.l[hb] += ((r.v[0] + r.v[1]) + (r.v[2] + r.v[3])) + ((r.v[4] + r.v[5]) + (r.v[6] + r.v[7]));
  } else {
    lds_char* prow = pbuf + (HB * w + hb) * (16 * kCT * 2) + n * 16;
    u32x2 v0, v1;
    v0[0] = pack_bf16(r.v[0], r.v[1]);
    v0[1] = pack_bf16(r.v[2], r.v[3]);
    v1[0] = pack_bf16(r.v[4], r.v[5]);
    v1[1] = pack_bf16(r.v[6], r.v[7]);
    ds_store_b64(prow + 256 * (quad >> 1) + 8 * (quad & 1), v0);        // tokens quad*4 .. +3
    ds_store_b64(prow + 256 * (2 + (quad >> 1)) + 8 * (quad & 1), v1);  // tokens 16 + quad*4 ..
  }
}

// The value product for dims DW*w .. DW*w + DW - 1 of every head.  A operand
// (V^T): tokens quad*8 .. +7 of one dim per lane, two transposed reads; B
// operand (P^T): one 16-byte slot.
template <int NW, int HB>
struct ValueOps {
  const lds_char* buf;
  const lds_char* pbuf;
  int w, n, quad;
  __device__ __forceinline__ u32x4 va(int mb) const {
    const int bc = (MlaCfg<NW, HB>::DW * w + mb * 16) * 2 + (n & 3) * 8;   // byte column
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

// The value product runs in groups of at most 4 B operands (head blocks) by
// every M-block, A operands two deep; with PV false only the softmax runs.
// The softmax stages of this chunk go between the MFMA groups of the previous
// chunk's value product, so one wave keeps both the MFMA pipe and the VALU
// busy.
template <int NW, int HB, bool PV>
__device__ __forceinline__ void values_and_softmax(MlaState<NW, HB>& st, const ValueOps<NW, HB>& vo,
                                                   const f32x4 (&sa)[HB][2], int tbase, int tend,
                                                   float cs, lds_char* pbuf, int w, int lane) {
  using C = MlaCfg<NW, HB>;
  constexpr int NBG = C::NB < 4 ? C::NB : 4;          // head blocks per group
  constexpr int NHALF = C::NB / NBG;                  // passes over the M-blocks
  constexpr int G = NHALF * C::MB;                    // MFMA groups
  constexpr int STAGES = 4 * HB;
  static_assert(C::NB % NBG == 0, "head block groups");
  SoftmaxRow row;
  auto stage = [&](auto kc) {
    constexpr int k = decltype(kc)::value;
    softmax_stage<NW, HB, k % 4>(row, sa[k / 4], st, k / 4, tbase, tend, cs, pbuf, w, lane);
  };
  if constexpr (!PV) {
    static_for<0, STAGES>(stage);
  } else {
    u32x4 pb[NBG];
    u32x4 va[2];
    static_for<0, G>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      constexpr int h = g / C::MB, mb = g % C::MB;
      if constexpr (mb == 0) {
#pragma unroll
        for (int i = 0; i < NBG; ++i) pb[i] = vo.pb(h * NBG + i);
        va[0] = vo.va(0);
      }
      if constexpr (mb + 1 < C::MB) va[(mb + 1) & 1] = vo.va(mb + 1);
#pragma unroll
      for (int i = 0; i < NBG; ++i) mfma_a(st.acc[mb][h * NBG + i], va[mb & 1], pb[i]);
      // softmax stage k after group (k * G) / STAGES
      static_for<0, STAGES>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr ((k * G) / STAGES == g) stage(kc);
      });
    });
  }
}

// Value product alone (the split's last chunk).
template <int NW, int HB>
__device__ __forceinline__ void values_only(MlaState<NW, HB>& st, const ValueOps<NW, HB>& vo) {
  using C = MlaCfg<NW, HB>;
  constexpr int NBG = C::NB < 4 ? C::NB : 4;
  constexpr int G = (C::NB / NBG) * C::MB;
  u32x4 pb[NBG];
  u32x4 va[2];
  static_for<0, G>([&](auto gc) {
    constexpr int g = decltype(gc)::value;
    constexpr int h = g / C::MB, mb = g % C::MB;
    if constexpr (mb == 0) {
#pragma unroll
      for (int i = 0; i < NBG; ++i) pb[i] = vo.pb(h * NBG + i);
      va[0] = vo.va(0);
    }
    if constexpr (mb + 1 < C::MB) va[(mb + 1) & 1] = vo.va(mb + 1);
#pragma unroll
    for (int i = 0; i < NBG; ++i) mfma_a(st.acc[mb][h * NBG + i], va[mb & 1], pb[i]);
  });
}

template <int NW, int HB, int BS>
__global__ __launch_bounds__(NW * 64) void mla_mfma_partial(Params p) {
  using C = MlaCfg<NW, HB>;
  __shared__ __attribute__((aligned(16))) char ring_lds[kRing * kChunkB];
  __shared__ __attribute__((aligned(16))) MlaLds<NW, HB> sm;
  __shared__ int ids_lds[BS == 1 ? kMaxIdsBS1 : 1];
  lds_char* const ring = (lds_char*)ring_lds;

  // 1-D grid of HG x S x B workgroups.  With two head groups, the two
  // workgroups of one (sequence, split) are 8 apart in dispatch order: the
  // same XCD (workgroups go round-robin to the 8 XCDs) at about the same time,
  // so the second reads the latent rows from that XCD's L2.
  const int HG = p.Hq / C::NH;
  int hg, u;
  const int L = blockIdx.x, g16 = L >> 4;
  if (HG == 2 && (g16 + 1) * 16 <= (int)gridDim.x) {
    hg = (L >> 3) & 1;
    u = (g16 << 3) | (L & 7);
  } else if (HG == 2) {                               // last, partial group of 16
    const int r = L - (g16 << 4);
    hg = r & 1;
    u = (g16 << 3) + (r >> 1);
  } else {
    hg = L % HG;
    u = L / HG;
  }
  const int b = u / p.S;
  const int s = split_of_block(u % p.S, b, p.S);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quad = lane >> 4, n = lane & 15;
  const int head0 = hg * C::NH;
  const int ctx = clampi(p.context_lens[b], 0, p.max_ctx);
  const int pages = (ctx + BS - 1) / BS;
  const int nsplit = splits_of(pages, p.c);
  if (s >= (nsplit > 0 ? nsplit : 1)) return;
  const int t0 = s * p.c * BS;
  const int t1 = min(ctx, (s * p.c + p.c) * BS);
  const int p1 = min(pages, s * p.c + p.c);
  const int nchunks = t1 > t0 ? (t1 - t0 + kCT - 1) / kCT : 0;
  const float cs = p.scale_log2;                      // > 0, checked by the host

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

  const int* bt = p.block_table + (size_t)b * p.maxb;
  const char* cbase = static_cast<const char*>(p.k);
  auto slot = [&](int ci) { return ring + (ci % kRing) * kChunkB; };
  auto pslot = [&](int ci) { return (lds_char*)sm.p[ci & 1]; };
  ChunkSource<NW, BS> src;
  src.bt = bt;
  src.cbase = cbase;
  src.t0 = t0;
  src.t1 = t1;
  src.p1 = p1;
  src.nblocks = p.nblocks;
  src.w = w;
  src.lane = lane;
  if constexpr (BS == 1) src.ids = ids_lds;
  for (;;) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) st.l[hb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) st.acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.bad = false;
    src.begin(s * p.c);
    // The first two chunks are issued even past the split's end (those loads
    // read the zero block), so the count in flight is known here and one wait
    // retires the query loads, which are older: no wait inside the loop has to
    // allow for them.
    src.issue(slot(0), 0);
    src.issue(slot(1), 1);
    constexpr int kInit = 2 * C::NWI;
    wait_vm<kInit <= 63 ? kInit : 0>();

    for (int ci = 0; ci < nchunks; ++ci) {
      // chunk ci has landed (this wave's loads, then, after the barrier,
      // every wave's); the probabilities of ci - 1 are complete; the value
      // product of ci - 2 is done, so its slot can be refilled
      if (ci + 1 < max(nchunks, 2)) wait_vm<C::NWI>(); else wait_vm<0>();
      lds_barrier();
      if (ci + 2 < nchunks) src.issue(slot(ci + 2), ci + 2);
      f32x4 sa[HB][2];
      chunk_scores<NW, HB>(slot(ci), st, sa, lane);
      const ValueOps<NW, HB> vo{slot(ci + kRing - 1), pslot(ci + 1), w, n, quad};
      if (ci > 0)
        values_and_softmax<NW, HB, true>(st, vo, sa, t0 + ci * kCT, t1, cs, pslot(ci), w, lane);
      else
        values_and_softmax<NW, HB, false>(st, vo, sa, t0 + ci * kCT, t1, cs, pslot(ci), w, lane);
    }
    if (nchunks > 0) {
      lds_barrier();                                  // the last chunk's probabilities
      const ValueOps<NW, HB> vo{slot(nchunks - 1), pslot(nchunks - 1), w, n, quad};
      values_only<NW, HB>(st, vo);
    }
    // Did any head's chunk max overflow the headroom over its reference max?
    // Every wave votes through LDS (the ring's first bytes: every load has
    // landed and every read of the ring is done after the barrier).
    wait_vm<0>();                                     // loads issued past the end of a short split
    lds_barrier();
    int* votes = (int*)ring_lds;
    if (lane == 0) votes[w] = __builtin_amdgcn_ballot_w64(st.bad) != 0;
    lds_barrier();
    int any = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) any |= votes[i];
    lds_barrier();                                    // votes read before the ring is refilled
    if (__builtin_amdgcn_readfirstlane(any) == 0) break;
    // Start over with every head's reference max raised to its largest chunk
    // max: no chunk can overflow then, so this happens at most once.
    st.m[0] = st.mtop[0];
    if constexpr (HB == 2) st.m[1] = st.mtop[1];
  }
  // the accumulators are read by VALU below: cover the last MFMA's latency
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // ---- finish: per-head statistics to every wave (in the ring's LDS, free
  // now), normalise, write
  float* stat_m = (float*)ring_lds;
  float* stat_l = stat_m + C::NH;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const float lt = sum_xor32(sum_xor16(st.l[hb]));
    if (quad == 0) {
      const int head = 16 * (HB * w + hb) + n;
      stat_m[head] = st.m[hb];
      stat_l[head] = lt;
    }
  }
  lds_barrier();
  const size_t row0 = (size_t)b * p.Hq + head0;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    const float mm = stat_m[nb * 16 + n];
    const float lt = stat_l[nb * 16 + n];
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
      const float mm = stat_m[head];
      const float lt = stat_l[head];
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
  const long blocks = (long)(p.Hq / MlaCfg<NW, HB>::NH) * p.S * p.B;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  if (p.bs == 1)
    hipLaunchKernelGGL((mla_mfma_partial<NW, HB, 1>), dim3((unsigned)blocks), dim3(NW * 64), 0, st,
                       p);
  else
    hipLaunchKernelGGL((mla_mfma_partial<NW, HB, 64>), dim3((unsigned)blocks), dim3(NW * 64), 0, st,
                       p);
  return hipGetLastError();
}

}  // namespace

bool mla_mfma_supported(bool bf16, int Dqk, int Dv, int bs, int Hq) {
  return bf16 && Dqk == kDqk && Dv == kDv && (bs == 64 || bs == 1) &&
         (Hq % 64 == 0 || Hq == 32 || Hq == 16);
}

int mla_heads_per_workgroup(int Hq) { return Hq % 64 == 0 ? 64 : Hq; }

int mla_max_split_tokens(int bs) { return bs == 1 ? kMaxIdsBS1 : 0x7fffffff; }

hipError_t launch_mla_mfma(const Params& p, hipStream_t st) {
  if (p.Hq % 64 == 0) return launch_cfg<4, 1>(p, st);
  if (p.Hq == 32) return launch_cfg<2, 1>(p, st);
  if (p.Hq == 16) return launch_cfg<1, 1>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
