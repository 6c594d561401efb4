// C ABI of libpa_decode: argument checks, the split plan, dispatch.
#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/pa_decode.h"
#include "pa_launch.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;
constexpr int kMaxSplits = 65535;          // grid y limit
constexpr long kFusedMergeBytes = 4 * 1024;   // largest per-unit partial set merged in-kernel
constexpr double kSplitBytesValu = 128.0 * 1024.0;   // KV bytes per workgroup, VALU kernel
constexpr double kSplitBytesMfma = 1024.0 * 1024.0;  // KV bytes per workgroup, MFMA kernel
constexpr int kMinSplitsLong = 8;                    // splits of the longest sequence (MFMA kernel, full grid)
constexpr double kShortUnitBytes = 4.0 * 1024 * 1024;  // longest unit (KV bytes) that is only halved
constexpr int kSchedSplitsLong = 10;                 // the same when the units run longest first
constexpr int kSchedSplitsMany = 3;                  // ... and the batch alone fills every slot twice
constexpr double kManyUnitBytes = 512.0 * 1024.0;    // smallest split of such a batch (KV bytes)
constexpr int kValuSplitsMany = 4;                   // longest sequence, VALU kernel, slots filled twice
constexpr double kScheduleUnitBytes = 384.0 * 1024.0;  // smallest unit (KV bytes) run longest first
constexpr double kMinSplitBytesValu = 32.0 * 1024.0;  // fewest KV bytes per workgroup, VALU kernel
constexpr double kMinSplitBytesMfma = 64.0 * 1024.0;  // fewest KV bytes per workgroup, MFMA kernel
constexpr int kMaxQLen = 16;                         // query rows per sequence
// Longest context: token indices, split ends ((s + 1) * c * bs) and page
// counts stay in int32 arithmetic inside the kernels.
constexpr int32_t kMaxContext = 1 << 29;

// Query rows per sequence (0 and 1 both mean one row).
int rows_of(const pa_shape& s) { return s.q_len > 1 ? s.q_len : 1; }

// Whether the caches hold FP8 E4M3 codes (kv_dtype 0 means the query dtype).
bool fp8_kv(const pa_shape& s) { return s.kv_dtype == PA_FP8_E4M3; }

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

enum class Kernel { None, MhaValu, GqaMfma, MlaMfma };

// Which partial kernel serves this shape (host-only, no HIP calls).
Kernel pick_kernel(const pa_shape& s, bool mla) {
  const bool bf16 = s.dtype == PA_BF16;
  if (mla) {
    if (fp8_kv(s))
      return bf16 && pa::mla_mfma_fp8_supported(s.head_dim, s.head_dim_v, s.block_size, s.num_q_heads)
                 ? Kernel::MlaMfma
                 : Kernel::None;
    return pa::mla_mfma_supported(bf16, s.head_dim, s.head_dim_v, s.block_size, s.num_q_heads)
               ? Kernel::MlaMfma
               : Kernel::None;
  }
  if (s.head_dim_v != s.head_dim) return Kernel::None;
  const int G = s.num_q_heads / s.num_kv_heads;
  const int ql = rows_of(s);
  if (fp8_kv(s)) {
    if (!bf16) return Kernel::None;
    if (pa::gqa_mfma_fp8_supported(s.head_dim, s.block_size, G, ql)) return Kernel::GqaMfma;
    if (ql == 1 && pa::mha_valu_fp8_supported(s.head_dim, s.block_size)) return Kernel::MhaValu;
    return Kernel::None;
  }
  if (pa::gqa_mfma_supported(bf16, s.head_dim, s.head_dim_v, s.block_size, G, ql))
    return Kernel::GqaMfma;
  if (ql == 1 && pa::mha_valu_supported(bf16, s.head_dim, s.block_size)) return Kernel::MhaValu;
  return Kernel::None;
}

// Shape checks that need no pointers (host-only).
pa_status check_shape(const pa_shape* s, bool mla) {
  if (!s) return PA_ERR_INVALID;
  if (s->batch > 65535) return PA_ERR_UNSUPPORTED;   // grid z limit
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->head_dim < 1 ||
      s->head_dim_v < 1 || s->block_size < 1 || s->max_blocks_per_seq < 1 || s->num_blocks < 1 ||
      s->max_context_len < 0)
    return PA_ERR_INVALID;
  if (s->num_q_heads % s->num_kv_heads != 0) return PA_ERR_INVALID;
  if (s->q_len < 0) return PA_ERR_INVALID;
  if (s->kv_dtype != 0 && s->kv_dtype != s->dtype && s->kv_dtype != PA_FP8_E4M3)
    return PA_ERR_INVALID;
  if (fp8_kv(*s) && (!std::isfinite(s->k_scale) || !(s->k_scale > 0.f) ||
                     !std::isfinite(s->v_scale) || !(s->v_scale > 0.f)))
    return PA_ERR_INVALID;
  if (s->q_len > kMaxQLen) return PA_ERR_UNSUPPORTED;
  if ((int64_t)s->max_context_len > (int64_t)s->max_blocks_per_seq * s->block_size)
    return PA_ERR_INVALID;
  if (s->max_context_len > kMaxContext) return PA_ERR_UNSUPPORTED;
  // rows (sequence, query row, head) are counted in int32 (grids, row indices)
  if ((int64_t)s->batch * (s->q_len > 1 ? s->q_len : 1) * s->num_q_heads > 0x7fffffffLL)
    return PA_ERR_UNSUPPORTED;
  if (s->dtype != PA_F32 && s->dtype != PA_BF16) return PA_ERR_INVALID;
  if (!std::isfinite(s->scale) || !(s->scale > 0.f)) return PA_ERR_INVALID;
  if (mla && (s->num_kv_heads != 1 || s->head_dim_v > s->head_dim)) return PA_ERR_INVALID;
  if (pick_kernel(*s, mla) == Kernel::None) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int max_pages(const pa_shape& s) {
  return (int)(((int64_t)s.max_context_len + s.block_size - 1) / s.block_size);
}

// Number of compute units of the current device, cached per device.
int device_cus() {
  static std::mutex mu;
  static int cache[kMaxDevices] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] > 0) return cache[dev];
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxDevices && cus > 0) {
    std::lock_guard<std::mutex> lk(mu);
    cache[dev] = cus;
  }
  return cus;
}

// Split plan (host only).  Each split is a fixed number of pages c, so
// ragged batches use fewer splits for shorter sequences (see header).  Chosen
// from measurements on MI355X (bf16, 128-dim heads, 16-token pages):
//  * a split should carry a fixed amount of KV per workgroup: ~128 KiB for
//    the VALU kernel (one head per workgroup, 4 workgroups per CU), ~1 MiB for
//    the MFMA kernel (a whole head group, 2 workgroups per CU; 2 MiB when a
//    batch with fewer units than CUs gets one 8-wave workgroup per CU).  Longer splits
//    leave a long tail on ragged batches; shorter ones pay each workgroup's
//    fixed prologue/epilogue more often;
//  * the grid must still hold at least one workgroup per CU if every sequence
//    were as long as the longest;
//  * each split's float32 partial (written, then read by the merge) should
//    stay a few percent of the KV bytes it summarises.
int heuristic_splits(const pa_shape& s, int cus, bool mla) {
  const int P = max_pages(s);
  if (P <= 1) return 1;
  if (cus <= 0) cus = 256;
  const Kernel k = pick_kernel(s, mla);
  const int esz = fp8_kv(s) ? 1 : (s.dtype == PA_BF16 ? 2 : 4);   // bytes per cache element
  long S;
  if (k == Kernel::MlaMfma) {
    // one workgroup per (head group, sequence, split): fill the CUs once
    const long groups = (long)s.batch * rows_of(s) *
                        (s.num_q_heads / pa::mla_heads_per_workgroup(s.num_q_heads, s.block_size));
    S = (cus + groups - 1) / groups;
    // one-token pages: a split holds at most mla_max_split_tokens ids
    const long max_c = pa::mla_max_split_tokens(s.block_size);
    const long s_min = ((long)P + max_c - 1) / max_c;
    if (S < s_min) S = s_min;
  } else {
    long units;
    int heads_per_wg;
    double target_bytes;
    if (k == Kernel::GqaMfma) {
      units = (long)s.batch * s.num_kv_heads;
      heads_per_wg = s.num_q_heads / s.num_kv_heads * rows_of(s);   // partial rows per workgroup
      // fewer units than CUs: one 8-wave workgroup per CU (gqa_waves) with
      // twice the bytes
      target_bytes = units < cus ? 2 * kSplitBytesMfma : kSplitBytesMfma;
    } else {
      units = (long)s.batch * s.num_q_heads;
      heads_per_wg = 1;
      // heads wider than 128 dims: the same tokens per split (their kernel
      // holds half the workgroups per CU; 256-dim heads, 16 x 16 of 1-4K
      // tokens: 107.6 us at 16 splits against 109.8 at 32)
      target_bytes = kSplitBytesValu * std::max(1.0, (s.head_dim + s.head_dim_v) / 256.0);
    }
    // FP8 caches hold half the bytes per token.  With at least one unit per
    // CU, splits keep the bf16 token count (the ragged batch: 186 against
    // 201 us with splits of the same bytes); when the CU count sizes the grid
    // instead, splits of the same bytes pay each workgroup's fixed cost half
    // as often (long-context GQA at 32 splits: 44 against 46 us at 64).
    const bool bf16_geometry = esz < 2 && units >= cus;
    const double page_bytes =
        (double)s.block_size * (s.head_dim + s.head_dim_v) * (bf16_geometry ? 2 : esz);
    const double part_bytes = 2.0 * heads_per_wg * (s.head_dim_v + 1) * 4.0;
    int c_min = (int)std::ceil(part_bytes / (0.03 * page_bytes));
    if (c_min < 1) c_min = 1;
    int c = (int)(target_bytes / page_bytes);
    // A batch with a unit per CU or more runs its workgroups in rounds; the
    // units differ in length, and workgroups as long as a whole short-batch
    // sequence leave a tail: the longest sequence of a batch with long units
    // gets at least kMinSplitsLong splits.
    const double long_unit_bytes = (double)P * page_bytes;   // the longest sequence's unit
    if (k == Kernel::GqaMfma && units >= cus && units < 4L * cus &&
        long_unit_bytes <= kShortUnitBytes) {
      // The units alone fill the grid and none is long: every further split
      // adds a workgroup's fixed cost and partials, so the longest sequence
      // is only halved, against the tail of a ragged batch.  Measured (bf16,
      // D128, bs16, decode call): 32 sequences x 8 KV heads at 8192 tokens,
      // 175 us at 2 splits against 190 at 8 (163 unsplit); 64 x 8 of
      // 1024-4096 tokens, 129 against 133 (141 unsplit); 128 x 4 of 512-2048,
      // 73 against 80; Llama-style MHA with 4 rows, 116 against 122.
      c = (P + 1) / 2;
    } else if (k == Kernel::GqaMfma && units >= cus) {
      const int c_long = (P + kMinSplitsLong - 1) / kMinSplitsLong;
      if (c > c_long) c = c_long;
      // Several sequences with large units run longest first (uses_schedule),
      // so a late unit no longer sets the tail and splits can be larger:
      // kSchedSplitsLong for the longest sequence.  The ragged batch: 350.6 us
      // at 10 splits against 357.5 at 15 (FP8 183.3 against 190.0); four
      // other draws of it: -2.9 % to +1.2 % (mean -1.4 %) against 15 splits,
      // while the best count varied from 7 to 10.
      const int c_sched = (P + kSchedSplitsLong - 1) / kSchedSplitsLong;
      if (s.batch > 1 && c_sched > c &&
          (double)c_sched * s.block_size * (s.head_dim + s.head_dim_v) * esz >= kScheduleUnitBytes)
        c = c_sched;
      // A batch whose (sequence, KV head) units alone fill every workgroup
      // slot (two per CU) twice over needs splitting only against a tail:
      // kSchedSplitsMany for the longest sequence, and no split below
      // kManyUnitBytes (a shorter longest sequence is not split at all).
      // Measured (64 q / 8 kv heads, D128): 128 sequences of 512-4096
      // tokens, 3 splits: 216.9 us against 254.8 at 8; 256 of log-uniform
      // 64-8192: 295.4 against 328.8; 256 of 64-1024 tokens, unsplit: 113.6
      // against 149.2 at 2; 512 of log-uniform 32-2048, 2 splits: 210.7
      // against 253.0 at 4 and 233 unsplit.
      if (s.batch > 1 && units >= 4L * cus) {
        const int c_many = std::max((P + kSchedSplitsMany - 1) / kSchedSplitsMany,
                                    (int)std::ceil(kManyUnitBytes / page_bytes));
        if (c_many > c) c = c_many;
      }
    }
    // The VALU kernel holds 4 workgroups per CU; a batch whose (sequence,
    // head) units alone fill those slots twice over gives the longest
    // sequence kValuSplitsMany splits (64 sequences x 32 heads of 1-4K
    // tokens: 437.8 us per step at 4 splits against 456.0 at 16; 128 x 32 of
    // log-uniform 128-8K tokens: 723.6 against 778.9 at 32).
    if (k == Kernel::MhaValu && s.batch > 1 && units >= 8L * cus) {
      const int c_many = (P + kValuSplitsMany - 1) / kValuSplitsMany;
      if (c_many > c) c = c_many;
    }
    if (c < c_min) c = c_min;
    S = (P + c - 1) / c;
    const long s_fill = (cus + units - 1) / units;
    if (S < s_fill) S = s_fill;
    // A problem too small to fill the CUs with useful work: filling them
    // anyway gives workgroups that read a few KiB each and a reduction launch
    // of the same cost as the work.  No split reads less than a minimum (the
    // launch is then bound by latency, not by how many CUs it occupies), so
    // tiny problems use few splits and merge them in-kernel, in one launch.
    const double unit_bytes = (double)P * s.block_size * (s.head_dim + s.head_dim_v) * esz;
    const double min_bytes = k == Kernel::GqaMfma ? kMinSplitBytesMfma : kMinSplitBytesValu;
    const long s_small = (long)(unit_bytes / min_bytes);
    if (S > s_small) S = s_small;
  }
  if (S > P) S = P;
  if (S > kMaxSplits) S = kMaxSplits;
  return S < 1 ? 1 : (int)S;
}

// Resolve num_splits (<= 0: heuristic), clamp to [1, P].  0 on failure.
int resolve_splits(const pa_shape& s, int32_t num_splits, bool mla) {
  const int P = max_pages(s);
  int S = num_splits;
  if (S <= 0) {
    const int cus = device_cus();
    if (cus <= 0) return 0;
    S = heuristic_splits(s, cus, mla);
  }
  if (S > P) S = P;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  return S;
}

// Workspace layout (S > 1), R = B * q_len * Hq rows, each region 256-byte
// aligned: counters i32 [R] | o_part [R][S][Dv] | lse_part f32 [R][S].
// The counters come first, at an offset that does not depend on S: calls with
// the same R find them where the previous call left them (zero), whatever
// their split counts, and the partials never overwrite them.
//
// o_part is float32, except on the MLA matrix-core path (bf16 latents),
// whose split outputs are stored as bfloat16: there the partials of 128
// heads x 512 dims per split are a sixth of the latent bytes a split reads
// (float32: a quarter), written once and read once by the reduction, and the
// output they merge into is bfloat16 as well.  The merge weights (lse_part)
// stay float32 everywhere.
size_t ws_rows(const pa_shape& s) { return (size_t)s.batch * rows_of(s) * s.num_q_heads; }
bool part_bf16(const pa_shape& s, bool mla) { return pick_kernel(s, mla) == Kernel::MlaMfma; }
size_t ws_counter_bytes(const pa_shape& s) { return align_up(ws_rows(s) * sizeof(int32_t)); }
size_t ws_opart_offset(const pa_shape& s) { return ws_counter_bytes(s); }
size_t ws_lse_offset(const pa_shape& s, int S, bool mla) {
  const size_t esz = part_bf16(s, mla) ? sizeof(uint16_t) : sizeof(float);
  return ws_opart_offset(s) + align_up(ws_rows(s) * S * s.head_dim_v * esz);
}
// A batch of several sequences on the grouped-query kernel runs its units in
// the order a schedule launch writes after lse_part: u32 [B * S] (pa_sched.hip),
// longest first, so that no long unit starts late and leaves a tail.  The
// launch costs ~6 us on MI355X, so it is used only where a unit can leave a
// tail much longer than that: units of at least kScheduleUnitBytes of KV
// (~30 us each at the per-workgroup share of HBM bandwidth; the ragged
// batch's bf16 units are 1 MiB: 370.7 -> 359.2 us, FP8 0.5 MiB: 201.4 ->
// 190.7 us; Llama-style MHA with 4 rows, 256 KiB units of near-equal
// sequences: 115.1 -> 116.8 us, so it keeps the plain grid order).
bool fuses(const pa_shape& s, int S, Kernel kern);
bool uses_schedule(const pa_shape& s, int S, bool mla) {
  if (S <= 1 || s.batch <= 1 || pick_kernel(s, mla) != Kernel::GqaMfma) return false;
  // a call that merges in-kernel stays one launch (its units are tiny anyway)
  if (fuses(s, S, Kernel::GqaMfma)) return false;
  if ((long long)s.batch * S >= (1LL << 31)) return false;
  const long long c = (max_pages(s) + S - 1) / S;
  const int esz = fp8_kv(s) ? 1 : (s.dtype == PA_BF16 ? 2 : 4);
  return (double)c * s.block_size * (s.head_dim + s.head_dim_v) * esz >= kScheduleUnitBytes;
}
size_t ws_sched_offset(const pa_shape& s, int S, bool mla) {
  return ws_lse_offset(s, S, mla) + align_up(ws_rows(s) * S * sizeof(float));
}
size_t workspace_bytes_for(const pa_shape& s, int S, bool mla) {
  if (S <= 1) return 0;
  return ws_sched_offset(s, S, mla) +
         (uses_schedule(s, S, mla) ? align_up((size_t)s.batch * S * sizeof(uint32_t)) : 0);
}

pa::Params make_params(const pa_shape& s, int S, bool mla, const void* q, const void* k,
                       const void* v, const int32_t* bt, const int32_t* ctx, void* out, float* lse,
                       void* ws) {
  pa::Params p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.block_table = bt;
  p.context_lens = ctx;
  p.out = out;
  p.lse = lse;
  p.B = s.batch;
  p.Hq = s.num_q_heads;
  p.Hkv = s.num_kv_heads;
  p.D = s.head_dim;
  p.Dv = s.head_dim_v;
  p.bs = s.block_size;
  p.maxb = s.max_blocks_per_seq;
  p.nblocks = s.num_blocks;
  p.max_ctx = s.max_context_len;
  p.ql = rows_of(s);
  p.S = S;
  const int P = max_pages(s);
  p.c = P > 0 ? (P + S - 1) / S : 1;
  p.scale_log2 = s.scale * 1.4426950408889634f * (fp8_kv(s) ? s.k_scale : 1.f);
  p.v_scale = fp8_kv(s) ? s.v_scale : 1.f;
  p.final_write = S == 1 ? 1 : 0;
  if (S > 1) {
    char* base = static_cast<char*>(ws);
    p.counters = reinterpret_cast<int32_t*>(base);
    if (part_bf16(s, mla))
      p.o_part16 = reinterpret_cast<uint16_t*>(base + ws_opart_offset(s));
    else
      p.o_part = reinterpret_cast<float*>(base + ws_opart_offset(s));
    p.lse_part = reinterpret_cast<float*>(base + ws_lse_offset(s, S, mla));
    if (uses_schedule(s, S, mla))
      p.sched = reinterpret_cast<uint32_t*>(base + ws_sched_offset(s, S, mla));
  }
  return p;
}

// Waves per workgroup of the grouped-query kernel: 8 when the grid holds at
// most one workgroup per CU (then every CU runs one; measured on the
// long-context workload at 32 splits: 82.3 us against 84.6 us for 4-wave
// workgroups at 64 splits, two per CU), else 4 (two workgroups per CU; 8
// waves measured 6 % slower on the ragged batch).
int gqa_waves(const pa_shape& s, int S) {
  const int cus = device_cus();
  const long wgs = (long)s.batch * s.num_kv_heads * S;
  return cus > 0 && wgs <= cus ? 8 : 4;
}

// Whether pa_decode merges in-kernel for this shape and split count.  The
// fused merge costs every workgroup a device-scope arrival atomic (a round
// trip it waits for) and leaves the merge to the last workgroup of each unit
// as a serial tail; a separate reduction launch merges all units in parallel
// for a few microseconds.  Measured on MI355X, the separate launch wins from
// 8 KiB of partials per unit up (batch 16 x 32 heads at 16 splits: 110 us
// against 116 us), so only tiny merges stay in-kernel.
bool fuses(const pa_shape& s, int S, Kernel kern) {
  if (S <= 1 || kern == Kernel::MlaMfma || kern == Kernel::None || rows_of(s) > 1) return false;
  const long unit_heads = kern == Kernel::GqaMfma ? s.num_q_heads / s.num_kv_heads : 1;
  const long merge_bytes = (long)S * unit_heads * (s.head_dim_v + 1) * 4;
  return merge_bytes <= kFusedMergeBytes;
}

// Launch the partial kernel.  With `fused` (and a kernel that supports it)
// the last workgroup of every (sequence, head unit) also merges the splits,
// so no reduction launch is needed; *needs_reduce tells the caller.
pa_status run_partial(const pa_shape* shape, const void* q, const void* k, const void* v,
                      const int32_t* bt, const int32_t* ctx, int32_t num_splits, void* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream, bool mla, bool fused,
                      int* S_out, bool* needs_reduce) {
  const pa_status st = check_shape(shape, mla);
  if (st != PA_OK) return st;
  if (!q || !k || (!mla && !v) || !bt || !ctx || !out) return PA_ERR_INVALID;
  // workspace check for an explicit split count needs no device query
  if (num_splits > 0) {
    const int S = resolve_splits(*shape, num_splits, mla);
    if (S > 1 && (!ws || ws_bytes < workspace_bytes_for(*shape, S, mla))) return PA_ERR_WORKSPACE;
  }
  const int S = resolve_splits(*shape, num_splits, mla);
  if (S < 1) return PA_ERR_HIP;
  if (S > 1 && (!ws || ws_bytes < workspace_bytes_for(*shape, S, mla))) return PA_ERR_WORKSPACE;
  const Kernel kern = pick_kernel(*shape, mla);
  if (kern == Kernel::MlaMfma) {
    const int P = max_pages(*shape);
    if ((P + S - 1) / S > pa::mla_max_split_tokens(shape->block_size)) return PA_ERR_UNSUPPORTED;
  }
  pa::Params p = make_params(*shape, S, mla, q, k, mla ? k : v, bt, ctx, out, lse, ws);
  // The fused merge runs in the last workgroup of each unit, after every
  // other split of the unit: cheap when the unit's partials are small, a
  // serial tail when they are large.  Above kFusedMergeBytes per unit the
  // separate reduction launch (all units in parallel) is faster.
  p.fused = (fused && fuses(*shape, S, kern)) ? 1 : 0;
  p.wg_waves = kern == Kernel::GqaMfma ? gqa_waves(*shape, S) : 0;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (kern) {
    case Kernel::MhaValu: e = pa::launch_mha_valu(p, shape->dtype == PA_BF16, fp8_kv(*shape), hs); break;
    case Kernel::GqaMfma:
      e = p.sched ? pa::launch_unit_schedule(p, hs) : hipSuccess;
      if (e == hipSuccess) e = pa::launch_gqa_mfma(p, fp8_kv(*shape), hs);
      break;
    case Kernel::MlaMfma: e = pa::launch_mla_mfma(p, fp8_kv(*shape), hs); break;
    default: return PA_ERR_UNSUPPORTED;
  }
  if (e != hipSuccess) return PA_ERR_HIP;
  if (S_out) *S_out = S;
  if (needs_reduce) *needs_reduce = S > 1 && !p.fused;
  return PA_OK;
}

pa_status run_reduce(const pa_shape* shape, const int32_t* ctx, int S, bool mla, const void* ws,
                     void* out, float* lse, void* stream) {
  if (S <= 1) return PA_OK;
  const pa::Params p = make_params(*shape, S, mla, nullptr, nullptr, nullptr, nullptr, ctx, out,
                                   lse, const_cast<void*>(ws));
  const hipError_t e = pa::launch_reduce(p, shape->dtype == PA_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Partials and arrival counters of pa_decode_static: a file-scope device
// array (each device holds its own copy until the process ends) in place of
// a caller's workspace.  In host code `scratch` is only a stand-in symbol;
// its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

struct ScratchSlot {
  void* ptr = nullptr;      // device address of this device's `scratch`
  size_t zero_rows = 0;     // rows whose arrival counters are known to be zero
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxDevices];

// This device's scratch slot, its address looked up on first use.
ScratchSlot* scratch_slot() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchSlot* slot = &g_scratch[dev];
  if (slot->ptr == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    slot->ptr = ptr;
    slot->zero_rows = 0;   // nothing known about the array's contents yet
  }
  return slot;
}

}  // namespace

extern "C" {

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported dtype/head_dim/block_size combination";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_SCRATCH: return "partials exceed the library's static scratch (64 MiB)";
    default: return "unknown status";
  }
}

int32_t pa_version(void) { return 100; }

int32_t pa_decode_launches(const pa_shape* shape, int32_t num_splits, int32_t mla) {
  if (check_shape(shape, mla != 0) != PA_OK) return 0;
  const int S = resolve_splits(*shape, num_splits, mla != 0);
  if (S < 1) return 0;
  if (S == 1) return 1;
  if (fuses(*shape, S, pick_kernel(*shape, mla != 0))) return 1;
  return uses_schedule(*shape, S, mla != 0) ? 3 : 2;
}

int32_t pa_choose_num_splits(const pa_shape* shape, int32_t num_cus, int32_t mla) {
  if (check_shape(shape, mla != 0) != PA_OK) return 0;
  int cus = num_cus;
  if (cus <= 0) cus = device_cus();
  if (cus <= 0) return 0;
  return heuristic_splits(*shape, cus, mla != 0);
}

size_t pa_decode_workspace_size(const pa_shape* shape, int32_t num_splits, int32_t mla) {
  if (check_shape(shape, mla != 0) != PA_OK) return 0;
  const int S = resolve_splits(*shape, num_splits, mla != 0);
  if (S < 1) return 0;
  return workspace_bytes_for(*shape, S, mla != 0);
}

pa_status pa_workspace_init(const pa_shape* shape, int32_t num_splits, int32_t mla,
                            void* workspace, size_t workspace_bytes, void* stream) {
  const pa_status st = check_shape(shape, mla != 0);
  if (st != PA_OK) return st;
  if (num_splits > 0) {
    const int S = resolve_splits(*shape, num_splits, mla != 0);
    if (S <= 1) return PA_OK;
    if (!workspace || workspace_bytes < workspace_bytes_for(*shape, S, mla != 0))
      return PA_ERR_WORKSPACE;
  }
  const int S = resolve_splits(*shape, num_splits, mla != 0);
  if (S < 1) return PA_ERR_HIP;
  if (S <= 1) return PA_OK;
  if (!workspace || workspace_bytes < workspace_bytes_for(*shape, S, mla != 0))
    return PA_ERR_WORKSPACE;
  int32_t* cnt = static_cast<int32_t*>(workspace);
  const size_t n = ws_rows(*shape);
  return pa::launch_zero_i32(cnt, n, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK
                                                                                    : PA_ERR_HIP;
}

pa_status pa_decode_partial(const pa_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* context_lens, int32_t num_splits, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return run_partial(shape, q, k_cache, v_cache, block_table, context_lens, num_splits, out, lse,
                     workspace, workspace_bytes, stream, false, false, nullptr, nullptr);
}

pa_status pa_decode_mla_partial(const pa_shape* shape, const void* q, const void* kv_cache,
                                const int32_t* block_table, const int32_t* context_lens,
                                int32_t num_splits, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return run_partial(shape, q, kv_cache, nullptr, block_table, context_lens, num_splits, out, lse,
                     workspace, workspace_bytes, stream, true, false, nullptr, nullptr);
}

pa_status pa_reduce(const pa_shape* shape, const int32_t* context_lens, int32_t num_splits,
                    int32_t mla, const void* workspace, size_t workspace_bytes, void* out,
                    float* lse, void* stream) {
  const pa_status st = check_shape(shape, mla != 0);
  if (st != PA_OK) return st;
  if (!context_lens || !out) return PA_ERR_INVALID;
  if (num_splits > 0) {
    const int S = resolve_splits(*shape, num_splits, mla != 0);
    if (S <= 1) return PA_OK;
    if (!workspace || workspace_bytes < workspace_bytes_for(*shape, S, mla != 0))
      return PA_ERR_WORKSPACE;
  }
  const int S = resolve_splits(*shape, num_splits, mla != 0);
  if (S < 1) return PA_ERR_HIP;
  if (S <= 1) return PA_OK;
  if (!workspace || workspace_bytes < workspace_bytes_for(*shape, S, mla != 0))
    return PA_ERR_WORKSPACE;
  return run_reduce(shape, context_lens, S, mla != 0, workspace, out, lse, stream);
}

pa_status pa_decode(const pa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_table, const int32_t* context_lens, int32_t num_splits,
                    void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  int S = 0;
  bool reduce = false;
  const pa_status st = run_partial(shape, q, k_cache, v_cache, block_table, context_lens, num_splits,
                                   out, lse, workspace, workspace_bytes, stream, false, true, &S,
                                   &reduce);
  if (st != PA_OK) return st;
  return reduce ? run_reduce(shape, context_lens, S, false, workspace, out, lse, stream) : PA_OK;
}

pa_status pa_decode_static(const pa_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* context_lens, int32_t num_splits, void* out,
                           float* lse, void* stream) {
  const pa_status st = check_shape(shape, false);
  if (st != PA_OK) return st;
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out) return PA_ERR_INVALID;
  const int S = resolve_splits(*shape, num_splits, false);
  if (S < 1) return PA_ERR_HIP;
  const size_t need = workspace_bytes_for(*shape, S, false);
  if (need > kScratchBytes) return PA_ERR_SCRATCH;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchSlot* slot = scratch_slot();
  if (slot == nullptr) return PA_ERR_HIP;
  const size_t rows = ws_rows(*shape);
  const bool merge_in_kernel = S > 1 && fuses(*shape, S, pick_kernel(*shape, false));
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (merge_in_kernel && slot->zero_rows < rows) {
    // counters a previous call may have covered with partials: zero them
    // (a fill kernel, safe under graph capture)
    if (pa::launch_zero_i32(static_cast<int32_t*>(slot->ptr), rows, hs) != hipSuccess)
      return PA_ERR_HIP;
    slot->zero_rows = rows;
  }
  int S_run = 0;
  bool reduce = false;
  const pa_status r = run_partial(shape, q, k_cache, v_cache, block_table, context_lens, S, out,
                                  lse, slot->ptr, kScratchBytes, stream, false, true, &S_run,
                                  &reduce);
  if (r != PA_OK) return r;
  // this call's partials follow its own counters: those of more rows may be gone
  if (rows < slot->zero_rows) slot->zero_rows = rows;
  return reduce ? run_reduce(shape, context_lens, S_run, false, slot->ptr, out, lse, stream) : PA_OK;
}

pa_status pa_decode_mla(const pa_shape* shape, const void* q, const void* kv_cache,
                        const int32_t* block_table, const int32_t* context_lens, int32_t num_splits,
                        void* out, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int S = 0;
  bool reduce = false;
  const pa_status st = run_partial(shape, q, kv_cache, nullptr, block_table, context_lens,
                                   num_splits, out, lse, workspace, workspace_bytes, stream, true,
                                   true, &S, &reduce);
  if (st != PA_OK) return st;
  return reduce ? run_reduce(shape, context_lens, S, true, workspace, out, lse, stream) : PA_OK;
}


// Shape checks of the append entry points: the decode's basic checks, without
// kernel support or scale (the append moves bytes only).
static pa_status check_append_shape(const pa_shape* s, bool mla) {
  if (!s) return PA_ERR_INVALID;
  if (s->batch > 65535) return PA_ERR_UNSUPPORTED;   // grid y limit
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->head_dim < 1 ||
      s->head_dim_v < 1 || s->block_size < 1 || s->max_blocks_per_seq < 1 || s->num_blocks < 1)
    return PA_ERR_INVALID;
  if (s->num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;   // grid x limit
  if (s->dtype != PA_F32 && s->dtype != PA_BF16) return PA_ERR_INVALID;
  if (s->kv_dtype != 0 && s->kv_dtype != s->dtype && s->kv_dtype != PA_FP8_E4M3)
    return PA_ERR_INVALID;
  if (mla && s->num_kv_heads != 1) return PA_ERR_INVALID;
  return PA_OK;
}

// Bytes per cache element of an append (the cache dtype).
static int cache_esize(const pa_shape& s) {
  if (s.kv_dtype == PA_FP8_E4M3) return 1;
  return s.dtype == PA_BF16 ? 2 : 4;
}

pa_status pa_append_kv(const pa_shape* shape, const void* k_new, const void* v_new, void* k_cache,
                       void* v_cache, const int32_t* block_table, const int32_t* context_lens,
                       void* stream) {
  const pa_status st = check_append_shape(shape, false);
  if (st != PA_OK) return st;
  if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !context_lens)
    return PA_ERR_INVALID;
  const pa_shape& s = *shape;
  pa::AppendParams a{k_new, v_new, k_cache, v_cache, block_table, context_lens,
                     s.batch, s.num_kv_heads, s.head_dim, s.head_dim_v, s.block_size,
                     s.max_blocks_per_seq, s.num_blocks};
  const hipError_t e = pa::launch_append(a, cache_esize(s), false, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_append_latent(const pa_shape* shape, const void* c_new, void* kv_cache,
                           const int32_t* block_table, const int32_t* context_lens,
                           void* stream) {
  const pa_status st = check_append_shape(shape, true);
  if (st != PA_OK) return st;
  if (!c_new || !kv_cache || !block_table || !context_lens) return PA_ERR_INVALID;
  const pa_shape& s = *shape;
  // FP8 latent rows only in the layouts the FP8 latent decode reads (576-wide
  // rows on 64-token or one-token pages): refuse to write caches nothing can read
  if (s.kv_dtype == PA_FP8_E4M3 && !(s.head_dim == 576 && (s.block_size == 64 || s.block_size == 1)))
    return PA_ERR_UNSUPPORTED;
  pa::AppendParams a{c_new, nullptr, kv_cache, nullptr, block_table, context_lens,
                     s.batch, 1, s.head_dim, 0, s.block_size, s.max_blocks_per_seq,
                     s.num_blocks};
  const hipError_t e = pa::launch_append(a, cache_esize(s), true, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return PA_ERR_INVALID;
  const hipError_t e =
      pa::launch_stream_read(src, bytes, sink, device_cus(), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
