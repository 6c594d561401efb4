// Kernel parameter block and launch entry points (internal to libpa_decode).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Everything a partial or reduce kernel needs, passed by value as the kernel
// argument.  Pointers are device pointers owned by the caller.
struct Params {
  const void* q;             // [B][ql][Hq][Dqk]
  const void* k;             // MHA/GQA: [nb][Hkv][bs][D]; MLA: latent [nb][bs][Dqk]
  const void* v;             // MHA/GQA: [nb][Hkv][Dv][bs]; MLA: unused (aliases k)
  const int32_t* block_table;  // [B][maxb]
  const int32_t* context_lens; // [B]
  void* out;                 // [B][ql][Hq][Dv] dtype
  float* lse;                // [B][ql][Hq] or nullptr
  float* o_part;             // [B][ql][Hq][S][Dv] float32 (S > 1), or null when o_part16 is set
  uint16_t* o_part16;        // the same layout in bfloat16 (S > 1, MLA matrix-core path), else null
  float* lse_part;           // [B][ql][Hq][S]     (S > 1)
  int32_t* counters;         // [B][Hq] arrival counters of the fused reduction (S > 1, ql == 1)
  uint32_t* sched;           // grouped-query kernel on a batch: [B * S] unit order, or null
                             // (entry: sequence | split << 16, kNoUnit for a slot without one)
  int32_t B, Hq, Hkv, D, Dv, bs, maxb, nblocks, max_ctx;
  int32_t ql;                // query rows per sequence (>= 1): rows are (b, j, h), j < ql
  int32_t S;                 // splits in the grid
  int32_t c;                 // pages per split
  float scale_log2;          // scale * log2(e) (* k_scale for FP8 caches)
  float v_scale;             // FP8 caches: factor of every value (1 otherwise)
  int32_t final_write;       // 1: S == 1, write out/lse directly
  int32_t fused;             // 1: the last workgroup of a unit merges the splits
  int32_t wg_waves;          // grouped-query kernel: waves per workgroup, 4 or 8
};

constexpr uint32_t kNoUnit = 0xFFFFFFFFu;

// Each returns hipSuccess or the launch error.  Shapes are validated by the caller.
hipError_t launch_mha_valu(const Params& p, bool bf16, bool fp8kv, hipStream_t st);
hipError_t launch_gqa_mfma(const Params& p, bool fp8kv, hipStream_t st);
hipError_t launch_mla_mfma(const Params& p, bool fp8kv, hipStream_t st);
hipError_t launch_reduce(const Params& p, bool bf16, hipStream_t st);
// Writes p.sched (longest units first) from the context lengths; one workgroup.
hipError_t launch_unit_schedule(const Params& p, hipStream_t st);
hipError_t launch_zero_i32(int32_t* dst, size_t n, hipStream_t st);

// Arguments of the paged KV append (MLA: k_new / k_cache are the latent
// row and pool, v_* unused, D the latent width).
struct AppendParams {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const int32_t* context_lens;
  int B, Hkv, D, Dv, bs, maxb, nblocks;
};
// esize: bytes per cache element (4 float32, 2 bfloat16, 1 FP8 code).
hipError_t launch_append(const AppendParams& a, int esize, bool mla, hipStream_t st);

// Streaming-read probe over `bytes` (a multiple of 16) of device memory.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int cus,
                              hipStream_t st);

// Which kernels exist (host-side predicates used by validation and dispatch).
bool mha_valu_supported(bool bf16, int D, int bs);
// G query heads per KV head, ql query rows: the kernel's 16 MFMA columns hold
// the G * ql (row, head) pairs of a KV head.
bool gqa_mfma_supported(bool bf16, int D, int Dv, int bs, int G, int ql);
// FP8 E4M3 caches (bf16 queries): which shapes each kernel takes.
bool gqa_mfma_fp8_supported(int D, int bs, int G, int ql);
bool mha_valu_fp8_supported(int D, int bs);
bool mla_mfma_supported(bool bf16, int Dqk, int Dv, int bs, int Hq);
// FP8 E4M3 latent cache (bf16 queries): the 128-head kernel on 64-token pages.
bool mla_mfma_fp8_supported(int Dqk, int Dv, int bs, int Hq);
// Query heads one MLA workgroup holds (the grid has Hq / this head groups).
int mla_heads_per_workgroup(int Hq, int bs);
// Longest split (tokens) the MLA kernel takes for this page size (one-token
// pages keep a split's token ids in LDS).
int mla_max_split_tokens(int bs);

}  // namespace pa
