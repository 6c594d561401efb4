/*
 * pa_decode.h - single-token decode attention over a paged KV cache, split-KV.
 *
 * C ABI of libpa_decode.so (gfx950 / MI355X).  Plain pointers and sizes only.
 *
 * What is computed (the definition every entry point reaches, up to rounding):
 *   For sequence b < batch, query head h < num_q_heads and logical token
 *   i < context_lens[b]:
 *       page  = block_table[b * max_blocks_per_seq + i / block_size]
 *       slot  = i % block_size,        g = h / (num_q_heads / num_kv_heads)
 *       s_i   = scale * <q[b][h][:], k_i>
 *       out[b][h][:] = sum_i exp(s_i - m) v_i / sum_i exp(s_i - m),  m = max_i s_i
 *       lse[b][h]    = m + ln(sum_i exp(s_i - m))          (natural log)
 *   This is scaled dot-product softmax attention of one query row per head
 *   (the wenku.it search page for "paged attention", its "Transformer
 *   introduction" snippet: each query scored against every key, scores
 *   re-weighting the values; the wenku.it search page for "Multi-head Latent
 *   Attention (MLA)": multi-head attention as h self-attentions), over KV
 *   memory managed in fixed pages as PagedAttention does (the "paged
 *   attention" search page, its vLLM README snippets).  It is evaluated with
 *   Flash-Decoding's three steps (the "flash decoding ++" entry, its
 *   three-steps snippet): the pages of
 *   a sequence are cut into contiguous splits, each split's attention is
 *   computed in parallel with its log-sum-exp, and the split results are
 *   rescaled and reduced into the exact output.
 *
 * Several query rows (q_len > 1: chunked prefill, draft verification): the
 *   rows are each sequence's last q_len tokens, whose K/V are already in the
 *   cache, and row j (position context_lens[b] - q_len + j) attends to
 *   positions 0 .. context_lens[b] - q_len + j.  The pages name the prefill
 *   stage and FlashAttention's exact attention over many query rows (the
 *   FlashMLA-ETAP related-papers page, its FlashAttention abstracts) but no
 *   mask; this causal reading reduces to the definition above at q_len = 1.
 *   A row that sees no token gives out = 0 and lse = -inf.
 *
 * Memory layouts (all row-major, contiguous, device memory):
 *   q            [batch][q_len][num_q_heads][head_dim]             dtype
 *   k_cache      [num_blocks][num_kv_heads][block_size][head_dim]  dtype
 *   v_cache      [num_blocks][num_kv_heads][head_dim_v][block_size] dtype
 *   kv_cache     [num_blocks][block_size][head_dim]  (MLA latent)  dtype
 *                keys are whole rows, values the first head_dim_v entries
 *   block_table  [batch][max_blocks_per_seq]                        int32
 *   context_lens [batch]                                            int32
 *   out          [batch][q_len][num_q_heads][head_dim_v]            dtype
 *   lse          [batch][q_len][num_q_heads]                        float32
 *   (q_len = 1 drops that axis: q [batch][num_q_heads][head_dim] etc.)
 *   dtype PA_F32 = float32, PA_BF16 = bfloat16 (accumulation is float32;
 *   bf16 outputs are rounded to nearest even).  The caches may instead hold
 *   FP8 E4M3 codes (kv_dtype, one byte per element, same layouts) with one
 *   scale per cache tensor; q and out stay bfloat16.  The pages name FP8 only
 *   as the hardware low precision FlashAttention-3 uses (the "llms-attention"
 *   post); this per-tensor-scale reading is the library's.
 *
 * Splits: with S = num_splits and P = ceil(max_context_len / block_size),
 *   every split covers c = ceil(P / S) pages; sequence b uses
 *   ceil(ceil(context_lens[b] / block_size) / c) splits (ragged batches
 *   therefore use fewer splits for shorter sequences).  num_splits <= 0 asks
 *   for pa_choose_num_splits().  S larger than P is legal (empty splits).
 *
 * Ownership and execution: every pointer is caller-owned device memory; the
 *   library allocates nothing and keeps no state beyond a per-device cache of
 *   the compute-unit count.  `stream` is a hipStream_t (NULL = default stream).
 *   Calls are asynchronous on `stream`; outputs are valid once it completes.
 *   Calls are thread-safe and reentrant; concurrent calls must not share a
 *   workspace.
 *
 * Errors: a status is returned, nothing is thrown.  Arguments are checked on
 *   the host before any HIP call; on failure nothing is launched.  Limits
 *   (PA_ERR_UNSUPPORTED beyond them): batch <= 65535, max_context_len <= 2^29,
 *   batch * q_len * num_q_heads < 2^31, at most 65535 splits.  Device-side
 *   context_lens are clamped to [0, max_context_len] and block ids to
 *   [0, num_blocks), so malformed tables cannot read outside the pools.
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID = 1,     /* NULL required pointer, non-positive size, inconsistent shape */
  PA_ERR_UNSUPPORTED = 2, /* well-formed but no kernel for this dtype/head_dim/block_size */
  PA_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than pa_decode_workspace_size() */
  PA_ERR_HIP = 4,         /* the HIP runtime reported an error (device query or launch) */
  PA_ERR_SCRATCH = 5      /* pa_decode_static: partials beyond its 64 MiB static scratch */
} pa_status;

/* PA_FP8_E4M3 is a cache dtype only (pa_shape.kv_dtype): OCP FP8 E4M3 codes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; subnormals;
 * S.1111.111 is NaN; no infinity), each read as its tensor's scale times the
 * code's value. */
typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

typedef struct pa_shape {
  int32_t batch;              /* B >= 1 */
  int32_t num_q_heads;        /* Hq >= 1 */
  int32_t num_kv_heads;       /* Hkv >= 1, divides Hq; must be 1 for MLA */
  int32_t head_dim;           /* Dqk: width of q and k (MLA: latent width) */
  int32_t head_dim_v;         /* Dv: width of v and out (MHA/GQA: == head_dim) */
  int32_t block_size;         /* tokens per page */
  int32_t max_blocks_per_seq; /* row length of block_table */
  int32_t num_blocks;         /* pages in the pool */
  int32_t max_context_len;    /* host-side upper bound of context_lens; sizes the grid */
  float scale;                /* score scale, finite and > 0, e.g. 1/sqrt(head_dim) */
  int32_t dtype;              /* pa_dtype of q, caches and out */
  int32_t q_len;              /* query rows per sequence, 0..16 (0 and 1: one row) */
  int32_t kv_dtype;           /* dtype of the caches: 0 = dtype, or PA_FP8_E4M3 (with PA_BF16 q) */
  float k_scale;              /* FP8 caches: a key is k_scale times its code's value (finite, > 0) */
  float v_scale;              /* FP8 caches: a value is v_scale times its code's value (finite, > 0) */
} pa_shape;

/* Human-readable name of a status code.  Never NULL. */
const char* pa_status_string(int32_t status);

/* Library version, major*10000 + minor*100 + patch. */
int32_t pa_version(void);

/*
 * Split-count heuristic (the split control that Flash-Decoding adds when
 * batch x heads alone cannot fill the GPU; the "flash decoding ++" entry,
 * its TRT-LLM multi_block_mode / vLLM PagedAttention V2 snippet).  Picks S so that the
 * partial kernel launches enough workgroups for `num_cus` compute units
 * while each split keeps enough pages to amortise its partial write; when the
 * batch runs its units longest first (pa_decode_launches == 3), splits are
 * larger, the fewer the more (sequence, KV head) units the batch has.
 * num_cus <= 0 queries the current HIP device.  Returns S >= 1, or 0 if the
 * shape is invalid (or the device query failed).  `mla` != 0 selects the
 * latent kernel's work unit.  Host only.
 */
int32_t pa_choose_num_splits(const pa_shape* shape, int32_t num_cus, int32_t mla);

/*
 * Kernel launches a pa_decode / pa_decode_mla call with this shape and split
 * count makes: 1 when S resolves to 1 or the splits are merged inside the
 * partial kernel (MHA/GQA, when a unit's partials are at most 4 KiB), 2 when
 * a separate reduction launch follows (MLA, larger partials), 3 when the
 * partial kernel is also preceded by the unit-order launch (the grouped-query
 * kernel on several sequences with units of at least 384 KiB of KV: the
 * (sequence, split) units then run longest first; see the workspace layout).
 * 0 on an invalid shape.  num_splits <= 0 resolves through the heuristic.
 * Host only.
 */
int32_t pa_decode_launches(const pa_shape* shape, int32_t num_splits, int32_t mla);

/*
 * Bytes of workspace a call with this shape and split count needs: int32
 * arrival counters [R] at offset 0, then partials o[R][S][head_dim_v]
 * (float32; bfloat16 for MLA, whose output is bfloat16 too) and float32
 * lse[R][S], R = batch * q_len * num_q_heads rows, and, when the call runs
 * its units longest first (pa_decode_launches == 3), the unit order u32
 * [batch][S] (written by the call itself), each region 256-byte aligned.  0 when S resolves to 1 (the partial kernel then writes
 * out/lse directly).  num_splits <= 0 resolves through the heuristic (which
 * may query the device).  Returns 0 on an invalid shape.  Host only.
 *
 * The counters (the first 4*R bytes) must be zero when a pa_decode call that
 * merges in-kernel starts (pa_decode_launches == 1 with S > 1).  Zero them
 * once for a new workspace (pa_workspace_init, or any memset to 0).  Every
 * call that completes leaves its counters zero and writes its partials after
 * them, so any sequence of calls with the same R keeps them zero, whatever
 * their split counts.  A call with a smaller R writes partials where a larger
 * R keeps counters: re-initialise before a call with a larger R than the
 * previous one, and after a faulted or aborted call.
 */
size_t pa_decode_workspace_size(const pa_shape* shape, int32_t num_splits, int32_t mla);

/*
 * Zero the counter region of `workspace` (its first 4*R bytes) for this shape
 * and split count, on `stream` (a fill kernel, safe to capture in a graph).
 * PA_OK when S resolves to 1 (no workspace needed).  Errors as for pa_decode.
 */
pa_status pa_workspace_init(const pa_shape* shape, int32_t num_splits, int32_t mla,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged split-KV decode attention, MHA and GQA (num_q_heads a multiple of
 * num_kv_heads).  Each workgroup computes one split's partial; the last
 * workgroup of each (sequence, head unit) to finish merges that unit's splits
 * with the log-sum-exp weights (a sequence that needs a single split is
 * written directly) -- one launch -- unless the unit's partials are large,
 * when a reduction launch merges every unit in parallel instead (see
 * pa_decode_launches).  `lse` may be NULL.  `workspace` may be
 * NULL only when S resolves to 1; its counters must be zero (see above).
 * Supported: PA_F32 with head_dim 64 or 128; PA_BF16 with head_dim 64, 128 or 256;
 * head_dim_v == head_dim; block_size 16 or 32.  With q_len > 1: PA_BF16,
 * head_dim 64 or 128, block_size 16 or 32 and (num_q_heads / num_kv_heads) *
 * q_len <= 16 (each KV tile is then read once for all rows and heads of its
 * group, as for PA_BF16 grouped heads with one row); the splits are merged by
 * a reduction launch.  FP8 caches (kv_dtype PA_FP8_E4M3): PA_BF16 q,
 * block_size 16 or 32, head_dim 64 or 128 with any q_len the bf16 path
 * takes, or head_dim 256 with one row; codes are widened to
 * bfloat16 exactly, k_scale folds into the score scale and v_scale into the
 * outputs.
 */
pa_status pa_decode(const pa_shape* shape, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_table,
                    const int32_t* context_lens, int32_t num_splits, void* out,
                    float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same computation, kernels and arguments as pa_decode;
 * the split partials and arrival counters live in a library-owned 64 MiB
 * device array (one per device, held until the process ends) instead of a
 * workspace.  The call allocates nothing.  A shape and split count whose
 * workspace (pa_decode_workspace_size) exceeds 64 MiB gives PA_ERR_SCRATCH,
 * with nothing launched.  Counters that an in-kernel merge needs and that an
 * earlier call may have overwritten are zeroed with a fill kernel on `stream`
 * first (at most one extra launch, when the row count grows).  Every call on
 * a device shares that device's array: calls that overlap on one device (other
 * streams, other host threads without ordering) race and give wrong results;
 * a faulted call leaves it in an unknown state.
 */
pa_status pa_decode_static(const pa_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* context_lens, int32_t num_splits, void* out,
                           float* lse, void* stream);

/*
 * MLA latent decode: every query head attends to one shared latent row per
 * token (the "Multi-head Latent Attention (MLA)" search page and the
 * FlashMLA-ETAP related-papers page, their MLA abstracts: MLA compresses the
 * KV cache into a latent vector and caches only it).  Keys are whole latent
 * rows (head_dim wide), values their first head_dim_v entries, read from the
 * same memory.  num_kv_heads must be 1.  Supported: PA_BF16, head_dim 576,
 * head_dim_v 512, num_q_heads 16, 32 or a multiple of 64; block_size 64, or
 * block_size 1: then block_table[b] is a per-sequence list of token (row)
 * ids, as a sparse top-k selection produces (the "llms-attention" post, its
 * DeepSeek V4 note on CSA and HCA: attention over the top 1024 entries plus
 * a 128-entry window, or densely over every entry), and a split may hold at
 * most 2048 tokens (PA_ERR_UNSUPPORTED for an explicit num_splits that needs
 * more; the heuristic never does).  Any q_len up to 16; its rows run as
 * further head groups, each with its own causal end.  FP8 latent caches
 * (kv_dtype PA_FP8_E4M3, one code per element, rows of 576 bytes): PA_BF16
 * q, the same head counts and block sizes; a key is k_scale times the row's
 * values, a value v_scale times its first 512 (codes widened to bfloat16
 * exactly in LDS, k_scale folded into the score scale, v_scale into the
 * outputs).
 */
pa_status pa_decode_mla(const pa_shape* shape, const void* q, const void* kv_cache,
                        const int32_t* block_table, const int32_t* context_lens,
                        int32_t num_splits, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * The two steps of the split-KV method as separate launches, so a caller can
 * time them, or gather partials computed elsewhere (for example other
 * devices' page ranges) before reducing.  The partial step writes every split
 * partial into `workspace` (or, when S resolves to 1, out/lse directly) and
 * does not touch the counters.
 * pa_reduce merges them: M = max_s lse_s, w_s = exp(lse_s - M),
 * out = sum_s w_s o_s / sum_s w_s, lse = M + ln(sum_s w_s) (the "flash
 * decoding ++" entry, the third of its three steps: rescale the split results
 * by their log-sum-exp and reduce).
 * pa_reduce with S == 1 does nothing and returns PA_OK.
 */
pa_status pa_decode_partial(const pa_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* context_lens, int32_t num_splits, void* out,
                            float* lse, void* workspace, size_t workspace_bytes,
                            void* stream);

pa_status pa_decode_mla_partial(const pa_shape* shape, const void* q, const void* kv_cache,
                                const int32_t* block_table, const int32_t* context_lens,
                                int32_t num_splits, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);

pa_status pa_reduce(const pa_shape* shape, const int32_t* context_lens, int32_t num_splits,
                    int32_t mla, const void* workspace, size_t workspace_bytes, void* out,
                    float* lse, void* stream);

/*
 * Paged KV append: write one new token per sequence into the cache at the
 * position that token takes, the step that precedes a decode call (the
 * "paged attention" search page, its vLLM README snippets: KV memory managed
 * in fixed pages through a block table).  With n = context_lens[b], the length BEFORE the append:
 *     page = block_table[b * max_blocks_per_seq + n / block_size]
 *     slot = n % block_size
 *     k_cache[page][g][slot][:]  = k_new[b][g][:]        g < num_kv_heads
 *     v_cache[page][g][:][slot]  = v_new[b][g][:]
 * after which a decode with context_lens[b] + 1 sees the token.  The caller
 * increments context_lens; the library does not.  k_new is
 * [batch][num_kv_heads][head_dim], v_new [batch][num_kv_heads][head_dim_v],
 * both dtype, device memory.  A sequence whose n is negative or not below
 * max_blocks_per_seq * block_size, or whose page id is outside
 * [0, num_blocks), writes nothing.  Any head dims; no workspace; scale and
 * num_q_heads are not used.  Errors: PA_ERR_INVALID for a bad shape or a NULL
 * pointer, PA_ERR_UNSUPPORTED for batch or num_kv_heads above 65535,
 * PA_ERR_HIP for a failed launch.
 */
pa_status pa_append_kv(const pa_shape* shape, const void* k_new, const void* v_new,
                       void* k_cache, void* v_cache, const int32_t* block_table,
                       const int32_t* context_lens, void* stream);

/*
 * MLA variant: kv_cache[page][slot][:] = c_new[b][:], c_new [batch][head_dim]
 * (the whole latent row: keys and values come from the same memory).
 * num_kv_heads must be 1.  With kv_dtype PA_FP8_E4M3, c_new holds the codes
 * (one byte per element) and the layout must be one the FP8 latent decode
 * reads (head_dim 576, block_size 64 or 1), else PA_ERR_UNSUPPORTED.
 * Otherwise as pa_append_kv.
 */
pa_status pa_append_latent(const pa_shape* shape, const void* c_new, void* kv_cache,
                           const int32_t* block_table, const int32_t* context_lens,
                           void* stream);

/*
 * Measurement helper, not part of the method: read `bytes` of device memory
 * at `src` with the streaming 128-bit loads the KV gather uses, on `stream`,
 * so a benchmark can report the read bandwidth this device reaches next to
 * its published HBM peak (the pages' roofline is the time to read the KV
 * cache from memory: the "flash decoding ++" entry, its upper-bound snippet).
 * `sink` is one caller-owned device word, written only in the (practically
 * impossible) case that the folded data equals a fixed constant, so the reads
 * cannot be optimised away and nothing is written.  `bytes` must be a
 * positive multiple of 16 and `src` 16-byte aligned (PA_ERR_INVALID
 * otherwise); PA_ERR_HIP on a failed launch.
 */
pa_status pa_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
