/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) DeepSeek MLA decode library.
 *
 * The operation (one query token per sequence, one latent KV head shared by
 * all query heads):
 *
 *   z[b,h,j]  = softmax_scale * ( q_nope[b,h,:] . latent_j + q_pe[b,h,:] . rope_j )
 *   lse[b,h]  = ln sum_{j < L_b} exp(z[b,h,j])
 *   out[b,h,:] = sum_{j < L_b} exp(z[b,h,j] - lse[b,h]) * latent_j
 *
 * where row j of sequence b's cache holds latent_j (512 values) and rope_j
 * (64 values), L_b = cache_seqlens[b], and the value row is the latent part of
 * the same cache row.  Sources: the TileLang MLA guide ("用 TileLang 编写高性能
 * DeepSeek MLA 内核"), sections "先看核心难点" (Q/K width 576 = 512 + 64,
 * V width 512), "Split Kernel" (two products summed into one score tile, base-2
 * online softmax with softmax_scale*log2(e) folded in), "Combine Kernel"
 * (log-sum-exp merge of split partials), "变体内核" (paged cache through
 * block_table with positions at or past cache_seqlens masked); and the FlashMLA
 * analysis ("DeepSeek开源周第一天：FlashMLA 深度分析"), whose parameter struct
 * lists the fields carried by mla_desc below (strides, block_table,
 * page_block_size, split metadata, partial-output buffers).
 *
 * Conventions for every entry point
 *   - Device pointers are plain HIP device addresses; host pointers are marked.
 *   - The caller owns every buffer.  No call allocates device memory; the
 *     one static array the library holds (mla_decode_noalloc's scratch) is
 *     created with the code when the library loads on a GPU.
 *   - Work is enqueued on `stream` only; no call synchronises the device.
 *     Inputs must stay alive until the stream reaches the call.
 *   - Return value: MLA_OK (0) or a negative mla_status.  On an argument error
 *     nothing is enqueued.  mla_last_error() gives a thread-local message.
 *   - Nothing is thrown across the ABI.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad stride, ...   */
  MLA_ERR_UNSUPPORTED = -2,   /* dims other than 512/64, dtype, misalignment     */
  MLA_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required      */
  MLA_ERR_HIP = -4            /* a HIP runtime call or launch failed             */
} mla_status;

typedef enum mla_dtype {
  MLA_DTYPE_F16 = 0,          /* IEEE binary16 for q, cache and out              */
  MLA_DTYPE_BF16 = 1          /* bfloat16 for q, cache and out                   */
} mla_dtype;

/*
 * Storage of the KV cache (mla_desc.kv_dtype).  The TileLang MLA guide lists
 * an FP8 KV-cache variant among its kernels ("变体内核",
 * example_mla_decode_kv_fp8) without fixing the format; this library reads it
 * as OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities, S.1111.111 is NaN; largest finite value 448; PyTorch's
 * float8_e4m3fn) with one fp32 scale for the whole cache: a stored byte x
 * stands for the value decode(x) * kv_scale.  Queries and output keep
 * `dtype`; the products run on `dtype` MFMAs with the decoded bytes, which
 * both 16-bit types hold exactly, and kv_scale multiplies the scores and the
 * output.
 */
typedef enum mla_kv_dtype {
  MLA_KV_AS_DTYPE = 0,        /* the cache holds `dtype` values                  */
  MLA_KV_FP8_E4M3 = 1         /* the cache holds E4M3 bytes (see above)          */
} mla_kv_dtype;

/* Latent (value) width and RoPE width; the only supported sizes. */
#define MLA_D_LATENT 512
#define MLA_D_ROPE 64
/* Split planning works in blocks of this many cache rows. */
#define MLA_SPLIT_BLOCK_ROWS 64
/* Largest number of splits of one sequence. */
#define MLA_MAX_SPLITS 1024
/* Cache row strides (kv_sr, kpe_sr) and query head strides (q_nope_sh,
 * q_pe_sh) must be below this many elements: the kernel forms in-tile row
 * offsets (31 rows or heads) in 32-bit and 24-bit arithmetic. */
#define MLA_MAX_ROW_STRIDE (1 << 22)

/*
 * Problem description.  All strides are in ELEMENTS (of the input dtype; of
 * the cache's storage for the cache strides, bytes with an FP8 cache) and must
 * keep every row start 16-byte aligned (multiples of 8 elements, 16 bytes for
 * an FP8 cache); kv_sr, kpe_sr, q_nope_sh and q_pe_sh must be below
 * MLA_MAX_ROW_STRIDE (MLA_ERR_UNSUPPORTED otherwise).
 *
 * Contiguous cache (block_table == NULL):
 *   kv_latent[b, j, 0, :] at kv_latent + b*kv_sb + j*kv_sr      (512 values)
 *   k_pe     [b, j, 0, :] at k_pe      + b*kpe_sb + j*kpe_sr    (64 values)
 *   for j < max_seqlen; every cache_seqlens[b] must be <= max_seqlen.
 * Paged cache (block_table != NULL), FlashMLA-style pool [P, page, 1, 576]:
 *   logical row j of sequence b is row (j % page_block_size) of physical page
 *   p = block_table[b*block_table_stride + j/page_block_size]; its latent part
 *   is at kv_latent + p*kv_sb + (j % page)*kv_sr and its RoPE part at
 *   k_pe + p*kpe_sb + (j % page)*kpe_sr.  For a single pool pass
 *   kv_latent = pool, k_pe = pool + 512, kv_sb = kpe_sb = page*576,
 *   kv_sr = kpe_sr = 576.  page_block_size must be a positive multiple of 32.
 *   Only entries for j < cache_seqlens[b] are read; other entries may hold
 *   anything (e.g. -1).  Entries that are read must lie in [0, num_pages);
 *   one outside is clamped into the pool (see mla_check_block_table).
 *
 * Several query tokens per sequence (speculative / multi-token decode; the
 * FlashMLA analysis's parameter struct carries seqlen_q and is_causal):
 * seqlen_q = s > 1 (at most 16) gives each sequence s query tokens, and
 * `heads` counts query ROWS, s x (heads per token), token-major: row
 * v = t * (heads / s) + h is head h of token t, and q/out strides address
 * rows.  The s new tokens are the last s rows of the cache: token t
 * (0-based, the newest last) sees rows j < L - (s - 1 - t), none if that is
 * below 1.  heads must be a multiple of s.  seqlen_q 0 or 1 is plain decode.
 */
typedef struct mla_desc {
  int32_t batch;               /* B >= 0                                         */
  int32_t heads;               /* H >= 1 query heads (one shared KV head)        */
  int32_t d_latent;            /* must be 512                                    */
  int32_t d_rope;              /* must be 64                                     */
  int32_t dtype;               /* mla_dtype of q_nope, q_pe, cache and out       */
  int32_t max_seqlen;          /* contiguous: rows per sequence in the cache     */
  int32_t page_block_size;     /* paged: rows per page                           */
  int32_t block_table_stride;  /* paged: int32 entries per block_table row       */
  int32_t num_pages;           /* paged: pages in the pool (documents the bound) */
  int32_t seqlen_q;            /* query tokens per sequence (0 or 1: one)        */
  int64_t q_nope_sb, q_nope_sh;  /* q_nope[b,h,:]  at q_nope + b*sb + h*sh       */
  int64_t q_pe_sb, q_pe_sh;      /* q_pe[b,h,:]    at q_pe + b*sb + h*sh         */
  int64_t kv_sb, kv_sr;          /* latent: batch (or page) stride, row stride   */
  int64_t kpe_sb, kpe_sr;        /* rope:   batch (or page) stride, row stride   */
  int64_t out_sb, out_sh;        /* out[b,h,:]     at out + b*sb + h*sh          */
  /* Appended fields (a zero-filled struct keeps the 16-bit behaviour):      */
  int32_t kv_dtype;              /* mla_kv_dtype of kv_latent and k_pe          */
  float kv_scale;                /* FP8 cache: finite and > 0, value =
                                    decode(byte) * kv_scale.  A 16-bit cache:
                                    0 or 1 (anything else is
                                    MLA_ERR_INVALID_ARG)                        */
} mla_desc;

/*
 * Split plan (what the planner writes; all int32, device- or host-resident).
 * A "work item" is one KV range of one sequence for all heads:
 *   work[4*w + 0] = b, work[4*w + 1] = split index k within b,
 *   work[4*w + 2] = first cache row, work[4*w + 3] = one past the last row.
 *   num_splits[b] = s_b; split_offset[b] = index of b's first work item, and
 *   split_offset[B] = total work items W.
 * Ranges follow the TileLang guide's paged variant ("Split-KV" item of its
 * optimisation list: per-sequence blocks_per_split and remaining_blocks): the
 * nb = ceil(L_b / 64) blocks of sequence b are dealt out in order, split k
 * getting floor(nb / s_b) blocks plus one more when k < nb mod s_b.
 *
 * With seqlen_q = s > 1 the splits above cut only a prefix that every query
 * token sees: rows [0, Lp) with Lp the largest multiple of 32 not above
 * L - (s - 1) (0 if that is negative).  Two more splits, the tails, take rows
 * [Lp, min(Lp + 32, L)) and [min(Lp + 32, L), L) (the second may be empty), so
 * s_b = num_split + 2 in forced mode.
 *
 * How s_b is chosen (num_split == 0, "planner" mode) is this library's own
 * rule, meant to fill the compute units: one work item per CU is the target,
 * so the planner finds the smallest per-item block budget t with
 *   sum_b max(1, ceil(nb_b / t)) <= max(B, C),  C = ceil(num_cus / head_groups)
 * (C minus the 2B tail splits when seqlen_q > 1 and 8B <= C)
 * and sets s_b = max(1, ceil(nb_b / t)) (+2 for the tails), the prefix count
 * capped at MLA_MAX_SPLITS.  head_groups = ceil(H / 128) with H the query
 * rows; nb_b counts the prefix's blocks (the tails, one tile each, come on top).
 * With num_split > 0 every s_b = num_split (+2 for the tails), including splits
 * that end up empty.
 */

/* Number of compute units of `device` (queried once, cached). */
int mla_num_cus(int device, int32_t* num_cus_out /* host */);

/*
 * Upper bound on the work items a plan can have for this description
 * (tail = 2 when desc->seqlen_q > 1, else 0):
 *   num_split > 0 : B * (num_split + tail)
 *   num_split == 0: max(B, C) + B * tail, C as above
 */
int mla_max_work(const mla_desc* desc, int32_t num_split, int32_t num_cus, int32_t* max_work_out /* host */);

/*
 * Bytes of device workspace mla_decode needs for this description.  The
 * bound is derived here from the split mode and the CU count (a caller
 * cannot know in advance how many splits the planner will choose), and the
 * size comes back through bytes_out beside a status, like every call:
 *   plan (int32): B + (B+1) + 4*max_work, rounded to 256 bytes;
 *   partial lse (fp32, base 2): max_work * H, rounded to 256 bytes;
 *   partial rows (fp16, normalised): max_work * H * 512, rounded to 256 bytes;
 *   fp32 copies of partial rows: max_work * H * 512, rounded to 256 bytes
 *   (a split writes the fp32 copy of a row only when one of its values lies
 *   beyond +-1, so that storing it in fp16 would cost more than 2^-12).
 */
int mla_workspace_size(const mla_desc* desc, int32_t num_split, int32_t num_cus, size_t* bytes_out /* host */);

/*
 * Host twin of the planner: same integers as the device planner.  The plan
 * comes back in three caller arrays, the layout mla_decode keeps in its
 * workspace, rather than in one plan struct, so that the two compare
 * directly.
 *   heads          query rows (as desc->heads); seqlen_q as desc->seqlen_q
 *   cache_seqlens  host int32[batch]
 *   num_splits     host int32[batch]            (out)
 *   split_offset   host int32[batch + 1]        (out)
 *   work           host int32[4 * max_work]     (out)
 *   max_work       capacity of `work` in items; MLA_ERR_INVALID_ARG if too small.
 */
int mla_plan_host(const int32_t* cache_seqlens, int32_t batch, int32_t heads, int32_t seqlen_q,
                  int32_t num_split, int32_t num_cus, int32_t* num_splits, int32_t* split_offset, int32_t* work,
                  int32_t max_work);

/*
 * Device planner: one workgroup reads cache_seqlens (device int32[batch]) and
 * writes num_splits / split_offset / work (device arrays as in mla_plan_host),
 * the plan mla_decode_planned takes.
 */
int mla_plan_device(const int32_t* cache_seqlens, int32_t batch, int32_t heads, int32_t seqlen_q,
                    int32_t num_split, int32_t num_cus, int32_t* num_splits, int32_t* split_offset, int32_t* work,
                    int32_t max_work, hipStream_t stream);

/*
 * MLA decode.  All array arguments are device pointers.
 *   q_nope [B, H, 512], q_pe [B, H, 64]     dtype, strides in desc
 *   kv_latent, k_pe                         cache (see mla_desc)
 *   block_table  int32, NULL for a contiguous cache
 *   cache_seqlens int32[B]; the lengths stay on the device, so they are
 *                  clamped in the kernels rather than checked (no status
 *                  reports them, as none could without a host
 *                  synchronisation): a negative length counts as 0, and a
 *                  contiguous cache's lengths are capped at desc->max_seqlen;
 *                  a paged cache's block_table entries likewise are clamped
 *                  into the pool (mla_check_block_table finds bad ones)
 *   softmax_scale  multiplies the raw dot products (typically 1/sqrt(576));
 *                  must be finite and > 0 (MLA_ERR_INVALID_ARG otherwise)
 *   num_split  0 = planner chooses s_b per sequence; > 0 forces s_b = num_split
 *   out   [B, H, 512] dtype (strides in desc)
 *   lse   fp32 [B, H] contiguous, natural log of the sum of exp(z)
 *   workspace  device buffer of at least mla_workspace_size() bytes, 256-byte
 *              aligned; its contents on entry do not matter.
 * A sequence with L_b = 0 gets out = 0 and lse = -inf.
 * Launches: the split kernel (in planner mode each of its workgroups runs the
 * planner rule itself and workgroup 0 writes the plan into the workspace),
 * then the combine kernel when any sequence has s_b > 1 (a single split
 * writes out/lse directly).
 * Calls that share a workspace must be ordered on one stream.
 */
int mla_decode(const void* q_nope, const void* q_pe, const void* kv_latent, const void* k_pe,
               const int32_t* block_table, const int32_t* cache_seqlens, float softmax_scale,
               int32_t num_split, void* out, float* lse, const mla_desc* desc, void* workspace,
               size_t workspace_bytes, hipStream_t stream);

/*
 * MLA decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and launches as
 * mla_decode; the workspace is a static device array of
 * MLA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  Nothing in this call allocates.  A problem whose
 * workspace (mla_workspace_size) exceeds that size returns MLA_ERR_WORKSPACE
 * and enqueues nothing.  A partial row (one work item, one query row) takes
 * 3076 bytes of it, so 100 MiB holds about 34,000 of them: 256 work items of
 * 128 query rows, for example, which is what the planner gives B = 64..256
 * sequences of 128 heads on 256 CUs.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or other host threads) race and give wrong results.
 * Calls on one stream are ordered and safe; the array's contents carry no
 * meaning from one call to the next.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)100 << 20)
int mla_decode_noalloc(const void* q_nope, const void* q_pe, const void* kv_latent, const void* k_pe,
                       const int32_t* block_table, const int32_t* cache_seqlens, float softmax_scale,
                       int32_t num_split, void* out, float* lse, const mla_desc* desc, hipStream_t stream);

/*
 * MLA decode with a plan made beforehand, for callers that decode the same
 * batch through many layers: one mla_plan_device call per decode step, then
 * this call per layer, whose split kernel reads its work item from the plan
 * instead of running the planner rule (FlashMLA's metadata call, whose tile
 * scheduler metadata and split counts every decode call then takes, plays
 * the same part: the FlashMLA analysis, "内存访问优化" section).
 * Arguments as for mla_decode, except:
 *   num_splits, split_offset, work  device arrays as mla_plan_device wrote
 *              them (or mla_plan_host's, copied to the device) for this
 *              call's cache_seqlens, desc->heads, desc->seqlen_q and the
 *              num_split and num_cus the plan was made with
 *   max_work   the capacity the plan was made with: mla_max_work(desc,
 *              num_split, num_cus)
 *   workspace  at least mla_workspace_size(desc, num_split, num_cus) bytes
 *              for that same num_split and num_cus (its plan region goes
 *              unused)
 * The plan is device data and is not checked against cache_seqlens: every
 * field the kernels read from it is clamped into range (sequence index,
 * split index, row range, item count, split offsets), so a plan made for
 * other lengths gives wrong results, never an access outside the buffers.
 * With several query tokens the work items run in slot order, not tails
 * first as in mla_decode (balance across the XCDs only).  Errors as for
 * mla_decode, plus MLA_ERR_INVALID_ARG for NULL or misaligned plan arrays
 * and max_work < 1.
 */
int mla_decode_planned(const void* q_nope, const void* q_pe, const void* kv_latent, const void* k_pe,
                       const int32_t* block_table, const int32_t* cache_seqlens, float softmax_scale,
                       const int32_t* num_splits, const int32_t* split_offset, const int32_t* work,
                       int32_t max_work, void* out, float* lse, const mla_desc* desc, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * Block-table check (paged cache).  mla_decode reads block_table entries
 * without checking them on the host (they are device memory): an entry it
 * reads that lies outside [0, desc->num_pages) is clamped into the pool, so
 * the call reads valid memory but rows other than the ones meant, and
 * returns MLA_OK.  This call detects such tables: one small kernel counts,
 * for each sequence b, the entries mla_decode would read (j <
 * ceil(L_b / page_block_size), L_b clamped as mla_decode clamps it) that lie
 * outside the pool, and writes the count to bad[b].  Entries past a
 * sequence's length are not read and not counted.
 *   block_table, cache_seqlens  as for mla_decode (device)
 *   desc   batch, page_block_size, block_table_stride, num_pages are used
 *   bad    device int32[batch] (out)
 * Enqueued on `stream`; errors as for mla_decode (MLA_ERR_INVALID_ARG for
 * NULL pointers or bad paging fields).
 */
int mla_check_block_table(const int32_t* block_table, const int32_t* cache_seqlens, const mla_desc* desc,
                          int32_t* bad, hipStream_t stream);

/* Thread-local text for the last non-OK status returned on this thread. */
const char* mla_last_error(void);

/*
 * Kernel timing for measurement.  While enabled, every mla_decode call times
 * its launches on its stream from their dispatch packets (start and stop
 * events of the launch itself): split_ms the split kernel, combine_ms the
 * combine (0 when no combine runs).  Events on the dispatch packets slow
 * the launches down by a few percent; use them to split a call's time
 * between its kernels, not as the call's time.
 * mla_timing_read() synchronises on those events and returns the summed
 * milliseconds and the number of calls since the last read (then resets).
 * Up to 4096 calls are recorded between reads; later ones are not timed.
 */
int mla_timing_enable(int enable);
int mla_timing_read(float* split_ms, float* combine_ms, int32_t* calls);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
