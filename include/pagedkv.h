/*
 * pagedkv.h — C ABI of libpagedkv.so: paged decode attention for gfx950 (MI355X).
 *
 * The operations follow the PagedAttention mechanism described on these pages:
 *   [blog]  "vLLM 部署与 PagedAttention 原理 · 检索整理（CSDN 频道批次）", item 2
 *           (the 2023 vLLM blog): the KV cache is cut into fixed-size token
 *           blocks reached through a per-sequence block table; blocks are taken
 *           on demand, so only the last block of a sequence wastes space;
 *           reference counts and copy-on-write let parallel samples share
 *           prompt blocks.
 *   [repo]  "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐 LLM 推理引擎",
 *           §2.1 PagedAttention: a block holds BLOCK_SIZE tokens of one head
 *           (16 x 128 = 2048 elements); the kernel computes QK dot products, a
 *           softmax normalisation and the weighted accumulation of V.
 *   [stack] "vLLM：从 PagedAttention 长出来的开源服务栈，200+ 模型架构与五维并行",
 *           section "把显存当虚拟内存管": logical-to-physical block mapping,
 *           non-contiguous physical blocks, waste confined to the last block.
 *
 * Conventions for every function below:
 *   - Data pointers are DEVICE pointers unless marked "host".  Bases must be
 *     16-byte aligned (256-byte alignment recommended).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     device work is enqueued asynchronously on it; the library never
 *     synchronises, never allocates device memory and keeps no state between
 *     calls (the block manager object is the one host-side exception).
 *   - Argument errors a host can see are reported by the return value BEFORE
 *     anything is launched.  The library never aborts or throws across the ABI.
 *   - Contents of device arrays (block ids, slots, context lengths) are the
 *     caller's contract and are not checked on the fast path.  Values outside
 *     the pool never cause an out-of-bounds access: a block id outside
 *     [0, num_blocks) is read from block 0 instead (that sequence's output is
 *     then unspecified) and an out-of-range slot or block pair is skipped.
 *
 * KV page layout (element offsets; one element = 2 bytes).  k_cache and v_cache
 * are separate buffers of pkv_cache_bytes() each.  Page (b, h) — block b, KV
 * head h — starts at element (b * num_kv_heads + h) * 2048.  Inside a page,
 * token t in [0,16) and dimension d in [0,128):
 *   K: (d / 8) * 128 + t * 8 + (d % 8)
 *   V: ((d / 16) / 2) * 512 + (16 * (t / 4) + d % 16) * 8 + ((d / 16) % 2) * 4 + t % 4
 * (integer division).  With these, each 64-lane wave reads a page as four fully
 * contiguous 1 KiB loads of 16 bytes per lane, and the bytes a lane receives
 * are the operand fragments of the 16x16x32 (K) and 16x16x16 (V) matrix-core
 * instructions; see pkv_k_index / pkv_v_index.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = 1,       /* bad argument: null pointer, bad count, small workspace, ... */
  PKV_ERR_UNSUPPORTED = 2,   /* block_size != 16, head_size != 128, unknown dtype */
  PKV_ERR_DEVICE = 3,        /* a HIP launch or runtime call failed */
  PKV_ERR_OUT_OF_BLOCKS = 4  /* block manager: the free list cannot cover the request */
} pkv_status;

typedef enum { PKV_F16 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

/* Shape of one layer's paged KV cache. */
typedef struct {
  int32_t num_blocks;   /* physical pool size */
  int32_t block_size;   /* tokens per block; must be 16 */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_size;    /* must be 128 */
  int32_t dtype;        /* pkv_dtype of the cache.  PKV_F16 / PKV_BF16: also the
                           dtype of q, out and the new k/v rows.  PKV_FP8_E4M3:
                           see the fp8 section below. */
} pkv_cache_desc;

/* Bytes of ONE of k_cache / v_cache: num_blocks * num_kv_heads * 2048 * element
 * bytes (2, or 1 for PKV_FP8_E4M3).  Returns 0 for an invalid or unsupported
 * descriptor. */
size_t pkv_cache_bytes(const pkv_cache_desc* cache);

/* Element offset of (block, head, token, dim) inside k_cache / v_cache, from the
 * layout formulas above (the fp8 formulas below for a PKV_FP8_E4M3 cache,
 * where an element is one byte).  -1 on out-of-range arguments.  Host-only
 * helpers. */
int64_t pkv_k_index(const pkv_cache_desc* cache, int32_t block, int32_t head, int32_t token, int32_t dim);
int64_t pkv_v_index(const pkv_cache_desc* cache, int32_t block, int32_t head, int32_t token, int32_t dim);

/* ---------------------------------------------------------------------------
 * paged_attn_decode — one query token per sequence attends to all
 * context_lens[s] tokens of its sequence ([repo] §2.1: QK dot products,
 * softmax normalisation, weighted sum of V), reading K/V pages through the
 * block table ([blog] item 2, [stack]).
 *
 *   out[s, h, :] = sum_t softmax_t(scale * q[s,h,:] . K[s,t,kvh,:]) * V[s,t,kvh,:]
 *   with kvh = h / (num_heads / num_kv_heads) and t < context_lens[s].
 *
 *   out           [num_seqs, num_heads, 128]   cache dtype, written (round to nearest even)
 *   q             [num_seqs, num_heads, 128]   cache dtype
 *   k_cache/v_cache                            pages as documented above
 *   block_tables  int32 [num_seqs, max_blocks_per_seq], row-major; entry j of
 *                 row s is the physical block of tokens 16j..16j+15.  Entries
 *                 at j >= ceil(context_lens[s] / 16) are never read.
 *   context_lens  int32 [num_seqs]; 1 <= context_lens[s] <= 16*max_blocks_per_seq
 *                 (a length of 0 yields a zero output row; longer lengths are
 *                 clamped to the table).
 *   scale         multiplies the logits before the softmax.
 *   num_kv_heads  must equal cache->num_kv_heads and divide num_heads.
 *   partition_tokens  0 = automatic; otherwise a multiple of 16 in [16, 4096]:
 *                 each sequence's context is cut into segments of this many
 *                 tokens; one work-group processes a segment, and a sequence
 *                 with several segments has their softmax statistics merged by
 *                 a log-sum-exp reduce kernel.  The automatic length depends
 *                 on the shapes only (never on the GPU or the lengths).
 *   workspace     device scratch of at least paged_attn_decode_workspace_size()
 *                 bytes, 16-byte aligned (NULL only when that size is 0).
 *                 Owned by the caller; contents on entry are irrelevant: the
 *                 call first writes the work list of this batch there (a
 *                 one-work-group pre-pass over context_lens), then the segment
 *                 partials.
 * Calls on one stream are ordered; two calls sharing a workspace on different
 * streams race.  num_seqs == 0 is a no-op.
 * ------------------------------------------------------------------------- */
pkv_status paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             float scale, int32_t num_kv_heads,
                             int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                             const pkv_cache_desc* cache, int32_t partition_tokens,
                             void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_decode split in two, for callers that decode several layers of
 * one batch: the work list depends only on context_lens and the shapes, so
 * paged_attn_decode_plan writes it into the workspace once, and
 * paged_attn_decode_run then runs the attention of any number of layers (each
 * with its own out, q and caches) from it.  Every run must use the same
 * workspace, num_seqs, num_heads, max_blocks_per_seq, cache shape,
 * partition_tokens and context_lens contents as the plan, and must follow it
 * on the same stream (or be ordered after it); runs sharing one workspace
 * must not overlap.  Arguments and errors as for paged_attn_decode. */
pkv_status paged_attn_decode_plan(const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                  int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                  int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                                  void* stream);
pkv_status paged_attn_decode_run(void* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 float scale, int32_t num_kv_heads,
                                 int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                 const pkv_cache_desc* cache, int32_t partition_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_decode_read_pages — a diagnostic: the page reads of
 * paged_attn_decode_run alone.  With the work list that paged_attn_decode_plan
 * wrote into `workspace` (same arguments), it runs the decode call's work
 * items, wave ranges and load instructions over every live K and V page of
 * the batch, with no dot products, softmax or output: its duration is the
 * ceiling the memory system puts on paged_attn_decode_run for this batch
 * ([repo] §2.1: the kernel's efficiency rests on how it reads the cache).
 *   sink   device uint32, 16-byte aligned; written only in the (practically
 *          never) case that the folded page words equal one fixed value.
 * 16-bit or fp8 caches; errors as paged_attn_decode_run. */
pkv_status paged_attn_decode_read_pages(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                        int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                        int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                                        uint32_t* sink, void* stream);

/* paged_attn_decode_noalloc — for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same call as paged_attn_decode without the workspace
 * arguments.  The work list and the segment partials live in a scratch array
 * inside the library, PKV_NOALLOC_SCRATCH_BYTES per GPU, reserved on every GPU
 * the library is loaded on and held until the process ends; its address is
 * looked up once per device on the first call made with that device current.
 * No hipMalloc/hipFree or other allocation happens in the call.
 *   - PKV_ERR_INVALID when paged_attn_decode_workspace_size() of these
 *     arguments exceeds PKV_NOALLOC_SCRATCH_BYTES (use paged_attn_decode with
 *     a caller workspace then), besides paged_attn_decode's own errors;
 *   - PKV_ERR_DEVICE if the scratch address cannot be obtained.
 * Every call on one GPU shares that GPU's scratch, and the run reads what the
 * call's own plan wrote there: calls that overlap on one GPU (two streams,
 * or two host threads) race and must be serialised by the caller.  Nothing in
 * the scratch has to start at any value. */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pkv_status paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     float scale, int32_t num_kv_heads,
                                     int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                     const pkv_cache_desc* cache, int32_t partition_tokens, void* stream);

/* Workspace bytes paged_attn_decode needs for these arguments: the work list
 * (up to 4096 sequences) and, when a sequence can span several segments, the
 * fp32 segment partials.  (size_t)-1 for invalid arguments. */
size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_heads,
                                        int32_t max_blocks_per_seq, int32_t partition_tokens,
                                        const pkv_cache_desc* cache);

/* Segment length in tokens that paged_attn_decode uses for these arguments
 * (resolves partition_tokens == 0).  -1 for invalid arguments. */
int32_t paged_attn_decode_partition_tokens(int32_t num_seqs, int32_t num_heads,
                                           int32_t max_blocks_per_seq, int32_t partition_tokens,
                                           const pkv_cache_desc* cache);

/* ---------------------------------------------------------------------------
 * reshape_and_cache — the slot-mapped cache write: for every token i with
 * slot_mapping[i] >= 0, the K and V rows of every KV head are written to block
 * slot / 16, offset slot % 16 ([blog] item 2: blocks are filled as tokens
 * arrive; the slot encoding block * 16 + offset is this library's convention).
 *
 *   k, v          [num_tokens, num_kv_heads, 128] cache dtype, contiguous
 *   slot_mapping  int32 [num_tokens]; negative = padding, skipped (so is a slot
 *                 >= num_blocks * 16); slots must be unique (two tokens writing
 *                 one slot race)
 * Bit-exact copy of the input bits.  num_tokens == 0 is a no-op.
 * ------------------------------------------------------------------------- */
pkv_status reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                             const int32_t* slot_mapping, int32_t num_tokens,
                             const pkv_cache_desc* cache, void* stream);

/* ---------------------------------------------------------------------------
 * copy_blocks — the copy-on-write block copy ([blog] item 2: a block shared
 * by parallel samples is copied before one of them writes to it).  For every
 * pair (src, dst) the whole block — all 16 slots of every KV head, K and V —
 * of src is copied to dst.
 *
 *   block_pairs   int32 [num_pairs, 2] row-major (src, dst); every dst distinct
 *                 and no dst equal to any src (else the copies race)
 * Bit-exact.  num_pairs == 0 is a no-op.
 * ------------------------------------------------------------------------- */
pkv_status copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                       const pkv_cache_desc* cache, void* stream);

/* ---------------------------------------------------------------------------
 * swap_blocks — whole blocks moved between two caches of one shape (the
 * number of blocks may differ), typically the device pool and a pool in pinned
 * host memory ([stack] "把显存当虚拟内存管": blocks can be swapped out when
 * device memory runs short, and back in).  For every pair (src, dst) block src
 * of (src_k, src_v) — all Hkv pages of K and of V — is copied to block dst of
 * (dst_k, dst_v).
 *
 *   dst_k/dst_v, src_k/src_v  device memory or pinned host memory (hipHostMalloc,
 *                 torch pin_memory); the GPU reads and writes host memory through
 *                 its device mapping, one launch for all pairs.  Pageable host
 *                 memory and unknown pointers are refused with PKV_ERR_INVALID
 *                 before anything is launched.
 *   block_pairs   int32 [num_pairs, 2] (src, dst), device or pinned host memory;
 *                 a pair with a block outside its pool is skipped; every dst
 *                 distinct (else the copies race)
 *   caches        same block_size, head_size, num_kv_heads and dtype
 * Bit-exact.  num_pairs == 0 is a no-op.
 * ------------------------------------------------------------------------- */
pkv_status swap_blocks(void* dst_k, void* dst_v, const pkv_cache_desc* dst_cache, const void* src_k,
                       const void* src_v, const pkv_cache_desc* src_cache, const int32_t* block_pairs,
                       int32_t num_pairs, void* stream);

/* ---------------------------------------------------------------------------
 * gather_cache — inspection helper: paged K/V of each sequence copied to a
 * contiguous [tokens, num_kv_heads, 128] array in logical token order.
 * Sequence s occupies rows out_offsets[s] .. out_offsets[s] + context_lens[s].
 *   out_offsets   int32 [num_seqs] (device)
 * Bit-exact.
 * ------------------------------------------------------------------------- */
pkv_status gather_cache(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens,
                        int32_t num_seqs, int32_t max_blocks_per_seq, const int32_t* out_offsets,
                        const pkv_cache_desc* cache, void* stream);

/* ---------------------------------------------------------------------------
 * fp8 KV cache ([repo] §三: the KV cache itself can be stored quantised; the
 * format and the scaling below are this library's reading).
 *
 * A PKV_FP8_E4M3 cache stores one byte per element: the OCP 8-bit floating-
 * point E4M3 code (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 holds subnormals (m/8) * 2^-6; no infinities; S.1111.111 is
 * NaN; largest finite magnitude 448).  K and V each have a float32 scale,
 * one per cache or one per KV head: the value a K code of head h stands for
 * is E4M3(code) * k_scale (or * k_head_scales[h]), and likewise for V.
 * Writing x gives the code nearest to the float32 quotient x / scale (one
 * correctly rounded float32 division), ties to the even mantissa, magnitudes
 * of 448 and beyond saturated to +-448, the sign of zero kept.  Queries,
 * outputs and the new k/v rows stay fp16 or bf16 (act_dtype).
 *
 * fp8 page layout (byte offsets; page (b, h) starts at byte (b*Hkv + h)*2048):
 *   K: (d / 64) * 1024 + (16 * ((d / 8) % 4) + t) * 16 + ((d / 32) % 2) * 8 + d % 8
 *   V: (d / 64) * 1024 + (16 * (t / 4) + d % 16) * 16 + ((d / 32) % 2) * 8
 *        + ((d / 16) % 2) * 4 + t % 4
 * A wave reads a page as two contiguous 1 KiB loads; widened to 16 bits, the
 * 16 bytes a lane receives are its fragments of the 16-bit layout.
 *
 * copy_blocks, gather_cache (codes, one byte per element), pkv_cache_bytes,
 * pkv_k_index / pkv_v_index, paged_attn_decode_plan, _workspace_size and
 * _partition_tokens accept a PKV_FP8_E4M3 cache as they are.
 * paged_attn_decode / _run and reshape_and_cache return PKV_ERR_UNSUPPORTED
 * for it: use the _fp8 entry points, which take the scales.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t act_dtype; /* PKV_F16 or PKV_BF16: dtype of q, out and the new k/v rows */
  float k_scale;     /* one K scale for the cache: finite and > 0 (ignored when k_head_scales is set) */
  float v_scale;     /* one V scale for the cache: finite and > 0 (ignored when v_head_scales is set) */
  /* Optional per-KV-head scales: NULL, or a device float32 array
   * [num_kv_heads] whose element h is the scale of every K (V) row of KV head
   * h in every block, replacing k_scale (v_scale).  4-byte aligned; the
   * values must be finite and > 0 (caller's contract, checked under
   * PKV_VALIDATE=1).  K and V choose independently. */
  const float* k_head_scales;
  const float* v_head_scales;
} pkv_fp8_scales;

/* reshape_and_cache into an fp8 cache: the rows (act_dtype) are encoded as
 * described above.  Arguments and errors otherwise as reshape_and_cache. */
pkv_status reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                                 const int32_t* slot_mapping, int32_t num_tokens,
                                 const pkv_cache_desc* cache, const pkv_fp8_scales* scales, void* stream);

/* paged_attn_decode over an fp8 cache: the same attention over the rows'
 * values E4M3(code) * scale, in fp32 on the GPU; q and out are act_dtype.
 * Arguments, workspace and errors otherwise as paged_attn_decode; the _run
 * form pairs with paged_attn_decode_plan as paged_attn_decode_run does. */
pkv_status paged_attn_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 float scale, int32_t num_kv_heads,
                                 int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                 const pkv_cache_desc* cache, const pkv_fp8_scales* scales,
                                 int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                                 void* stream);
pkv_status paged_attn_decode_run_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     float scale, int32_t num_kv_heads,
                                     int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                     const pkv_cache_desc* cache, const pkv_fp8_scales* scales,
                                     int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* decode_step_prologue — what a decode step runs before its attention, in one
 * launch: copy_blocks(block_pairs), then reshape_and_cache(k, v,
 * slot_mapping), then paged_attn_decode_plan(context_lens, ...) into the
 * workspace ([blog] item 2: a block shared by parallel samples is copied
 * before a sample writes into it).  Arguments, contracts and results are
 * those of the three calls in that order (then call paged_attn_decode_run
 * with the same workspace), with one more condition: a token written into the
 * SOURCE block of a pair lies at an offset that is also written in that
 * pair's destination.  A decode step satisfies it: the samples that share a
 * partial block append at the same position, the copies into their fresh
 * blocks and the last sample in place.  16-bit caches (PKV_ERR_UNSUPPORTED
 * for an fp8 cache: decode_step_prologue_fp8 below is its form).  With more
 * than 65,536 tokens the three kernels are launched separately (the fused
 * copy reads the whole slot mapping per copied page).  num_pairs == 0,
 * num_tokens == 0 and num_seqs == 0 are allowed. */
pkv_status decode_step_prologue(const void* k, const void* v, void* k_cache, void* v_cache,
                                const int32_t* slot_mapping, int32_t num_tokens,
                                const int32_t* block_pairs, int32_t num_pairs,
                                const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                                void* stream);
/* The same for an fp8 cache: copy_blocks, then reshape_and_cache_fp8(k, v,
 * slot_mapping, scales), then the plan, in one launch.  A copied page that
 * receives new tokens gets their E4M3 codes from the same encoding as the
 * write (each element divided by its row's scale, then rounded to E4M3), so
 * the result is bit-identical to the three calls.  scales: as
 * reshape_and_cache_fp8 (PKV_ERR_INVALID when null or for a 16-bit cache);
 * everything else as decode_step_prologue. */
pkv_status decode_step_prologue_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int32_t num_tokens,
                                    const int32_t* block_pairs, int32_t num_pairs,
                                    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                    int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                    const pkv_fp8_scales* scales, int32_t partition_tokens,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * paged_attn_prefill — multi-token-query attention over the paged cache, for
 * chunked prefill ([repo] §2.2: the prefill of a long prompt is cut into
 * chunks that run alongside decode; the causal reading below is this
 * library's).  Sequence s has context_lens[s] tokens in the cache, the last
 * C_s = query_start[s+1] - query_start[s] of which are its chunk (already
 * written by reshape_and_cache).  Chunk query j sits at position
 * p = context_lens[s] - C_s + j and attends to cache tokens 0..p:
 *
 *   out[query_start[s] + j, h, :] =
 *       sum_{t <= p} softmax_t(scale * q[query_start[s]+j, h, :] . K[s,t,kvh,:]) V[s,t,kvh,:]
 *
 *   q, out           [num_query_tokens, num_heads, 128], cache dtype (16-bit
 *                    caches) or act_dtype (fp8 form)
 *   query_start      int32 [num_seqs + 1], non-decreasing, query_start[0] = 0,
 *                    query_start[num_seqs] = num_query_tokens, C_s <= context_lens[s]
 *   max_query_len    >= every C_s (sizes the grid; queries of a longer chunk
 *                    past max_query_len are not written)
 *   other arguments  as paged_attn_decode; the workspace holds fp32 segment
 *                    partials per (query token, head) when a work-group's key
 *                    range spans several segments; its size is
 *                    paged_attn_prefill_workspace_size().
 * One work-group takes 128 (query position, head) rows of one KV head (two
 * 16-row tiles per wave) and streams the keys up to its last position on the
 * matrix cores; keys beyond a row's position are masked.  Tolerance and
 * errors as decode.
 * ------------------------------------------------------------------------- */
size_t paged_attn_prefill_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                         int32_t num_query_tokens, int32_t max_query_len,
                                         int32_t partition_tokens, const pkv_cache_desc* cache);
pkv_status paged_attn_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              const int32_t* query_start, float scale, int32_t num_kv_heads,
                              int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                              int32_t num_query_tokens, int32_t max_query_len,
                              const pkv_cache_desc* cache, int32_t partition_tokens,
                              void* workspace, size_t workspace_bytes, void* stream);
/* The same over an fp8 cache (see the fp8 section above). */
pkv_status paged_attn_prefill_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* query_start, float scale, int32_t num_kv_heads,
                                  int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  int32_t num_query_tokens, int32_t max_query_len,
                                  const pkv_cache_desc* cache, const pkv_fp8_scales* scales,
                                  int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                                  void* stream);

const char* pkv_status_string(pkv_status s);
const char* pkv_version(void);

/* ---------------------------------------------------------------------------
 * Host block manager ([blog] item 2; [stack] "把显存当虚拟内存管").  Pure host
 * code; no GPU needed.  Sequences are identified by caller-chosen int32 ids.
 *
 *   - the free list starts as free_order (a permutation of 0..num_blocks-1;
 *     NULL = 0,1,2,...) and blocks are taken from its front; freed blocks are
 *     appended to its back in block-table order;
 *   - add: a new sequence with num_tokens tokens takes ceil(num_tokens/16)
 *     blocks (ref = 1) and writes their slots (block*16 + offset) to slots_out
 *     (host, may be NULL);
 *   - fork: child shares every block of parent (ref += 1 each);
 *   - append_slot: room for one more token.  At a block boundary a fresh block
 *     is taken; otherwise if the last block is shared (ref > 1) a fresh block
 *     replaces it in this sequence's table, the pair (old, new) is reported for
 *     copy_blocks and the old block's ref drops by one (so the last sharer to
 *     append writes in place);
 *   - step: append_slot for each listed sequence in order, all or nothing;
 *   - free: ref -= 1 for each block; blocks reaching 0 return to the free list.
 * Every call either succeeds completely or returns an error without changing
 * state (PKV_ERR_OUT_OF_BLOCKS when the free list is short, PKV_ERR_INVALID
 * for unknown/duplicate ids or bad sizes).
 * ------------------------------------------------------------------------- */
typedef struct pkv_block_manager pkv_block_manager;

/* free_order: host int32 [num_blocks] or NULL.  Returns NULL on bad arguments. */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order);
void pkv_bm_destroy(pkv_block_manager* bm);

pkv_status pkv_bm_add(pkv_block_manager* bm, int32_t seq, int32_t num_tokens, int32_t* slots_out);
pkv_status pkv_bm_fork(pkv_block_manager* bm, int32_t parent, int32_t child);
/* slot_out: host int32; cow_pair_out: host int32[2], (-1, -1) when no copy. */
pkv_status pkv_bm_append_slot(pkv_block_manager* bm, int32_t seq, int32_t* slot_out, int32_t* cow_pair_out);
/* slot_mapping_out: host int32 [n]; pairs_out: host int32 [n][2] capacity;
 * num_pairs_out: host int32. */
pkv_status pkv_bm_step(pkv_block_manager* bm, const int32_t* seqs, int32_t n,
                       int32_t* slot_mapping_out, int32_t* pairs_out, int32_t* num_pairs_out);
pkv_status pkv_bm_free(pkv_block_manager* bm, int32_t seq);
/* table_out: host int32 [n][max_blocks], -1 padded; context_lens_out: host
 * int32 [n] or NULL.  PKV_ERR_INVALID if a sequence has more than max_blocks. */
pkv_status pkv_bm_block_table(const pkv_block_manager* bm, const int32_t* seqs, int32_t n,
                              int32_t max_blocks, int32_t* table_out, int32_t* context_lens_out);
/* blocks available to new allocations: the free list plus the evictable blocks
 * of the prefix cache */
int32_t pkv_bm_num_free(const pkv_block_manager* bm);
int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block);   /* -1 if out of range */
int32_t pkv_bm_length(const pkv_block_manager* bm, int32_t seq);       /* -1 if unknown */
int32_t pkv_bm_num_seq_blocks(const pkv_block_manager* bm, int32_t seq); /* -1 if unknown */
/* allocated-but-unused slots of one sequence (at most 15); -1 if unknown */
int32_t pkv_bm_waste(const pkv_block_manager* bm, int32_t seq);
/* free list contents front to back (evictable blocks not included): host int32
 * [capacity]; returns the free list's length */
int32_t pkv_bm_free_list(const pkv_block_manager* bm, int32_t* out, int32_t capacity);

/* Prefix caching across requests ([repo] §2.2: the KV cache of an identical
 * prefix, such as a system prompt, is computed once and reused by later
 * requests; the policy below is this library's reading).
 *   - A full block whose token ids are known is registered under the key
 *     (its chain's previous block, its 16 token ids); the key of a block thus
 *     names its whole token prefix.  Only full blocks are registered.
 *   - add_cached: a new sequence with token_ids (host int32 [num_tokens])
 *     reuses the longest run of registered full blocks matching its first
 *     tokens (refcount + 1), takes fresh blocks for the rest, registers its
 *     fresh full blocks, and reports in num_cached_out the tokens whose K/V are
 *     already in the cache (a multiple of 16: only the other tokens need the
 *     slot-mapped write); slots_out as for pkv_bm_add.
 *   - append_token: append_slot for a token with a known id; the block it
 *     completes is registered (unless that content is registered already).
 *     pkv_bm_append_slot / pkv_bm_step append tokens without ids: a
 *     sequence's blocks after such a token are never registered.
 *   - A registered block whose refcount drops to 0 is evictable, not free: a
 *     later hit revives it; allocations take free-list blocks first and then
 *     evict the least recently freed evictable block, dropping its key.
 *   - Sequences added with pkv_bm_add register nothing: without add_cached /
 *     append_token the manager behaves exactly as described above.
 * Errors and all-or-nothing behaviour as for the other calls. */
pkv_status pkv_bm_add_cached(pkv_block_manager* bm, int32_t seq, int32_t num_tokens, const int32_t* token_ids,
                             int32_t* slots_out, int32_t* num_cached_out);
pkv_status pkv_bm_append_token(pkv_block_manager* bm, int32_t seq, int32_t token_id, int32_t* slot_out,
                               int32_t* cow_pair_out);
int32_t pkv_bm_num_evictable(const pkv_block_manager* bm);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
