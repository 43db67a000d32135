/*
 * msa.h -- C ABI of the MI355X (gfx950) Multi-Segment Attention library.
 *
 * Multi-Segment Attention (MSA) computes attention for a decode query, or a
 * chunk of prefill queries, over only the blocks of a paged KV cache that
 * survived lossless eviction.  The surviving blocks of each sequence are cut
 * into maximal physically-contiguous segments, attention runs over the
 * segments inside one launch, and the per-split partials are stitched by a
 * log-sum-exp normaliser.
 *   Source: "AsymCache：把 KV Cache 决策摆到 GPU 注意力内核的同一张桌子上"
 *   (papers.ananclaw.com explainer of arXiv 2606.02964), section
 *   "核心方法 / 1. Multi-Segment Attention (MSA)", its pseudocode (a split
 *   of the alive blocks into contiguous segments, attention per segment,
 *   results summed with a per-segment normaliser) and the paragraph after
 *   it; "Multi-Segment Attention: Enabling Efficient KV-Cache
 *   Management for Faster LLM Serving" (gptget.net), Methodology and Key
 *   Results (one kernel processes many disjoint segments).
 *
 * Conventions for every call
 *   - All array pointers are DEVICE pointers, owned by the caller; the
 *     library keeps none of them after the call returns.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the null stream).  MSA_OK means "validated and enqueued", not
 *     "finished".  No call synchronises with the host.
 *   - The library allocates no memory and keeps no state between calls.
 *     Scratch memory is a caller-provided `workspace` whose size comes from
 *     the matching *_workspace_size function.  Calls that share a workspace
 *     must be ordered on one stream.
 *   - Host-detectable argument errors return a negative msa_status before
 *     anything is enqueued.  Data errors that only the device can see are
 *     reported through a device error word (MSA_DEVERR_* bits): the plan
 *     overwrites its `dev_error`; decode and prefill OR their bit into the
 *     `dev_error` they are given (pass the plan's word to collect a whole
 *     plan + attention step in one place).  The kernels never read or write
 *     outside the buffers described here, whatever the data.
 *   - Logarithms are natural: LSE = ln(sum exp(score)), score = scale*q.k.
 *
 * Memory layouts (row-major, innermost last)
 *   K/V pool    [P, block_size, Hkv, D]   dtype; P = num_phys_blocks
 *               (token-major, MSA_LAYOUT_NHD: the default; the *_ex calls
 *               also take the head-major [P, Hkv, block_size, D],
 *               MSA_LAYOUT_HND, in which each KV head's rows of a block are
 *               one contiguous run)
 *   decode Q    [B, Hq, D]                dtype
 *   decode O    [B, Hq, D]                dtype;  LSE [B, Hq] float32
 *   prefill Q   [B, C, Hq, D]             dtype
 *   prefill O   [B, C, Hq, D]             dtype;  LSE [B, C, Hq] float32
 *   Query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
 *
 * Supported kernels: block_size 16; Hq/Hkv in {1, 2, 4, 8}; decode and
 * prefill in bfloat16 or float32 with D 64 or 128.  The tuned kernels cover
 * decode in bfloat16 (D 64, 128) and float32 (D 64) and prefill in bfloat16
 * with D 128; the other pairs (decode float32 D 128, prefill bfloat16 D 64,
 * prefill float32 D 64 and 128) run on a plain float32 vector-ALU kernel with
 * the same results and no throughput target.  Anything else returns
 * MSA_ERR_UNSUPPORTED (msa_attention_supported answers without launching).
 * The plan accepts any block_size >= 1.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_VERSION 2

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, Hq % Hkv != 0, ... */
  MSA_ERR_UNSUPPORTED = -2, /* dtype / head_dim / block_size / group size not built */
  MSA_ERR_CAPACITY = -3,    /* workspace or output capacity too small */
  MSA_ERR_DEVICE = -4       /* a HIP runtime call failed (launch error) */
} msa_status;

typedef enum { MSA_F32 = 0, MSA_BF16 = 1 } msa_dtype;

/* Order of the dimensions inside one pool block (see Memory layouts). */
typedef enum { MSA_LAYOUT_NHD = 0, MSA_LAYOUT_HND = 1 } msa_kv_layout;

/* Bits of the device error word. */
#define MSA_DEVERR_PHYS_RANGE 1 /* plan: an alive block's physical id is outside [0, P); it was treated as evicted */
#define MSA_DEVERR_CAPACITY 2   /* plan: more segments than seg_capacity; extra records dropped, indptr clamped */
#define MSA_DEVERR_CTX_RANGE 4  /* plan: ctx_len < 0 or > max_blocks*block_size; clamped into range */
#define MSA_DEVERR_TRUNCATED 8  /* decode/prefill: a sequence has more alive tokens than max_ctx_len
                                   allows for; its keys were cut at the grid's capacity */

/* Which decode kernel runs (msa_decode_ex).  AUTO picks per shape (see
 * msa_decode); VECTOR is the vector-ALU kernel (every supported shape);
 * MATRIX the matrix-core kernel with one workgroup per (sequence, KV head,
 * split), built for bf16 with D 128 and Hq/Hkv 4 or 8 only; BLOCK the
 * matrix-core kernel with one workgroup per work item that streams whole KV
 * blocks for all KV heads and, for up to 256 sequences, streams a prefix
 * that several sequences share (same first physical block at logical block
 * 0) once for up to 8 of them; built for bf16, D 128, Hkv 8, Hq/Hkv 4 or 8
 * and B <= 512 (MSA_ERR_UNSUPPORTED otherwise). */
typedef enum {
  MSA_DECODE_AUTO = 0,
  MSA_DECODE_VECTOR = 1,
  MSA_DECODE_MATRIX = 2,
  MSA_DECODE_BLOCK = 3
} msa_decode_kernel;

/* One segment: a maximal run of alive blocks of one sequence that are
 * consecutive both in logical index and in physical id.  24 bytes, plain
 * int32 fields.  Tokens of the segment sit at logical positions
 * logical_block*block_size + t and physical block phys_block + t/block_size,
 * slot t%block_size, for t < num_tokens.  alive_token_start is the number of
 * alive tokens of the sequence that precede the segment. */
typedef struct {
  int32_t seq;
  int32_t logical_block;
  int32_t phys_block;
  int32_t num_blocks;
  int32_t num_tokens;
  int32_t alive_token_start;
} msa_segment;

/* ------------------------------------------------------------------------ */
/* a1: segment plan                                                          */
/* ------------------------------------------------------------------------ */

/* Workspace bytes msa_plan_segments needs for B sequences. */
size_t msa_plan_workspace_size(int32_t B);

/* split_into_contiguous_segments (P1, MSA pseudocode; the split follows the
 * physical layout, and the hole an evicted block leaves breaks a run).
 *
 * Reading used: logical block l+1 continues the segment holding block l iff
 * both are alive and phys(l+1) == phys(l)+1.  Records are written per
 * sequence in logical order, sequences in order; seg_indptr is the CSR
 * offset array, so the segments of sequence b are
 * segs[seg_indptr[b] .. seg_indptr[b+1]).
 *
 *   block_table  int32 [B, max_blocks]  physical id of each logical block;
 *                entries of dead blocks are ignored (any value)
 *   alive        uint8 [B, max_blocks]  nonzero = block resident
 *   ctx_len      int32 [B]              tokens of each sequence; only blocks
 *                l < ceil(ctx_len/block_size) are considered
 *   segs         msa_segment [seg_capacity]   output
 *   seg_indptr   int32 [B+1]            output
 *   dev_error    int32 [1]              output, required: overwritten with the
 *                OR of MSA_DEVERR_* bits found by this call (0 = none)
 *   workspace    >= msa_plan_workspace_size(B) bytes
 * seg_capacity >= B*max_blocks can never overflow.  The plan is valid for as
 * long as table, alive and ctx_len are unchanged; attention over a stale
 * plan reads the pool where the plan says (in bounds) but is undefined. */
int msa_plan_segments(const int32_t* block_table, const uint8_t* alive, const int32_t* ctx_len,
                      int32_t B, int32_t max_blocks, int32_t block_size, int32_t num_phys_blocks,
                      msa_segment* segs, int32_t seg_capacity, int32_t* seg_indptr,
                      int32_t* dev_error, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* a2+a3(+a5): decode                                                        */
/* ------------------------------------------------------------------------ */

/* Workspace bytes for msa_decode with the same shape arguments.  Zero when
 * one split covers max_ctx_len and the block kernel cannot run for the shape
 * (then no partials and no merge launch); where it can, enough for either
 * kernel. */
size_t msa_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t max_ctx_len, int32_t block_size, int32_t split_blocks);

/* multi_segment_attention for one decode query per sequence (P1 MSA
 * pseudocode; P2 Key Results: one kernel over many disjoint segments).
 *
 * The query of sequence b attends to every alive token of b (it sits after
 * all of them: no mask).  Work split: each sequence's nA alive blocks are
 * cut into ceil(nA / split_blocks) near-equal splits of at most split_blocks
 * blocks (0 = chosen by the library); every split walks its segments in
 * logical order and folds them into a running (max, sum-exp, unnormalised
 * output).  The per-head kernels run one workgroup per (sequence, KV head,
 * split) and choose split_blocks on the host from B, Hkv and max_ctx_len;
 * the block kernel runs one workgroup per split for all KV heads and, with
 * split_blocks 0, chooses the split length on the device from the plan's
 * alive counts.  The automatic choice (msa_decode, MSA_DECODE_AUTO) is the
 * block kernel where it is built, B <= 256 and B * ceil(max_ctx_len / 16)
 * >= 6144 (enough blocks for 256 work items of 24 blocks), except when one
 * workgroup per (sequence, KV head) fills the 256 CUs and no context exceeds
 * 256 blocks.
 * When a sequence has more than one partial they go to `workspace` and a
 * merge kernel stitches them by log-sum-exp (as msa_merge_partials).
 *
 *   q            [B, Hq, D] dtype           k_pool, v_pool  [P, 16, Hkv, D] dtype
 *   segs, seg_indptr   a plan from msa_plan_segments over the same pool
 *   max_ctx_len  >= every sequence's number of alive tokens (sizes the grid;
 *                a sequence with more alive tokens is cut to its first
 *                ceil(ceil(max_ctx_len/16) / split_blocks) x split_blocks
 *                alive blocks in logical order -- memory-safe, but the
 *                result then covers only those keys, and the cut sets
 *                MSA_DEVERR_TRUNCATED in dev_error)
 *   scale        softmax scale; <= 0 selects 1/sqrt(D)
 *   out          [B, Hq, D] dtype           lse_out  [B, Hq] float32, may be NULL
 *   dev_error    int32 [1], may be NULL: MSA_DEVERR_TRUNCATED is ORed in
 *                when a sequence was cut at the grid (understated
 *                max_ctx_len); the word is never cleared by this call
 * A sequence with no alive token gets out = 0 and lse = -inf.  Accumulation
 * is float32 throughout; for bf16 with D 128 and Hq/Hkv 4 or 8 the scores
 * and the output run on bf16 matrix cores, so the softmax weights are rounded
 * to bf16 for the P x V product (as in msa_prefill_chunk). */
int msa_decode(const void* q, const void* k_pool, const void* v_pool, int32_t num_phys_blocks,
               int32_t block_size, const msa_segment* segs, const int32_t* seg_indptr, int32_t B,
               int32_t Hq, int32_t Hkv, int32_t D, int32_t max_ctx_len, msa_dtype dtype,
               float scale, int32_t split_blocks, void* out, float* lse_out, void* workspace,
               size_t workspace_bytes, int32_t* dev_error, void* stream);

/* msa_decode over pools in the block layout kv_layout, with the decode
 * kernel chosen by `kernel` (msa_decode itself is this call with
 * MSA_LAYOUT_NHD and MSA_DECODE_AUTO).  Same arguments, results and errors;
 * a kv_layout or kernel value other than those above returns
 * MSA_ERR_INVALID_ARG, MSA_DECODE_MATRIX or MSA_DECODE_BLOCK on a shape it
 * was not built for MSA_ERR_UNSUPPORTED.  Both layouts give bitwise-identical
 * results on the same values with the same kernel; the kernels agree within
 * the bf16 tolerance (the matrix-core kernels round the softmax weights to
 * bf16 for P x V, and split differently). */
int msa_decode_ex(const void* q, const void* k_pool, const void* v_pool, int32_t num_phys_blocks,
                  int32_t block_size, const msa_segment* segs, const int32_t* seg_indptr,
                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_ctx_len,
                  msa_dtype dtype, float scale, int32_t split_blocks, void* out, float* lse_out,
                  void* workspace, size_t workspace_bytes, msa_kv_layout kv_layout,
                  msa_decode_kernel kernel, int32_t* dev_error, void* stream);

/* msa_decode for callers that cannot allocate device memory at call time
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument; the split partials go to a
 * library-owned device array of msa_decode_noalloc_capacity() bytes
 * (32 MiB), one per GPU, held until the process ends.  Everything else --
 * arguments, kernels, results, errors -- is msa_decode's.  Returns
 * MSA_ERR_CAPACITY when msa_decode_workspace_size for the same arguments
 * exceeds the array, MSA_ERR_DEVICE if its device address cannot be looked
 * up.  The array's address is looked up once per device on the first call
 * that needs it, for the current device, which must be the device of
 * `stream`.  No call allocates.  All calls on one GPU share the array:
 * calls that overlap in time on the same GPU race on it and must be ordered
 * by the caller (one stream, or events). */
size_t msa_decode_noalloc_capacity(void);
int msa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                       int32_t num_phys_blocks, int32_t block_size, const msa_segment* segs,
                       const int32_t* seg_indptr, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                       int32_t max_ctx_len, msa_dtype dtype, float scale, int32_t split_blocks,
                       void* out, float* lse_out, int32_t* dev_error, void* stream);

/* ------------------------------------------------------------------------ */
/* a2+a4(+a5): chunked prefill                                               */
/* ------------------------------------------------------------------------ */

size_t msa_prefill_workspace_size(int32_t B, int32_t C, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t max_ctx_len, int32_t block_size, int32_t split_blocks);

/* multi_segment_attention for a chunk of C query rows per sequence (P1 MSA
 * pseudocode; P1 "3. 自适应分块调度器": prefill runs in chunks).
 *
 * Row i of sequence b sits at logical position q_pos0[b] + i; key at
 * logical position p is visible to it iff p <= q_pos0[b] + i (causal by
 * logical position; evicted tokens are simply absent).  The chunk's own K/V
 * must already be written into the pool as alive blocks covered by the
 * plan.  QK^T and PV run on bf16 MFMA with float32 accumulation; the
 * softmax weights are rounded to bf16 for PV.
 *
 *   q       [B, C, Hq, D] bf16     q_pos0  int32 [B] (device)
 *   out     [B, C, Hq, D] bf16     lse_out [B, C, Hq] float32, may be NULL
 *   max_ctx_len  as for msa_decode: bounds every sequence's alive tokens
 *                (the chunk's included) and sizes the grid; a longer
 *                sequence is cut the same way and sets MSA_DEVERR_TRUNCATED
 *   dev_error    int32 [1], may be NULL: as for msa_decode
 *   split_blocks  0 = automatic: the alive-key stream is split only when the
 *                 (row tile, KV head, sequence) work items do not cover the
 *                 chip's 256 CUs; otherwise it is cut into near-equal splits
 *                 of at most that many blocks.  Splits are merged by
 *                 log-sum-exp through `workspace`.
 * A row that sees no key gets out = 0 and lse = -inf.
 * Errors (returned before any launch): MSA_ERR_INVALID_ARG for null
 * pointers, C <= 0 or bad shapes; MSA_ERR_UNSUPPORTED for shapes not built
 * (msa_attention_supported) and when B x splits > 65535 or, with more than
 * one split, C > 65535 (launch-grid limits); MSA_ERR_CAPACITY when a split
 * is needed and the workspace is missing or smaller than
 * msa_prefill_workspace_size. */
int msa_prefill_chunk(const void* q, int32_t C, const int32_t* q_pos0, const void* k_pool,
                      const void* v_pool, int32_t num_phys_blocks, int32_t block_size,
                      const msa_segment* segs, const int32_t* seg_indptr, int32_t B, int32_t Hq,
                      int32_t Hkv, int32_t D, int32_t max_ctx_len, msa_dtype dtype, float scale,
                      int32_t split_blocks, void* out, float* lse_out, void* workspace,
                      size_t workspace_bytes, int32_t* dev_error, void* stream);

/* msa_prefill_chunk over pools in the block layout kv_layout (as
 * msa_decode_ex). */
int msa_prefill_chunk_ex(const void* q, int32_t C, const int32_t* q_pos0, const void* k_pool,
                         const void* v_pool, int32_t num_phys_blocks, int32_t block_size,
                         const msa_segment* segs, const int32_t* seg_indptr, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t max_ctx_len, msa_dtype dtype,
                         float scale, int32_t split_blocks, void* out, float* lse_out,
                         void* workspace, size_t workspace_bytes, msa_kv_layout kv_layout,
                         int32_t* dev_error, void* stream);

/* Chunk length for the next msa_prefill_chunk call of an adaptive chunking
 * scheduler (P1 "3. 自适应分块调度器": prefill of a long prompt runs in
 * chunks whose size follows the attention kernel's occupancy).
 *
 * msa_prefill_chunk runs one workgroup per (256/(Hq/Hkv) query positions,
 * KV head, sequence), one workgroup per compute unit.  The call returns the
 * smallest multiple of those 256/(Hq/Hkv) positions whose workgroups cover
 * all `compute_units` (<= 0 selects 256, MI355X); below it the kernel must
 * split the key stream (partials and a merge), above it the rate per flop
 * stays flat while each chunk, and the decode steps waiting on it, takes
 * longer.  The result is capped at max_rows and at remaining_tokens (the
 * prompt tokens still to prefill, per sequence), and a remainder shorter
 * than one position tile is folded into this chunk when max_rows allows.
 * Returns the chunk length (0 when remaining_tokens is 0), or a negative
 * msa_status: INVALID_ARG for non-positive B, Hq, Hkv or max_rows, negative
 * remaining_tokens or Hq % Hkv != 0; UNSUPPORTED for a group size the
 * prefill kernel was not built for.  Host only, no device work. */
int32_t msa_prefill_chunk_rows(int32_t B, int32_t Hq, int32_t Hkv, int32_t remaining_tokens,
                               int32_t max_rows, int32_t compute_units);

/* ------------------------------------------------------------------------ */
/* a5: log-sum-exp merge of partials                                         */
/* ------------------------------------------------------------------------ */

/* The sum of per-segment results scaled by a per-segment normaliser (P1 MSA
 * pseudocode), with the normaliser read as the log-sum-exp weight.
 *
 * Partials of sequence b are rows [part_indptr[b], part_indptr[b+1]) of
 *   o_part  float32 [N, R, H, D]   unnormalised output  sum_j exp(s_j - m) v_j
 *   m_part  float32 [N, R, H]      running max m (natural-log units; -inf = empty)
 *   l_part  float32 [N, R, H]      sum_j exp(s_j - m)
 * merged (in a fixed order, so deterministically):
 *   M = max_i m_i,  w_i = exp(m_i - M) (0 if m_i = -inf),  L = sum_i w_i l_i,
 *   out = sum_i w_i o_i / L,  lse = M + ln L;  all empty -> out 0, lse -inf.
 * o_part of an empty partial (m = -inf) may hold anything (NaN included): it
 * is read but never used.
 *   out  [B, R, H, D] out_dtype      lse_out [B, R, H] float32, may be NULL
 * R is 1 for decode and C for prefill. */
int msa_merge_partials(const float* o_part, const float* m_part, const float* l_part,
                       const int32_t* part_indptr, int32_t B, int32_t R, int32_t H, int32_t D,
                       msa_dtype out_dtype, void* out, float* lse_out, void* stream);

/* ------------------------------------------------------------------------ */
/* Gather-then-attend baseline (not on the MSA path)                          */
/* ------------------------------------------------------------------------ */

/* The detour MSA avoids (P1, "Core method 1: MSA": without a multi-segment
 * kernel, the surviving blocks are first gathered into one contiguous
 * buffer, then a contiguous kernel runs; P2, Key Results, compares the two).
 * Copies every sequence's alive K/V blocks, in logical order, into dense
 * pools where alive block j of sequence b becomes block b*blocks_per_seq + j,
 * and writes the matching plan: one segment per sequence
 *   {b, logical_block 0, phys_block b*blocks_per_seq, nA_b, A_b, 0}
 * (nA_b = alive blocks, A_b = alive tokens, both cut at blocks_per_seq) and
 * dense_indptr = 0, 1, ..., B.  msa_decode over (dense pools, dense plan)
 * then computes the same attention with a single segment per sequence.
 * Logical positions are renumbered, so the dense plan suits decode only.
 *
 *   k_pool, v_pool   [P, 16, Hkv, D] dtype (device, read); whole blocks are
 *                    copied, so head-major [P, Hkv, 16, D] pools work alike
 *                    (pass the same block_size and Hkv) and give head-major
 *                    dense pools
 *   segs, seg_indptr a plan of those pools (device)
 *   dense_k, dense_v [B * blocks_per_seq, 16, Hkv, D] dtype (device, written)
 *   dense_segs       [B] msa_segment (device, written)
 *   dense_indptr     [B + 1] int32 (device, written)
 * Dense blocks past a sequence's alive blocks are left untouched.
 * Returns INVALID_ARG for null pointers or non-positive sizes, UNSUPPORTED
 * for other dtypes or block sizes, DEVICE on a launch error. */
int msa_gather_alive(const void* k_pool, const void* v_pool, int32_t num_phys_blocks,
                     int32_t block_size, const msa_segment* segs, const int32_t* seg_indptr,
                     int32_t B, int32_t Hkv, int32_t D, msa_dtype dtype, int32_t blocks_per_seq,
                     void* dense_k, void* dense_v, msa_segment* dense_segs,
                     int32_t* dense_indptr, void* stream);

/* ------------------------------------------------------------------------ */

/* 1 if the attention kernels were built for this shape, else 0.
 * prefill = 0 asks about msa_decode, 1 about msa_prefill_chunk;
 * group_size = Hq / Hkv.  No device work, no side effects. */
int msa_attention_supported(int prefill, msa_dtype dtype, int32_t head_dim, int32_t group_size,
                            int32_t block_size);

const char* msa_status_string(int status);
int msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
