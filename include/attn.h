/*
 * attn.h -- C ABI of libattn.so: scaled-dot-product attention with online
 * softmax on AMD Instinct MI355X (gfx950).
 *
 * The attention operations come from "Tutorial: Adding a New Kernel to RL.cu"
 * (skillsmp.com add-cuda-kernel page), attention.cuh listing:
 *   - attn_prefill: causal (or non-causal) GQA prefill, the "Flash Attention 2
 *     -- Prefill" section of that header;
 *   - attn_decode_paged: single-token decode against a paged KV cache, the
 *     "Paged Attention -- Decode" section of that header, run as split-K
 *     flash-decoding (named as the next step in the "Remaining Gap vs
 *     nano-vllm" section of the GRPO-CUDA project memory page) with a
 *     log-sum-exp merge.
 * The cache append and the QK-norm + rotary step around them follow the
 * GRPO-CUDA project memory page, and the cross-attention module the
 * POPCORNBENCH cross-attention trace (sections cited at each declaration).
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers (HIP device memory or memory the device can
 *     address), except where stated.  The caller owns every buffer; the library
 *     allocates nothing, keeps no state between calls and is reentrant, with
 *     one exception: attn_decode_paged_scratch uses a fixed array of its own
 *     in device memory (see there).
 *   - fp16 tensors are IEEE binary16, dense, row-major, with the layouts given
 *     below; every fp16 base pointer must be 16-byte aligned, int32 pointers
 *     4-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the default stream)
 *     and the call returns without synchronising.  A non-OK status means
 *     nothing was enqueued, except ATTN_ERR_LAUNCH (the launch itself failed).
 *   - Arguments are validated on the host before any HIP call; an invalid
 *     argument never touches the GPU.
 *   - The softmax scale is 1/sqrt(head_dim) (the launch wrappers of the
 *     attention.cu listing), applied to fp32 dot products; accumulation is
 *     fp32; outputs are rounded to fp16 with round-to-nearest-even.
 *
 * Where this ABI is its own design rather than the pages':
 *   - attn_abi_version, attn_status_string, the status codes and the
 *     *_workspace_size queries have no counterpart on the pages (whose
 *     launchers return nothing and abort on a CUDA error);
 *   - `stream` is a void* carrying a hipStream_t, so that this header needs
 *     no HIP include; the pages' launch wrappers take the runtime's stream
 *     type;
 *   - attn_decode_paged takes num_blocks (to bound every table entry) and a
 *     caller workspace for split-K decoding, which the pages' decode
 *     signature does not have;
 *   - attn_prefill takes S_q, S_kv and `causal` where the pages have one S
 *     and always mask.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status_t {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, size <= 0, H_q % H_kv != 0,
                               causal with S_q != S_kv, misaligned pointer */
  ATTN_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, block_size,
                               H_q / H_kv ratio outside the supported set */
  ATTN_ERR_WORKSPACE = 3,   /* workspace non-NULL but smaller than required,
                               or more than attn_decode_paged_scratch's
                               fixed array holds */
  ATTN_ERR_LAUNCH = 4,      /* the HIP runtime refused a kernel launch */
  ATTN_STATUS_MAX_ENUM = 0x7fffffff /* never returned: makes every int from 0
                                       to INT_MAX a valid attn_status_t, so
                                       attn_status_string may be passed any
                                       such code */
} attn_status_t;

/* Version of this ABI; bumped on any incompatible change. */
int attn_abi_version(void);

/* Human-readable name of a status code (static string, never NULL;
   "ATTN_ERR_UNKNOWN" for a value that is no status). */
const char* attn_status_string(attn_status_t status);

/*
 * Prefill: O = softmax(Q K^T / sqrt(D) + mask) V for every query row.
 *
 *   q  [B, S_q,  H_q,  D] fp16      k, v [B, S_kv, H_kv, D] fp16
 *   o  [B, S_q,  H_q,  D] fp16 (written)
 *
 * GQA: H_q % H_kv == 0; query head h reads kv head (h * H_kv) / H_q
 * (integer division), as the attention.cuh header states.
 * causal != 0: row i attends to keys 0..i (the header's causal mask); this
 * requires S_q == S_kv (the pages define causal prefill for one S only).
 * causal == 0: every row attends to all S_kv keys (cross-attention).
 * head_dim (D): 32, 64 or 128.  Any B, S_q, S_kv >= 1 (ragged tails are
 * masked inside the kernel), with (ceil(S_kv / 64) + 3) * 64 * H_kv * D * 2
 * < 2^31 (one batch entry's K or V, rounded up to whole 64-key tiles plus
 * three tiles of staging margin, below 2 GiB, so that 32-bit byte offsets
 * reach it; larger is ATTN_ERR_UNSUPPORTED).
 */
attn_status_t attn_prefill(const void* q, const void* k, const void* v, void* o,
                           int B, int S_q, int S_kv, int H_q, int H_kv,
                           int head_dim, int causal, void* stream);

/*
 * Bytes of device workspace attn_decode_paged needs for split-K decoding of
 * up to num_seqs sequences with tables max_blocks_per_seq wide.  Returns 0 if
 * no workspace is needed (every sequence fits one split), and 0 for invalid
 * or unsupported arguments (attn_decode_paged reports those).  The size
 * depends on the shape only: up to 4096 sequences it is
 * ((num_seqs * H_kv + 1024) * (H_q / H_kv) * 130 + num_seqs + 1) * 4 bytes,
 * independent of the table width; beyond that (or past 32-bit positions)
 * num_seqs * H_q * splits * 130 * 4.
 */
size_t attn_decode_paged_workspace_size(int num_seqs, int H_q, int H_kv,
                                        int head_dim, int max_blocks_per_seq,
                                        int block_size);

/*
 * Paged decode: one new query token per sequence attends to its whole cached
 * context, in logical order, through the block table.
 *
 *   q            [num_seqs, H_q, D] fp16
 *   k_cache      [num_blocks, H_kv, block_size, D] fp16
 *   v_cache      [num_blocks, H_kv, block_size, D] fp16
 *   out          [num_seqs, H_q, D] fp16 (written)
 *   block_tables [num_seqs, max_blocks_per_seq] int32: logical block ->
 *                physical block; only entries for blocks below
 *                ceil(seq_lens[s] / block_size) are read
 *   seq_lens     [num_seqs] int32: context length including the new token
 *
 * Token t of sequence s is k_cache[block_tables[s][t / block_size], g,
 * t % block_size, :] with g = (h * H_kv) / H_q for query head h (the decode
 * section of the attention.cuh header and the "KV Cache design" section of
 * the project memory page).  head_dim must be 128 and block_size 16 (the
 * only specialisation the pages build); H_q / H_kv must be 1..8.
 *
 * num_blocks (not in the pages' signature) bounds the table: the kernel
 * never reads a block outside [0, num_blocks).
 *
 * workspace: device memory of at least attn_decode_paged_workspace_size(...)
 * bytes selects split-K decoding (this library's design; the pages' project
 * memory names flash-decoding split-K as the fix for long contexts): the
 * visible blocks of every (sequence, kv head) are cut into pieces processed
 * in parallel, then merged by log-sum-exp.  Up to 4096 sequences the cut is
 * balanced: every kv head's blocks, sequence after sequence, form equal runs
 * (one workgroup each, as many as the GPU holds at once), each sequence
 * charged a fixed cost of 6 blocks so runs over many short sequences take
 * fewer blocks; beyond that, fixed-length chunks.  NULL selects the
 * single-pass kernel (one workgroup walks a whole sequence).  Both give the
 * same result within fp32 rounding.
 *
 * Device-side preconditions (not checkable without a synchronisation):
 *   1 <= seq_lens[s] <= max_blocks_per_seq * block_size and every table entry
 *   read lies in [0, num_blocks).  A sequence that breaks them gets NaN in all
 *   of its output rows; seq_lens[s] <= 0 gets an all-zero row.  No
 *   out-of-bounds access happens in either case.
 */
attn_status_t attn_decode_paged(const void* q, const void* k_cache,
                                const void* v_cache, void* out,
                                const int32_t* block_tables,
                                const int32_t* seq_lens, int num_seqs, int H_q,
                                int H_kv, int head_dim, int max_blocks_per_seq,
                                int block_size, int64_t num_blocks,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Size in bytes of the device array behind attn_decode_paged_scratch (one
 * copy per device).
 */
#define ATTN_DECODE_SCRATCH_BYTES (16u << 20)

/*
 * Paged decode that allocates nothing and takes no workspace, for callers
 * that cannot allocate device memory around the call: code being captured
 * into a HIP graph, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, layouts, preconditions and result are those of
 * attn_decode_paged given a workspace of
 * attn_decode_paged_workspace_size(...) bytes (split-K decoding; the same
 * kernels run).  The split-K partials live instead in an array of
 * ATTN_DECODE_SCRATCH_BYTES bytes that the library holds in the memory of
 * each device it runs on until the process ends.
 *
 *   - A call whose workspace size exceeds ATTN_DECODE_SCRATCH_BYTES returns
 *     ATTN_ERR_WORKSPACE and enqueues nothing (e.g. H_q = 16, H_kv = 8
 *     allows up to 1887 sequences of any table width; use attn_decode_paged
 *     for more).
 *   - The array of the CURRENT device is used; a non-NULL stream must belong
 *     to that device (else ATTN_ERR_INVALID_ARG).  Its device address is
 *     looked up on the first call on each device (under a lock), so make one
 *     call on a device before capturing a graph there.
 *   - Every call on a device shares that device's array.  Calls whose work
 *     overlaps on one device (other streams, other host threads, concurrent
 *     graph replays) race on it and give wrong results: order them.
 *     Sequential calls need no clearing between them; each call rewrites
 *     every part of the array that it reads.
 */
attn_status_t attn_decode_paged_scratch(const void* q, const void* k_cache,
                                        const void* v_cache, void* out,
                                        const int32_t* block_tables,
                                        const int32_t* seq_lens, int num_seqs,
                                        int H_q, int H_kv, int head_dim,
                                        int max_blocks_per_seq, int block_size,
                                        int64_t num_blocks, void* stream);

/*
 * Bytes of device workspace attn_decode_paged_shared_prefix needs; 0 for
 * invalid or unsupported arguments.
 */
size_t attn_decode_paged_shared_prefix_workspace_size(int num_seqs, int H_q, int H_kv,
                                                      int head_dim, int max_blocks_per_seq,
                                                      int block_size, int num_groups,
                                                      int max_group_size);

/*
 * Paged decode of forked sequences: the result of attn_decode_paged over the
 * same arguments, with every group's shared prompt blocks read once for the
 * whole group instead of once per sequence (cascade attention).  GRPO
 * samples several completions of one prompt, and the engine forks the
 * prompt's cache by copying table entries only ("GRPO-CUDA Project Memory"
 * page, "KV Cache design": paged_kv_cache_fork, no KV copy).
 *
 *   q, k_cache, v_cache, out, block_tables, seq_lens, num_seqs, H_q, H_kv,
 *   head_dim, max_blocks_per_seq, block_size, num_blocks: as attn_decode_paged
 *   group_start   [num_groups + 1] int32: sequences group_start[i] ..
 *                 group_start[i+1]-1 form group i (group_start[0] = 0,
 *                 group_start[num_groups] = num_seqs, nondecreasing)
 *   prefix_blocks [num_groups] int32: the number of leading table entries
 *                 that every sequence of group i shares (the prompt's whole
 *                 blocks; 0 = no sharing)
 *   max_group_size: an upper bound on every group's size
 *
 * Each group's prefix is attended once per kv head for all of its query
 * rows (group size x H_q/H_kv of them, in MFMA column blocks of 32), through
 * the table of the group's first sequence; every sequence's remaining blocks
 * go through the split-K decode kernel, and the partial results are combined
 * by log-sum-exp.  With num_seqs * H_kv >= 2048 every sequence's own blocks
 * form one split that also combines the prefix partials (two launches on
 * `stream`); below that, splits are shorter and a merge kernel combines
 * them (three launches).
 *
 * workspace: at least attn_decode_paged_shared_prefix_workspace_size(...)
 * bytes (NULL or smaller is ATTN_ERR_WORKSPACE).
 * Device-side preconditions, besides those of attn_decode_paged: the group
 * arrays follow the rules above, every sequence of a group holds at least
 * prefix_blocks * block_size tokens, and the prefix entries of all tables of
 * a group are equal (not checked: the first table's entries are used).  A
 * sequence that breaks a checked one gets NaN rows; seq_lens <= 0 gives an
 * all-zero row.
 */
attn_status_t attn_decode_paged_shared_prefix(const void* q, const void* k_cache,
                                              const void* v_cache, void* out,
                                              const int32_t* block_tables,
                                              const int32_t* seq_lens, int num_seqs,
                                              int H_q, int H_kv, int head_dim,
                                              int max_blocks_per_seq, int block_size,
                                              int64_t num_blocks,
                                              const int32_t* group_start,
                                              const int32_t* prefix_blocks,
                                              int num_groups, int max_group_size,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream);

/*
 * Paged KV append: write new keys and values into the paged caches that
 * attn_decode_paged reads -- the write side of the same data structure
 * ("GRPO-CUDA Project Memory" page, "KV Cache design": slot_mapping[token] =
 * physical_block * block_size + in-block offset, int64; "Known bugs fixed":
 * padding tokens carry slot -1 and are skipped).
 *
 *   k_new, v_new  [num_tokens, H_kv, head_dim] fp16 (e.g. a prefill's K/V
 *                 [B, S, H_kv, D] seen as B*S tokens)
 *   k_cache, v_cache [num_blocks, H_kv, block_size, head_dim] fp16 (updated)
 *   slot_mapping  [num_tokens] int64
 *
 * Token i's rows go to cache[slot / block_size, h, slot % block_size, :] for
 * every head h.  Slots outside [0, num_blocks * block_size), -1 included,
 * are skipped.  Two tokens with the same slot race (the result for that slot
 * is unspecified).  head_dim must be a multiple of 8; any block_size >= 1.
 * num_tokens == 0 is a no-op.
 */
attn_status_t attn_kv_append(const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, int64_t num_tokens,
                             int H_kv, int head_dim, int block_size,
                             int64_t num_blocks, void* stream);

/*
 * RoPE table: fill the fp32 tables the rotation reads ("GRPO-CUDA Project
 * Memory" page, "RoPE design": NeoX split-half, table [max_seq_len, D/2]
 * precomputed once).  Pair i of a head at position p turns by the angle
 * p * theta^(-2i/D):
 *
 *   cos_table[p * (head_dim/2) + i] = cos(p * theta^(-2i/head_dim))
 *   sin_table[p * (head_dim/2) + i] = sin(...)           p < max_pos
 *
 * theta is the model's rotary base (not on the pages; Qwen3 configurations
 * use 1e6).  The angle, cosine and sine are evaluated in fp64 and rounded to
 * fp32 once.  head_dim must be even and positive; tables 16-byte aligned.
 */
attn_status_t attn_rope_table(float* cos_table, float* sin_table, int max_pos,
                              int head_dim, double theta, void* stream);

/*
 * QK-norm + rotary embedding, in place (the Qwen3 order: RMSNorm on every
 * query and key head, then the NeoX rotation; "GRPO-CUDA Project Memory"
 * page, "Qwen3 key dims", "Qwen3-Specific Notes" and "RoPE design").
 *
 *   q         [num_tokens, H_q, head_dim] fp16 (updated)
 *   k         [num_tokens, H_kv, head_dim] fp16 (updated)
 *   q_weight, k_weight  [head_dim] fp16 RMSNorm weights, or NULL for the
 *             rotation only (both NULL or both set)
 *   cos_table, sin_table  [max_pos, head_dim/2] fp32 (attn_rope_table)
 *   positions [num_tokens] int32: the token's position in its sequence
 *
 * Per head: y_d = x_d / sqrt(mean_e x_e^2 + eps) * w_d, then for
 * i < D/2: out_i = y_i cos - y_{i+D/2} sin, out_{i+D/2} = y_{i+D/2} cos +
 * y_i sin, with the position's table entries.  fp32 throughout, one
 * rounding to fp16 at the end.  head_dim: 32, 64 or 128.  A [B, S, H, D]
 * prefill tensor is num_tokens = B*S.  num_tokens == 0 is a no-op (the
 * pointers are then not checked).
 * Device-side precondition: 0 <= positions[t] < max_pos; a token that
 * breaks it gets NaN in all of its q and k rows (no out-of-bounds access).
 */
attn_status_t attn_qk_norm_rope(void* q, void* k, const void* q_weight,
                                const void* k_weight, const float* cos_table,
                                const float* sin_table, const int32_t* positions,
                                int64_t num_tokens, int H_q, int H_kv,
                                int head_dim, int max_pos, float eps,
                                void* stream);

/*
 * attn_qk_norm_rope fused with the paged KV append: as above, and in the
 * same pass every token's rotated key rows and its value rows
 * v [num_tokens, H_kv, head_dim] fp16 (read only) are written to
 * k_cache / v_cache [num_blocks, H_kv, block_size, head_dim] at
 * slot_mapping[t] (int64; slots outside [0, num_blocks * block_size),
 * -1 included, are skipped), exactly as attn_kv_append places them.  This is
 * the step between the projections and attention in the pages' Qwen3 layer
 * order ("QK-norm -> RoPE -> KV append -> attn").  A token with a bad
 * position writes NaN key rows to its slot.
 * q may be NULL (then q_weight must be NULL too): keys and values only, for
 * a prefill that normalises and rotates Q as it loads it
 * (attn_prefill_qk_norm_rope); k_weight alone then selects the key norm.
 */
attn_status_t attn_qk_norm_rope_append(void* q, void* k, const void* v,
                                       const void* q_weight, const void* k_weight,
                                       const float* cos_table, const float* sin_table,
                                       const int32_t* positions, int64_t num_tokens,
                                       int H_q, int H_kv, int head_dim, int max_pos,
                                       float eps, void* k_cache, void* v_cache,
                                       const int64_t* slot_mapping, int block_size,
                                       int64_t num_blocks, void* stream);

/*
 * Causal (or not) GQA prefill with the Qwen3 QK-norm + RoPE of the queries
 * fused into the query load ("GRPO-CUDA Project Memory" page, "RoPE design"
 * and the Qwen3 notes): the result of attn_qk_norm_rope on q (per-head
 * RMSNorm with q_weight, or none when NULL, then the NeoX rotation at
 * positions[b * S_q + i], fp32, one rounding to fp16) followed by
 * attn_prefill, without writing the rotated q anywhere (q is read only).
 * The keys must already be normalised and rotated, e.g. by
 * attn_qk_norm_rope_append with q = NULL, which also fills the cache.
 *
 *   q, k, v, o, B, S_q, S_kv, H_q, H_kv, head_dim, causal: as attn_prefill
 *   q_weight  [head_dim] fp16 or NULL
 *   cos_table, sin_table [max_pos, head_dim/2] fp32 (attn_rope_table)
 *   positions [B * S_q] int32, or NULL: query row i of every sequence is at
 *             position i (a prefill from the start of the sequence; the
 *             table lookups then wait for nothing)
 *
 * Same validation and errors as attn_prefill, plus INVALID_ARG for a NULL
 * table, max_pos <= 0, eps < 0 or a misaligned table (16 bytes), weight
 * (16 bytes) or positions array (4 bytes).  Device-side precondition
 * 0 <= position < max_pos; a query row that breaks it comes out NaN.
 */
attn_status_t attn_prefill_qk_norm_rope(const void* q, const void* k, const void* v, void* o,
                                        const void* q_weight, const float* cos_table,
                                        const float* sin_table, const int32_t* positions,
                                        int B, int S_q, int S_kv, int H_q, int H_kv,
                                        int head_dim, int max_pos, float eps, int causal,
                                        void* stream);

/*
 * Bytes of device workspace attn_cross_attention needs (the projected q, k,
 * v and the attention output, fp16).  0 for invalid or unsupported
 * arguments (attn_cross_attention reports those).
 */
size_t attn_cross_attention_workspace_size(int B, int T_q, int T_k, int dim, int H);

/*
 * One layer of multi-head cross-attention with rotary embeddings, the module
 * of the cross-attention trace (POPCORNBENCH "Kimi-K2.6" page: the problem
 * statement and its nn.Linear notes): no bias, dropout p = 0.
 *
 *   x_q   [B, T_q, dim] fp16        x_kv [B, T_k, dim] fp16
 *   w_q, w_k, w_v, w_o [dim, dim] fp16, nn.Linear layout [out, in]
 *   cos_table, sin_table [max_pos, dim/H / 2] fp32 (attn_rope_table with
 *                         head_dim = dim / H and the module's rotary base)
 *   out   [B, T_q, dim] fp16 (written)
 *
 *   Q = x_q w_q^T,  K = x_kv w_k^T,  V = x_kv w_v^T; head h is columns
 *   h*D .. h*D+D-1 (D = dim / H).  Q and K rows are rotated over adjacent
 *   pairs (2j, 2j+1) by the angle of their position in the sequence
 *   (0..T-1) and pair j; then per head softmax(Q K^T / sqrt(D)) V without a
 *   mask; out = concat(heads) w_o^T.
 *
 * Three launches on `stream`: the Q/K/V projections with the rotation, the
 * attention (the non-causal prefill kernel), the output projection.  fp32
 * accumulation; the projected Q, K, V and the attention output are rounded
 * to fp16 in between (the MFMA operand precision).  workspace: at least
 * attn_cross_attention_workspace_size(...) bytes, 256-byte aligned (NULL or
 * smaller is ATTN_ERR_WORKSPACE).  D must be 32, 64 or 128, dim a multiple
 * of 32, max_pos >= max(T_q, T_k).  32-bit byte offsets bound the sizes
 * (larger is ATTN_ERR_UNSUPPORTED): ceil(B * max(T_q, T_k) / 32) * 32 * dim
 * * 2 < 2^31 (the projections address whole 32-row tiles), dim * dim * 2 <
 * 2^31, and (ceil(T_k / 64) + 3) * 64 * dim * 2 < 2^31 (the attention step,
 * as for attn_prefill).
 */
attn_status_t attn_cross_attention(const void* x_q, const void* x_kv, const void* w_q,
                                   const void* w_k, const void* w_v, const void* w_o,
                                   const float* cos_table, const float* sin_table,
                                   int max_pos, void* out, int B, int T_q, int T_k, int dim,
                                   int H, void* workspace, size_t workspace_bytes,
                                   void* stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* ATTN_H_ */
