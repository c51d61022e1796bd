// attn_internal.h -- shared declarations between the C-ABI front end and the
// gfx950 kernels of libattn.so.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// log2(e): softmax is evaluated as exp2((s - m) * scale * log2(e)).
constexpr float kLog2e = 1.4426950408889634f;

struct PrefillArgs {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  _Float16* o;
  int B, S_q, S_kv, H_q, H_kv;
  int n_qtiles;      // ceil(S_q / BLOCK_M)
  float scale_log2;  // log2(e) / sqrt(D)
  // Optional per-head RMSNorm + NeoX rotation of Q as it is loaded (off when
  // cos_table is null): Q row (b, i) turns by the table row positions[b*S_q+i].
  const _Float16* q_weight = nullptr;  // [D] or null (rotation only)
  const float* cos_table = nullptr;    // [max_pos, D/2]
  const float* sin_table = nullptr;
  const int32_t* positions = nullptr;  // [B * S_q], or null: row i of each sequence is at i
  int max_pos = 0;
  float eps = 0.0f;
};

struct DecodeArgs {
  const _Float16* q;
  const _Float16* k_cache;
  const _Float16* v_cache;
  _Float16* out;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_o;   // [num_seqs, H_q, n_split_max, D] partial outputs (unnormalised)
  float* ws_ml;  // [num_seqs, H_q, n_split_max, 2] partial (max, sum), log2 domain
  int64_t num_blocks;
  int num_seqs, H_q, H_kv;
  int max_blocks_per_seq;
  int split_blocks;  // KV blocks per split
  int n_split_max;   // ceil(max_blocks_per_seq / split_blocks)
  float scale_log2;
  // Shared-prefix (cascade) mode, off when group_start is null: sequences
  // group_start[i] .. group_start[i+1]-1 share their first prefix_blocks[i]
  // table entries.  Those blocks are attended once per group by the prefix
  // kernel (partials in slots [0, prefix_slots)); the split kernel covers the
  // rest (slots prefix_slots + split) and, with one split per sequence,
  // folds in the prefix partials; otherwise the merge kernel does.
  const int32_t* group_start;
  const int32_t* prefix_blocks;
  int num_groups;
  int max_group_size;
  int prefix_slots;         // ceil(max_blocks_per_seq / kPrefixChunkBlocks), 0 when off
  int slot_stride;          // workspace slots per (sequence, query head)
  // [num_seqs] (workspace): each sequence's prefix blocks, or -1 when its
  // group breaks a checked rule; written by the prefix launch
  int32_t* seq_skip;
  // Balanced mode (plain decode with partials), off when workers == 0: the
  // (sequence, kv head, block) order is cut into `workers` equal runs, one
  // per workgroup; a (sequence, kv head) that one run covers is finished by
  // it, the others leave partials in slot (s * H_kv + g + run) of ws_o /
  // ws_ml (G heads per slot) for the merge.  run_prefix [num_seqs + 1]
  // (workspace) receives the blocks per kv head before each sequence.
  int workers;
  int32_t* run_prefix;
};

struct KvAppendArgs {
  const _Float16* k_new;  // [num_tokens, H_kv, head_dim]
  const _Float16* v_new;
  _Float16* k_cache;      // [num_blocks, H_kv, block_size, head_dim]
  _Float16* v_cache;
  const int64_t* slot_mapping;  // [num_tokens]
  int64_t num_tokens;
  int64_t num_blocks;
  int H_kv, head_dim, block_size;
};

struct RopeArgs {
  _Float16* q;                 // [num_tokens, H_q, D], updated in place
  _Float16* k;                 // [num_tokens, H_kv, D], updated in place
  const _Float16* v;           // [num_tokens, H_kv, D] (append only)
  const _Float16* q_weight;    // [D] or null (no norm)
  const _Float16* k_weight;
  const float* cos_table;      // [max_pos, D/2]
  const float* sin_table;
  const int32_t* positions;    // [num_tokens]
  _Float16* k_cache;           // [num_blocks, H_kv, block_size, D] (append only)
  _Float16* v_cache;
  const int64_t* slot_mapping; // [num_tokens] (append only)
  int64_t num_tokens;
  int64_t num_blocks;
  int H_q, H_kv, max_pos, block_size;
  float eps;
};

// One matrix of a projection launch: y[M, N] = x[M, K] w[N, K]^T, with the
// adjacent-pair rotary epilogue when rope != 0 (position = row % T).
struct ProjJob {
  const _Float16* x;
  const _Float16* w;
  _Float16* y;
  int M, T, rope;
  int64_t tiles;  // (ceil(M / 32)) * (N / 32)
};
struct ProjArgs {
  ProjJob job[3];
  int n_jobs;
  int K, N, head_dim;
  const float* cos_table;  // [max_pos, head_dim / 2]
  const float* sin_table;
};

// Launchers: enqueue on `stream`, return the launch status.
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, bool causal, hipStream_t stream);
// head_dim 128 without the fused Q rotation: two row blocks per wavefront
hipError_t launch_prefill_dual(const PrefillArgs& a, bool causal, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int group, hipStream_t stream);
hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream);
hipError_t launch_qk_norm_rope(const RopeArgs& a, int head_dim, bool append, hipStream_t stream);
hipError_t launch_proj(const ProjArgs& a, hipStream_t stream);
hipError_t launch_rope_table(float* cos_t, float* sin_t, int max_pos, int head_dim, double theta,
                             hipStream_t stream);

// Decode split policy (shared by the workspace-size query and the launch).
constexpr int kDecodeBlockSize = 16;
constexpr int kDecodeHeadDim = 128;
int decode_split_blocks(int num_seqs, int H_kv, int max_blocks_per_seq);
constexpr int kPrefixChunkBlocks = 64;  // prefix blocks per prefix-kernel workgroup
constexpr int kDecodeSingleSplitPairs = 2048;  // shared-prefix decode: one split per sequence from here
constexpr int kDecodeWorkers = 1024;      // balanced decode: runs (4 resident workgroups x 256 CUs)
constexpr int kDecodeMinRun = 16;         // balanced decode: fewest blocks per run
constexpr int kDecodeBalancedMaxSeqs = 4096;  // balanced decode: sequences whose prefix fits LDS

// Shared-prefix mode: the group gi of sequence s (group_start ascending,
// group_start[0] = 0, group_start[num_groups] = num_seqs) and its shared
// leading blocks.  False when the arrays break those rules for s, the prefix
// is negative or wider than the table, or the group exceeds max_group_size;
// the merge then reports NaN for the sequence.
__device__ __forceinline__ bool decode_group_of(const DecodeArgs& a, int s, int& gi, int& skip) {
  int lo = 0, hi = a.num_groups;
  if (a.group_start[0] > s || a.group_start[hi] <= s) return false;
  while (hi - lo > 1) {  // largest lo with group_start[lo] <= s
    const int mid = (lo + hi) >> 1;
    if (a.group_start[mid] <= s) lo = mid;
    else hi = mid;
  }
  if (a.group_start[lo + 1] <= s) return false;
  gi = lo;
  skip = a.prefix_blocks[lo];
  return skip >= 0 && skip <= a.max_blocks_per_seq && a.group_start[lo] >= 0 &&
         a.group_start[lo + 1] <= a.num_seqs &&
         a.group_start[lo + 1] - a.group_start[lo] <= a.max_group_size;
}
// Prefix kernel plus, in the same launch, the per-sequence seq_skip table.
hipError_t launch_decode_prefix(const DecodeArgs& a, int group, hipStream_t stream);

}  // namespace attn
