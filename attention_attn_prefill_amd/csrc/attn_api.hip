// attn_api.hip -- the extern "C" entry points of libattn.so (see
// include/attn.h): host-side argument validation, then kernel launches on the
// caller's stream.  No allocation and no synchronisation; the only global
// state is the per-device address of attn_decode_paged_scratch's array.
#include "../../include/attn.h"

#include <math.h>

#include <mutex>

#include "attn_internal.h"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kAbiVersion = 1;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Everything attn_decode_paged checks before the workspace (shared with the
// workspace-size query so both agree on what is valid).
attn_status_t check_decode_shape(int num_seqs, int H_q, int H_kv, int head_dim,
                                 int max_blocks_per_seq, int block_size) {
  if (num_seqs <= 0 || H_q <= 0 || H_kv <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
      block_size <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (H_q % H_kv != 0) return ATTN_ERR_INVALID_ARG;
  if (head_dim != attn::kDecodeHeadDim || block_size != attn::kDecodeBlockSize)
    return ATTN_ERR_UNSUPPORTED;
  if (H_q / H_kv > 8) return ATTN_ERR_UNSUPPORTED;
  // tokens per sequence must fit an int
  if ((int64_t)max_blocks_per_seq * block_size > (int64_t)0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

struct DecodePlan {
  int split_blocks;
  int n_split_max;
  bool balanced;    // equal runs of the (sequence, kv head, block) order
  size_t ws_bytes;  // 0 when no merge pass is needed
};

// Plain decode: one split per (sequence, kv head) when the table is short
// enough for that to fill the chip (no workspace needed).  Otherwise the
// balanced mode (up to kDecodeBalancedMaxSeqs sequences, whose block prefix
// fits LDS): kDecodeWorkers runs, partials in (num_seqs * H_kv +
// kDecodeWorkers) slots of G heads, then the block prefix.  Beyond that,
// fixed-length splits with num_seqs * H_q * n_split_max partial slots.
DecodePlan plan_decode(int num_seqs, int H_q, int H_kv, int max_blocks_per_seq) {
  DecodePlan p;
  p.split_blocks = attn::decode_split_blocks(num_seqs, H_kv, max_blocks_per_seq);
  p.n_split_max = (int)ceil_div64(max_blocks_per_seq, p.split_blocks);
  p.balanced = false;
  if (p.n_split_max <= 1) {
    p.ws_bytes = 0;
  } else if (num_seqs <= attn::kDecodeBalancedMaxSeqs &&
             (int64_t)num_seqs * (max_blocks_per_seq + 16) * H_kv < (int64_t)0x7fffffff &&
             ((int64_t)num_seqs * H_kv + attn::kDecodeWorkers) * (H_q / H_kv) * (attn::kDecodeHeadDim + 2) <
                 (int64_t)0x7fffffff) {
    p.balanced = true;
    const int64_t slots = ((int64_t)num_seqs * H_kv + attn::kDecodeWorkers) * (H_q / H_kv);
    p.ws_bytes = (size_t)(slots * (attn::kDecodeHeadDim + 2) + num_seqs + 1) * sizeof(float);
  } else {
    const int64_t slots = (int64_t)num_seqs * H_q * p.n_split_max;
    p.ws_bytes = (size_t)slots * (attn::kDecodeHeadDim + 2) * sizeof(float);
  }
  return p;
}

}  // namespace

ATTN_EXPORT int attn_abi_version(void) { return kAbiVersion; }

ATTN_EXPORT const char* attn_status_string(attn_status_t status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH";
    case ATTN_STATUS_MAX_ENUM: break;
  }
  return "ATTN_ERR_UNKNOWN";
}

static attn_status_t prefill_args(const void* q, const void* k, const void* v, void* o, int B, int S_q,
                                  int S_kv, int H_q, int H_kv, int head_dim, int causal,
                                  attn::PrefillArgs& a) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
  if (B <= 0 || S_q <= 0 || S_kv <= 0 || H_q <= 0 || H_kv <= 0 || head_dim <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (H_q % H_kv != 0) return ATTN_ERR_INVALID_ARG;
  if (causal && S_q != S_kv) return ATTN_ERR_INVALID_ARG;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return ATTN_ERR_INVALID_ARG;
  // one workgroup per (128 query rows, q head, batch) must fit a 1-D grid
  if (ceil_div64(S_q, 128) * H_q * B > (int64_t)0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  // K/V rows of one batch entry are addressed with 32-bit byte offsets; the
  // kernels address whole 64-key tiles and stage up to three tiles past the
  // last one (those loads fall outside the buffer range and read zero)
  if ((ceil_div64(S_kv, 64) + 3) * 64 * H_kv * head_dim * 2 >= ((int64_t)1 << 31)) return ATTN_ERR_UNSUPPORTED;

  a.q = static_cast<const _Float16*>(q);
  a.k = static_cast<const _Float16*>(k);
  a.v = static_cast<const _Float16*>(v);
  a.o = static_cast<_Float16*>(o);
  a.B = B;
  a.S_q = S_q;
  a.S_kv = S_kv;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.n_qtiles = 0;  // set by the launcher
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
  return ATTN_OK;
}

ATTN_EXPORT attn_status_t attn_prefill(const void* q, const void* k, const void* v, void* o, int B,
                                       int S_q, int S_kv, int H_q, int H_kv, int head_dim,
                                       int causal, void* stream) {
  attn::PrefillArgs a;
  const attn_status_t st = prefill_args(q, k, v, o, B, S_q, S_kv, H_q, H_kv, head_dim, causal, a);
  if (st != ATTN_OK) return st;
  const hipError_t e = attn::launch_prefill(a, head_dim, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_EXPORT attn_status_t attn_prefill_qk_norm_rope(const void* q, const void* k, const void* v, void* o,
                                                    const void* q_weight, const float* cos_table,
                                                    const float* sin_table, const int32_t* positions,
                                                    int B, int S_q, int S_kv, int H_q, int H_kv,
                                                    int head_dim, int max_pos, float eps, int causal,
                                                    void* stream) {
  attn::PrefillArgs a;
  const attn_status_t st = prefill_args(q, k, v, o, B, S_q, S_kv, H_q, H_kv, head_dim, causal, a);
  if (st != ATTN_OK) return st;
  if (!cos_table || !sin_table || max_pos <= 0 || !(eps >= 0.0f)) return ATTN_ERR_INVALID_ARG;
  if (!aligned(cos_table, 16) || !aligned(sin_table, 16) || (positions && !aligned(positions, 4)) ||
      (q_weight && !aligned(q_weight, 16)))
    return ATTN_ERR_INVALID_ARG;
  if ((int64_t)max_pos * (head_dim / 2) >= ((int64_t)1 << 40)) return ATTN_ERR_UNSUPPORTED;
  a.q_weight = static_cast<const _Float16*>(q_weight);
  a.cos_table = cos_table;
  a.sin_table = sin_table;
  a.positions = positions;
  a.max_pos = max_pos;
  a.eps = eps;
  const hipError_t e = attn::launch_prefill(a, head_dim, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_EXPORT size_t attn_decode_paged_workspace_size(int num_seqs, int H_q, int H_kv, int head_dim,
                                                    int max_blocks_per_seq, int block_size) {
  if (check_decode_shape(num_seqs, H_q, H_kv, head_dim, max_blocks_per_seq, block_size) != ATTN_OK)
    return 0;
  return plan_decode(num_seqs, H_q, H_kv, max_blocks_per_seq).ws_bytes;
}

// Validation, planning and launch of plain paged decode.  `ws` (may be null)
// holds `ws_bytes` bytes; null means the single-pass path, one split per
// (sequence, kv head).
static attn_status_t decode_paged(const void* q, const void* k_cache, const void* v_cache, void* out,
                                  const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                                  int H_q, int H_kv, int head_dim, int max_blocks_per_seq,
                                  int block_size, int64_t num_blocks, float* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  DecodePlan plan = plan_decode(num_seqs, H_q, H_kv, max_blocks_per_seq);
  if (ws == nullptr || plan.ws_bytes == 0) {
    // single pass: one split covers the whole table width
    plan.split_blocks = max_blocks_per_seq;
    plan.n_split_max = 1;
    plan.balanced = false;
  } else if (ws_bytes < plan.ws_bytes) {
    return ATTN_ERR_WORKSPACE;
  }
  if ((int64_t)plan.n_split_max * H_kv * num_seqs > (int64_t)0x7fffffff) return ATTN_ERR_UNSUPPORTED;

  attn::DecodeArgs a;
  a.q = static_cast<const _Float16*>(q);
  a.k_cache = static_cast<const _Float16*>(k_cache);
  a.v_cache = static_cast<const _Float16*>(v_cache);
  a.out = static_cast<_Float16*>(out);
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  const int64_t slots = plan.balanced
                            ? ((int64_t)num_seqs * H_kv + attn::kDecodeWorkers) * (H_q / H_kv)
                            : (int64_t)num_seqs * H_q * plan.n_split_max;
  a.ws_o = plan.n_split_max > 1 ? ws : nullptr;
  a.ws_ml = plan.n_split_max > 1 ? ws + slots * attn::kDecodeHeadDim : nullptr;
  a.workers = plan.balanced ? attn::kDecodeWorkers : 0;
  a.run_prefix = plan.balanced ? reinterpret_cast<int32_t*>(ws + slots * (attn::kDecodeHeadDim + 2)) : nullptr;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.split_blocks = plan.split_blocks;
  a.n_split_max = plan.n_split_max;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
  a.group_start = nullptr;  // plain decode
  a.seq_skip = nullptr;
  a.prefix_blocks = nullptr;
  a.num_groups = 0;
  a.max_group_size = 0;
  a.prefix_slots = 0;
  a.slot_stride = plan.n_split_max;
  const hipError_t e = attn::launch_decode(a, H_q / H_kv, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

static attn_status_t check_decode_args(const void* q, const void* k_cache, const void* v_cache,
                                       const void* out, const int32_t* block_tables,
                                       const int32_t* seq_lens, int num_seqs, int H_q, int H_kv,
                                       int head_dim, int max_blocks_per_seq, int block_size,
                                       int64_t num_blocks) {
  if (!q || !k_cache || !v_cache || !out || !block_tables || !seq_lens) return ATTN_ERR_INVALID_ARG;
  const attn_status_t st =
      check_decode_shape(num_seqs, H_q, H_kv, head_dim, max_blocks_per_seq, block_size);
  if (st != ATTN_OK) return st;
  if (num_blocks <= 0) return ATTN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

ATTN_EXPORT attn_status_t attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                                            void* out, const int32_t* block_tables,
                                            const int32_t* seq_lens, int num_seqs, int H_q,
                                            int H_kv, int head_dim, int max_blocks_per_seq,
                                            int block_size, int64_t num_blocks, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  const attn_status_t st = check_decode_args(q, k_cache, v_cache, out, block_tables, seq_lens, num_seqs,
                                             H_q, H_kv, head_dim, max_blocks_per_seq, block_size,
                                             num_blocks);
  if (st != ATTN_OK) return st;
  if (workspace && !aligned(workspace, 16)) return ATTN_ERR_INVALID_ARG;
  return decode_paged(q, k_cache, v_cache, out, block_tables, seq_lens, num_seqs, H_q, H_kv, head_dim,
                      max_blocks_per_seq, block_size, num_blocks, static_cast<float*>(workspace),
                      workspace_bytes, static_cast<hipStream_t>(stream));
}

// ---- paged decode without allocation ---------------------------------------
// The split-K partials go to a library-owned array in device memory instead of
// a caller workspace.  Each device holds its own copy from the library's load
// until the process ends; its address differs per device and is looked up
// (with that device current) on the first call there.  Nothing in it needs
// clearing: the merge reads only the partial slots that the same call's split
// kernel wrote.
namespace {

constexpr size_t kScratchBytes = (size_t)ATTN_DECODE_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices];  // per device, set once under the mutex

// Device address of `scratch` on device `dev` (current).  Null on failure.
float* scratch_on(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  return g_scratch_ptr[dev];
}

}  // namespace

ATTN_EXPORT attn_status_t attn_decode_paged_scratch(const void* q, const void* k_cache,
                                                    const void* v_cache, void* out,
                                                    const int32_t* block_tables,
                                                    const int32_t* seq_lens, int num_seqs, int H_q,
                                                    int H_kv, int head_dim, int max_blocks_per_seq,
                                                    int block_size, int64_t num_blocks, void* stream) {
  const attn_status_t st = check_decode_args(q, k_cache, v_cache, out, block_tables, seq_lens, num_seqs,
                                             H_q, H_kv, head_dim, max_blocks_per_seq, block_size,
                                             num_blocks);
  if (st != ATTN_OK) return st;
  const DecodePlan plan = plan_decode(num_seqs, H_q, H_kv, max_blocks_per_seq);
  if (plan.ws_bytes > kScratchBytes) return ATTN_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  float* ws = nullptr;
  if (plan.ws_bytes > 0) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
    if (s != nullptr) {
      // the scratch looked up below is the current device's: the stream must
      // belong to it
      hipDevice_t sdev = -1;
      if (hipStreamGetDevice(s, &sdev) != hipSuccess) return ATTN_ERR_LAUNCH;
      if (sdev != dev) return ATTN_ERR_INVALID_ARG;
    }
    ws = scratch_on(dev);
    if (ws == nullptr) return ATTN_ERR_LAUNCH;
  }
  return decode_paged(q, k_cache, v_cache, out, block_tables, seq_lens, num_seqs, H_q, H_kv, head_dim,
                      max_blocks_per_seq, block_size, num_blocks, ws, kScratchBytes, s);
}

// ---- shared-prefix (forked) paged decode ----------------------------------
// Workspace: per (sequence, query head) the prefix-chunk partials and the
// suffix-split partials: slot_stride * (D + 2) floats.
struct SharedPlan {
  int split_blocks, n_split_max, prefix_slots;
  int64_t ws_bytes;
};

static SharedPlan plan_shared(int num_seqs, int H_q, int H_kv, int max_blocks_per_seq) {
  SharedPlan p;
  p.split_blocks = attn::decode_split_blocks(num_seqs, H_kv, max_blocks_per_seq);
  // Enough (sequence, kv head) pairs to fill the chip with one workgroup
  // each: one split per sequence, so the split kernel folds in the prefix
  // partials and no merge kernel runs.  The private part of a forked
  // sequence is its generated tokens, short next to the shared prompt.
  if ((int64_t)num_seqs * H_kv >= attn::kDecodeSingleSplitPairs) p.split_blocks = max_blocks_per_seq;
  p.n_split_max = (int)ceil_div64(max_blocks_per_seq, p.split_blocks);
  p.prefix_slots = (int)ceil_div64(max_blocks_per_seq, attn::kPrefixChunkBlocks);
  // partial o and (max, sum) per slot, then the per-sequence prefix lengths
  p.ws_bytes = (int64_t)num_seqs * H_q * (p.prefix_slots + p.n_split_max) * (attn::kDecodeHeadDim + 2) * 4 +
               (int64_t)num_seqs * 4;
  return p;
}

static attn_status_t check_shared(int num_seqs, int H_q, int H_kv, int head_dim, int max_blocks_per_seq,
                                  int block_size, int num_groups, int max_group_size) {
  const attn_status_t st = check_decode_shape(num_seqs, H_q, H_kv, head_dim, max_blocks_per_seq, block_size);
  if (st != ATTN_OK) return st;
  if (num_groups <= 0 || num_groups > num_seqs || max_group_size <= 0 || max_group_size > num_seqs)
    return ATTN_ERR_INVALID_ARG;
  const SharedPlan p = plan_shared(num_seqs, H_q, H_kv, max_blocks_per_seq);
  const int64_t col_blocks = ceil_div64((int64_t)max_group_size * (H_q / H_kv), 32);
  if ((int64_t)p.prefix_slots * num_groups * H_kv * col_blocks + ceil_div64(num_seqs, 256) > (int64_t)0x7fffffff ||
      (int64_t)p.n_split_max * H_kv * num_seqs > (int64_t)0x7fffffff)
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

ATTN_EXPORT size_t attn_decode_paged_shared_prefix_workspace_size(int num_seqs, int H_q, int H_kv,
                                                                 int head_dim, int max_blocks_per_seq,
                                                                 int block_size, int num_groups,
                                                                 int max_group_size) {
  if (check_shared(num_seqs, H_q, H_kv, head_dim, max_blocks_per_seq, block_size, num_groups,
                   max_group_size) != ATTN_OK)
    return 0;
  return (size_t)plan_shared(num_seqs, H_q, H_kv, max_blocks_per_seq).ws_bytes;
}

ATTN_EXPORT attn_status_t attn_decode_paged_shared_prefix(
    const void* q, const void* k_cache, const void* v_cache, void* out, const int32_t* block_tables,
    const int32_t* seq_lens, int num_seqs, int H_q, int H_kv, int head_dim, int max_blocks_per_seq,
    int block_size, int64_t num_blocks, const int32_t* group_start, const int32_t* prefix_blocks,
    int num_groups, int max_group_size, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !out || !block_tables || !seq_lens || !group_start || !prefix_blocks)
    return ATTN_ERR_INVALID_ARG;
  const attn_status_t st = check_shared(num_seqs, H_q, H_kv, head_dim, max_blocks_per_seq, block_size,
                                        num_groups, max_group_size);
  if (st != ATTN_OK) return st;
  if (num_blocks <= 0) return ATTN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(group_start, 4) ||
      !aligned(prefix_blocks, 4))
    return ATTN_ERR_INVALID_ARG;
  const SharedPlan plan = plan_shared(num_seqs, H_q, H_kv, max_blocks_per_seq);
  if (!workspace || (int64_t)workspace_bytes < plan.ws_bytes || !aligned(workspace, 16))
    return ATTN_ERR_WORKSPACE;

  attn::DecodeArgs a;
  a.q = static_cast<const _Float16*>(q);
  a.k_cache = static_cast<const _Float16*>(k_cache);
  a.v_cache = static_cast<const _Float16*>(v_cache);
  a.out = static_cast<_Float16*>(out);
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  const int64_t slots = (int64_t)num_seqs * H_q * (plan.prefix_slots + plan.n_split_max);
  a.ws_o = static_cast<float*>(workspace);
  a.ws_ml = a.ws_o + slots * attn::kDecodeHeadDim;
  a.seq_skip = reinterpret_cast<int32_t*>(a.ws_ml + slots * 2);
  a.workers = 0;  // fixed-length splits after the prefix
  a.run_prefix = nullptr;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.split_blocks = plan.split_blocks;
  a.n_split_max = plan.n_split_max;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
  a.group_start = group_start;
  a.prefix_blocks = prefix_blocks;
  a.num_groups = num_groups;
  a.max_group_size = max_group_size;
  a.prefix_slots = plan.prefix_slots;
  a.slot_stride = plan.prefix_slots + plan.n_split_max;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (attn::launch_decode_prefix(a, H_q / H_kv, s) != hipSuccess) return ATTN_ERR_LAUNCH;
  return attn::launch_decode(a, H_q / H_kv, s) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_EXPORT attn_status_t attn_kv_append(const void* k_new, const void* v_new, void* k_cache,
                                         void* v_cache, const int64_t* slot_mapping,
                                         int64_t num_tokens, int H_kv, int head_dim, int block_size,
                                         int64_t num_blocks, void* stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return ATTN_ERR_INVALID_ARG;
  if (num_tokens < 0 || H_kv <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (head_dim % 8 != 0) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return ATTN_ERR_INVALID_ARG;
  if (ceil_div64(num_tokens, 4) > (int64_t)0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  if (num_tokens == 0) return ATTN_OK;
  attn::KvAppendArgs a;
  a.k_new = static_cast<const _Float16*>(k_new);
  a.v_new = static_cast<const _Float16*>(v_new);
  a.k_cache = static_cast<_Float16*>(k_cache);
  a.v_cache = static_cast<_Float16*>(v_cache);
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_blocks = num_blocks;
  a.H_kv = H_kv;
  a.head_dim = head_dim;
  a.block_size = block_size;
  const hipError_t e = attn::launch_kv_append(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_EXPORT attn_status_t attn_rope_table(float* cos_table, float* sin_table, int max_pos,
                                          int head_dim, double theta, void* stream) {
  if (!cos_table || !sin_table || max_pos <= 0 || head_dim <= 0 || (head_dim & 1) || !(theta > 0.0))
    return ATTN_ERR_INVALID_ARG;
  if (!aligned(cos_table, 16) || !aligned(sin_table, 16)) return ATTN_ERR_INVALID_ARG;
  if (ceil_div64((int64_t)max_pos * (head_dim / 2), 256) > (int64_t)0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  const hipError_t e = attn::launch_rope_table(cos_table, sin_table, max_pos, head_dim, theta,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

static attn_status_t qk_norm_rope_common(void* q, void* k, const void* v, const void* q_weight,
                                         const void* k_weight, const float* cos_table,
                                         const float* sin_table, const int32_t* positions,
                                         int64_t num_tokens, int H_q, int H_kv, int head_dim,
                                         int max_pos, float eps, void* k_cache, void* v_cache,
                                         const int64_t* slot_mapping, int block_size,
                                         int64_t num_blocks, bool append, void* stream) {
  if (num_tokens < 0 || H_q <= 0 || H_kv <= 0 || head_dim <= 0 || max_pos <= 0 || !(eps >= 0.0f))
    return ATTN_ERR_INVALID_ARG;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (num_tokens == 0) return ATTN_OK;  // nothing is read or written
  // q may be null when appending (K-only: Q is rotated by the prefill that
  // reads it); then q_weight must be null too
  if ((!q && !append) || !k || !cos_table || !sin_table || !positions) return ATTN_ERR_INVALID_ARG;
  if (q ? (q_weight == nullptr) != (k_weight == nullptr) : q_weight != nullptr) return ATTN_ERR_INVALID_ARG;
  if ((q && !aligned(q, 16)) || !aligned(k, 16) || !aligned(cos_table, 16) || !aligned(sin_table, 16) ||
      !aligned(positions, 4) || (q_weight && !aligned(q_weight, 16)) || (k_weight && !aligned(k_weight, 16)))
    return ATTN_ERR_INVALID_ARG;
  if (append) {
    if (!v || !k_cache || !v_cache || !slot_mapping || block_size <= 0 || num_blocks <= 0)
      return ATTN_ERR_INVALID_ARG;
    if (!aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
      return ATTN_ERR_INVALID_ARG;
  }
  const int64_t rows_per_block = (64 / (head_dim / 8)) * 4;
  const int64_t heads = (q ? (int64_t)H_q : 0) + (int64_t)H_kv * (append ? 2 : 1);
  if (num_tokens > ((int64_t)1 << 40) / heads ||
      ceil_div64(num_tokens * heads, rows_per_block) > (int64_t)0x7fffffff)
    return ATTN_ERR_UNSUPPORTED;
  attn::RopeArgs a;
  a.q = static_cast<_Float16*>(q);
  a.k = static_cast<_Float16*>(k);
  a.v = static_cast<const _Float16*>(v);
  a.q_weight = static_cast<const _Float16*>(q_weight);
  a.k_weight = static_cast<const _Float16*>(k_weight);
  a.cos_table = cos_table;
  a.sin_table = sin_table;
  a.positions = positions;
  a.k_cache = static_cast<_Float16*>(k_cache);
  a.v_cache = static_cast<_Float16*>(v_cache);
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_blocks = append ? num_blocks : 0;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.max_pos = max_pos;
  a.block_size = append ? block_size : 1;
  a.eps = eps;
  const hipError_t e = attn::launch_qk_norm_rope(a, head_dim, append, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_EXPORT attn_status_t attn_qk_norm_rope(void* q, void* k, const void* q_weight,
                                            const void* k_weight, const float* cos_table,
                                            const float* sin_table, const int32_t* positions,
                                            int64_t num_tokens, int H_q, int H_kv, int head_dim,
                                            int max_pos, float eps, void* stream) {
  return qk_norm_rope_common(q, k, nullptr, q_weight, k_weight, cos_table, sin_table, positions,
                             num_tokens, H_q, H_kv, head_dim, max_pos, eps, nullptr, nullptr,
                             nullptr, 0, 0, false, stream);
}

ATTN_EXPORT attn_status_t attn_qk_norm_rope_append(void* q, void* k, const void* v,
                                                   const void* q_weight, const void* k_weight,
                                                   const float* cos_table, const float* sin_table,
                                                   const int32_t* positions, int64_t num_tokens,
                                                   int H_q, int H_kv, int head_dim, int max_pos,
                                                   float eps, void* k_cache, void* v_cache,
                                                   const int64_t* slot_mapping, int block_size,
                                                   int64_t num_blocks, void* stream) {
  return qk_norm_rope_common(q, k, v, q_weight, k_weight, cos_table, sin_table, positions,
                             num_tokens, H_q, H_kv, head_dim, max_pos, eps, k_cache, v_cache,
                             slot_mapping, block_size, num_blocks, true, stream);
}

// ---- cross-attention module ------------------------------------------------
// Workspace: q [B*T_q, dim], k and v [B*T_k, dim], the attention output
// [B*T_q, dim], fp16, each part 256-byte aligned.
static int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

static attn_status_t check_cross(int B, int T_q, int T_k, int dim, int H) {
  if (B <= 0 || T_q <= 0 || T_k <= 0 || dim <= 0 || H <= 0 || dim % H) return ATTN_ERR_INVALID_ARG;
  const int D = dim / H;
  if (D != 32 && D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (dim % 32) return ATTN_ERR_UNSUPPORTED;
  // 32-bit byte offsets: the projections address whole 32-row tiles of every
  // operand, and the attention step (the prefill rules) whole 64-key tiles
  // of one batch entry's K/V plus three tiles of staging margin
  const int64_t rows = (int64_t)B * (T_q > T_k ? T_q : T_k);
  if (ceil_div64(rows, 32) * 32 * dim * 2 >= ((int64_t)1 << 31) ||
      (int64_t)dim * dim * 2 >= ((int64_t)1 << 31))
    return ATTN_ERR_UNSUPPORTED;
  if ((ceil_div64(T_k, 64) + 3) * 64 * dim * 2 >= ((int64_t)1 << 31)) return ATTN_ERR_UNSUPPORTED;
  if (ceil_div64(T_q, 128) * H * B > (int64_t)0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

static int64_t cross_ws_bytes(int B, int T_q, int T_k, int dim) {
  const int64_t q = align256((int64_t)B * T_q * dim * 2);
  const int64_t kv = align256((int64_t)B * T_k * dim * 2);
  return 2 * q + 2 * kv;
}

ATTN_EXPORT size_t attn_cross_attention_workspace_size(int B, int T_q, int T_k, int dim, int H) {
  if (check_cross(B, T_q, T_k, dim, H) != ATTN_OK) return 0;
  return (size_t)cross_ws_bytes(B, T_q, T_k, dim);
}

ATTN_EXPORT attn_status_t attn_cross_attention(const void* x_q, const void* x_kv, const void* w_q,
                                               const void* w_k, const void* w_v, const void* w_o,
                                               const float* cos_table, const float* sin_table,
                                               int max_pos, void* out, int B, int T_q, int T_k,
                                               int dim, int H, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  if (!x_q || !x_kv || !w_q || !w_k || !w_v || !w_o || !cos_table || !sin_table || !out)
    return ATTN_ERR_INVALID_ARG;
  const attn_status_t st = check_cross(B, T_q, T_k, dim, H);
  if (st != ATTN_OK) return st;
  if (max_pos < T_q || max_pos < T_k) return ATTN_ERR_INVALID_ARG;
  if (!aligned(x_q, 16) || !aligned(x_kv, 16) || !aligned(w_q, 16) || !aligned(w_k, 16) ||
      !aligned(w_v, 16) || !aligned(w_o, 16) || !aligned(out, 16) || !aligned(cos_table, 4) ||
      !aligned(sin_table, 4))
    return ATTN_ERR_INVALID_ARG;
  const int64_t need = cross_ws_bytes(B, T_q, T_k, dim);
  if (!workspace || (int64_t)workspace_bytes < need || !aligned(workspace, 256)) return ATTN_ERR_WORKSPACE;
  const int D = dim / H;
  char* ws = static_cast<char*>(workspace);
  const int64_t qb = align256((int64_t)B * T_q * dim * 2), kvb = align256((int64_t)B * T_k * dim * 2);
  _Float16* q = reinterpret_cast<_Float16*>(ws);
  _Float16* k = reinterpret_cast<_Float16*>(ws + qb);
  _Float16* v = reinterpret_cast<_Float16*>(ws + qb + kvb);
  _Float16* att = reinterpret_cast<_Float16*>(ws + qb + 2 * kvb);
  hipStream_t s = static_cast<hipStream_t>(stream);

  const int64_t col_tiles = dim / 32;
  attn::ProjArgs p{};
  p.K = dim;
  p.N = dim;
  p.head_dim = D;
  p.cos_table = cos_table;
  p.sin_table = sin_table;
  p.n_jobs = 3;
  p.job[0] = {static_cast<const _Float16*>(x_q), static_cast<const _Float16*>(w_q), q, B * T_q, T_q, 1,
              ceil_div64((int64_t)B * T_q, 32) * col_tiles};
  p.job[1] = {static_cast<const _Float16*>(x_kv), static_cast<const _Float16*>(w_k), k, B * T_k, T_k, 1,
              ceil_div64((int64_t)B * T_k, 32) * col_tiles};
  p.job[2] = {static_cast<const _Float16*>(x_kv), static_cast<const _Float16*>(w_v), v, B * T_k, T_k, 0,
              ceil_div64((int64_t)B * T_k, 32) * col_tiles};
  if (attn::launch_proj(p, s) != hipSuccess) return ATTN_ERR_LAUNCH;

  attn::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = att;
  a.B = B;
  a.S_q = T_q;
  a.S_kv = T_k;
  a.H_q = H;
  a.H_kv = H;
  a.n_qtiles = 0;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  if (attn::launch_prefill(a, D, false, s) != hipSuccess) return ATTN_ERR_LAUNCH;

  attn::ProjArgs po{};
  po.K = dim;
  po.N = dim;
  po.head_dim = D;
  po.n_jobs = 1;
  po.job[0] = {att, static_cast<const _Float16*>(w_o), static_cast<_Float16*>(out), B * T_q, T_q, 0,
               ceil_div64((int64_t)B * T_q, 32) * col_tiles};
  return attn::launch_proj(po, s) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
