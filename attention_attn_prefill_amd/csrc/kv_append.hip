// kv_append.hip -- write new keys/values into the paged KV cache on gfx950.
//
// The write side of the paged cache ("GRPO-CUDA Project Memory", "KV Cache
// design": slot_mapping[token] = physical_block * block_size + in-block
// offset, int64; "Known bugs fixed": padding tokens carry slot -1 and are
// skipped).  Token i's rows k_new[i, h, :] / v_new[i, h, :] go to
// cache[slot / block_size, h, slot % block_size, :].
//
// Pure data movement, HBM-bound: every byte is read once (non-temporal
// loads) and written once.  Calls that move less than kStreamingBytes store
// non-temporally too; larger ones store through L2.  Measured at H_kv 8, D
// 128: non-temporal stores run 5-8 % faster up to 12288 tokens (100 MB
// moved), where the write-back of dirty L2 lines at the kernel's end weighs
// most, and level off near 5.5 TB/s.  Regular stores reach 6.1-6.6 TB/s from
// 24576 tokens on, and the two cross near 16384 tokens (128 MiB).
// One wavefront per token; its H_kv * D halfs are moved as 16-byte vectors,
// lane-contiguous on the read side (the token's rows are contiguous) and
// 16 lanes per 2*D-byte cache row on the write side.  Slots outside
// [0, num_blocks * block_size) -- including -1 -- are skipped.
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int64_t kStreamingBytes = (int64_t)128 << 20;

template <bool NT_STORES>
__global__ __launch_bounds__(64 * kWaves) void kv_append_kernel(KvAppendArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t token = (int64_t)blockIdx.x * kWaves + wave;
  if (token >= a.num_tokens) return;
  const int64_t slot = a.slot_mapping[token];
  if (slot < 0 || slot >= a.num_blocks * (int64_t)a.block_size) return;
  const int64_t block = slot / a.block_size;
  const int off = (int)(slot - block * a.block_size);

  const int vec_per_row = a.head_dim / 8;
  const int vecs = a.H_kv * vec_per_row;
  const half8_t* ks = reinterpret_cast<const half8_t*>(a.k_new + token * a.H_kv * a.head_dim);
  const half8_t* vs = reinterpret_cast<const half8_t*>(a.v_new + token * a.H_kv * a.head_dim);
  for (int v = lane; v < vecs; v += 64) {
    const int h = v / vec_per_row;
    const int c = v - h * vec_per_row;
    const int64_t dst = ((block * a.H_kv + h) * a.block_size + off) * a.head_dim + 8 * c;
    const half8_t kx = __builtin_nontemporal_load(ks + v);
    const half8_t vx = __builtin_nontemporal_load(vs + v);
    if (NT_STORES) {
      __builtin_nontemporal_store(kx, reinterpret_cast<half8_t*>(a.k_cache + dst));
      __builtin_nontemporal_store(vx, reinterpret_cast<half8_t*>(a.v_cache + dst));
    } else {
      *reinterpret_cast<half8_t*>(a.k_cache + dst) = kx;
      *reinterpret_cast<half8_t*>(a.v_cache + dst) = vx;
    }
  }
}

}  // namespace

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream) {
  KvAppendArgs args = a;
  void* kargs[] = {&args};
  const int64_t blocks = (a.num_tokens + kWaves - 1) / kWaves;
  // bytes moved: K and V rows, each read once and written once
  const int64_t moved = a.num_tokens * a.H_kv * a.head_dim * 2 * 4;
  const void* fn = moved < kStreamingBytes ? reinterpret_cast<const void*>(&kv_append_kernel<true>)
                                           : reinterpret_cast<const void*>(&kv_append_kernel<false>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(64 * kWaves), kargs, 0, stream);
}

}  // namespace attn
