// kv_append.hip -- write new keys/values into the paged KV cache on gfx950.
//
// The write side of the paged cache ("GRPO-CUDA Project Memory", "KV Cache
// design": slot_mapping[token] = physical_block * block_size + in-block
// offset, int64; "Known bugs fixed": padding tokens carry slot -1 and are
// skipped).  Token i's rows k_new[i, h, :] / v_new[i, h, :] go to
// cache[slot / block_size, h, slot % block_size, :].
//
// Pure data movement, HBM-bound: every byte is read once and written once,
// by non-temporal loads and stores.
// One wavefront per token; its H_kv * D halfs are moved as 16-byte vectors,
// lane-contiguous on the read side (the token's rows are contiguous) and
// 16 lanes per 2*D-byte cache row on the write side.  Slots outside
// [0, num_blocks * block_size) -- including -1 -- are skipped.
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kWaves = 4;

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
    // non-temporal both ways: this launch touches each byte once, and the
    // cache rows are read by later calls, not from this launch's L2
    __builtin_nontemporal_store(kx, reinterpret_cast<half8_t*>(a.k_cache + dst));
    __builtin_nontemporal_store(vx, reinterpret_cast<half8_t*>(a.v_cache + dst));
  }
}

}  // namespace

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream) {
  KvAppendArgs args = a;
  void* kargs[] = {&args};
  const int64_t blocks = (a.num_tokens + kWaves - 1) / kWaves;
  return hipLaunchKernel(reinterpret_cast<const void*>(&kv_append_kernel), dim3((unsigned)blocks),
                         dim3(64 * kWaves), kargs, 0, stream);
}

}  // namespace attn
