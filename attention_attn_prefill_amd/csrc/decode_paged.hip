// decode_paged.hip -- single-token attention over a paged KV cache, split-K
// ("flash-decoding") with a log-sum-exp merge, for gfx950.
//
// What is computed follows "Tutorial: Adding a New Kernel to RL.cu",
// attention.cuh / attention.cu decode sections: q [num_seqs,H_q,D], caches
// [num_blocks,H_kv,16,D], block_tables maps logical to physical blocks,
// seq_lens counts the context including the new token; token t lives at
// cache[bt[s][t/16], g, t%16, :].  The pages' kernel runs one thread per
// (sequence, head) and walks every token serially; the project memory page
// ("Remaining Gap vs nano-vllm") names split-K flash-decoding as the fix.
//
// Design (bandwidth-bound: every visible K and V byte is read exactly once)
//   * grid (kv head g, sequence, split) with the split index slowest, so the
//     round-robin deal of workgroups to the 8 XCDs is balanced; a split covers
//     split_blocks consecutive logical blocks (16..128, the largest that still
//     leaves 8 workgroups per CU).  All G = H_q/H_kv query heads of kv head g
//     are served by the same workgroup, so each K/V byte is fetched once;
//   * inside a workgroup, wavefront w takes blocks w, w+4, ...; a block of
//     one kv head is a contiguous 4 KB slab per tensor, read as four
//     1 KB wavefront loads (lane l: token 4i + l/16, dims 8*(l%16)..+7).
//     The next block's slab is in flight while the current one is reduced,
//     and table entries arrive 64 at a time (one per lane, broadcast with
//     readlane);
//   * scores: fp16 dot2 products into fp32, reduced over the 16 lanes of a
//     token with DPP row operations;
//   * each 16-lane group keeps its own running (max, sum, o[8 dims]) per
//     query head, so no cross-group exchange happens inside the loop; at the
//     end the four groups of a wavefront merge with lane shuffles and the
//     four wavefronts through LDS;
//   * the split's (max, sum, unnormalised o) go to the workspace, and a
//     second kernel merges splits: M = max m_c, L = sum l_c 2^(m_c - M),
//     O = sum o_c 2^(m_c - M) / L (scores are kept in the log2 domain).
//     A sequence that fits one split is finished by the first kernel;
//   * balanced mode (plain decode with a workspace, up to 4096 sequences):
//     splits of a fixed length leave workgroups of very different lengths
//     when sequence lengths vary, and the last ones run with much of the
//     chip idle.  Instead each kv head's blocks, sequence after sequence and
//     each sequence charged a fixed cost of a few blocks, are cut into equal
//     runs, one workgroup each, as many as the GPU holds at once.  Run i of
//     every kv head covers the same (sequence, block) range and those
//     workgroups start together, so the kv heads' slabs of a physical block
//     are read at about the same time.  A run's part of a sequence is one
//     piece: a whole (sequence, kv head) is written out directly, the others
//     leave partials for the merge.  Every workgroup builds the prefix over
//     seq_lens in LDS to find its start;
//   * shared-prefix mode (forked sequences): a sequence's splits start after
//     its group's prefix blocks, whose partials the prefix kernel has
//     written; with one split per sequence the split kernel folds them in
//     itself, otherwise the merge kernel combines prefix and splits.
#include "attn_internal.h"

#include <math.h>

#include <atomic>

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int D = kDecodeHeadDim;     // 128
constexpr int BS = kDecodeBlockSize;  // 16

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Sum over the 16 lanes of a DPP row, result in every lane of the row.
__device__ __forceinline__ float row16_sum(float x) {
  // quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_ror:4 = 0x124, row_ror:8 = 0x128
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ float dot8(const half8_t& a, const half8_t& b) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2_t x = {a[2 * i], a[2 * i + 1]};
    const half2_t y = {b[2 * i], b[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2(x, y, acc, false);
  }
  return acc;
}

// Per-wavefront state of a workgroup's range, combined after a barrier.
template <int G>
struct DecodeLds {
  float m[kWaves][G];
  float l[kWaves][G];
  __attribute__((aligned(16))) float o[kWaves][G][D];
  int bad;
};

// Attention of the G query heads of kv head g of sequence s over its logical
// blocks [blk_begin, blk_end) (L visible tokens): each wavefront leaves its
// (max, sum, unnormalised o) per head in sm, the 16-lane groups of the
// wavefront already merged.  A table entry outside the pool sets sm.bad.
// The caller synchronises before and after.
template <int G>
__device__ __forceinline__ void attend_blocks(const DecodeArgs& a, int s, int g, int blk_begin, int blk_end,
                                              int L, DecodeLds<G>& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane >> 4;  // token slot inside a 4-token wavefront load
  const int dl = lane & 15;   // this lane's dims: 8*dl .. 8*dl+7

  half8_t qv[G];
#pragma unroll
  for (int j = 0; j < G; ++j)
    qv[j] = *reinterpret_cast<const half8_t*>(a.q + ((int64_t)s * a.H_q + g * G + j) * D + 8 * dl);

  float m[G], lsum[G], o[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    lsum[j] = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) o[j][d] = 0.0f;
  }

  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int64_t block_stride = (int64_t)a.H_kv * BS * D;
  // this lane's element offset inside a (block, kv head) slab
  const int64_t lane_off = (int64_t)g * BS * D + grp * D + 8 * dl;

  // Blocks of this wavefront: blk_begin + wave + i*kWaves, i < nb.  Their
  // table entries are fetched 64 at a time, one per lane, and broadcast
  // with readlane; the K/V slab of block i+1 is in flight while block i is
  // being reduced.
  const int nb = (blk_end - blk_begin - wave + kWaves - 1) / kWaves;
  int tab = 0;
  auto table_chunk = [&](int chunk) {
    const int i = chunk * 64 + lane;
    const int blk = blk_begin + wave + i * kWaves;
    tab = (i < nb) ? bt[blk] : 0;
  };
  auto fetch = [&](int i, half8_t (&kr)[4], half8_t (&vr)[4]) {
    if ((i & 63) == 0) table_chunk(i >> 6);
    int phys = __builtin_amdgcn_readlane(tab, i & 63);
    if (phys < 0 || (int64_t)phys >= a.num_blocks) {
      sm.bad = 1;  // the whole sequence reports NaN; read block 0 instead
      phys = 0;
    }
    const _Float16* kb = a.k_cache + (int64_t)phys * block_stride + lane_off;
    const _Float16* vb = a.v_cache + (int64_t)phys * block_stride + lane_off;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kr[u] = __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(kb + 4 * u * D));
      vr[u] = __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(vb + 4 * u * D));
    }
  };
  auto reduce = [&](int i, const half8_t (&kr)[4], const half8_t (&vr)[4]) {
    const int tok0 = (blk_begin + wave + i * kWaves) * BS;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float sc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float dot = row16_sum(dot8(qv[j], kr[u]));
        sc[u] = (tok0 + 4 * u + grp < L) ? dot * a.scale_log2 : -INFINITY;
      }
      const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      const float m_new = fmaxf(m[j], mx);
      if (m_new == -INFINITY) continue;  // no visible token for this group yet
      const float alpha = __builtin_amdgcn_exp2f(m[j] - m_new);
      float p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) p[u] = __builtin_amdgcn_exp2f(sc[u] - m_new);
      lsum[j] = lsum[j] * alpha + (p[0] + p[1]) + (p[2] + p[3]);
      m[j] = m_new;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        float acc = o[j][d] * alpha;
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = fmaf(p[u], (float)vr[u][d], acc);
        o[j][d] = acc;
      }
    }
  };

  half8_t ka[4], va[4], kb2[4], vb2[4];
  if (nb > 0) fetch(0, ka, va);
  for (int i = 0; i < nb; i += 2) {
    if (i + 1 < nb) fetch(i + 1, kb2, vb2);
    reduce(i, ka, va);
    if (i + 1 < nb) {
      if (i + 2 < nb) fetch(i + 2, ka, va);
      reduce(i + 1, kb2, vb2);
    }
  }

  // merge the four lane groups of each wavefront (lanes l, l^16, l^32, l^48
  // hold the same dims for different tokens), then the wavefronts via LDS
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float mm = m[j];
    mm = fmaxf(mm, __shfl_xor(mm, 16));
    mm = fmaxf(mm, __shfl_xor(mm, 32));
    const float w = (m[j] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m[j] - mm);
    float ls = lsum[j] * w;
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      float x = o[j][d] * w;
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      o[j][d] = x;
    }
    if (grp == 0) {
      if (dl == 0) {
        sm.m[wave][j] = mm;
        sm.l[wave][j] = ls;
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) sm.o[wave][j][8 * dl + d] = o[j][d];
    }
  }
}

// The four wavefronts' states of head j, dim d, combined.
template <int G>
__device__ __forceinline__ void combine_waves(const DecodeLds<G>& sm, int j, int d, float& M, float& Ls,
                                              float& Os) {
  M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) M = fmaxf(M, sm.m[k][j]);
  Ls = 0.0f;
  Os = 0.0f;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    const float mk = sm.m[k][j];
    const float w = (mk == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mk - M);
    Ls = fmaf(sm.l[k][j], w, Ls);
    Os = fmaf(sm.o[k][j][d], w, Os);
  }
}

template <int G>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  // linear block id -> (kv head, sequence, split), split slowest: consecutive
  // workgroups (which the dispatcher deals round-robin to the 8 XCDs) are
  // different (sequence, head) pairs of the same split, so every XCD gets an
  // even share of full splits, and the partial or empty last splits of short
  // sequences come at the end of the grid.
  const int pairs = a.num_seqs * a.H_kv;
  const int split = blockIdx.x / pairs;
  const int g = (blockIdx.x - split * pairs) % a.H_kv;
  const int s = (blockIdx.x - split * pairs) / a.H_kv;
  const int tid = threadIdx.x;

  __shared__ DecodeLds<G> sm;

  const int L_raw = a.seq_lens[s];
  const int cap = a.max_blocks_per_seq * BS;
  const bool len_bad = L_raw > cap;
  const int L = len_bad ? cap : L_raw;
  // shared-prefix mode: the first `skip` blocks belong to the group's
  // prefix.  With one split per sequence this kernel also folds in the
  // prefix partials and writes the output (no merge kernel); otherwise the
  // merge kernel reports broken preconditions.
  const bool shared_direct = a.group_start && a.n_split_max == 1;
  int skip = 0;
  bool pre_bad = false;
  if (a.group_start) {
    // the prefix must be valid (seq_skip >= 0) and fit the sequence
    skip = a.seq_skip[s];
    pre_bad = skip < 0 || skip * BS > L;
    if (pre_bad) {
      if (!shared_direct) return;
      skip = 0;
    }
  }
  const int rem_blocks = (L + BS - 1) / BS - skip;
  const int n_split = (L > 0 && rem_blocks > 0) ? (rem_blocks + a.split_blocks - 1) / a.split_blocks : 0;
  // this workgroup writes the final output (one split, or shared direct)
  const bool direct = (n_split <= 1 && !a.group_start) || shared_direct;

  if (L <= 0 || (shared_direct && (pre_bad || len_bad))) {
    // zero-length context: an all-zero row; a broken precondition in shared
    // direct mode: NaN rows.  Written once (by the merge kernel in the other
    // shared-prefix mode)
    if (split == 0 && (!a.group_start || shared_direct)) {
      const _Float16 fill = (_Float16)(L_raw <= 0 ? 0.0f : __builtin_nanf(""));
      for (int idx = tid; idx < G * D; idx += kThreads) {
        const int j = idx / D, d = idx - j * D;
        a.out[((int64_t)s * a.H_q + g * G + j) * D + d] = fill;
      }
    }
    return;
  }
  // empty split (in shared direct mode split 0 runs even with no own
  // blocks: the sequence is its prefix, and the output is still written here)
  if (split >= (shared_direct ? 1 : n_split)) return;

  if (tid == 0) sm.bad = len_bad ? 1 : 0;
  __syncthreads();

  const int blk_begin = skip + split * a.split_blocks;
  const int blk_end = min(blk_begin + a.split_blocks, (L + BS - 1) / BS);

  attend_blocks<G>(a, s, g, blk_begin, blk_end, L, sm);
  __syncthreads();

  const bool bad = sm.bad != 0;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int j = idx / D;
    const int d = idx - j * D;
    float M, Ls, Os;
    combine_waves<G>(sm, j, d, M, Ls, Os);
    const int h = g * G + j;
    if (bad) {
      M = Ls = Os = __builtin_nanf("");
    }
    if (shared_direct) {
      // fold in the prefix chunks' partials (written by the prefix kernel
      // earlier on the stream); a NaN partial keeps the row NaN
      // (four slots per round trip, combined online)
      const int n_pre = (skip + kPrefixChunkBlocks - 1) / kPrefixChunkBlocks;
      const int64_t base = ((int64_t)s * a.H_q + h) * a.slot_stride;
      float Mt = M;
      for (int c0 = 0; c0 < n_pre; c0 += 4) {
        float mc[4], lc[4], oc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool ok = c0 + u < n_pre;
          const int64_t slot = base + (ok ? c0 + u : 0);
          mc[u] = ok ? a.ws_ml[slot * 2] : -INFINITY;
          lc[u] = ok ? a.ws_ml[slot * 2 + 1] : 0.0f;
          oc[u] = ok ? a.ws_o[slot * D + d] : 0.0f;
        }
        float mn = Mt;
#pragma unroll
        for (int u = 0; u < 4; ++u) mn = fmaxf(mn, mc[u]);
        const float wown = (Mt == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(Mt - mn);
        Ls *= wown;
        Os *= wown;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float w = (mc[u] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mc[u] - mn);
          Ls = fmaf(lc[u], w, Ls);
          Os = fmaf(oc[u], w, Os);
        }
        Mt = mn;
      }
    }
    if (direct) {
      a.out[((int64_t)s * a.H_q + h) * D + d] = (_Float16)(Os / Ls);
    } else {
      const int64_t slot = ((int64_t)s * a.H_q + h) * a.slot_stride + a.prefix_slots + split;
      a.ws_o[slot * D + d] = Os;
      if (d == 0) {
        a.ws_ml[slot * 2 + 0] = M;
        a.ws_ml[slot * 2 + 1] = Ls;
      }
    }
  }
}

// One workgroup of D threads per (sequence, query head): merge the splits
// (and, in shared-prefix mode, the group's prefix chunks).
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  const int s = blockIdx.x / a.H_q;
  const int h = blockIdx.x - s * a.H_q;
  const int d = threadIdx.x;
  const int L_raw = a.seq_lens[s];
  const int cap = a.max_blocks_per_seq * BS;
  const int L = L_raw > cap ? cap : L_raw;
  _Float16* dst = a.out + ((int64_t)s * a.H_q + h) * D + d;
  const int64_t base = ((int64_t)s * a.H_q + h) * a.slot_stride;
  int n_pre = 0, first_split = 0, skip = 0;
  if (a.group_start) {
    if (L_raw <= 0) {
      *dst = (_Float16)0.0f;
      return;
    }
    // the prefix must be valid and fit the sequence (whole visible blocks)
    skip = a.seq_skip[s];
    if (skip < 0 || L_raw > cap || skip * BS > L) {
      *dst = (_Float16)__builtin_nanf("");
      return;
    }
    n_pre = (skip + kPrefixChunkBlocks - 1) / kPrefixChunkBlocks;
    first_split = a.prefix_slots;
  }
  const int rem_blocks = (L + BS - 1) / BS - skip;
  const int n_split = (L > 0 && rem_blocks > 0) ? (rem_blocks + a.split_blocks - 1) / a.split_blocks : 0;
  if (!a.group_start && n_split <= 1) return;  // finished by the split kernel
  float M = -INFINITY;
  for (int c = 0; c < n_pre; ++c) M = fmaxf(M, a.ws_ml[(base + c) * 2]);
  for (int c = 0; c < n_split; ++c) M = fmaxf(M, a.ws_ml[(base + first_split + c) * 2]);
  float Ls = 0.0f, Os = 0.0f;
  auto add = [&](int64_t slot) {
    const float mc = a.ws_ml[slot * 2];
    const float w = (mc == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mc - M);
    Ls = fmaf(a.ws_ml[slot * 2 + 1], w, Ls);
    Os = fmaf(a.ws_o[slot * D + d], w, Os);
  };
  for (int c = 0; c < n_pre; ++c) add(base + c);
  for (int c = 0; c < n_split; ++c) add(base + first_split + c);
  *dst = (_Float16)(Os / Ls);
}

// Fixed cost of a piece (table and first K/V round trips, the combine, the
// partial write) in units of one block's streaming: every sequence with
// blocks is charged this much in front of its blocks when runs are cut, so
// runs over many short sequences take fewer blocks.
#ifndef DECODE_PIECE_COST
#define DECODE_PIECE_COST 6
#endif
constexpr int kPieceCost = DECODE_PIECE_COST;

// Cost units per run of the balanced mode: the T units of one kv head over
// its `runs` runs, rounded up, and at least kDecodeMinRun (the balanced
// kernel and its merge must agree on it).
__device__ __forceinline__ int balanced_run(int T, int runs) {
  const int r = (T + runs - 1) / runs;
  return r > kDecodeMinRun ? r : kDecodeMinRun;
}

// Balanced mode.  Every kv head has the same sequence of cost units:
// sequence after sequence, kPieceCost units then its blocks (nothing for an
// empty sequence), T in all.  They are cut into runs = workers / H_kv runs of
// R = balanced_run(T, runs) units; workgroup w takes run i = w / H_kv of kv
// head g = w % H_kv, and the blocks whose units fall in it.  Run i
// covers the same (sequence, block) range in every kv head, and those H_kv
// workgroups are dispatched together, so the H_kv slabs of a physical block
// (one contiguous 32 KB at H_kv = 8) are read at about the same time, as in
// the split grid.  The piece of sequence s in run i of kv head g leaves its
// partials in slot g (num_seqs + runs) + s + i: s + i grows along a kv head's
// pieces, so slots are unique.
template <int G>
__global__ __launch_bounds__(kThreads, G <= 2 ? 4 : 1) void decode_balanced_kernel(DecodeArgs a) {
  __shared__ DecodeLds<G> sm;
  __shared__ int pre[kDecodeBalancedMaxSeqs + 1];  // cost units per kv head before each sequence
  __shared__ int wsum[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = a.num_seqs;  // <= kDecodeBalancedMaxSeqs (host check)
  const int cap = a.max_blocks_per_seq * BS;
  // visible blocks of sequence i (lengths past the table are cut to it; the
  // sequence still reports NaN below)
  auto nblk = [&](int i) {
    const int lr = a.seq_lens[i];
    const int l = lr > cap ? cap : lr;
    return l > 0 ? (l + BS - 1) / BS + kPieceCost : 0;  // cost units of sequence i
  };
  // exclusive prefix over the sequences: thread t sums entries
  // [t per, (t + 1) per), the sums are scanned across the workgroup, and each
  // thread writes the prefix of its entries
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  int loc = 0;
  for (int i = i0; i < i1; ++i) loc += nblk(i);
  int inc = loc;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int run = inc - loc;
  for (int k = 0; k < wave; ++k) run += wsum[k];
  for (int i = i0; i < i1; ++i) {
    pre[i] = run;
    run += nblk(i);
  }
  if (tid == kThreads - 1) pre[n] = run;  // the last thread's end is the total
  __syncthreads();
  // the merge kernel needs the same prefix
  if (blockIdx.x == 0)
    for (int i = tid; i <= n; i += kThreads) a.run_prefix[i] = pre[i];

  const int runs = a.workers / a.H_kv;
  const int g = (int)blockIdx.x % a.H_kv;
  const int run_i = (int)blockIdx.x / a.H_kv;
  const int T = pre[n];
  const int R = balanced_run(T, runs);
  if (run_i >= runs) return;
  const int64_t y0 = (int64_t)run_i * R;
  if (y0 >= T) return;
  const int y = (int)y0;
  const int end = (int)min((int64_t)T, y0 + R);
  // the first sequence that reaches into the run: the last s with pre[s] <=
  // y (pre[0] = 0 <= y < pre[n])
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= y) lo = mid;
    else hi = mid;
  }
  for (int s = lo; s < n && pre[s] < end; ++s) {
    const int span = pre[s + 1] - pre[s];
    if (span == 0) continue;  // empty sequence
    const int nb = span - kPieceCost;
    const int first = pre[s] + kPieceCost;  // unit of block 0
    const int b0 = max(0, y - first), b1 = min(nb, end - first);
    if (b1 <= b0) continue;  // only the sequence's fixed units fall in this run
    const int lr = a.seq_lens[s];
    const bool len_bad = lr > cap;
    __syncthreads();  // the previous piece's combine has read sm
    if (tid == 0) sm.bad = len_bad ? 1 : 0;
    __syncthreads();
    attend_blocks<G>(a, s, g, b0, b1, len_bad ? cap : lr, sm);
    __syncthreads();
    const bool bad = sm.bad != 0;
    const bool whole = b0 == 0 && b1 == nb;
    const int slot = g * (n + runs) + s + run_i;  // host: the whole workspace is < 2^31 floats
    // the bases, redefined here, keep the compiler from holding per-lane
    // store addresses across the block loop (at G = 2 that costs a spill)
    _Float16* outp = a.out;
    float* wso = a.ws_o;
    float* wsml = a.ws_ml;
    asm volatile("" : "+s"(outp), "+s"(wso), "+s"(wsml));
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int j = idx / D;
      const int d = idx - j * D;
      float M, Ls, Os;
      combine_waves<G>(sm, j, d, M, Ls, Os);
      if (bad) M = Ls = Os = __builtin_nanf("");
      if (whole) {
        outp[((int64_t)s * a.H_q + g * G + j) * D + d] = (_Float16)(Os / Ls);
      } else {
        wso[(slot * G + j) * D + d] = Os;
        if (d == 0) {
          wsml[(slot * G + j) * 2 + 0] = M;
          wsml[(slot * G + j) * 2 + 1] = Ls;
        }
      }
    }
  }
}

// One workgroup of D threads per (sequence, query head) in balanced mode:
// zero rows for empty sequences, and the partials of a (sequence, kv head)
// that spans several runs (runs i0..i1 of its kv head).
__global__ __launch_bounds__(D) void decode_balanced_merge_kernel(DecodeArgs a) {
  const int s = blockIdx.x / a.H_q;
  const int h = blockIdx.x - s * a.H_q;
  const int d = threadIdx.x;
  const int G = a.H_q / a.H_kv;
  const int g = h / G, j = h - g * G;
  _Float16* dst = a.out + ((int64_t)s * a.H_q + h) * D + d;
  const int p0 = a.run_prefix[s];
  const int span = a.run_prefix[s + 1] - p0;
  if (span == 0) {  // no visible token: a zero row
    *dst = (_Float16)0.0f;
    return;
  }
  const int runs = a.workers / a.H_kv;
  const int R = balanced_run(a.run_prefix[a.num_seqs], runs);
  // the runs that hold blocks of the sequence (units p0 + kPieceCost ..
  // p0 + span - 1)
  const int i0 = (p0 + kPieceCost) / R, i1 = (p0 + span - 1) / R;
  if (i0 == i1) return;  // one run held it whole and wrote it
  const int64_t base = (int64_t)g * (a.num_seqs + runs) + s;
  float M = -INFINITY;
  for (int i = i0; i <= i1; ++i) M = fmaxf(M, a.ws_ml[((base + i) * G + j) * 2]);
  float Ls = 0.0f, Os = 0.0f;
  for (int i = i0; i <= i1; ++i) {
    const int64_t slot = (base + i) * G + j;
    const float mc = a.ws_ml[slot * 2];
    const float wt = (mc == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mc - M);
    Ls = fmaf(a.ws_ml[slot * 2 + 1], wt, Ls);
    Os = fmaf(a.ws_o[slot * D + d], wt, Os);
  }
  *dst = (_Float16)(Os / Ls);
}

// Runs of the balanced mode on the current device: as many as workgroups of
// the balanced kernel fit on it at once (one round, all ending together),
// at most the kDecodeWorkers the workspace holds slots for.  Cached per
// device.
template <int G>
int balanced_workers() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kDecodeWorkers;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&decode_balanced_kernel<G>),
                                                   kThreads, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0)
    return kDecodeWorkers;
  const int w = cus * per_cu < kDecodeWorkers ? cus * per_cu : kDecodeWorkers;
  if (dev < kMaxDevices) cached[dev].store(w, std::memory_order_relaxed);
  return w;
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  DecodeArgs args = a;
  void* kargs[] = {&args};
  if (a.workers > 0) {
    args.workers = balanced_workers<G>();  // <= a.workers, the slots the workspace holds
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_balanced_kernel<G>),
                                   dim3((unsigned)a.workers), dim3(kThreads), kargs, 0, stream);
    if (e != hipSuccess) return e;
    return hipLaunchKernel(reinterpret_cast<const void*>(&decode_balanced_merge_kernel),
                           dim3((unsigned)(a.num_seqs * a.H_q)), dim3(D), kargs, 0, stream);
  }
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_split_kernel<G>),
                                 dim3((unsigned)((int64_t)a.n_split_max * a.H_kv * a.num_seqs)), dim3(kThreads), kargs, 0, stream);
  if (e != hipSuccess || a.n_split_max <= 1) return e;  // one split: finished by the split kernel
  return hipLaunchKernel(reinterpret_cast<const void*>(&decode_merge_kernel),
                         dim3((unsigned)(a.num_seqs * a.H_q)), dim3(D), kargs, 0, stream);
}

}  // namespace

// Largest split (in 16-token blocks) that still gives at least 8 workgroups
// per CU over the table width: long splits amortise each workgroup's start-up
// and partial write, many workgroups keep every CU's memory queue full.
int decode_split_blocks(int num_seqs, int H_kv, int max_blocks_per_seq) {
  const int64_t pairs = (int64_t)num_seqs * H_kv;
  const int64_t want = 8 * 256;
  for (int split = 128; split > 16; split /= 2)
    if (pairs * ((max_blocks_per_seq + split - 1) / split) >= want) return split;
  return 16;
}

hipError_t launch_decode(const DecodeArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 3: return launch_g<3>(a, stream);
    case 4: return launch_g<4>(a, stream);
    case 5: return launch_g<5>(a, stream);
    case 6: return launch_g<6>(a, stream);
    case 7: return launch_g<7>(a, stream);
    case 8: return launch_g<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
