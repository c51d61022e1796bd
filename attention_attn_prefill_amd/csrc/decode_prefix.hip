// decode_prefix.hip -- the shared prefix of forked sequences in paged decode
// (cascade attention), gfx950.
//
// GRPO samples several completions from one prompt; the engine forks the
// prompt's cache by copying block-table pointers only ("GRPO-CUDA Project
// Memory", "KV Cache design": paged_kv_cache_fork), so the sequences of a
// group share their leading physical blocks.  Plain paged decode reads those
// blocks once per sequence.  Here each group's prefix is read once for all of
// its query rows:
//   * the query rows of a group and kv head g are the G = H_q/H_kv heads of
//     g for every sequence of the group, R = group size * G rows; they are
//     the 32 MFMA columns of one workgroup (more rows take more column
//     blocks, each re-reading the prefix);
//   * a workgroup takes kPrefixChunkBlocks prefix blocks (read through the
//     group's first table row: the prefix entries of every table in the group
//     are the same blocks); its 4 wavefronts take 32-key tiles (two blocks)
//     in turn;
//   * per tile: S^T[32 keys x 32 rows] = K Q^T with v_mfma_f32_32x32x16_f16,
//     the K operand read straight from the cache (lane l: key l % 32, 16
//     bytes at dims 8 * (l / 32) + 16 * step), the Q fragment held in VGPRs;
//     online softmax in the log2 domain (each row's 32 scores sit in lanes l
//     and l + 32); O^T[D x 32] += V^T P^T with the V tile staged row-major
//     in the wavefront's own LDS region and the V^T operand read with the
//     transposing ds_read_b64_tr_b16, P^T taken from the score accumulator;
//   * the wavefronts merge through LDS and the workgroup writes one partial
//     (unnormalised o, max, sum) per query row into the decode workspace
//     slot of its chunk; the decode merge kernel combines these with the
//     per-sequence suffix splits.
#include "attn_internal.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int D = kDecodeHeadDim;     // 128
constexpr int BS = kDecodeBlockSize;  // 16
constexpr int VROW = D + 32;          // LDS row stride of the V tile (halfs): 4 rows of a tr read hit disjoint banks
constexpr int CB = kPrefixChunkBlocks;

typedef short short4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ short4_t lds_read_tr(const _Float16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
}

// V^T operand of 16 keys (chunk c of the 32-key tile) for d tile dt, in the
// key order of the P^T operand taken from the score accumulator: keys
// 16c + 4*hf + (0..3), then 16c + 8 + 4*hf + (0..3).
__device__ __forceinline__ half8_t pv_operand(const _Float16* vl, int dt, int c) {
  const short4_t lo = lds_read_tr(vl + 16 * c * VROW + dt * 32);
  const short4_t hi = lds_read_tr(vl + (16 * c + 8) * VROW + dt * 32);
  const short4_t lohi[2] = {lo, hi};
  return __builtin_bit_cast(half8_t, lohi);
}

__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int G>
__global__ __launch_bounds__(64 * kWaves) void prefix_chunk_kernel(DecodeArgs a, int col_blocks) {
  // block id -> (chunk, group, kv head, column block), chunk slowest
  const int per_chunk = a.num_groups * a.H_kv * col_blocks;
  const int chunk = blockIdx.x / per_chunk;
  int rest = blockIdx.x - chunk * per_chunk;
  const int cb = rest % col_blocks;
  rest /= col_blocks;
  const int g = rest % a.H_kv;
  const int gi = rest / a.H_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;

  __shared__ __attribute__((aligned(16))) _Float16 v_lds[kWaves][32 * VROW];
  __shared__ float sm_m[kWaves][32];
  __shared__ float sm_l[kWaves][32];
  __shared__ __attribute__((aligned(16))) float sm_o[kWaves][32][D + 4];
  __shared__ int sm_bad;

  // group and chunk extents; anything inconsistent is left to the merge
  // kernel, which reports NaN for the group's sequences
  const int gs = a.group_start[gi], ge = a.group_start[gi + 1];
  if (gs < 0 || ge > a.num_seqs || ge < gs || ge - gs > a.max_group_size) return;
  const int rows = (ge - gs) * G;
  if (32 * cb >= rows) return;
  const int P = a.prefix_blocks[gi];
  if (P < 0 || P > a.max_blocks_per_seq) return;
  const int b_begin = chunk * CB;
  if (b_begin >= P) return;
  const int b_end = min(b_begin + CB, P);
  if (tid == 0) sm_bad = 0;
  __syncthreads();

  // this lane's query row (MFMA column) and its Q fragment
  const int r = 32 * cb + col;
  const bool valid_row = r < rows;
  const int s = gs + (valid_row ? r / G : 0);
  const int h = g * G + (valid_row ? r % G : 0);
  half8_t qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = valid_row ? *reinterpret_cast<const half8_t*>(a.q + ((int64_t)s * a.H_q + h) * D + 16 * ks + 8 * hf)
                       : half8_t{};

  const int32_t* bt = a.block_tables + (int64_t)gs * a.max_blocks_per_seq;
  const int64_t slab = (int64_t)a.H_kv * BS * D;  // elements per physical block
  const int64_t head_off = (int64_t)g * BS * D;
  _Float16* vl = v_lds[wave];
  // transposing-read offset of this lane inside the V tile
  const int v_lane = (4 * hf + (lane & 15) / 4) * VROW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  float m = -INFINITY, l = 0.0f;
  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};

  const int n_tiles = (b_end - b_begin + 1) / 2;
  for (int t = wave; t < n_tiles; t += kWaves) {
    const int b0 = b_begin + 2 * t;
    const bool has1 = b0 + 1 < b_end;
    int p0 = bt[b0];
    int p1 = has1 ? bt[b0 + 1] : p0;
    if (p0 < 0 || (int64_t)p0 >= a.num_blocks || p1 < 0 || (int64_t)p1 >= a.num_blocks) {
      sm_bad = 1;  // the group reports NaN; read block 0 instead
      p0 = p1 = 0;
    }
    // K operand: key col (block col / 16, row col % 16)
    const _Float16* kp = a.k_cache + (int64_t)(col < 16 ? p0 : p1) * slab + head_off + (col & 15) * D + 8 * hf;
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const half8_t kf = *reinterpret_cast<const half8_t*>(kp + 16 * ks);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], sc, 0, 0, 0);
    }
    // stage V rows (key kk = lane / 16 + 4u, dims 8 * (lane % 16)) into LDS
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kk = (lane >> 4) + 4 * u;
      const _Float16* vp = a.v_cache + (int64_t)(kk < 16 ? p0 : p1) * slab + head_off + (kk & 15) * D + 8 * (lane & 15);
      *reinterpret_cast<half8_t*>(vl + kk * VROW + 8 * (lane & 15)) = *reinterpret_cast<const half8_t*>(vp);
    }
    // scores (log2 domain); keys of a missing second block are masked.
    // Accumulator element i holds key 8 * (i / 4) + 4 * hf + i % 4.
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 8 * (i >> 2) + 4 * hf + (i & 3);
      sc[i] = (key < 16 || has1) ? sc[i] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    mx = half_swap_max(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - m_new);
    half8_t pf[2];
    float ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(sc[i] - m_new);
      ps += p;
      pf[i >> 3][i & 7] = (_Float16)p;
    }
    l = l * alpha + ps;
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pv_operand(vl + v_lane, dt, c), pf[c], o[dt], 0, 0, 0);
  }

  // per-wavefront results: row col's sum is split over lanes col, col + 32
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    const float lrow = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (hf == 0) {
      sm_m[wave][col] = m;
      sm_l[wave][col] = lrow;
    }
    // O^T element (d = dt*32 + 8*(i/4) + 4*hf + i%4, row col)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sm_o[wave][col][dt * 32 + 8 * (i >> 2) + 4 * hf + (i & 3)] = o[dt][i];
  }
  __syncthreads();

  // merge the wavefronts and write one partial per valid row
  const bool bad = sm_bad != 0;
  for (int idx = tid; idx < 32 * D; idx += 64 * kWaves) {
    const int rr = idx / D, d = idx - rr * D;
    const int row = 32 * cb + rr;
    if (row >= rows) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][rr]);
    float Ls = 0.0f, Os = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][rr];
      const float wt = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      Ls = fmaf(sm_l[w][rr], wt, Ls);
      Os = fmaf(sm_o[w][rr][d], wt, Os);
    }
    if (bad) M = Ls = Os = __builtin_nanf("");
    const int ss = gs + row / G, hh = g * G + row % G;
    const int64_t slot = ((int64_t)ss * a.H_q + hh) * a.slot_stride + chunk;
    a.ws_o[slot * D + d] = Os;
    if (d == 0) {
      a.ws_ml[slot * 2 + 0] = M;
      a.ws_ml[slot * 2 + 1] = Ls;
    }
  }
}

template <int G>
hipError_t launch_prefix_g(const DecodeArgs& a, hipStream_t stream) {
  const int col_blocks = (a.max_group_size * G + 31) / 32;
  const int64_t blocks = (int64_t)a.prefix_slots * a.num_groups * a.H_kv * col_blocks;
  DecodeArgs args = a;
  int cbs = col_blocks;
  void* kargs[] = {&args, &cbs};
  return hipLaunchKernel(reinterpret_cast<const void*>(&prefix_chunk_kernel<G>), dim3((unsigned)blocks),
                         dim3(64 * kWaves), kargs, 0, stream);
}

}  // namespace

hipError_t launch_decode_prefix(const DecodeArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_prefix_g<1>(a, stream);
    case 2: return launch_prefix_g<2>(a, stream);
    case 3: return launch_prefix_g<3>(a, stream);
    case 4: return launch_prefix_g<4>(a, stream);
    case 5: return launch_prefix_g<5>(a, stream);
    case 6: return launch_prefix_g<6>(a, stream);
    case 7: return launch_prefix_g<7>(a, stream);
    case 8: return launch_prefix_g<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
