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
//     are the same blocks) as 32-key tiles (two blocks);
//   * the tiles stream through a ring of kStages LDS stages filled by
//     buffer-to-LDS loads (no registers held while in flight), kStages - 1
//     tiles ahead; each wavefront fills a quarter of every tile;
//   * every wavefront computes the whole score tile S^T[32 keys x 32 rows] =
//     K Q^T with v_mfma_f32_32x32x16_f16 (K from LDS, Q in VGPRs) and the
//     same online softmax in the log2 domain, and owns one 32-wide slice of
//     the head dimension of O^T += V^T P^T (V^T read with the transposing
//     ds_read_b64_tr_b16, P^T taken from the score accumulator), so the
//     wavefronts never merge: each writes its slice of the partial
//     (unnormalised o) and wavefront 0 the (max, sum) of every row into the
//     decode workspace slot of its chunk; the decode merge kernel combines
//     these with the per-sequence suffix splits.
// LDS tiles are unpadded 256-byte key rows.  K: 16-byte chunk c of row r sits
// at chunk c ^ (r % 16), so the 16 rows one K-operand read touches spread
// over all banks.  V: 64-byte segment s of row r sits at s ^ (r % 4), so the
// four rows of a transposing read hit four different segments.  The loads
// put each lane's 16 bytes at the swizzled place directly.
#include "attn_internal.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int D = kDecodeHeadDim;     // 128
constexpr int BS = kDecodeBlockSize;  // 16
constexpr int CB = kPrefixChunkBlocks;
constexpr int kStages = 4;
constexpr int kTileHalfs = 32 * D;    // one 32-key tile of K or V
static_assert(CB % 2 == 0 && CB <= 64, "a chunk is whole 2-block tiles, its table entries one per lane");

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

typedef short short4_t __attribute__((ext_vector_type(4)));

// The V^T operands of a whole 32-key tile: four transposing reads at the
// lane's LDS byte address + 0, 8, 16 and 24 rows.  Written as one asm block
// that waits for its own reads: the compiler cannot tell these reads from
// the buffer-to-LDS loads still in flight into other stages and would
// otherwise wait for all of them first; the ring protocol (vmcnt wait and
// barrier before a tile is read) already orders them.  The outputs are
// early-clobber: a read's destination must not be the address register
// that a later read of the block still uses (its data can land before the
// later read issues).
__device__ __forceinline__ void lds_read_tr_tile(uint32_t addr, short4_t (&r)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:4096\n\t"
      "ds_read_b64_tr_b16 %3, %4 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(addr)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const _Float16* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) _Float16*)p);
}

__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_swap_add(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// buffer resource over one (block, kv head) slab of 4 KB
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const _Float16* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, BS * D * 2, 0x00020000);
}

// Wait until at most `ahead` tiles (4 buffer-to-LDS loads per lane each)
// are still in flight behind the current one.
__device__ __forceinline__ void wait_tiles(int ahead) {
  static_assert(kStages >= 2 && kStages <= 8, "vmcnt immediates below cover up to six tiles ahead");
  switch (ahead) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
  }
}

template <int G>
__global__ __launch_bounds__(64 * kWaves) void prefix_chunk_kernel(DecodeArgs a, int col_blocks) {
  // block id -> (chunk, group, kv head, column block), chunk slowest
  const int per_chunk = a.num_groups * a.H_kv * col_blocks;
  const int main_blocks = a.prefix_slots * per_chunk;
  if ((int)blockIdx.x >= main_blocks) {
    // the trailing workgroups record every sequence's prefix length (or -1
    // when its group breaks a checked rule) for the split and merge kernels
    const int s = ((int)blockIdx.x - main_blocks) * (64 * kWaves) + (int)threadIdx.x;
    if (s < a.num_seqs) {
      int gi, skip;
      a.seq_skip[s] = decode_group_of(a, s, gi, skip) ? skip : -1;
    }
    return;
  }
  const int chunk = blockIdx.x / per_chunk;
  int rest = blockIdx.x - chunk * per_chunk;
  const int cb = rest % col_blocks;
  rest /= col_blocks;
  const int g = rest % a.H_kv;
  const int gi = rest / a.H_kv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;

  __shared__ __attribute__((aligned(1024))) _Float16 ring[kStages][2][kTileHalfs];

  // group and chunk extents (uniform over the workgroup); anything
  // inconsistent is left to the merge kernel, which reports NaN
  const int gs = a.group_start[gi], ge = a.group_start[gi + 1];
  if (gs < 0 || ge > a.num_seqs || ge < gs || ge - gs > a.max_group_size) return;
  const int rows = (ge - gs) * G;
  if (32 * cb >= rows) return;
  const int P = a.prefix_blocks[gi];
  if (P < 0 || P > a.max_blocks_per_seq) return;
  const int b_begin = chunk * CB;
  if (b_begin >= P) return;
  const int nb = min(CB, P - b_begin);
  const int n_tiles = (nb + 1) / 2;

  // the chunk's table entries, one per lane; a bad entry turns the group's
  // rows NaN and block 0 is read in its place
  const int32_t* bt = a.block_tables + (int64_t)gs * a.max_blocks_per_seq + b_begin;
  int ent = lane < nb ? bt[lane] : 0;
  const bool ent_bad = ent < 0 || (int64_t)ent >= a.num_blocks;
  const bool bad = __builtin_amdgcn_ballot_w64(ent_bad) != 0;
  if (ent_bad) ent = 0;

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
  // take the Q loads' wait here, before the tile loads are in flight
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(qf[ks]));

  // loads: wavefront w fills key rows 8w .. 8w + 7 of each tile (block w / 2
  // of the pair), two 4-row loads of 1 KB for K and two for V; lane i of a
  // load lands at row R0 + i / 16, 16-byte place i % 16
  const int64_t slab = (int64_t)a.H_kv * BS * D;
  const int64_t head_off = (int64_t)g * BS * D;
  int voff_k[2], voff_v[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rr = 8 * (wave & 1) + 4 * j + (lane >> 4);  // row inside the block
    const int pl = lane & 15;                             // place inside the LDS row
    voff_k[j] = rr * 256 + 16 * (pl ^ rr);
    voff_v[j] = rr * 256 + 16 * (4 * ((pl >> 2) ^ (rr & 3)) + (pl & 3));
  }
  auto issue = [&](int t) {
    const int e0 = __builtin_amdgcn_readlane(ent, 2 * t);
    const int e1 = 2 * t + 1 < nb ? __builtin_amdgcn_readlane(ent, 2 * t + 1) : e0;
    const int64_t blk = (wave < 2 ? e0 : e1) * slab + head_off;
    const __amdgpu_buffer_rsrc_t kr = slab_rsrc(a.k_cache + blk);
    const __amdgpu_buffer_rsrc_t vr = slab_rsrc(a.v_cache + blk);
    _Float16* kd = ring[t % kStages][0] + 8 * wave * D;
    _Float16* vd = ring[t % kStages][1] + 8 * wave * D;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, LDS_PTR(kd + 4 * j * D), 16, voff_k[j], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, LDS_PTR(vd + 4 * j * D), 16, voff_v[j], 0, 0, 0);
    }
  };

  // K operand: key col, 16-byte chunk 2 ks + hf at chunk (2 ks + hf) ^ (col % 16)
  const int k_row = col * D;
  const int k_x = col & 15;
  // V^T operand of 16 keys (chunk c of the tile) for this wavefront's d
  // slice, in the key order of the P^T operand taken from the score
  // accumulator (keys 16c + 4hf + 0..3, then 16c + 8 + 4hf + 0..3); the
  // four rows of a read differ in row % 4 = (lane % 16) / 4
  const int vq = (lane & 15) >> 2;
  const int v_lane = (4 * hf + vq) * D + 32 * (wave ^ vq) + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  float m = -INFINITY, l = 0.0f;
  f32x16_t o = f32x16_t{};

#pragma unroll
  for (int t = 0; t < kStages - 1; ++t)
    if (t < n_tiles) issue(t);

  for (int t = 0; t < n_tiles; ++t) {
    wait_tiles(min(kStages - 2, n_tiles - 1 - t));
    // tile t is in LDS for every wavefront, and every wavefront is done
    // with tile t - 1, whose stage is refilled next.  A bare barrier: the
    // waits it needs are explicit (the loads' vmcnt above; every LDS read of
    // tile t - 1 has been waited for by its consumer), and a fenced barrier
    // would wait for the tiles still in flight.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + kStages - 1 < n_tiles) issue(t + kStages - 1);

    const _Float16* kl = ring[t % kStages][0];
    const _Float16* vl = ring[t % kStages][1];
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const half8_t kf = *reinterpret_cast<const half8_t*>(kl + k_row + 8 * ((2 * ks + hf) ^ k_x));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], sc, 0, 0, 0);
    }
    // scores (log2 domain); keys of a missing second block are masked.
    // Accumulator element i holds key 8 * (i / 4) + 4 * hf + i % 4.
    const bool has1 = 2 * t + 1 < nb;
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
    o *= alpha;
    short4_t vt[4];  // rows +0, +8 (keys 0..15) and +16, +24 (keys 16..31)
    lds_read_tr_tile(lds_addr(vl + v_lane), vt);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const short4_t lohi[2] = {vt[2 * c], vt[2 * c + 1]};
      o = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, lohi), pf[c], o, 0, 0, 0);
    }
  }

  // row col's sum is split over lanes col and col + 32
  const float lrow = half_swap_add(l);
  if (!valid_row) return;
  const float nan = __builtin_nanf("");
  const int64_t slot = ((int64_t)s * a.H_q + h) * a.slot_stride + chunk;
  // O^T element i: d = 32 wave + 8 (i / 4) + 4 hf + i % 4, row col
  float* od = a.ws_o + slot * D + 32 * wave + 4 * hf;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    float4 v4 = {o[4 * q4], o[4 * q4 + 1], o[4 * q4 + 2], o[4 * q4 + 3]};
    if (bad) v4 = {nan, nan, nan, nan};
    *reinterpret_cast<float4*>(od + 8 * q4) = v4;
  }
  if (wave == 0 && hf == 0) {
    a.ws_ml[slot * 2 + 0] = bad ? nan : m;
    a.ws_ml[slot * 2 + 1] = bad ? nan : lrow;
  }
}

template <int G>
hipError_t launch_prefix_g(const DecodeArgs& a, hipStream_t stream) {
  const int col_blocks = (a.max_group_size * G + 31) / 32;
  const int64_t blocks = (int64_t)a.prefix_slots * a.num_groups * a.H_kv * col_blocks +
                        (a.num_seqs + 64 * kWaves - 1) / (64 * kWaves);
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
