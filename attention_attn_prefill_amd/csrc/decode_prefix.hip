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
//   * a workgroup is one wavefront: the tiles stream through its own ring of
//     kStages LDS stages, filled by buffer-to-LDS loads (no registers held
//     while in flight) kStages - 1 tiles ahead; a tile is read once its
//     loads are counted done (vmcnt), with no barrier, and its stage is
//     refilled only after the reads of the tile that used it have returned;
//   * per tile, S^T[32 keys x 32 rows] = K Q^T on v_mfma_f32_32x32x16_f16 (K
//     from LDS, Q in VGPRs, two accumulators over alternate k-steps), online
//     softmax in the log2 domain with a lazy reference point, and
//     O^T[128 x 32] += V^T P^T in four 32-wide slices (V^T read with the
//     transposing ds_read_b64_tr_b16, P^T taken from the score accumulator).
//     One wavefront computes each score tile once; with several wavefronts
//     sharing a tile, each recomputed the scores, which cost more than the
//     barrier-free single wavefront loses in latency hiding;
//   * the workgroup writes one partial (unnormalised o, max, sum) per query
//     row into the decode workspace slot of its chunk; the split kernel (one
//     split per sequence) or the merge kernel folds these into the
//     per-sequence suffix.
// LDS tiles are unpadded 256-byte key rows.  K: 16-byte chunk c of row r sits
// at chunk c ^ (r % 16), so the 16 rows one K-operand read touches spread
// over all banks.  V: 64-byte segment s of row r sits at s ^ (r % 4), so the
// four rows of a transposing read hit four different segments.  The loads
// put each lane's 16 bytes at the swizzled place directly.
#include "attn_internal.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kWaves = 1;                  // wavefronts per workgroup
constexpr int D = kDecodeHeadDim;          // 128
constexpr int BS = kDecodeBlockSize;       // 16
constexpr int CB = kPrefixChunkBlocks;
constexpr int kSlices = 4 / kWaves;        // 32-wide head-dim slices of O per wavefront
constexpr int kRowsPerWave = 32 / kWaves;  // tile rows each wavefront loads
constexpr int kLoads = kRowsPerWave / 4;   // 1 KB loads per tensor, tile and wavefront
constexpr int kStages = 4;
static_assert(kWaves == 1 || kWaves == 4, "the transposing-read blocks cover one or four slices");
constexpr int kTileHalfs = 32 * D;    // one 32-key tile of K or V
constexpr float kLazyLog2 = 8.0f;     // rescale only past 2^8
static_assert(CB % 2 == 0 && CB <= 64, "a chunk is whole 2-block tiles, its table entries one per lane");

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

typedef short short4_t __attribute__((ext_vector_type(4)));

// The V^T operands of a whole 32-key tile: four transposing reads at the
// lane's LDS byte address + 0, 8, 16 and 24 rows.  Written as one asm block
// that waits for its own reads: the compiler cannot tell these reads from
// the buffer-to-LDS loads still in flight into other stages and would
// otherwise wait for all of them first; the ring protocol (the vmcnt wait
// before a tile is read, and a barrier when several wavefronts share it)
// already orders them.  The outputs are
// early-clobber: a read's destination must not be the address register
// that a later read of the block still uses (its data can land before the
// later read issues).
[[maybe_unused]] __device__ __forceinline__ void lds_read_tr_tile(const uint32_t (&addr)[1], short4_t (&r)[1][4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:4096\n\t"
      "ds_read_b64_tr_b16 %3, %4 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[0][2]), "=&v"(r[0][3])
      : "v"(addr[0])
      : "memory");
}

// The same for four head-dim slices (a wavefront that owns all of O):
// sixteen reads, one wait.
[[maybe_unused]] __device__ __forceinline__ void lds_read_tr_tile(const uint32_t (&addr)[4], short4_t (&r)[4][4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %3, %16 offset:6144\n\t"
      "ds_read_b64_tr_b16 %4, %17\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %7, %17 offset:6144\n\t"
      "ds_read_b64_tr_b16 %8, %18\n\t"
      "ds_read_b64_tr_b16 %9, %18 offset:2048\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %11, %18 offset:6144\n\t"
      "ds_read_b64_tr_b16 %12, %19\n\t"
      "ds_read_b64_tr_b16 %13, %19 offset:2048\n\t"
      "ds_read_b64_tr_b16 %14, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[0][2]), "=&v"(r[0][3]),
        "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[1][2]), "=&v"(r[1][3]),
        "=&v"(r[2][0]), "=&v"(r[2][1]), "=&v"(r[2][2]), "=&v"(r[2][3]),
        "=&v"(r[3][0]), "=&v"(r[3][1]), "=&v"(r[3][2]), "=&v"(r[3][3])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
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

// Wait until at most `ahead` tiles (2 * kLoads buffer-to-LDS loads per lane
// each) are still in flight behind the current one.
__device__ __forceinline__ void wait_tiles(int ahead) {
  static_assert((kStages - 2) * 2 * kLoads <= 48, "vmcnt immediates below cover up to 48 loads");
  switch (ahead * 2 * kLoads) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 48: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;  // always safe
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

  // loads: wavefront w fills key rows kRowsPerWave * w .. + kRowsPerWave - 1
  // of each tile with 4-row loads of 1 KB per tensor; lane i of a load
  // lands at row R0 + i / 16, 16-byte place i % 16
  const int64_t slab = (int64_t)a.H_kv * BS * D;
  const int64_t head_off = (int64_t)g * BS * D;
  int voff_k[kLoads], voff_v[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int rr = (kRowsPerWave * wave + 4 * j + (lane >> 4)) & 15;  // row inside its block
    const int pl = lane & 15;                                         // place inside the LDS row
    voff_k[j] = rr * 256 + 16 * (pl ^ rr);
    voff_v[j] = rr * 256 + 16 * (4 * ((pl >> 2) ^ (rr & 3)) + (pl & 3));
  }
  auto issue = [&](int t) {
    const int e0 = __builtin_amdgcn_readlane(ent, 2 * t);
    const int e1 = 2 * t + 1 < nb ? __builtin_amdgcn_readlane(ent, 2 * t + 1) : e0;
    _Float16* kd = ring[t % kStages][0] + kRowsPerWave * wave * D;
    _Float16* vd = ring[t % kStages][1] + kRowsPerWave * wave * D;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      // this load's rows lie in block (kRowsPerWave * wave + 4 j) / 16 of the pair
      const int64_t blk = ((kRowsPerWave * wave + 4 * j) < 16 ? e0 : e1) * slab + head_off;
      // non-temporal (aux = 2): each slab is read once per launch
      __builtin_amdgcn_raw_ptr_buffer_load_lds(slab_rsrc(a.k_cache + blk), LDS_PTR(kd + 4 * j * D), 16,
                                               voff_k[j], 0, 0, 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(slab_rsrc(a.v_cache + blk), LDS_PTR(vd + 4 * j * D), 16,
                                               voff_v[j], 0, 0, 2);
    }
  };

  // K operand: key col, 16-byte chunk 2 ks + hf at chunk (2 ks + hf) ^ (col % 16)
  const int k_row = col * D;
  const int k_x = col & 15;
  // V^T operand of 16 keys (chunk c of the tile) for d slice dt, in the key
  // order of the P^T operand taken from the score accumulator (keys
  // 16c + 4hf + 0..3, then 16c + 8 + 4hf + 0..3); the four rows of a read
  // differ in row % 4 = (lane % 16) / 4
  const int vq = (lane & 15) >> 2;
  const int v_row = (4 * hf + vq) * D + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  float m = -INFINITY, l = 0.0f;
  f32x16_t o[kSlices];
#pragma unroll
  for (int sl = 0; sl < kSlices; ++sl) o[sl] = f32x16_t{};

#pragma unroll
  for (int t = 0; t < kStages - 1; ++t)
    if (t < n_tiles) issue(t);

  for (int t = 0; t < n_tiles; ++t) {
    wait_tiles(min(kStages - 2, n_tiles - 1 - t));
    // tile t is in LDS, and the reads of tile t - 1 (whose stage is
    // refilled next) have all returned: their consumers waited for them.
    // With several wavefronts, a bare barrier makes that hold for all of
    // them (a fenced one would also wait for the tiles still in flight).
    if constexpr (kWaves > 1) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
    }
    asm volatile("" ::: "memory");
    if (t + kStages - 1 < n_tiles) issue(t + kStages - 1);

    const _Float16* kl = ring[t % kStages][0];
    const _Float16* vl = ring[t % kStages][1];
    // two accumulators (even and odd k-steps): two chains of four
    // dependent MFMAs instead of one of eight
    f32x16_t sa = f32x16_t{}, sb = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const half8_t kf = *reinterpret_cast<const half8_t*>(kl + k_row + 8 * ((2 * ks + hf) ^ k_x));
      if (ks & 1) sb = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], sb, 0, 0, 0);
      else sa = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], sa, 0, 0, 0);
    }
    f32x16_t sc = sa + sb;
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
    // lazy reference point: m (and o, l with it) moves only when some row's
    // weights would pass 2^8; any reference cancels in o / l and in the
    // log-sum-exp merge, and weights up to 2^8 are exact enough in fp16
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazyLog2) != 0) {
      const float m_new = fmaxf(m, mx);
      const float alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl) o[sl] *= alpha;
      m = m_new;
    }
    half8_t pf[2];
    float ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(sc[i] - m);
      ps += p;
      pf[i >> 3][i & 7] = (_Float16)p;
    }
    l += ps;
    // per slice: rows +0, +8 (keys 0..15) and +16, +24 (keys 16..31)
    uint32_t va[kSlices];
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl) va[sl] = lds_addr(vl + v_row + 32 * ((kSlices * wave + sl) ^ vq));
    short4_t vt[kSlices][4];
    lds_read_tr_tile(va, vt);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl) {
        const short4_t lohi[2] = {vt[sl][2 * c], vt[sl][2 * c + 1]};
        o[sl] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, lohi), pf[c], o[sl], 0, 0, 0);
      }
  }

  // row col's sum is split over lanes col and col + 32
  const float lrow = half_swap_add(l);
  if (!valid_row) return;
  const float nan = __builtin_nanf("");
  const int64_t slot = ((int64_t)s * a.H_q + h) * a.slot_stride + chunk;
  // O^T element i of slice dt: d = 32 dt + 8 (i / 4) + 4 hf + i % 4, row col
#pragma unroll
  for (int sl = 0; sl < kSlices; ++sl) {
    float* od = a.ws_o + slot * D + 32 * (kSlices * wave + sl) + 4 * hf;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4 v4 = {o[sl][4 * q4], o[sl][4 * q4 + 1], o[sl][4 * q4 + 2], o[sl][4 * q4 + 3]};
      if (bad) v4 = {nan, nan, nan, nan};
      *reinterpret_cast<float4*>(od + 8 * q4) = v4;
    }
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
