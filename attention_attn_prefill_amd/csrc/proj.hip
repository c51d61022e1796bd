// proj.hip -- the linear layers of the cross-attention module on gfx950:
// Y = X W^T (nn.Linear layout, W [N, K]) with an optional rotary epilogue.
//
// The module (POPCORNBENCH cross-attention trace, problem statement and its
// nn.Linear notes): Q/K/V projections, RoPE on Q and K over adjacent pairs
// (2j, 2j+1) at the row's position in its sequence, attention, and the output
// projection.  Its sizes are small (the pages' case is 4 x 64 queries,
// 4 x 128 keys, dim 256), so the layers are latency-bound MFMA tiles:
//   * a workgroup owns one 32 x 32 output tile, and its four wavefronts
//     split K: each walks a quarter of the k-steps of 16 with
//     v_mfma_f32_32x32x16_f16, with up to kPrefetch steps of operands in
//     flight (all of them for K up to 256).  The four partial tiles are
//     summed through LDS in wavefront order, so the result does not depend
//     on timing.  Both operands come straight from global memory: lane l
//     reads 16 bytes of row (l % 32) of X, and 16 bytes of row (l % 32) of
//     W (a column of W^T), at k-offset 8 * (l / 32);
//   * rows past M read as zeros through a raw buffer resource and are not
//     stored;
//   * the rotary epilogue: output column n sits in lane n % 32 of the
//     accumulator, so the pair partner of column n (n xor 1) is the
//     neighbouring lane.  Rotation in fp32 from the shared fp32 cos/sin table
//     (same frequencies as the NeoX table: pos * theta^(-2j/D)), then one
//     rounding to fp16;
//   * one launch runs several independent jobs (the Q, K and V projections)
//     so the three of them cost one launch.
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kWaves = 4;     // wavefronts per workgroup, each a quarter of K
constexpr int kTile = 32;
constexpr int kPrefetch = 4;  // k-steps of operands in flight per wavefront

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  const int range = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, range, 0x00020000);
}

__device__ __forceinline__ half8_t load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(half8_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__global__ __launch_bounds__(64 * kWaves) void proj_kernel(ProjArgs a) {
  // which job and which 32 x 32 tile of it (one tile per workgroup)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int64_t tile = blockIdx.x;
  // the job index is workgroup-uniform; fixed indices keep the argument
  // block out of private memory
  int j;
  if (tile < a.job[0].tiles) {
    j = 0;
  } else if (a.n_jobs > 1 && tile < a.job[0].tiles + a.job[1].tiles) {
    j = 1;
    tile -= a.job[0].tiles;
  } else if (a.n_jobs > 2 && tile < a.job[0].tiles + a.job[1].tiles + a.job[2].tiles) {
    j = 2;
    tile -= a.job[0].tiles + a.job[1].tiles;
  } else {
    return;
  }
  const ProjJob job = j == 0 ? a.job[0] : (j == 1 ? a.job[1] : a.job[2]);
  const int K = a.K, N = a.N;
  const int col_tiles = N / kTile;
  const int m0 = (int)(tile / col_tiles) * kTile;
  const int n0 = (int)(tile % col_tiles) * kTile;
  const int c = lane & 31, hk = lane >> 5;

  const __amdgpu_buffer_rsrc_t xr = rsrc_of(job.x, (int64_t)job.M * K * 2);
  const __amdgpu_buffer_rsrc_t wr = rsrc_of(job.w, (int64_t)N * K * 2);
  // this wavefront's k-steps: [s_begin, s_end)
  const int steps = K / 16;
  const int per_wave = (steps + kWaves - 1) / kWaves;
  const int s_begin = wave * per_wave;
  const int s_end = min(steps, s_begin + per_wave);
  const int xoff = ((m0 + c) * K + 8 * hk) * 2 + 32 * s_begin;
  const int woff = ((n0 + c) * K + 8 * hk) * 2 + 32 * s_begin;
  const int n_steps = max(0, s_end - s_begin);

  // the rotary table entries of this lane's 16 outputs (column n0 + c,
  // rows m0 + 8 (r / 4) + 4 hk + r % 4) go out with the operand loads
  const int n = n0 + c;
  float cs[16], sn[16];
  if (job.rope && wave == 0) {
    const int D = a.head_dim;
    const int pair = (n % D) >> 1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 8 * (r >> 2) + 4 * hk + (r & 3);
      const int pos = (m < job.M ? m : 0) % job.T;
      cs[r] = a.cos_table[(int64_t)pos * (D / 2) + pair];
      sn[r] = a.sin_table[(int64_t)pos * (D / 2) + pair];
    }
  }

  f32x16_t acc = f32x16_t{};
  half8_t ra[kPrefetch], rb[kPrefetch];
#pragma unroll
  for (int s = 0; s < kPrefetch; ++s) {
    if (s < n_steps) {
      ra[s] = load16(xr, xoff + 32 * s);
      rb[s] = load16(wr, woff + 32 * s);
    }
  }
  for (int s0 = 0; s0 < n_steps; s0 += kPrefetch) {
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u) {
      const int s = s0 + u;
      if (s < n_steps) {
        const half8_t fa = ra[u], fb = rb[u];
        if (s + kPrefetch < n_steps) {
          ra[u] = load16(xr, xoff + 32 * (s + kPrefetch));
          rb[u] = load16(wr, woff + 32 * (s + kPrefetch));
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, fb, acc, 0, 0, 0);
      }
    }
  }

  // sum the partial tiles: wavefronts 1.. hand theirs to wavefront 0, which
  // adds them in order (element-major, lane-contiguous: no bank conflicts)
  __shared__ float red[kWaves - 1][16][64];
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave - 1][i][lane] = acc[i];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += red[w][i][lane];

  // epilogue: lane holds column n0 + c, rows m0 + 8 * (r / 4) + 4 * hk + r % 4
  if (job.rope) {
    const bool odd = n & 1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float u = acc[r];
      const float p = __shfl_xor(u, 1, 64);
      // even column: a c - b s; odd column: a s + b c (a even, b odd)
      acc[r] = odd ? fmaf(p, sn[r], u * cs[r]) : fmaf(u, cs[r], -p * sn[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + 8 * (r >> 2) + 4 * hk + (r & 3);
    if (m < job.M) job.y[(int64_t)m * N + n] = (_Float16)acc[r];
  }
}

}  // namespace

hipError_t launch_proj(const ProjArgs& a, hipStream_t stream) {
  int64_t tiles = 0;
  for (int j = 0; j < a.n_jobs; ++j) tiles += a.job[j].tiles;
  ProjArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&proj_kernel), dim3((unsigned)tiles), dim3(64 * kWaves),
                         kargs, 0, stream);
}

}  // namespace attn
