// prefill_fwd.hip -- causal / non-causal GQA attention prefill for gfx950.
//
// Computes O = softmax(Q K^T / sqrt(D) + mask) V over [B,S,H,D] fp16 tensors
// with fp32 accumulation ("Tutorial: Adding a New Kernel to RL.cu",
// attention.cuh prefill section and the attention.cu prefill kernel: GQA kv
// head = h*H_kv/H_q, causal mask j <= i, online softmax with running max m,
// running sum l and rescale factor exp(m_old - m_new)).  The pages' kernel
// gives each thread one query row and walks keys one by one with scalar
// fp32 dot products; here both contractions run on the matrix cores.
//
// Work decomposition
//   * a workgroup = 4 wavefronts = 128 query rows of one (batch, q head);
//     each wavefront owns 32 rows for the whole kernel;
//   * keys stream through LDS in tiles of 64: K row-major [64][D+8] and V
//     transposed [D][64+8] (the padding keeps the MFMA operand reads free of
//     bank conflicts);
//   * per tile and wavefront:
//       S^T[64 x 32] = K_tile[64 x D] . Q_w^T[D x 32]   (v_mfma_f32_32x32x16_f16)
//     so each query's 64 scores sit in two lanes (l and l+32) of the
//     accumulator; the row max needs one v_permlane32_swap, the rest of the
//     softmax is lane-local;
//       O^T[D x 32] += V_tile^T[D x 64] . P^T[64 x 32]  (same instruction)
//     where P^T is the score accumulator rounded to fp16 in place: the key
//     order inside each 16-key chunk of the transposed V tile is permuted so
//     that the accumulator layout of S^T is exactly the B-operand layout of
//     P^T, with no data movement between lanes;
//   * causal: tiles strictly above the diagonal are never loaded; only tiles
//     crossing the diagonal (or the ragged end) are masked element-wise;
//   * workgroups are issued longest-first (last query tiles first) so the
//     causal triangle's long tiles do not trail at the end of the grid.
#include "attn_internal.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockM = 32 * kWaves;  // query rows per workgroup
constexpr int kBlockN = 64;           // keys per tile

__device__ __forceinline__ float wave_half_swap_max(float x) {
  // max of x over lanes l and l^32 (both halves end with the same value)
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_half_swap_add(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position group (of 4 keys) inside a 16-key chunk of the transposed V tile
// for key group a = key/4 % 4: the B operand of the PV product for lane half
// hf holds, at k = 8*hf + i, the score of key 4*hf + i (i < 4) or
// 8 + 4*hf + (i - 4) (i >= 4), so key groups {0,1,2,3} sit at positions
// {0,2,1,3}.
__device__ __forceinline__ int vt_pos_group(int a) { return (a == 1) ? 2 : (a == 2) ? 1 : a; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void prefill_fwd_kernel(PrefillArgs a) {
  constexpr int KS = D / 16;           // k-steps of the QK^T contraction
  constexpr int DT = D / 32;           // 32-wide d tiles of O^T
  constexpr int KROW = D + 8;          // LDS row stride of K (halfs)
  constexpr int VROW = kBlockN + 8;    // LDS row stride of V^T (halfs)
  constexpr int VEC_PER_ROW = D / 8;   // 16-byte vectors per key row

  __shared__ __attribute__((aligned(16))) _Float16 k_lds[kBlockN * KROW];
  __shared__ __attribute__((aligned(16))) _Float16 vt_lds[D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;  // query column of S^T / O^T owned by this lane
  const int hf = lane >> 5;   // which half of the k-range this lane supplies

  // Longest-first issue order: the slowest-varying part of the linear block
  // id is the query tile, counted from the end.
  const int combos = a.H_q * a.B;
  const int id = blockIdx.x;
  const int qt = a.n_qtiles - 1 - id / combos;
  const int rem = id - (id / combos) * combos;
  const int h = rem % a.H_q;
  const int b = rem / a.H_q;
  const int g = (int)(((int64_t)h * a.H_kv) / a.H_q);

  const int q0 = qt * kBlockM;
  const int qw = q0 + wave * 32;  // first row of this wavefront
  const int qrow = qw + col;      // this lane's query row
  const int64_t q_row_stride = (int64_t)a.H_q * D;
  const int64_t kv_row_stride = (int64_t)a.H_kv * D;

  // Q fragment (B operand of S^T = K Q^T): q[qrow][16*ks + 8*hf + 0..7]
  half8_t qf[KS];
  if (qrow < a.S_q) {
    const _Float16* qp = a.q + ((int64_t)b * a.S_q + qrow) * q_row_stride + (int64_t)h * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const half8_t*>(qp + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = half8_t{};
  }

  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16_t{};
  float m = -INFINITY;  // running max of raw dot products (scale applied later)
  float l = 0.0f;       // running sum of this lane's share of exp2 weights

  int n_tiles = (a.S_kv + kBlockN - 1) / kBlockN;
  if (CAUSAL) {
    const int last_row = min(q0 + kBlockM, a.S_q) - 1;
    n_tiles = min(n_tiles, last_row / kBlockN + 1);
  }
  const int wave_last_row = min(qw + 31, a.S_q - 1);

  const _Float16* kbase = a.k + (int64_t)b * a.S_kv * kv_row_stride + (int64_t)g * D;
  const _Float16* vbase = a.v + (int64_t)b * a.S_kv * kv_row_stride + (int64_t)g * D;

  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = t * kBlockN;
    __syncthreads();  // every wavefront is done reading the previous tile

    // K tile: row r, 16-byte vector c; consecutive threads cover one row.
    for (int idx = tid; idx < kBlockN * VEC_PER_ROW; idx += kThreads) {
      const int r = idx / VEC_PER_ROW;
      const int c = idx - r * VEC_PER_ROW;
      const int key = kv0 + r;
      half8_t val = half8_t{};
      if (key < a.S_kv) val = *reinterpret_cast<const half8_t*>(kbase + (int64_t)key * kv_row_stride + 8 * c);
      *reinterpret_cast<half8_t*>(&k_lds[r * KROW + 8 * c]) = val;
    }
    // V tile, transposed: 4 consecutive keys x 8 d values per work item,
    // written as 8 columns of 4 keys at the permuted position group.
    for (int idx = tid; idx < (kBlockN / 4) * VEC_PER_ROW; idx += kThreads) {
      const int kg = idx % (kBlockN / 4);
      const int c = idx / (kBlockN / 4);
      half8_t rows[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = kv0 + 4 * kg + j;
        rows[j] = half8_t{};
        if (key < a.S_kv) rows[j] = *reinterpret_cast<const half8_t*>(vbase + (int64_t)key * kv_row_stride + 8 * c);
      }
      const int pos = (kg >> 2) * 16 + vt_pos_group(kg & 3) * 4;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        half4_t col4 = {rows[0][i], rows[1][i], rows[2][i], rows[3][i]};
        *reinterpret_cast<half4_t*>(&vt_lds[(8 * c + i) * VROW + pos]) = col4;
      }
    }
    __syncthreads();

    if (qw >= a.S_q) continue;                   // wavefront past the last row
    if (CAUSAL && kv0 > wave_last_row) continue;  // tile entirely above the diagonal

    // S^T = K Q^T for the two 32-key halves of the tile
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const half8_t kf = *reinterpret_cast<const half8_t*>(&k_lds[(kb * 32 + col) * KROW + 16 * ks + 8 * hf]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], s[kb], 0, 0, 0);
      }
    }

    // element-wise mask only where the tile crosses the diagonal or the end
    const bool need_mask = (CAUSAL && kv0 + kBlockN - 1 > qw) || (kv0 + kBlockN > a.S_kv);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
          const bool masked = (CAUSAL && key > qrow) || key >= a.S_kv;
          if (masked) s[kb][r] = -INFINITY;
        }
      }
    }

    // online softmax (fp32): new max, rescale factor, exp2 weights
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = wave_half_swap_max(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f((m - m_new) * a.scale_log2);
    const float mb = m_new * a.scale_log2;

    half8_t pf[4];
    float psum = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[c >> 1][8 * (c & 1) + i], a.scale_log2, -mb));
        psum += p;
        pf[c][i] = (_Float16)p;
      }
    }
    l = fmaf(l, alpha, psum);
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const half8_t vf = *reinterpret_cast<const half8_t*>(&vt_lds[(dt * 32 + col) * VROW + 16 * c + 8 * hf]);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[c], o[dt], 0, 0, 0);
      }
    }
  }

  // epilogue: combine the two half-row sums, normalise, round to fp16
  if (qw >= a.S_q) return;
  l = wave_half_swap_add(l);
  if (qrow >= a.S_q) return;
  const float inv = 1.0f / l;
  _Float16* op = a.o + ((int64_t)b * a.S_q + qrow) * q_row_stride + (int64_t)h * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      half4_t out;
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = (_Float16)(o[dt][rg * 4 + j] * inv);
      *reinterpret_cast<half4_t*>(op + dt * 32 + rg * 8 + hf * 4) = out;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.n_qtiles * a.H_q * a.B;
  PrefillArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&prefill_fwd_kernel<D, CAUSAL>),
                         dim3((unsigned)blocks), dim3(kThreads), kargs, 0, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a_in, int head_dim, bool causal, hipStream_t stream) {
  PrefillArgs a = a_in;
  a.n_qtiles = (a.S_q + kBlockM - 1) / kBlockM;
  switch (head_dim) {
    case 32: return causal ? launch_t<32, true>(a, stream) : launch_t<32, false>(a, stream);
    case 64: return causal ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
    case 128: return causal ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
