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
//   * a workgroup serves HP query heads that share one kv head (HP = 2 when
//     H_q/H_kv is even, else 1) and 128 query rows of each: 4*HP wavefronts,
//     each owning 32 rows of one head for the whole kernel.  Both heads read
//     the same K/V tiles, so each tile is staged once for 2x the math;
//   * keys stream through LDS in tiles of 64, double-buffered: K row-major
//     [64][D+8] and V transposed [D][64+8] (the padding keeps the 16-byte MFMA
//     operand reads free of bank conflicts).  The global loads of tile t+1 are
//     issued before the math of tile t and land in LDS after it, so one
//     barrier per tile suffices and the load latency hides behind the MFMAs;
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
//   * online softmax with a lazy reference point: the running max used for
//     the exponentials is only moved (and O, l rescaled) when a tile's max
//     exceeds it by more than 2^8 in the exp2 domain.  The result is the same
//     in real arithmetic (any reference point cancels in O/l); the weights stay
//     below 2^8, far inside fp16 range.  The row sum l adds up the fp16 weights
//     that actually enter the PV product (v_dot2_f32_f16 against ones);
//   * causal: tiles strictly above the diagonal are never loaded; only tiles
//     crossing the diagonal (or the ragged end) are masked element-wise;
//   * workgroups are issued longest-first (last query tiles first) so the
//     causal triangle's long tiles do not trail at the end of the grid.
#include "attn_internal.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kRowsPerWave = 32;
constexpr int kWavesPerHead = 4;
constexpr int kBlockM = kRowsPerWave * kWavesPerHead;  // query rows per head per workgroup
constexpr int kBlockN = 64;                            // keys per tile
constexpr float kLazyLog2 = 8.0f;                      // rescale only past 2^8

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

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

template <int D, int HP>
struct TileStage {
  static constexpr int kThreads = 64 * kWavesPerHead * HP;
  static constexpr int VEC_PER_ROW = D / 8;                              // 16-byte vectors per key row
  static constexpr int K_VECS = kBlockN * VEC_PER_ROW;                   // K tile vectors
  static constexpr int V_ITEMS = (kBlockN / 4) * VEC_PER_ROW;           // (4 keys x 8 dims) items
  static constexpr int K_PER_T = (K_VECS + kThreads - 1) / kThreads;
  static constexpr int V_PER_T = (V_ITEMS + kThreads - 1) / kThreads;
  half8_t kreg[K_PER_T];
  half8_t vreg[V_PER_T][4];
};

template <int D, int HP>
__device__ __forceinline__ void stage_load(TileStage<D, HP>& st, const _Float16* kbase,
                                           const _Float16* vbase, int64_t row_stride, int kv0,
                                           int S_kv, int tid) {
  using TS = TileStage<D, HP>;
  const int last = S_kv - 1;
#pragma unroll
  for (int u = 0; u < TS::K_PER_T; ++u) {
    const int idx = tid + u * TS::kThreads;
    if (idx < TS::K_VECS) {
      const int r = idx / TS::VEC_PER_ROW;
      const int c = idx - r * TS::VEC_PER_ROW;
      const int key = min(kv0 + r, last);  // rows past the end repeat a valid row; they are masked
      st.kreg[u] = *reinterpret_cast<const half8_t*>(kbase + (int64_t)key * row_stride + 8 * c);
    }
  }
#pragma unroll
  for (int u = 0; u < TS::V_PER_T; ++u) {
    const int idx = tid + u * TS::kThreads;
    if (idx < TS::V_ITEMS) {
      const int kg = idx % (kBlockN / 4);
      const int c = idx / (kBlockN / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = min(kv0 + 4 * kg + j, last);
        st.vreg[u][j] = *reinterpret_cast<const half8_t*>(vbase + (int64_t)key * row_stride + 8 * c);
      }
    }
  }
}

template <int D, int HP>
__device__ __forceinline__ void stage_store(const TileStage<D, HP>& st, _Float16* k_lds,
                                            _Float16* vt_lds, int tid) {
  using TS = TileStage<D, HP>;
  constexpr int KROW = D + 8;
  constexpr int VROW = kBlockN + 8;
#pragma unroll
  for (int u = 0; u < TS::K_PER_T; ++u) {
    const int idx = tid + u * TS::kThreads;
    if (idx < TS::K_VECS) {
      const int r = idx / TS::VEC_PER_ROW;
      const int c = idx - r * TS::VEC_PER_ROW;
      *reinterpret_cast<half8_t*>(&k_lds[r * KROW + 8 * c]) = st.kreg[u];
    }
  }
#pragma unroll
  for (int u = 0; u < TS::V_PER_T; ++u) {
    const int idx = tid + u * TS::kThreads;
    if (idx < TS::V_ITEMS) {
      const int kg = idx % (kBlockN / 4);
      const int c = idx / (kBlockN / 4);
      const int pos = (kg >> 2) * 16 + vt_pos_group(kg & 3) * 4;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        half4_t col4 = {st.vreg[u][0][i], st.vreg[u][1][i], st.vreg[u][2][i], st.vreg[u][3][i]};
        *reinterpret_cast<half4_t*>(&vt_lds[(8 * c + i) * VROW + pos]) = col4;
      }
    }
  }
}

template <int D, bool CAUSAL, int HP>
__global__ __launch_bounds__(64 * kWavesPerHead * HP, 2) void prefill_fwd_kernel(PrefillArgs a) {
  constexpr int kThreads = 64 * kWavesPerHead * HP;
  constexpr int KS = D / 16;           // k-steps of the QK^T contraction
  constexpr int DT = D / 32;           // 32-wide d tiles of O^T
  constexpr int KROW = D + 8;          // LDS row stride of K (halfs)
  constexpr int VROW = kBlockN + 8;    // LDS row stride of V^T (halfs)
  constexpr int K_LDS = kBlockN * KROW;
  constexpr int V_LDS = D * VROW;

  __shared__ __attribute__((aligned(16))) _Float16 k_lds[2][K_LDS];
  __shared__ __attribute__((aligned(16))) _Float16 vt_lds[2][V_LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;  // query column of S^T / O^T owned by this lane
  const int hf = lane >> 5;   // which half of the k-range this lane supplies

  // Longest-first issue order: the slowest-varying part of the linear block
  // id is the query tile, counted from the end.
  const int head_groups = a.H_q / HP;
  const int combos = head_groups * a.B;
  const int id = blockIdx.x;
  const int qt = a.n_qtiles - 1 - id / combos;
  const int rem = id - (id / combos) * combos;
  const int hg = rem % head_groups;
  const int b = rem / head_groups;
  const int h = hg * HP + wave / kWavesPerHead;
  const int g = (int)(((int64_t)hg * HP * a.H_kv) / a.H_q);  // shared by the HP heads

  const int q0 = qt * kBlockM;
  const int qw = q0 + (wave % kWavesPerHead) * kRowsPerWave;  // first row of this wavefront
  const int qrow = qw + col;                                  // this lane's query row
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
  float m = -INFINITY;  // reference point of the exponentials (raw dot-product units)
  float l = 0.0f;       // this lane's share of the sum of fp16 weights
  const float c2 = a.scale_log2;
  const float lazy_raw = kLazyLog2 / c2;
  const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};

  int n_tiles = (a.S_kv + kBlockN - 1) / kBlockN;
  if (CAUSAL) {
    const int last_row = min(q0 + kBlockM, a.S_q) - 1;
    n_tiles = min(n_tiles, last_row / kBlockN + 1);
  }
  const int wave_last_row = min(qw + kRowsPerWave - 1, a.S_q - 1);

  const _Float16* kbase = a.k + (int64_t)b * a.S_kv * kv_row_stride + (int64_t)g * D;
  const _Float16* vbase = a.v + (int64_t)b * a.S_kv * kv_row_stride + (int64_t)g * D;

  TileStage<D, HP> st;
  stage_load<D, HP>(st, kbase, vbase, kv_row_stride, 0, a.S_kv, tid);
  stage_store<D, HP>(st, k_lds[0], vt_lds[0], tid);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = t * kBlockN;
    const int buf = t & 1;
    const bool has_next = t + 1 < n_tiles;
    if (has_next) stage_load<D, HP>(st, kbase, vbase, kv_row_stride, kv0 + kBlockN, a.S_kv, tid);

    const bool active = qw < a.S_q && !(CAUSAL && kv0 > wave_last_row);
    if (active) {
      const _Float16* kl = k_lds[buf];
      const _Float16* vl = vt_lds[buf];
      // S^T = K Q^T for the two 32-key halves of the tile
      f32x16_t s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const half8_t kf = *reinterpret_cast<const half8_t*>(&kl[(kb * 32 + col) * KROW + 16 * ks + 8 * hf]);
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

      // tile max of this query over both lane halves
      float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[0][r], s[0][r + 1]));
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[1][r], s[1][r + 1]));
      mx = wave_half_swap_max(mx);

      // move the reference point only when some row's weights would pass 2^8
      if (__builtin_amdgcn_ballot_w64(mx > m + lazy_raw) != 0) {
        const float m_new = fmaxf(m, mx);
        const float alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m - m_new) * c2);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      }
      const float mb = m * c2;

      half8_t pf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pf[c][i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[c >> 1][8 * (c & 1) + i], c2, -mb));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const half2_t pp = {pf[c][2 * i], pf[c][2 * i + 1]};
          l = __builtin_amdgcn_fdot2(pp, ones, l, false);
        }
      }

      // O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const half8_t vf = *reinterpret_cast<const half8_t*>(&vl[(dt * 32 + col) * VROW + 16 * c + 8 * hf]);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[c], o[dt], 0, 0, 0);
        }
      }
    }

    if (has_next) stage_store<D, HP>(st, k_lds[buf ^ 1], vt_lds[buf ^ 1], tid);
    __syncthreads();
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

template <int D, bool CAUSAL, int HP>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.n_qtiles * (a.H_q / HP) * a.B;
  PrefillArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&prefill_fwd_kernel<D, CAUSAL, HP>),
                         dim3((unsigned)blocks), dim3(64 * kWavesPerHead * HP), kargs, 0, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_hp(const PrefillArgs& a, hipStream_t stream) {
  const bool pair = ((a.H_q / a.H_kv) % 2) == 0;
  return pair ? launch_t<D, CAUSAL, 2>(a, stream) : launch_t<D, CAUSAL, 1>(a, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a_in, int head_dim, bool causal, hipStream_t stream) {
  PrefillArgs a = a_in;
  a.n_qtiles = (a.S_q + kBlockM - 1) / kBlockM;
  switch (head_dim) {
    case 32: return causal ? launch_hp<32, true>(a, stream) : launch_hp<32, false>(a, stream);
    case 64: return causal ? launch_hp<64, true>(a, stream) : launch_hp<64, false>(a, stream);
    case 128: return causal ? launch_hp<128, true>(a, stream) : launch_hp<128, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
