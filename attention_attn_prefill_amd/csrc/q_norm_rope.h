// q_norm_rope.h -- the per-head RMSNorm + NeoX rotation of a query row's
// fragment as a prefill kernel loads it (the "Qwen3" and "RoPE design"
// sections of the GRPO-CUDA project memory page: QK-norm over D before the
// rotation; pairs (i, i + D/2) turned by the table row of the token's
// position).  Shared by the prefill kernels of libattn.so; not installed.
#pragma once

#include "attn_internal.h"

namespace attn {
namespace qnr {

// sum of x over lanes l and l ^ 32 (both halves end with the same value)
__device__ __forceinline__ float half_swap_add(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// RMSNorm (when q_weight is set) and NeoX rotation of the Q fragment of one
// lane (dims 16 ks + 8 hf + j of its query row), in fp32, rounded to fp16
// once.  Its loads go out in two waves so that their latency overlaps the
// first K/V tile loads: the position (issue_pos), then the weight slices and
// the table rows once the position is known (issue_rest), then the
// arithmetic (apply).  Without a positions array the position is the row's
// index in its sequence.
// Rows past S_q stay zero.  apply() returns false for a position outside
// [0, max_pos): that row's fragment is zero (the kernels using this are
// built without NaN semantics, so no NaN enters the arithmetic) and their
// epilogue stores NaN bits for it.  Every lane of the wavefront takes part
// in apply() (the row sum is exchanged with lane l ^ 32).
template <int D>
struct QNormRope {
  static constexpr int KS = D / 16, HK = KS / 2;
  half8_t w[KS];
  f32x4_t c[HK][2], s[HK][2];
  int pos;
  bool valid, ok;

  __device__ __forceinline__ void issue(const PrefillArgs& a, int b, int qrow, int hf) {
    issue_pos(a, b, qrow);
    issue_rest(a, hf);
  }
  // The two halves of issue().  A kernel that issues its tile loads in
  // between should take the position first: loads retire in order, so the
  // table rows, which need the position, would otherwise wait for every
  // tile load issued ahead of it.
  __device__ __forceinline__ void issue_pos(const PrefillArgs& a, int b, int qrow) {
    valid = qrow < a.S_q;
    if (a.positions) pos = valid ? a.positions[(int64_t)b * a.S_q + qrow] : 0;
    else pos = qrow;
  }
  __device__ __forceinline__ void issue_rest(const PrefillArgs& a, int hf) {
    tables(a, hf);
    if (a.q_weight) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) w[ks] = *reinterpret_cast<const half8_t*>(a.q_weight + 16 * ks + 8 * hf);
    }
  }
  __device__ __forceinline__ void tables(const PrefillArgs& a, int hf) {
    ok = pos >= 0 && pos < a.max_pos;
    const int64_t trow = (int64_t)(ok ? pos : 0) * (D / 2);
#pragma unroll
    for (int ks = 0; ks < HK; ++ks) {
      const f32x4_t* ct = reinterpret_cast<const f32x4_t*>(a.cos_table + trow + 16 * ks + 8 * hf);
      const f32x4_t* st = reinterpret_cast<const f32x4_t*>(a.sin_table + trow + 16 * ks + 8 * hf);
      c[ks][0] = ct[0];
      c[ks][1] = ct[1];
      s[ks][0] = st[0];
      s[ks][1] = st[1];
    }
  }
  __device__ __forceinline__ bool apply(const PrefillArgs& a, half8_t (&qf)[KS]) const {
    float y[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) y[ks][j] = (float)qf[ks][j];
    if (a.q_weight) {
      float ss = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(y[ks][j], y[ks][j], ss);
      ss = half_swap_add(ss);
      // v_rsq_f32 directly: the math library's rsqrtf is not inlined into
      // code built without NaN semantics and would become a call; for
      // the normal arguments a mean square plus eps gives, it is the same
      // instruction
      const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) y[ks][j] = y[ks][j] * inv * (float)w[ks][j];
    }
#pragma unroll
    for (int ks = 0; ks < HK; ++ks) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float cj = c[ks][j >> 2][j & 3], sj = s[ks][j >> 2][j & 3];
        const float lo = y[ks][j], hi = y[ks + HK][j];
        const float rlo = fmaf(lo, cj, -hi * sj);
        const float rhi = fmaf(hi, cj, lo * sj);
        qf[ks][j] = (valid && ok) ? (_Float16)rlo : (_Float16)0.0f;
        qf[ks + HK][j] = (valid && ok) ? (_Float16)rhi : (_Float16)0.0f;
      }
    }
    return !valid || ok;
  }
};

}  // namespace qnr
}  // namespace attn
