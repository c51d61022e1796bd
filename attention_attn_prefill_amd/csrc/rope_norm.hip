// rope_norm.hip -- fused per-head RMSNorm + NeoX rotary embedding on gfx950,
// optionally fused with the paged-cache append.
//
// Qwen3 applies RMSNorm to every query and key head before the rotary
// embedding ("GRPO-CUDA Project Memory", Qwen3 notes).  The rotation is the
// NeoX split-half form with an fp32 table [max_pos, D/2] and fp32 arithmetic
// ("RoPE design"):
//   out_i       = y_i * cos_i - y_{i+D/2} * sin_i
//   out_{i+D/2} = y_{i+D/2} * cos_i + y_i * sin_i,       i in [0, D/2)
// where y is the normalised head, y_d = x_d / sqrt(mean(x^2) + eps) * w_d.
//
// One pass over the activations, HBM-bound:
//   * a "row" is one (token, head) of q or k (and, when appending, of v);
//     D/8 lanes own a row, 8 consecutive halfs (16 bytes) per lane, so a
//     wavefront covers 64/(D/8) rows of contiguous memory;
//   * the mean square is reduced over the row's lanes with lane shuffles;
//     the split-half partner of a lane's elements sits D/16 lanes away in the
//     same row (lane xor D/16), so the rotation needs one shuffle per value;
//   * norm and rotation stay in fp32; the result is rounded to fp16 once and
//     written back in place (and, when appending, to the token's cache slot);
//   * a position outside [0, max_pos) has no table row: the row comes out
//     NaN, which the caller can see (the same convention as bad block tables
//     in paged decode).
// The table is built once by rope_table_kernel in fp64 (angle, cosine, sine)
// and rounded to fp32, so it is within half an fp32 ulp of the exact values.
#include "attn_internal.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float lane_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

template <int D, bool APPEND>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(RopeArgs a) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPW = 64 / LPR;       // rows per wavefront
  constexpr int RPB = RPW * (kThreads / 64);
  constexpr int HALF = D / 2;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR;          // which 8-element slice of the row
  const int64_t row = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 6) * RPW + lane / LPR;

  const int64_t rq = a.q ? a.num_tokens * a.H_q : 0;  // no q rows in K-only mode
  const int64_t rk = a.num_tokens * a.H_kv;
  const int64_t total = rq + rk + (APPEND ? rk : 0);
  if (row >= total) return;  // whole rows only: the shuffles stay inside a row

  // which tensor, token and head this row is
  int kind;  // 0 = q, 1 = k, 2 = v (append only)
  int64_t r;
  int H;
  _Float16* base;
  if (row < rq) {
    kind = 0; r = row; H = a.H_q; base = a.q;
  } else if (row < rq + rk) {
    kind = 1; r = row - rq; H = a.H_kv; base = a.k;
  } else {
    kind = 2; r = row - rq - rk; H = a.H_kv; base = const_cast<_Float16*>(a.v);
  }
  const int64_t token = r / H;
  const int head = (int)(r - token * H);
  half8_t* src = reinterpret_cast<half8_t*>(base + r * D) + sub;
  // Every load that depends on no other goes out first (the row, its norm
  // weight, the token's position and slot), the table row as soon as the
  // position is in: two round trips, not five.
  const half8_t xin = *src;
  const _Float16* w = kind == 0 ? a.q_weight : a.k_weight;
  const bool norm = kind != 2 && w != nullptr;
  half8_t wv = {};
  if (norm) wv = *(reinterpret_cast<const half8_t*>(w) + sub);
  const int pos = kind != 2 ? a.positions[token] : 0;
  int64_t slot = -1;
  if (APPEND && kind != 0) slot = a.slot_mapping[token];
  const bool ok = pos >= 0 && pos < a.max_pos;
  const bool first = sub < LPR / 2;  // elements in [0, D/2)
  const int i0 = (sub % (LPR / 2)) * 8;
  float cs[8] = {}, sn[8] = {};
  if (kind != 2 && ok) {
    const f32x4_t* ct = reinterpret_cast<const f32x4_t*>(a.cos_table + (int64_t)pos * HALF + i0);
    const f32x4_t* st = reinterpret_cast<const f32x4_t*>(a.sin_table + (int64_t)pos * HALF + i0);
    const f32x4_t c0 = ct[0], c1 = ct[1], s0 = st[0], s1 = st[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cs[j] = c0[j]; cs[j + 4] = c1[j];
      sn[j] = s0[j]; sn[j + 4] = s1[j];
    }
  }

  half8_t res;
  if (kind == 2) {
    res = xin;  // values are only copied into the cache
  } else {
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = (float)xin[j];
    if (norm) {
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(y[j], y[j], ss);
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1) ss += lane_xor(ss, m);
      const float inv = rsqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = y[j] * inv * (float)wv[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = lane_xor(y[j], LPR / 2);  // the split-half partner
      const float o = first ? fmaf(y[j], cs[j], -p * sn[j]) : fmaf(y[j], cs[j], p * sn[j]);
      res[j] = (_Float16)(ok ? o : __builtin_nanf(""));
    }
    // non-temporal stores (in place and into the cache): nothing in this
    // launch reads them back
    __builtin_nontemporal_store(res, src);
  }

  if (APPEND && kind != 0) {
    if (slot >= 0 && slot < a.num_blocks * (int64_t)a.block_size) {
      const int64_t blk = slot / a.block_size;
      const int off = (int)(slot - blk * a.block_size);
      _Float16* cache = kind == 1 ? a.k_cache : a.v_cache;
      __builtin_nontemporal_store(res, reinterpret_cast<half8_t*>(cache + ((blk * a.H_kv + head) * a.block_size + off) * D) + sub);
    }
  }
}

__global__ void rope_table_kernel(float* cos_t, float* sin_t, int max_pos, int D, double theta) {
  const int half = D / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)max_pos * half) return;
  const int p = (int)(idx / half);
  const int i = (int)(idx - (int64_t)p * half);
  const double angle = (double)p * pow(theta, -2.0 * (double)i / (double)D);
  double s, c;
  sincos(angle, &s, &c);
  cos_t[idx] = (float)c;
  sin_t[idx] = (float)s;
}

template <int D>
hipError_t launch_d(const RopeArgs& a, bool append, hipStream_t stream) {
  constexpr int RPB = (64 / (D / 8)) * (kThreads / 64);
  const int64_t rows = a.num_tokens * ((a.q ? a.H_q : 0) + a.H_kv * (append ? 2 : 1));
  const int64_t blocks = (rows + RPB - 1) / RPB;
  RopeArgs args = a;
  void* kargs[] = {&args};
  const void* f = append ? reinterpret_cast<const void*>(&qk_norm_rope_kernel<D, true>)
                         : reinterpret_cast<const void*>(&qk_norm_rope_kernel<D, false>);
  return hipLaunchKernel(f, dim3((unsigned)blocks), dim3(kThreads), kargs, 0, stream);
}

}  // namespace

hipError_t launch_qk_norm_rope(const RopeArgs& a, int head_dim, bool append, hipStream_t stream) {
  switch (head_dim) {
    case 32: return launch_d<32>(a, append, stream);
    case 64: return launch_d<64>(a, append, stream);
    case 128: return launch_d<128>(a, append, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rope_table(float* cos_t, float* sin_t, int max_pos, int head_dim, double theta,
                             hipStream_t stream) {
  const int64_t n = (int64_t)max_pos * (head_dim / 2);
  const int64_t blocks = (n + 255) / 256;
  void* kargs[] = {&cos_t, &sin_t, &max_pos, &head_dim, &theta};
  return hipLaunchKernel(reinterpret_cast<const void*>(&rope_table_kernel), dim3((unsigned)blocks), dim3(256),
                         kargs, 0, stream);
}

}  // namespace attn
