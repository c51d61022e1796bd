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
//   * keys stream through LDS in tiles of 64, double-buffered, both row-major:
//     K [64][D+8] and V [64][D+32] (the padding keeps the MFMA operand reads
//     free of bank conflicts).  The global loads of the next tiles are issued
//     before the math of the current one and land in LDS after it, so one
//     barrier per tile suffices and the load latency hides behind the MFMAs;
//   * per tile and wavefront:
//       S^T[64 x 32] = K_tile[64 x D] . Q_w^T[D x 32]   (v_mfma_f32_32x32x16_f16)
//     so each query's 64 scores sit in two lanes (l and l+32) of the
//     accumulator; the row max needs one v_permlane32_swap, the rest of the
//     softmax is lane-local;
//       O^T[D x 32] += V_tile^T[D x 64] . P^T[64 x 32]  (same instruction)
//     where P^T is the score accumulator rounded to fp16 in place (no data
//     movement between lanes), and the V^T operand is read from the
//     row-major V tile with the transposing ds_read_b64_tr_b16, two reads per
//     operand, in the key order that the S^T accumulator layout dictates;
//   * online softmax with a lazy reference point: the running max used for
//     the exponentials is only moved (and O, l rescaled) when a tile's max
//     exceeds it by more than 2^8 in the exp2 domain.  The result is the same
//     in real arithmetic (any reference point cancels in O/l); the weights stay
//     below 2^8, far inside fp16 range.  The row sum l adds up the fp16 weights
//     that actually enter the PV product (v_dot2_f32_f16 against ones);
//   * with two heads per workgroup the wavefronts of the two heads that share
//     a SIMD run each step in opposite order (MFMA phase then softmax, and
//     softmax then MFMA phase), at raised issue priority during their MFMA
//     phase, so one wavefront's exponentials overlap the other's matrix work;
//   * causal: tiles strictly above the diagonal are never loaded; only tiles
//     crossing the diagonal (or the ragged end) are masked element-wise;
//   * a workgroup runs query tiles i and n-1-i back to back: under the causal
//     mask every such pair costs the same, so the grid has no tail of long
//     tiles (an odd middle tile runs alone, last);
//   * optionally (ROPE) Q gets the Qwen3 per-head RMSNorm and NeoX rotation
//     as it is loaded ("GRPO-CUDA Project Memory", Qwen3 notes and "RoPE
//     design"), in fp32, rounded to fp16 once: a lane holds dims
//     16ks + 8hf + (0..7), so the split-half partner of dim d < D/2 (d + D/2,
//     k-step ks + KS/2) is in the same lane, and the mean square needs one
//     swap with lane l ^ 32, which holds the rest of the row.  Q is read
//     once per wavefront, so this costs nothing next to the tile loop;
//     K is rotated once, by the pass that also writes it to the cache.
#include "attn_internal.h"
#include "q_norm_rope.h"

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


// A raw buffer resource over [p, p + bytes).  The base address is passed
// through readfirstlane so the descriptor lives in SGPRs (it is workgroup-
// uniform); a VGPR descriptor would turn every load into a waterfall loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const _Float16* p, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Workgroup barrier that orders LDS accesses only.  The wavefronts of a
// workgroup exchange data through LDS alone, so the barrier need not wait for
// outstanding global loads or stores (__syncthreads() does: its workgroup
// fence covers global memory too, and a query tile's output stores or the
// next tiles' loads would then be waited out at every barrier).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Row stride (halfs) of the V tile in LDS.  The PV operand is read with
// ds_read_b64_tr_b16, where the 16 lanes of a group read 4 key rows x 16
// dims; a stride of 16 dwords modulo the 64 banks keeps those rows on
// disjoint banks.
template <int D>
struct VLayout {
  static constexpr int VROW = (D == 32) ? 32 : D + 32;
};

// Per-thread staging of the K and V tiles: global -> registers (issued early)
// -> LDS (written after the math of the current tile).  Both tiles are
// written row-major, one 16-byte vector per (row, 8 dims).
// Loads go through buffer resources whose range is the kv head's rows
// [0, S_kv): rows past the end read as zeros (and are masked), with no
// clamping arithmetic and 32-bit offsets.
template <int D, int HP>
struct Stager {
  static constexpr int kThreads = 64 * kWavesPerHead * HP;
  static constexpr int VEC_PER_ROW = D / 8;                     // 16-byte vectors per key row
  static constexpr int VECS = kBlockN * VEC_PER_ROW;
  static constexpr int PER_T = (VECS + kThreads - 1) / kThreads;
  static constexpr int KROW = D + 8;
  static constexpr int VROW = VLayout<D>::VROW;

  half8_t kreg[PER_T];
  half8_t vreg[PER_T];
  __amdgpu_buffer_rsrc_t krsrc, vrsrc;
  int row_bytes;  // bytes between consecutive key rows (H_kv * D * 2)

  __device__ __forceinline__ void init(const _Float16* kbase, const _Float16* vbase, int row_stride,
                                       int S_kv) {
    row_bytes = row_stride * 2;
    const int range = S_kv * row_bytes;  // host guarantees < 2^31
    krsrc = make_rsrc(kbase, range);
    vrsrc = make_rsrc(vbase, range);
  }
  __device__ __forceinline__ static bool mine(int u, int tid) { return tid + u * kThreads < VECS; }

  __device__ __forceinline__ void load_k(int kv0, int tid) { load_k_into(kreg, kv0, tid); }
  __device__ __forceinline__ void load_k_into(half8_t (&dst)[PER_T], int kv0, int tid) const {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      if (!mine(u, tid)) continue;
      const int idx = tid + u * kThreads;
      const int r = idx / VEC_PER_ROW, c = idx % VEC_PER_ROW;
      dst[u] = __builtin_bit_cast(half8_t, __builtin_amdgcn_raw_buffer_load_b128(krsrc, (kv0 + r) * row_bytes + 16 * c, 0, 0));
    }
  }
  __device__ __forceinline__ void load_v(int kv0, int tid) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      if (!mine(u, tid)) continue;
      const int idx = tid + u * kThreads;
      const int r = idx / VEC_PER_ROW, c = idx % VEC_PER_ROW;
      vreg[u] = __builtin_bit_cast(half8_t, __builtin_amdgcn_raw_buffer_load_b128(vrsrc, (kv0 + r) * row_bytes + 16 * c, 0, 0));
    }
  }
  __device__ __forceinline__ void store_k(_Float16* k_lds, int tid) const { store_k_from(kreg, k_lds, tid); }
  __device__ __forceinline__ static void store_k_from(const half8_t (&src)[PER_T], _Float16* k_lds, int tid) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      if (!mine(u, tid)) continue;
      const int idx = tid + u * kThreads;
      const int r = idx / VEC_PER_ROW, c = idx % VEC_PER_ROW;
      *reinterpret_cast<half8_t*>(&k_lds[r * KROW + 8 * c]) = src[u];
    }
  }
  __device__ __forceinline__ void store_v(_Float16* v_lds, int tid) const {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      if (!mine(u, tid)) continue;
      const int idx = tid + u * kThreads;
      const int r = idx / VEC_PER_ROW, c = idx % VEC_PER_ROW;
      *reinterpret_cast<half8_t*>(&v_lds[r * VROW + 8 * c]) = vreg[u];
    }
  }
};

typedef short short4_t __attribute__((ext_vector_type(4)));

// 4 fp16 values through the transposing LDS read: in each 16-lane group,
// lanes 4j..4j+3 read 16 consecutive halfs of row j and lane i receives
// column i of rows 0..3.
__device__ __forceinline__ short4_t lds_read_tr(const _Float16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(p));
}

// PV operand V^T[32 dims x 16 keys] for lane l: dims dt*32 + l%32, keys
// 16c + 4*hf + (0..3) then 16c + 8 + 4*hf + (0..3) -- the key order of the
// B operand taken straight from the S^T accumulator (registers 8(c%2)..+7 of
// the 32-key half c/2).  `vl` already holds this lane's row/column offset.
template <int VROW>
__device__ __forceinline__ half8_t pv_operand(const _Float16* vl, int dt, int c) {
  const short4_t lo = lds_read_tr(vl + 16 * c * VROW + dt * 32);
  const short4_t hi = lds_read_tr(vl + (16 * c + 8) * VROW + dt * 32);
  const short4_t lohi[2] = {lo, hi};
  return __builtin_bit_cast(half8_t, lohi);
}

// S^T tile (64 keys x 32 queries) = K_tile . Q_w^T from an LDS K buffer.
// The two 32-key accumulators alternate so consecutive MFMAs are
// independent, and operand reads run four MFMAs ahead of their use.
template <int D>
__device__ __forceinline__ void qk_tile(f32x16_t (&s)[2], const _Float16* kl, const half8_t (&qf)[D / 16]) {
  constexpr int KROW = D + 8;
  constexpr int N = 2 * (D / 16);
  constexpr int R = 4;
  half8_t ring[R];
  s[0] = f32x16_t{};
  s[1] = f32x16_t{};
#pragma unroll
  for (int n = 0; n < R; ++n) ring[n] = *reinterpret_cast<const half8_t*>(&kl[(n & 1) * 32 * KROW + 16 * (n >> 1)]);
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int kb = n & 1, ks = n >> 1;
    const half8_t kf = ring[n % R];
    if (n + R < N)
      ring[n % R] = *reinterpret_cast<const half8_t*>(&kl[((n + R) & 1) * 32 * KROW + 16 * ((n + R) >> 1)]);
    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], s[kb], 0, 0, 0);
  }
}

// Issue order of a GEMM phase: kLdsAhead operand reads first, then each
// MFMA followed by up to two more reads, so the LDS reads of later operands
// are in flight while earlier MFMAs run (the scheduler otherwise keeps only
// one or two reads ahead and each MFMA group waits out a full LDS latency).
constexpr int kLdsAhead = 8;

template <int I, int NM, int REM>
struct IssueChain {
  static __device__ __forceinline__ void run() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int k = REM < 2 ? REM : 2;
    if constexpr (k > 0) __builtin_amdgcn_sched_group_barrier(0x100, k, 0);  // LDS reads
    IssueChain<I + 1, NM, REM - k>::run();
  }
};
template <int NM, int REM>
struct IssueChain<NM, NM, REM> {
  static __device__ __forceinline__ void run() {}
};

// All per-wavefront state of one prefill workgroup, and the per-tile step.
template <int D, bool CAUSAL, int HP>
struct Prefill {
  static constexpr int KS = D / 16;         // k-steps of the QK^T contraction
  static constexpr int DT = D / 32;         // 32-wide d tiles of O^T
  static constexpr int KROW = D + 8;        // LDS row stride of K (halfs)
  static constexpr int VROW = VLayout<D>::VROW;  // LDS row stride of V (halfs)
  static constexpr int K_LDS = kBlockN * KROW;
  static constexpr int V_LDS = kBlockN * VROW;

  _Float16* k_lds;
  _Float16* vt_lds;
  const _Float16* kbase;
  const _Float16* vbase;
  int64_t kv_row_stride;
  int S_kv, n_tiles, tid, qw, qrow, hf, k_lane, v_lane;
  float c2, lazy_raw;
  Stager<D, HP> st;
  half8_t qf[KS];
  f32x16_t o[DT];
  float m, l;

  // Stage the next tiles: K runs one tile ahead of V (the math of step t
  // reads K(t+1) for the next scores and V(t) for this tile's PV product).
  __device__ __forceinline__ void issue_loads(int t) {
    if (t + 2 < n_tiles) st.load_k((t + 2) * kBlockN, tid);
    if (t + 1 < n_tiles) st.load_v((t + 1) * kBlockN, tid);
  }
  __device__ __forceinline__ void commit_loads(int t) {
    // K(t+2) goes into the slot that held K(t); K(0) is read by the QK
    // product that precedes the loop, so before the first store every
    // wavefront must be past that read
    if (t == 0) lds_barrier();
    if (t + 2 < n_tiles) st.store_k(k_lds + (t & 1) * K_LDS, tid);
    if (t + 1 < n_tiles) st.store_v(vt_lds + ((t + 1) & 1) * V_LDS, tid);
    lds_barrier();
  }

  __device__ __forceinline__ void qk(f32x16_t (&s)[2], int t) const {
    qk_tile<D>(s, k_lds + (t & 1) * K_LDS + k_lane, qf);
  }

  half8_t pf[4];  // fp16 weights of the tile whose PV product is next

  // Mask (only where the tile crosses the diagonal or the end of the keys),
  // tile max of each query over both lane halves, and the lazy move of the
  // reference point: only when some row's weights would pass 2^8.
  __device__ __forceinline__ void mask_max_rescale(int t, f32x16_t (&sc)[2]) {
    const int kv0 = t * kBlockN;
    const bool need_mask = (CAUSAL && kv0 + kBlockN - 1 > qw) || (kv0 + kBlockN > S_kv);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
          const bool masked = (CAUSAL && key > qrow) || key >= S_kv;
          if (masked) sc[kb][r] = -INFINITY;
        }
      }
    }
    float mx = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sc[0][r], sc[0][r + 1]));
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sc[1][r], sc[1][r + 1]));
    mx = wave_half_swap_max(mx);
    if (__builtin_amdgcn_ballot_w64(mx > m + lazy_raw) != 0) {
      const float m_new = fmaxf(m, mx);
      const float alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m - m_new) * c2);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
  }

  // fp16 weights exp2(s*c2 - m*c2) -> pf, and the row sum of exactly those
  // fp16 values (four independent partial sums)
  __device__ __forceinline__ void weights(const f32x16_t (&sc)[2]) {
    const float mb = m * c2;
    const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
    float lp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pf[c][i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(sc[c >> 1][8 * (c & 1) + i], c2, -mb));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half2_t pp = {pf[c][2 * i], pf[c][2 * i + 1]};
        lp[i] = __builtin_amdgcn_fdot2(pp, ones, lp[i], false);
      }
    }
    l += (lp[0] + lp[1]) + (lp[2] + lp[3]);
  }

  // O^T += V^T P^T for tile t, the DT accumulators alternating, operand
  // reads four ahead
  __device__ __forceinline__ void pv(int t) {
    const _Float16* vl = vt_lds + (t & 1) * V_LDS + v_lane;
    constexpr int N = DT * 4;
    constexpr int R = 4;
    half8_t ring[R];
#pragma unroll
    for (int n = 0; n < R; ++n) ring[n] = pv_operand<VROW>(vl, n % DT, n / DT);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int dt = n % DT, c = n / DT;
      const half8_t vf = ring[n % R];
      if (n + R < N) ring[n % R] = pv_operand<VROW>(vl, (n + R) % DT, (n + R) / DT);
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[c], o[dt], 0, 0, 0);
    }
  }

  // One step of the one-head schedule: softmax of tile t's scores and its PV
  // product; when NEXT, the scores of tile t+1 are computed in the same basic
  // block so that the scheduler can interleave those MFMAs with this tile's
  // exponentials.
  template <bool NEXT>
  __device__ __forceinline__ void step(int t, f32x16_t (&sc)[2], f32x16_t (&sn)[2]) {
    issue_loads(t);
    mask_max_rescale(t, sc);
    if (NEXT) qk(sn, t + 1);
    weights(sc);
    pv(t);
    commit_loads(t);
  }

  // ---- the two phases of the ping-pong schedule (HP == 2) ----

  // VALU phase: tile t's scores sc -> fp16 weights pf
  __device__ __forceinline__ void softmax(int t, f32x16_t (&sc)[2]) {
    mask_max_rescale(t, sc);
    weights(sc);
  }

  // MFMA phase: the scores of tile t+1 into sn (when QK), then O += P(t) V(t).
  // The wavefront raises its issue priority for the phase, so on a SIMD the
  // MFMAs of this wavefront go first and the other's VALU fills the gaps.
  template <bool QK>
  __device__ __forceinline__ void gemm(int t, f32x16_t (&sn)[2]) {
    __builtin_amdgcn_s_setprio(1);
    if (QK) qk(sn, t + 1);
    pv(t);
    // QK: 2*(D/16) MFMAs, one b128 read each; PV: 4*DT MFMAs, two reads each
    constexpr int NM = (QK ? 2 * KS : 0) + 4 * DT;
    constexpr int NR = (QK ? 2 * KS : 0) + 8 * DT;
    __builtin_amdgcn_sched_group_barrier(0x100, kLdsAhead, 0);
    IssueChain<0, NM, NR - kLdsAhead>::run();
    __builtin_amdgcn_s_setprio(0);
  }

  // a tile this wavefront does not compute (above its diagonal): staging only
  __device__ __forceinline__ void idle_step(int t) {
    issue_loads(t);
    commit_loads(t);
  }
};

// One query tile (128 rows of each of the HP heads of head group hg, batch b)
// against its keys, from the first K/V tile to the last.
template <int D, bool CAUSAL, int HP, bool ROPE>
__device__ __forceinline__ void prefill_qtile(const PrefillArgs& a, int qt, int hg, int b,
                                              _Float16* k_lds, _Float16* vt_lds) {

  using P = Prefill<D, CAUSAL, HP>;

  P p;
  p.k_lds = k_lds;
  p.vt_lds = vt_lds;
  p.tid = (int)__builtin_amdgcn_workitem_id_x();  // threadIdx.x (see the kernel)
  const int lane = p.tid & 63;
  const int wave = p.tid >> 6;
  const int col = lane & 31;  // query column of S^T / O^T owned by this lane
  p.hf = lane >> 5;           // which half of the k-range this lane supplies

  const int h = hg * HP + wave / kWavesPerHead;
  const int g = (int)(((int64_t)hg * HP * a.H_kv) / a.H_q);  // shared by the HP heads

  const int q0 = qt * kBlockM;
  p.qw = q0 + (wave % kWavesPerHead) * kRowsPerWave;  // first row of this wavefront
  p.qrow = p.qw + col;                                // this lane's query row
  const int64_t q_row_stride = (int64_t)a.H_q * D;
  p.kv_row_stride = (int64_t)a.H_kv * D;
  p.S_kv = a.S_kv;

  // the row's position goes out first: the table rows need it, and loads
  // retire in order
  qnr::QNormRope<D> qr;
  if constexpr (ROPE) qr.issue_pos(a, b, p.qrow);
  // Q fragment (B operand of S^T = K Q^T): q[qrow][16*ks + 8*hf + 0..7]
  if (p.qrow < a.S_q) {
    const _Float16* qp = a.q + ((int64_t)b * a.S_q + p.qrow) * q_row_stride + (int64_t)h * D + 8 * p.hf;
#pragma unroll
    for (int ks = 0; ks < P::KS; ++ks) p.qf[ks] = *reinterpret_cast<const half8_t*>(qp + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < P::KS; ++ks) p.qf[ks] = half8_t{};
  }
#pragma unroll
  for (int dt = 0; dt < P::DT; ++dt) p.o[dt] = f32x16_t{};
  p.m = -INFINITY;  // reference point of the exponentials (raw dot-product units)
  p.l = 0.0f;       // this lane's share of the sum of fp16 weights
  p.c2 = a.scale_log2;
  p.lazy_raw = kLazyLog2 / p.c2;

  int n_tiles = (a.S_kv + kBlockN - 1) / kBlockN;
  if (CAUSAL) {
    const int last_row = min(q0 + kBlockM, a.S_q) - 1;
    n_tiles = min(n_tiles, last_row / kBlockN + 1);
  }
  p.n_tiles = n_tiles;
  const int wave_last_row = min(p.qw + kRowsPerWave - 1, a.S_q - 1);
  // tiles this wavefront computes: [0, wave_tiles)
  int wave_tiles = p.qw < a.S_q ? n_tiles : 0;
  if (CAUSAL) wave_tiles = min(wave_tiles, wave_last_row / kBlockN + 1);

  p.kbase = a.k + (int64_t)b * a.S_kv * p.kv_row_stride + (int64_t)g * D;
  p.vbase = a.v + (int64_t)b * a.S_kv * p.kv_row_stride + (int64_t)g * D;
  p.k_lane = col * P::KROW + 8 * p.hf;
  // transposed V reads: 16-lane group G = lane/16 covers dims 16*(G%2)..+15
  // of keys 4*hf + (lane%16)/4, four dims per lane
  p.v_lane = (4 * p.hf + (lane & 15) / 4) * P::VROW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // prologue: K(0), V(0) and K(1) into LDS
  p.st.init(p.kbase, p.vbase, (int)p.kv_row_stride, a.S_kv);
  if constexpr (ROPE) qr.issue_rest(a, p.hf);  // the weights and table rows
  // K(0), V(0) and K(1) in flight together: one global round trip
  half8_t k1[Stager<D, HP>::PER_T];
  p.st.load_k(0, p.tid);
  p.st.load_v(0, p.tid);
  if (n_tiles > 1) p.st.load_k_into(k1, kBlockN, p.tid);
  bool q_ok = true;
  if constexpr (ROPE) q_ok = qr.apply(a, p.qf);
  p.st.store_k(k_lds, p.tid);
  p.st.store_v(vt_lds, p.tid);
  if (n_tiles > 1) Stager<D, HP>::store_k_from(k1, k_lds + P::K_LDS, p.tid);
  lds_barrier();

  // Every wavefront takes part in all n_tiles staging steps (and barriers);
  // it computes tiles [0, wave_tiles).
  if constexpr (HP == 2) {
    // Ping-pong: SIMD s runs wavefront s (first head) and s + 4 (second head)
    // on the same rows.  Per step the first runs its MFMA phase, then its
    // softmax; the second its softmax, then its MFMA phase.  Each SIMD so
    // pairs one wavefront's MFMAs with the other's VALU work instead of both
    // doing the same kind of work at once.
    //   first head,  step t: QK(t+1), PV(t) | softmax(t+1)
    //   second head, step t: softmax(t)     | QK(t+1), PV(t)
    f32x16_t sc[2];
    const bool first = wave < kWavesPerHead;
    if (wave_tiles > 0) {
      p.qk(sc, 0);
      if (first) p.softmax(0, sc);
    }
    int t = 0;
    for (; t < wave_tiles; ++t) {
      p.issue_loads(t);
      const bool more = t + 1 < wave_tiles;
      if (first) {
        if (more) p.template gemm<true>(t, sc); else p.template gemm<false>(t, sc);
        __builtin_amdgcn_sched_barrier(0);  // keep the phases apart
        if (more) p.softmax(t + 1, sc);
      } else {
        p.softmax(t, sc);
        __builtin_amdgcn_sched_barrier(0);
        if (more) p.template gemm<true>(t, sc); else p.template gemm<false>(t, sc);
      }
      p.commit_loads(t);
    }
    for (; t < n_tiles; ++t) p.idle_step(t);
  } else {
  // One head per workgroup: the scores of tile t+1 are computed inside step t,
  // among tile t's exponentials.  Pairs of steps swap the two score buffers so
  // no copy is needed.
  f32x16_t sa[2], sb[2];
  if (wave_tiles > 0) p.qk(sa, 0);
  int t = 0;
  for (; t + 2 < wave_tiles; t += 2) {
    p.template step<true>(t, sa, sb);
    p.template step<true>(t + 1, sb, sa);
  }
  if (t + 1 < wave_tiles) {
    p.template step<true>(t, sa, sb);
    p.template step<false>(t + 1, sb, sa);
    t += 2;
  } else if (t < wave_tiles) {
    p.template step<false>(t, sa, sb);
    t += 1;
  }
  for (; t < n_tiles; ++t) p.idle_step(t);
  }

  // epilogue: combine the two half-row sums, normalise, round to fp16.
  // A lane holds 4-dim pieces of one row, so storing them directly would
  // scatter 8-byte writes over 32 rows per instruction.  Instead each
  // wavefront puts its 32 x D tile row-major into its own part of the K/V
  // tiles' LDS (free: every wavefront is past the last step's barrier, and
  // the next query tile writes it only after the workgroup barrier that
  // follows), reads it back as 16-byte row pieces and stores whole rows.
  if (p.qw >= a.S_q) return;
  const float lsum = wave_half_swap_add(p.l);
  const float inv = 1.0f / lsum;
  // row stride (halfs): a multiple of 8 for the 16-byte reads; with it the
  // 4 tiles of a head fit the V tiles (first head) and the K tiles (second)
  constexpr int OROW = (D == 32) ? D : D + 8;
  static_assert(4 * kRowsPerWave * OROW <= 2 * P::V_LDS && 4 * kRowsPerWave * OROW <= 2 * P::K_LDS,
                "output tiles must fit the K/V tiles' LDS");
  _Float16* ot = (wave < kWavesPerHead ? vt_lds : k_lds) + (wave % kWavesPerHead) * kRowsPerWave * OROW;
#pragma unroll
  for (int dt = 0; dt < P::DT; ++dt) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      half4_t out;
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = (_Float16)(p.o[dt][rg * 4 + j] * inv);
      if (ROPE && !q_ok) out = __builtin_bit_cast(half4_t, 0x7e007e007e007e00ull);  // quiet NaN bits
      *reinterpret_cast<half4_t*>(ot + col * OROW + dt * 32 + rg * 8 + p.hf * 4) = out;
    }
  }
  // the lanes read rows other lanes of this wavefront wrote
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  constexpr int PIECES = D / 8;             // 16-byte pieces per row
  constexpr int ROWS_PER = 64 / PIECES;     // rows per 64-lane store
  const int pr = lane / PIECES, pc = lane % PIECES;
#pragma unroll
  for (int i = 0; i < kRowsPerWave / ROWS_PER; ++i) {
    const int r = i * ROWS_PER + pr;
    const half8_t v8 = *reinterpret_cast<const half8_t*>(ot + r * OROW + 8 * pc);
    if (p.qw + r < a.S_q)
      *reinterpret_cast<half8_t*>(a.o + ((int64_t)b * a.S_q + p.qw + r) * q_row_stride + (int64_t)h * D + 8 * pc) = v8;
  }
}

// Work unit of a workgroup: query tiles qt and n_qtiles-1-qt of one (head
// group, batch).  Under the causal mask tile i costs i+1 units of 128 keys,
// so every pair costs the same n_qtiles+1 units and the grid has no
// long-tile tail; an odd middle tile runs alone, after all pairs.
template <int D, bool CAUSAL, int HP, bool ROPE>
__global__ __launch_bounds__(64 * kWavesPerHead * HP, 2) void prefill_fwd_kernel(PrefillArgs a) {
  using P = Prefill<D, CAUSAL, HP>;
  // K runs one tile ahead of V: at step t the math reads K(t+1) and V(t)
  __shared__ __attribute__((aligned(16))) _Float16 k_lds[2 * P::K_LDS];
  __shared__ __attribute__((aligned(16))) _Float16 vt_lds[2 * P::V_LDS];

  const int head_groups = a.H_q / HP;
  const int combos = head_groups * a.B;
  // The raw work-group / work-item id builtins: this file is built without NaN
  // semantics, so the device library's blockIdx / threadIdx helpers (built
  // with them) are not inlined and would become calls.
  const int id = (int)__builtin_amdgcn_workgroup_id_x();
  const int pair = id / combos;
  const int rem = id - pair * combos;
  const int hg = rem % head_groups;
  const int b = rem / head_groups;
  const int lo = pair, hi = a.n_qtiles - 1 - pair;
  prefill_qtile<D, CAUSAL, HP, ROPE>(a, hi, hg, b, k_lds, vt_lds);
  if (lo < hi) {
    lds_barrier();  // the first tile's last LDS reads are done (its output stores may still be in flight)
    prefill_qtile<D, CAUSAL, HP, ROPE>(a, lo, hg, b, k_lds, vt_lds);
  }
}

template <int D, bool CAUSAL, int HP, bool ROPE>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)((a.n_qtiles + 1) / 2) * (a.H_q / HP) * a.B;
  PrefillArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&prefill_fwd_kernel<D, CAUSAL, HP, ROPE>),
                         dim3((unsigned)blocks), dim3(64 * kWavesPerHead * HP), kargs, 0, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_hp(const PrefillArgs& a, hipStream_t stream) {
  const bool pair = ((a.H_q / a.H_kv) % 2) == 0;
  if (a.cos_table)
    return pair ? launch_t<D, CAUSAL, 2, true>(a, stream) : launch_t<D, CAUSAL, 1, true>(a, stream);
  return pair ? launch_t<D, CAUSAL, 2, false>(a, stream) : launch_t<D, CAUSAL, 1, false>(a, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a_in, int head_dim, bool causal, hipStream_t stream) {
  if (head_dim == 128) return launch_prefill_dual(a_in, causal, stream);
  PrefillArgs a = a_in;
  a.n_qtiles = (a.S_q + kBlockM - 1) / kBlockM;
  switch (head_dim) {
    case 32: return causal ? launch_hp<32, true>(a, stream) : launch_hp<32, false>(a, stream);
    case 64: return causal ? launch_hp<64, true>(a, stream) : launch_hp<64, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
