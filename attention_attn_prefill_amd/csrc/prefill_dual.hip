// prefill_dual.hip -- causal / non-causal GQA attention prefill for gfx950
// at head_dim 128, with two 32-row query blocks per wavefront.
//
// Computes O = softmax(Q K^T / sqrt(D) + mask) V over [B,S,H,D] fp16 tensors
// with fp32 accumulation ("Tutorial: Adding a New Kernel to RL.cu",
// attention.cuh prefill section and the attention.cu prefill kernel: GQA kv
// head = h*H_kv/H_q, causal mask j <= i, online softmax with a running max,
// a running sum and rescaling by exp(m_old - m_new)).  Both contractions run
// on v_mfma_f32_32x32x16_f16.
//
// What shapes this kernel is LDS operand traffic.  A wavefront that owns one
// 32-row query block reads 1 KB of K or V operand from LDS per 32x32x16
// MFMA; with every SIMD busy that is as many LDS bytes per clock as the CU
// can deliver.  Here a wavefront owns two row blocks that multiply the same
// operands:
//   * the same 32 rows of the two query heads that share a kv head (H_q/H_kv
//     even), or 64 consecutive rows of one head otherwise;
//   * S^T[32 keys x 32 queries] = K . Q^T with K as the A operand, so one K
//     read serves both blocks' B operands (their Q fragments), and
//     O^T[D x 32] += V^T . P^T with V^T (read by ds_read_b64_tr_b16) as the
//     A operand, one read for both blocks' P^T;
//   * registers: two Q fragments (64), two output accumulators (128), two
//     pairs of score accumulators (64) -- one wavefront per SIMD, four per
//     workgroup, 128 (two heads) or 256 (one head) query rows per workgroup.
// With no second wavefront on the SIMD to hide the softmax behind, the
// wavefront overlaps it with its own matrix work.  Keys advance in 32-key
// sub-blocks; step u issues
//     S(u+1) = K(u+1) Q^T            16 MFMAs, 8 K operand reads
//     P(u)   = exp2(S(u)), row sums  ~100 VALU instructions
//     O     += V(u-1)^T P(u-1)^T    16 MFMAs, 8 V operands (16 reads)
// which are independent of each other, in one basic block, interleaved
// chunk by chunk (one MFMA and its share of the softmax per chunk; the LDS
// reads in the even chunks, which carry no fp16 packing or row-sum adds).
//
// Scores stay exact: S^T accumulates the fp16 products of Q and K in fp32
// from zero, and the weight of a key is exp2(s * log2(e)/sqrt(D) - m) with m
// the row's reference point in log2 units (one fma and one v_exp_f32).
//
// Fixed reference point per query tile: the reference of a row is the exact
// max of its first sub-block and then stays put, so O and the row sum l are
// never rescaled inside the loop (the usual online-softmax rescale exp(m_old -
// m_new) becomes a no-op).  What can go wrong is fp16 overflow of a weight
// when later keys score far above the first ones; each lane keeps the
// running max of its per-sub-block row-sum shares, and a share of at most
// 2^15 bounds every weight of those 16 keys below the fp16 limit.  If any
// wavefront of the workgroup saw a larger share, the query tile is computed
// again: a first pass of QK products takes the exact max of every row, and the
// second pass runs against it (every weight <= 1).  The result does not depend
// on which path ran (any reference cancels in O/l); on typical scores the
// check never fires.  The row sum adds the fp32 weights before their
// rounding to fp16.
//
// Staging: K and V tiles of 64 keys, double-buffered in LDS, row-major
// (K [64][D+8], V [64][D+32]: the padding keeps the operand reads nearly
// free of bank conflicts), copied from HBM straight into LDS by buffer
// loads over the kv head's rows [0, S_kv) (rows past the end read as zero
// and are masked).  K runs one tile ahead of V: the two steps of iteration
// t read K(t+1) and V(t); the first step copies K(t+2) and the second
// V(t+1) into the slots that K(t) and V(t-1) held, and a vmcnt(0) wait and
// one LDS barrier end the iteration.
//
// Causal: all four wavefronts run every step of the workgroup's key range;
// sub-blocks before a wavefront's diagonal run unmasked, the rest with the
// element mask (those past the diagonal come out all zero); tiles above the
// workgroup's last row are never loaded.  A workgroup runs query tiles
// n-1-i and i back to back, so every workgroup does the same work.
#include "gfx950_device.h"
#include "q_norm_rope.h"

#include <math.h>

#include <type_traits>

namespace attn {
namespace {

using dev::half_swap_add;
using dev::half_swap_max;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;              // wavefronts per workgroup, one per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;              // keys per staged K/V tile
constexpr float kShareMax = 32768.0f;  // largest row-sum share that keeps fp16 weights finite
constexpr uint32_t kPadOffset = 0x80000000u;  // a load offset past any buffer range

// ROPE: Q's per-head RMSNorm and NeoX rotation are applied as it is loaded
// (attn_prefill_qk_norm_rope); the rest of the kernel is unchanged.
template <bool CAUSAL, int HP, bool ROPE>
struct Dual {
  static constexpr int D = 128;
  static constexpr int KS = D / 16;                          // k-steps of QK^T
  static constexpr int DT = D / 32;                          // 32-dim tiles of O^T
  static constexpr int KROW = D + 8;                         // LDS row stride of K (halfs)
  static constexpr int VROW = D + 32;                        // LDS row stride of V (halfs)
  static constexpr int K_LDS = kTile * KROW;
  static constexpr int V_LDS = kTile * VROW;
  static constexpr int LDS_HALFS = 2 * K_LDS + 2 * V_LDS;  // the K/V slots (a spare 1 KB follows)
  static constexpr int VEC_ROW = D / 8;                      // 16-byte vectors per key row
  static constexpr int K_BLOCKS = kTile * KROW * 2 / 1024;   // 1 KB LDS blocks per K tile (17)
  static constexpr int V_BLOCKS = kTile * VROW * 2 / 1024;   // 1 KB LDS blocks per V tile (20)
  static constexpr int K_COPIES = (K_BLOCKS + kWaves - 1) / kWaves;  // copies per wavefront and tile
  static constexpr int V_COPIES = (V_BLOCKS + kWaves - 1) / kWaves;
  static constexpr int COPIES = K_COPIES + V_COPIES;
  static constexpr int ROWS_WG = HP == 2 ? 4 * 32 : 4 * 64;  // query rows per head and workgroup
  static constexpr int OROW = D + 8;                         // LDS row stride of the output tiles
  static constexpr int OUT_LDS = 8 * 32 * OROW;               // output tiles (an LDS array of their own)
  static constexpr int SMEM_HALFS = LDS_HALFS + 512;            // the K/V slots and the spare block
  static_assert(K_BLOCKS * 1024 == kTile * KROW * 2 && V_BLOCKS * 1024 == kTile * VROW * 2,
                "tiles must be whole 1 KB blocks");
  static_assert((SMEM_HALFS + OUT_LDS) * 2 <= 160 * 1024, "LDS of one workgroup");

  _Float16* smem;   // the K/V slots and the spare block
  _Float16* osmem;  // the output tiles of the epilogue
  int tid, lane, hf, col;
  int wave;  // wavefront index in the workgroup (uniform: from readfirstlane)
  int k_lane, v_lane;  // this lane's offsets in a K / V tile (halfs)
  __amdgpu_buffer_rsrc_t krsrc, vrsrc;
  uint32_t row_bytes;
  // per-lane byte offsets (within a tile) of the 1 KB LDS blocks this
  // wavefront copies: row * row_bytes + 16 * chunk, or kPadOffset where the
  // block position is row padding (an out-of-range load writes zeros there)
  uint32_t k_off[K_COPIES], v_off[V_COPIES];
  // LDS byte address of the block each copy fills, per slot (the spare block
  // for a dummy copy); uniform, so they live in SGPRs and a copy costs one
  // scalar select into M0.  Given as integers, the copies carry no pointer
  // the compiler could relate to the operand reads, so it places no wait for
  // them before those reads (the iteration's vmcnt(0) and barrier order them)
  uint32_t k_dst[2][K_COPIES], v_dst[2][V_COPIES];
  int S_kv;
  int mask_from;  // first sub-block that may need the element mask
  int n_tiles;    // K/V tiles the workgroup stages
  // K/V tile t of the pass sits in slot (t + par0) & 1.  Copies of tiles
  // next_base and next_base + 1 (past the pass's keys) fetch the next query
  // tile's tiles 0 and 1 instead (next_base is out of reach otherwise).
  int par0;
  int next_base;
  int row0[2];    // first query row of each row block
  int head[2];    // query head of each row block
  int b;          // batch entry
  half8_t qf[2][KS];
  f32x16_t o[2][DT];
  f32x16_t s[2][2];    // [sub-block parity][row block]
  half2_t p[2][2][8];  // fp16 weights [parity][row block][key pair]: pairs 4c..4c+3 form 16-key chunk c
  float mb[2];         // reference point (log2 units)
  float c2;            // log2(e) / sqrt(D)
  float l[2], lsum[2];
  float share_max;     // largest row-sum share of this lane so far
  // ROPE: the norm + rotation state of a query row (the two blocks of a
  // two-head workgroup share their row; a one-head workgroup's blocks take
  // it in turn) and whether each row's position was valid (else its output
  // is NaN)
  qnr::QNormRope<D> qr;
  bool q_ok[2];

  // ---- staging -----------------------------------------------------------
  // Tiles go from HBM straight into LDS (buffer loads with the LDS bit), in
  // 1 KB blocks of the padded row layout, block i of a tile by wavefront
  // i % 4.  A wavefront whose share is one block short copies a dummy block
  // (zeros into a spare 1 KB) so that every wavefront issues the same number
  // of copies.
  template <int ROW>
  __device__ __forceinline__ void copy_offsets(uint32_t* off, int copies) {
    constexpr int ROWB = ROW * 2;
    for (int j = 0; j < copies; ++j) {
      const int bo = (wave + kWaves * j) * 1024 + 16 * lane;  // byte in the tile
      const int r = bo / ROWB, c = (bo - r * ROWB) / 16;
      off[j] = c < VEC_ROW ? (uint32_t)r * row_bytes + 16u * c : kPadOffset;
    }
  }
  __device__ __forceinline__ void copy_dsts() {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) _Float16*)smem;
    const uint32_t spare = lds0 + LDS_HALFS * 2;  // the spare block past the tiles
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
      for (int j = 0; j < K_COPIES; ++j) {
        const int i = wave + kWaves * j;
        k_dst[sl][j] = i < K_BLOCKS ? lds0 + (sl * K_LDS + i * 512) * 2 : spare;
      }
#pragma unroll
      for (int j = 0; j < V_COPIES; ++j) {
        const int i = wave + kWaves * j;
        v_dst[sl][j] = i < V_BLOCKS ? lds0 + (2 * K_LDS + sl * V_LDS + i * 512) * 2 : spare;
      }
    }
  }
  // copy n of the tile pair (K tile tk, V tile tv); n < COPIES
  __device__ __forceinline__ void copy(int n, int tk, int tv) {
    if (n < K_COPIES) {
      const int src_t = tk >= next_base ? tk - next_base : tk;
      const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)src_t * kTile * row_bytes);
      dev::buffer_load16_lds_at(krsrc, ((tk + par0) & 1) ? k_dst[1][n] : k_dst[0][n], (int)(k_off[n] + base));
    } else {
      const int j = n - K_COPIES;
      const int src_t = tv >= next_base ? tv - next_base : tv;
      const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)src_t * kTile * row_bytes);
      dev::buffer_load16_lds_at(vrsrc, ((tv + par0) & 1) ? v_dst[1][j] : v_dst[0][j], (int)(v_off[j] + base));
    }
  }
  __device__ __forceinline__ void copy_tiles(int tk, int tv) {
#pragma unroll
    for (int n = 0; n < COPIES; ++n) copy(n, tk, tv);
  }
  // iteration t copies K(t+2) and V(t+1) into the slots that K(t) and
  // V(t-1) held; past the last tile the copies read zeros (outside the
  // buffer range) into slots nothing reads any more
  __device__ __forceinline__ void stage(int t) { copy_tiles(t + 2, t + 1); }
  // prologue of a pass: K(0), V(0) and K(1) in LDS
  __device__ __forceinline__ void stage_prologue() {
    copy_tiles(0, 0);
#pragma unroll
    for (int n = 0; n < K_COPIES; ++n) copy(n, 1, 0);
    dev::wait_vmcnt0();
  }

  // ---- the parts of a step -----------------------------------------------
  // S^T of sub-block uu (keys 32uu..32uu+31, parity PAR = uu & 1) for both
  // row blocks, into s[PAR] (raw dot products, fp32)
  template <int PAR>
  __device__ __forceinline__ void qk(int uu) {
    const _Float16* kb = smem + (((uu >> 1) + par0) & 1) * K_LDS + k_lane + PAR * 32 * KROW;
    half8_t kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const half8_t*>(kb + 16 * ks);
    f32x16_t acc[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[g] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int g = 0; g < 2; ++g) acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks], qf[g][ks], acc[g], 0, 0, 0);
    s[PAR][0] = acc[0];
    s[PAR][1] = acc[1];
  }

  // element mask of sub-block uu (causal diagonal, ragged end of the keys)
  template <int PAR>
  __device__ __forceinline__ void mask(int uu) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int row = row0[g] + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * uu + 8 * (r >> 2) + 4 * hf + (r & 3);
        if ((CAUSAL && key > row) || key >= S_kv) s[PAR][g][r] = -INFINITY;
      }
    }
  }

  // fp16 pair of score elements r, r+1 (r even) of row block g into p[PAR]
  // (one v_cvt_pk_f16_f32, kept where it is issued)
  template <int PAR>
  __device__ __forceinline__ void put_pair(int g, int r, float a, float b) {
    half2_t h = {(_Float16)a, (_Float16)b};
    asm volatile("" : "+v"(h));
    p[PAR][g][r >> 1] = h;
  }
  // B operand of the PV product: 16-key chunk c of p[PAR][g]
  template <int PAR>
  __device__ __forceinline__ half8_t p_chunk(int g, int c) const {
    const half2_t q4[4] = {p[PAR][g][4 * c], p[PAR][g][4 * c + 1], p[PAR][g][4 * c + 2], p[PAR][g][4 * c + 3]};
    return __builtin_bit_cast(half8_t, q4);
  }

  __device__ __forceinline__ static float max16(const f32x16_t& x) {
    float a = fmaxf(fmaxf(x[0], x[1]), x[2]);
    float b = fmaxf(fmaxf(x[3], x[4]), x[5]);
    float c = fmaxf(fmaxf(x[6], x[7]), x[8]);
    float d = fmaxf(fmaxf(x[9], x[10]), x[11]);
    float e = fmaxf(fmaxf(x[12], x[13]), x[14]);
    return fmaxf(fmaxf(fmaxf(a, b), fmaxf(c, d)), fmaxf(e, x[15]));
  }

  // weights of the sub-block in s[PAR]: p = fp16(exp2(s * c2 - mb)) and this
  // lane's share of their row sum (the fp32 weights)
  template <int PAR>
  __device__ __forceinline__ void weights() {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(s[PAR][g][r], c2, -mb[g]));
#pragma unroll
      for (int r = 0; r < 16; r += 2) p[PAR][g][r >> 1] = half2_t{(_Float16)e[r], (_Float16)e[r + 1]};
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = e[2 * i] + e[2 * i + 1];
      lsum[g] = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    }
    share_max = fmaxf(share_max, fmaxf(lsum[0], lsum[1]));
  }

  // Step u (parity PAR) of the loop: S(u+1) = K Q^T into s[PAR ^ 1], the
  // softmax of s[PAR] into p[PAR], and O += V^T P(u-1)^T.  STAGE 1 issues
  // the iteration's K tile copies in the first chunks of the step, STAGE 2
  // its V tile copies (one half of the staging in each step of an iteration
  // costs less issue time than all of it in one).
  //
  // The three parts are independent, and a wavefront is alone on its SIMD,
  // so the instruction order is spelled out: 32 chunks, each one MFMA (16 of
  // QK, then 16 of PV), the fma of one score element, the exponential of the
  // element before it, every other (odd) chunk the fp16 pair and the
  // row-sum adds of two earlier elements, and in the even chunks the LDS
  // operand reads, six to eight MFMAs before their use.  A scheduling fence
  // after every chunk keeps the compiler from regrouping MFMAs and VALU work
  // into runs.
  //
  // The first K operands of a step are read AHEAD / 2 = 3 k-steps ahead of
  // its first MFMA.  The second step of an iteration reads the same K tile
  // as the first, already resident, so the first step reads them for it in
  // its last chunks (PRE_OUT, into kpre) and the second step starts on them
  // (PRE_IN) instead of waiting on fresh LDS reads.  The first step's K tile
  // only becomes visible at the iteration's barrier.
  static constexpr int PRE = 3;
  template <int PAR, bool MASK, int STAGE, bool PRE_IN, bool PRE_OUT>
  __device__ __forceinline__ void step(int u, int t, half8_t (&kpre)[PRE]) {
    constexpr int PP = PAR ^ 1;
    constexpr int AHEAD = 6;  // chunks between an operand read and its MFMA
    static_assert(AHEAD == 2 * PRE, "the prefetched K operands are the up-front ones");
#pragma unroll
    for (int g = 0; g < 2; ++g) l[g] += lsum[g];
    if (MASK) mask<PAR>(u);
    const _Float16* kb = smem + ((((u + 1) >> 1) + par0) & 1) * K_LDS + k_lane + PP * 32 * KROW;
    const _Float16* vl = smem + 2 * K_LDS + ((((u - 1) >> 1) + par0) & 1) * V_LDS + v_lane;
    half8_t kf[KS];
    dev::short4_t vr[16];
    f32x16_t acc[2];
    float x[32], y[32];
    float ls[2][2];  // two running partial row sums per block
    // K k-step ks feeds chunks 2ks, 2ks+1; V operand op (= c * 4 + dt) feeds
    // chunks 16 + 2op, 17 + 2op and takes two transposed reads
    auto read_k = [&](int ks) { kf[ks] = *reinterpret_cast<const half8_t*>(kb + 16 * ks); };
    auto read_v = [&](int v) {
      const int op = v >> 1, c = op >> 2, dt = op & 3, cc = 2 * PP + c;
      vr[v] = dev::lds_read_tr(vl + (16 * cc + 8 * (v & 1)) * VROW + dt * 32);
    };
#pragma unroll
    for (int ks = 0; 2 * ks < AHEAD; ++ks) {
      if (PRE_IN) kf[ks] = kpre[ks];
      else read_k(ks);
    }
    // the next step's K sub-block (u + 2, parity PAR), for PRE_OUT
    const _Float16* kb_next = smem + ((((u + 2) >> 1) + par0) & 1) * K_LDS + k_lane + PAR * 32 * KROW;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i < 16) {
        const int ks = i >> 1, g = i & 1;
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks], qf[g][ks], ks == 0 ? f32x16_t{} : acc[g], 0, 0, 0);
      } else {
        const int j = i - 16, op = j >> 1, g = j & 1, c = op >> 2, dt = op & 3;
        const dev::short4_t lohi[2] = {vr[2 * op], vr[2 * op + 1]};
        o[g][dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, lohi), p_chunk<PP>(g, c), o[g][dt], 0, 0, 0);
      }
      x[i] = fmaf(s[PAR][i >> 4][i & 15], c2, -mb[i >> 4]);
      if (i >= 1) y[i - 1] = __builtin_amdgcn_exp2f(x[i - 1]);
      if (i >= 3 && (i & 1)) {
        const int e = i - 3, g = e >> 4, r = e & 15;
        put_pair<PAR>(g, r, y[e], y[e + 1]);
        // the first pair of each partial sum starts it (no add of zero)
        if (r < 4) ls[g][(r >> 1) & 1] = y[e] + y[e + 1];
        else ls[g][(r >> 1) & 1] += y[e] + y[e + 1];
        // keep the add in this chunk (otherwise it sinks to the loop latch)
        asm volatile("" : "+v"(ls[g][(r >> 1) & 1]));
      }
      // the reads of chunk i + AHEAD, on even chunks only: a K k-step, or
      // both halves of a V operand (LDS reads cost least next to MFMAs in the
      // chunks without the fp16 packing and the row-sum adds)
      const int n = i + AHEAD;
      if (n < 16 && !(n & 1)) read_k(n >> 1);
      if (n >= 16 - 2 && n < 32 - 2 && !(n & 1)) {
        read_v(n - 14);
        read_v(n - 13);
      }
      if (PRE_OUT && i >= 32 - PRE - 2 && i < 32 - 2) {
        const int ks = i - (32 - PRE - 2);
        kpre[ks] = *reinterpret_cast<const half8_t*>(kb_next + 16 * ks);
      }
      if (STAGE == 1 && i < K_COPIES) copy(i, t + 2, t + 1);
      if (STAGE == 2 && i < V_COPIES) copy(K_COPIES + i, t + 2, t + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    y[31] = __builtin_amdgcn_exp2f(x[31]);
#pragma unroll
    for (int e = 30; e < 32; e += 2) {
      const int g = e >> 4, r = e & 15;
      put_pair<PAR>(g, r, y[e], y[e + 1]);
      ls[g][(r >> 1) & 1] += y[e] + y[e + 1];
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) lsum[g] = ls[g][0] + ls[g][1];
    share_max = fmaxf(share_max, fmaxf(lsum[0], lsum[1]));
    s[PP][0] = acc[0];
    s[PP][1] = acc[1];
  }

  // One pass over the keys, with the Q fragments loaded and K(0), V(0),
  // K(1) in LDS (published by the caller's barrier).  KNOWN_REF: the references mb are
  // the exact row maxima; else the first sub-block sets them.
  // Returns true when a row-sum share above kShareMax was seen anywhere in the
  // workgroup (workgroup-uniform).
  template <bool KNOWN_REF>
  __device__ __forceinline__ bool run(int* flags) {
    // the Q fragments are only ever MFMA operands: keep them in AGPRs so the
    // accumulators, which the softmax reads, fit in VGPRs
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(qf[g][ks]));
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[g][dt] = f32x16_t{};
      l[g] = 0.0f;
      lsum[g] = 0.0f;
    }
    share_max = 0.0f;

    // first sub-blocks: S(0) and S(1) (both from K(0)) and the softmax of
    // S(0); without known references the exact max of S(0) becomes the
    // reference of each row
    qk<0>(0);
    qk<1>(1);
    if (mask_from == 0) mask<0>(0);
    if (!KNOWN_REF) {
#pragma unroll
      for (int g = 0; g < 2; ++g) mb[g] = half_swap_max(max16(s[0][g])) * c2;
    }
    weights<0>();
    // S(0), S(1) read K(0)'s slot, which iteration 0 overwrites; those reads
    // have returned (their products are taken), so no fence is needed, and
    // a fenced barrier would wait for the previous tile's output stores
    dev::plain_barrier();

    // Every wavefront runs every step of the workgroup's key range.  Steps
    // past its own diagonal (or past the keys) are masked to -inf: their
    // weights are zero and they add nothing, and a wavefront waiting at the
    // barrier instead would not finish sooner.  The last step's softmax works
    // on a sub-block past the staged tiles; it is masked too.
    // Two loops with one path each (branches between step variants inside
    // one loop cost the register allocator dearly): the iterations whose two
    // sub-blocks lie before this wavefront's first diagonal sub-block, then
    // the rest with the element mask on (a sub-block that needs no mask keeps
    // every key under it).
    int t = 0;
    half8_t kpre[PRE];
    for (; t < n_tiles && 2 * t + 2 < mask_from; ++t) {
      step<1, false, 1, false, true>(2 * t + 1, t, kpre);
      step<0, false, 2, true, false>(2 * t + 2, t, kpre);
      dev::wait_vmcnt0();
      dev::lds_barrier();
    }
    for (; t < n_tiles; ++t) {
      step<1, true, 1, false, true>(2 * t + 1, t, kpre);
      step<0, true, 2, true, false>(2 * t + 2, t, kpre);
      dev::wait_vmcnt0();
      dev::lds_barrier();
    }
    if (KNOWN_REF) return false;
    // the ballot runs with every lane active, the store from one lane
    const bool over = __builtin_amdgcn_ballot_w64(share_max > kShareMax) != 0;
    if (lane == 0) flags[wave] = over;
    dev::lds_barrier();
    return (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
  }

  // First pass of the recomputation: the exact max of every row over its
  // visible keys (QK products only), as the reference mb.
  __device__ __forceinline__ void row_max_pass() {
    stage_prologue();
    float m[2] = {-INFINITY, -INFINITY};
    dev::lds_barrier();
    auto take = [&](auto par, int uu) {
      constexpr int PAR = decltype(par)::value;
      qk<PAR>(uu);
      if (uu >= mask_from) mask<PAR>(uu);
#pragma unroll
      for (int g = 0; g < 2; ++g) m[g] = fmaxf(m[g], max16(s[PAR][g]));
    };
    take(std::integral_constant<int, 0>{}, 0);
    take(std::integral_constant<int, 1>{}, 1);
    dev::lds_barrier();
    for (int t = 0; t < n_tiles; ++t) {
      stage(t);
      if (t + 1 < n_tiles) {
        take(std::integral_constant<int, 0>{}, 2 * t + 2);
        take(std::integral_constant<int, 1>{}, 2 * t + 3);
      }
      dev::wait_vmcnt0();
      dev::lds_barrier();
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) mb[g] = half_swap_max(m[g]) * c2;
  }

  // ---- per query tile ------------------------------------------------------
  // Geometry of query tile qt (the K/V side, same for every tile of the
  // workgroup, is set up once by the kernel).
  __device__ __forceinline__ void setup(const PrefillArgs& a, int qt, int hg) {
    const int q0 = qt * ROWS_WG;
    if (HP == 2) {
      row0[0] = row0[1] = q0 + wave * 32;
      head[0] = 2 * hg;
      head[1] = 2 * hg + 1;
    } else {
      row0[0] = q0 + wave * 64;
      row0[1] = row0[0] + 32;
      head[0] = head[1] = hg;
    }
    const int kv_sub = (a.S_kv + 31) / 32;
    int n_sub_wg;
    if (CAUSAL) {
      mask_from = row0[0] / 32;  // this wavefront's first diagonal sub-block
      n_sub_wg = (min(q0 + ROWS_WG, a.S_q) - 1) / 32 + 1;
    } else {
      mask_from = (a.S_kv % 32) ? kv_sub - 1 : kv_sub;
      n_sub_wg = kv_sub;
    }
    n_tiles = (n_sub_wg + 1) / 2;
  }

  // Q fragments (B operand of S^T = K Q^T: q[row][16*ks + 8*hf + 0..7]),
  // and with COPIES the copies of K(0), V(0), K(1) into LDS; the caller
  // waits for them.  Loads per wavefront: 2 * KS for Q, 2 * K_COPIES +
  // V_COPIES copies.
  template <bool COPIES>
  __device__ __forceinline__ void issue_tile_loads(const PrefillArgs& a) {
    const int64_t q_row_stride = (int64_t)a.H_q * D;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      // rows past S_q load row 0 (their results are never stored)
      const int row = row0[g] + col < a.S_q ? row0[g] + col : 0;
      const _Float16* qp = a.q + ((int64_t)b * a.S_q + row) * q_row_stride + (int64_t)head[g] * D + 8 * hf;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[g][ks] = *reinterpret_cast<const half8_t*>(qp + 16 * ks);
    }
    if (COPIES) {
      copy_tiles(0, 0);
#pragma unroll
      for (int n = 0; n < K_COPIES; ++n) copy(n, 1, 0);
    }
  }
  // ROPE: the position of the first row block's query row, issued ahead of
  // the tile loads (the table rows need it, and loads retire in order); then
  // the norm weights and table rows; the arithmetic once they (and the Q
  // fragments) are in
  __device__ __forceinline__ void rope_pos(const PrefillArgs& a) {
    if constexpr (ROPE) qr.issue_pos(a, b, row0[0] + col);
  }
  __device__ __forceinline__ void rope_rest(const PrefillArgs& a) {
    if constexpr (ROPE) qr.issue_rest(a, hf);
  }
  __device__ __forceinline__ void rope_apply(const PrefillArgs& a) {
    if constexpr (ROPE) {
      q_ok[0] = qr.apply(a, qf[0]);
      if (HP == 1) {
        // the second block's rows (32 further on) in turn
        qr.issue(a, b, row0[1] + col, hf);
      }
      q_ok[1] = qr.apply(a, qf[1]);
    }
  }

  // the whole query tile: first pass, and the recomputation when a
  // row-sum share overflowed
  __device__ __forceinline__ void compute(int* flags) {
    if (run<false>(flags)) {
      row_max_pass();
      stage_prologue();
      dev::lds_barrier();
      run<true>(flags);
    }
  }

  // Epilogue of a query tile (rows rows0, heads heads): normalise, round to
  // fp16, and store whole rows through this wavefront's part of the output
  // LDS.  Returns true when every row was stored (16 stores per wavefront,
  // the count the caller may wait on), false for a ragged last tile.
  __device__ __forceinline__ bool epilogue(const PrefillArgs& a, const int (&rows0)[2], const int (&heads)[2]) {
    if (rows0[0] >= a.S_q) return false;
    const int64_t q_row_stride = (int64_t)a.H_q * D;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float inv = 1.0f / half_swap_add(l[g]);
      _Float16* ot = osmem + (wave * 2 + g) * 32 * OROW;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          half4_t out;
#pragma unroll
          for (int j = 0; j < 4; ++j) out[j] = (_Float16)(o[g][dt][rg * 4 + j] * inv);
          if (ROPE && !q_ok[g]) out = __builtin_bit_cast(half4_t, 0x7e007e007e007e00ull);  // quiet NaN bits
          *reinterpret_cast<half4_t*>(ot + col * OROW + dt * 32 + rg * 8 + hf * 4) = out;
        }
      }
    }
    // the lanes read rows that other lanes of this wavefront wrote: a
    // wavefront's LDS instructions execute in issue order, so only the
    // compiler must keep the reads after the writes (a fence would also wait
    // for the next tile's loads, issued before this epilogue)
    asm volatile("" ::: "memory");
    constexpr int PIECES = D / 8;          // 16-byte pieces per row
    constexpr int ROWS_PER = 64 / PIECES;  // rows per 64-lane store
    const int pr = lane / PIECES, pc = lane % PIECES;
    const bool full = rows0[1] + 31 < a.S_q;
    // all of a block's row pieces are read back before its stores go out, so
    // the LDS reads overlap instead of each waiting before its own store
    constexpr int PER_G = 32 / ROWS_PER;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const _Float16* ot = osmem + (wave * 2 + g) * 32 * OROW;
      half8_t v8[PER_G];
#pragma unroll
      for (int i = 0; i < PER_G; ++i) v8[i] = *reinterpret_cast<const half8_t*>(ot + (i * ROWS_PER + pr) * OROW + 8 * pc);
      // non-temporal stores: nothing in this launch reads the output back,
      // so it need not stay in L2 next to the K/V rows, nor be held there
      // until the write-back at the kernel's end
#pragma unroll
      for (int i = 0; i < PER_G; ++i) {
        const int row = rows0[g] + i * ROWS_PER + pr;
        if (full || row < a.S_q)
          __builtin_nontemporal_store(
              v8[i], reinterpret_cast<half8_t*>(a.o + ((int64_t)b * a.S_q + row) * q_row_stride + (int64_t)heads[g] * D + 8 * pc));
      }
    }
    return full;
  }
};

// Work unit of a workgroup: query tiles qt and n_qtiles-1-qt of one (head
// group, batch).  Under the causal mask tile i costs i+1 units of keys, so
// every pair costs the same and the grid has no long-tile tail; an odd
// middle tile runs alone.  Both tiles read the same kv head, so the K/V side
// is set up once.  The second tile's Q loads and first K/V copies go out
// before the first tile's epilogue, which then overlaps their latency.
template <bool CAUSAL, int HP, bool ROPE>
__global__ __launch_bounds__(kThreads, 1) void prefill_dual_kernel(PrefillArgs a) {
  using W = Dual<CAUSAL, HP, ROPE>;
  constexpr int D = W::D;
  __shared__ __attribute__((aligned(16))) _Float16 smem[W::SMEM_HALFS];
  __shared__ __attribute__((aligned(16))) _Float16 osmem[W::OUT_LDS];
  __shared__ int flags[kWaves];
  const int head_groups = a.H_q / HP;
  const int combos = head_groups * a.B;
  // the raw work-group / work-item id builtins: this file is built without
  // NaN semantics, so the device library's blockIdx / threadIdx helpers
  // (built with them) are not inlined and would become calls
  const int id = (int)__builtin_amdgcn_workgroup_id_x();
  const int pair = id / combos;
  const int rem = id - pair * combos;
  const int hg = rem % head_groups;
  const int lo = pair, hi = a.n_qtiles - 1 - pair;

  W w;
  w.smem = smem;
  w.osmem = osmem;
  w.tid = (int)__builtin_amdgcn_workitem_id_x();
  w.lane = w.tid & 63;
  // the wavefront index is uniform; readfirstlane lets the compiler see that,
  // so everything derived from it (row blocks, sub-block counts) is scalar
  w.wave = __builtin_amdgcn_readfirstlane(w.tid >> 6);
  w.col = w.lane & 31;
  w.hf = w.lane >> 5;
  w.S_kv = a.S_kv;
  w.b = rem / head_groups;
  w.c2 = a.scale_log2;
  w.k_lane = w.col * W::KROW + 8 * w.hf;
  w.v_lane = dev::pv_lane_offset<W::VROW>(w.lane);
  const int g_kv = (int)(((int64_t)hg * HP * a.H_kv) / a.H_q);
  const int64_t kv_row_stride = (int64_t)a.H_kv * D;
  const _Float16* kbase = a.k + (int64_t)w.b * a.S_kv * kv_row_stride + (int64_t)g_kv * D;
  const _Float16* vbase = a.v + (int64_t)w.b * a.S_kv * kv_row_stride + (int64_t)g_kv * D;
  w.row_bytes = (uint32_t)kv_row_stride * 2u;
  const int range = (int)((uint32_t)a.S_kv * w.row_bytes);  // host guarantees < 2^31
  w.krsrc = dev::make_rsrc(kbase, range);
  w.vrsrc = dev::make_rsrc(vbase, range);
  w.template copy_offsets<W::KROW>(w.k_off, W::K_COPIES);
  w.template copy_offsets<W::VROW>(w.v_off, W::V_COPIES);
  w.copy_dsts();

  w.setup(a, hi, hg);
  w.par0 = 0;
  // both tiles read the same K/V rows from key 0 on: the first pass's last
  // two iterations copy the second tile's K(0), V(0), K(1) (see next_base)
  w.next_base = lo < hi ? w.n_tiles : 0x40000000;
  w.rope_pos(a);
  w.template issue_tile_loads<true>(a);
  w.rope_rest(a);
  dev::wait_vmcnt0();
  w.rope_apply(a);
  dev::lds_barrier();
  w.compute(flags);
  if (lo < hi) {
    // K(0), V(0), K(1) of the second tile are in LDS already (the first
    // pass's last iterations copied them, in the slots after its own last
    // tiles) and the Q fragments are dead: start the second tile's Q loads,
    // then store the first tile
    const int rows0[2] = {w.row0[0], w.row0[1]};
    const int heads[2] = {w.head[0], w.head[1]};
    const int n_first = w.n_tiles;
    w.setup(a, lo, hg);
    w.par0 = n_first & 1;
    w.next_base = 0x40000000;
    w.rope_pos(a);  // one register, held across the epilogue
    w.template issue_tile_loads<false>(a);
    const bool full = w.epilogue(a, rows0, heads);
    if (ROPE) {
      // the rest of the rotation's loads go out once the first tile's
      // outputs (and their registers) are gone (the position is in by now);
      // loads retire in order, so waiting for them waits for the 16 output
      // stores as well
      w.rope_rest(a);
      dev::wait_vmcnt0();
      w.rope_apply(a);
    } else if (full) {
      dev::wait_vmcnt<2 * (D / 8) * 32 / 64>();  // its 16 stores may stay in flight
    } else {
      dev::wait_vmcnt0();
    }
    dev::plain_barrier();
    w.compute(flags);
  }
  w.epilogue(a, w.row0, w.head);
}

template <bool CAUSAL, int HP, bool ROPE>
hipError_t launch_dual_t(const PrefillArgs& a_in, hipStream_t stream) {
  PrefillArgs a = a_in;
  constexpr int ROWS_WG = Dual<CAUSAL, HP, ROPE>::ROWS_WG;
  a.n_qtiles = (a.S_q + ROWS_WG - 1) / ROWS_WG;
  const int64_t blocks = (int64_t)((a.n_qtiles + 1) / 2) * (a.H_q / HP) * a.B;
  void* kargs[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&prefill_dual_kernel<CAUSAL, HP, ROPE>),
                         dim3((unsigned)blocks), dim3(kThreads), kargs, 0, stream);
}

template <bool ROPE>
hipError_t launch_dual_r(const PrefillArgs& a, bool causal, hipStream_t stream) {
  const bool pair = ((a.H_q / a.H_kv) % 2) == 0;
  if (causal) return pair ? launch_dual_t<true, 2, ROPE>(a, stream) : launch_dual_t<true, 1, ROPE>(a, stream);
  return pair ? launch_dual_t<false, 2, ROPE>(a, stream) : launch_dual_t<false, 1, ROPE>(a, stream);
}

}  // namespace

hipError_t launch_prefill_dual(const PrefillArgs& a, bool causal, hipStream_t stream) {
  return a.cos_table ? launch_dual_r<true>(a, causal, stream) : launch_dual_r<false>(a, causal, stream);
}

}  // namespace attn
