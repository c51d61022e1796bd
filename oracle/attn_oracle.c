/*
 * attn_oracle.c -- plain fp64 CPU oracle for scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header or constant with the HIP library, and the HIP library never calls it.
 *
 * What it computes (the plain definition; the pages' online-softmax kernels
 * reach the same value up to rounding order):
 *
 *   For one query row q and its visible key set J:
 *     s_j  = (sum_d q_d * k_{j,d}) / sqrt(D)                 j in J
 *     m    = max_j s_j
 *     P_j  = exp(s_j - m) / sum_{j' in J} exp(s_j' - m)
 *     o_d  = sum_{j in J} P_j * v_{j,d}
 *
 *   Prefill ("Tutorial: Adding a New Kernel to RL.cu", the attention.cuh
 *   listing, prefill section; and the CPU reference in test_attention.cu):
 *     Q, K, V laid out [B, S, H, D]; O laid out [B, S_q, H_q, D].
 *     GQA: H_q % H_kv == 0 and kv head g = (h * H_kv) / H_q (integer division).
 *     Causal: row i sees keys 0..i; non-causal: all S_kv keys.
 *
 *   Paged decode (same page, attention.cuh listing, decode section; and the
 *   "KV Cache design" section of the GRPO-CUDA project memory page):
 *     q [num_seqs, H_q, D]; caches [num_blocks, H_kv, block_size, D];
 *     block_tables [num_seqs, max_blocks_per_seq] maps logical block -> physical;
 *     seq_lens[s] counts every context token including the new one.
 *     Token t of sequence s lives at cache[bt[s][t / bs], g, t % bs, :].
 *     All seq_lens[s] tokens are visible, in logical order.
 *
 * Readings taken where the pages are silent (each listed in the design notes):
 *   - causal with S_q != S_kv is undefined on the pages: rejected (-1).
 *   - seq_len <= 0 is a precondition violation on the pages; the oracle writes
 *     a zero row for it, and the same is documented for the GPU path.
 *   - inputs are IEEE binary16 bit patterns, decoded exactly to fp64 here; the
 *     scale is 1/sqrt(D) in fp64.
 *
 * Every function below works one output row at a time, in the order of the
 * definition above: gather the visible keys, score them, take the max,
 * exponentiate, normalise, and sum the weighted value rows.  OpenMP only
 * distributes independent rows over threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- IEEE 754 binary16 -> fp64 (exact) -------------------------------- */
/* sign(1) | exponent(5, bias 15) | fraction(10).
 * normal:    (1 + f/1024) * 2^(e-15) = (1024 + f) * 2^(e-25)
 * subnormal: (f/1024) * 2^-14        = f * 2^-24
 * e == 31:   infinity (f == 0) or NaN.                                       */
static double half_bits_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1f;
  const int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

static double g_h2d[65536];
static int g_h2d_ready = 0;

static void init_table(void) {
  if (g_h2d_ready) return;
  for (int i = 0; i < 65536; ++i) g_h2d[i] = half_bits_to_double((uint16_t)i);
  g_h2d_ready = 1;
}

/* Exposed so the tests can check the decoder against an independent one. */
double oracle_half_to_double(uint16_t h) { return half_bits_to_double(h); }

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- one softmax-attention row ----------------------------------------- */
/* q:      D decoded query values
 * krow/vrow: n pointers to the visible key / value rows (binary16 bits)
 * scores: scratch of n doubles
 * out:    D outputs; *lse receives m + log(sum exp(s - m)) (natural log)      */
static void attend_row(const double* q, const uint16_t* const* krow,
                       const uint16_t* const* vrow, int64_t n, int D,
                       double* scores, double* out, double* lse) {
  if (n <= 0) {
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (lse) *lse = -INFINITY;
    return;
  }
  const double scale = 1.0 / sqrt((double)D);

  /* scores s_j = (q . k_j) / sqrt(D) */
  for (int64_t j = 0; j < n; ++j) {
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += q[d] * g_h2d[krow[j][d]];
    scores[j] = dot * scale;
  }

  /* m = max_j s_j */
  double m = scores[0];
  for (int64_t j = 1; j < n; ++j)
    if (scores[j] > m) m = scores[j];

  /* exp(s_j - m) and their sum */
  double z = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    scores[j] = exp(scores[j] - m);
    z += scores[j];
  }

  /* P_j = exp(s_j - m) / z */
  for (int64_t j = 0; j < n; ++j) scores[j] /= z;

  /* o = sum_j P_j v_j */
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double p = scores[j];
    for (int d = 0; d < D; ++d) out[d] += p * g_h2d[vrow[j][d]];
  }
  if (lse) *lse = m + log(z);
}

/* ---- prefill ----------------------------------------------------------- */
/* q [B,S_q,H_q,D], k/v [B,S_kv,H_kv,D] binary16 bits, row-major.
 * rows: optional list of n_rows flat row ids r = (b*S_q + i)*H_q + h; when
 *       NULL every row is computed and out is [B,S_q,H_q,D] (fp64), else out
 *       is [n_rows, D] in list order.
 * lse:  optional, one value per computed row.
 * Returns 0, or -1 on invalid arguments.                                     */
int oracle_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   double* out, int B, int S_q, int S_kv, int H_q, int H_kv,
                   int D, int causal, const int64_t* rows, int64_t n_rows,
                   double* lse) {
  if (!q || !k || !v || !out) return -1;
  if (B <= 0 || S_q <= 0 || S_kv <= 0 || H_q <= 0 || H_kv <= 0 || D <= 0)
    return -1;
  if (H_q % H_kv != 0) return -1;
  if (causal && S_q != S_kv) return -1;
  init_table();

  const int64_t total = (int64_t)B * S_q * H_q;
  const int64_t count = rows ? n_rows : total;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= total) return -1;

  int err = 0;
#pragma omp parallel
  {
    double* qd = (double*)malloc(sizeof(double) * D);
    double* scores = (double*)malloc(sizeof(double) * (size_t)S_kv);
    const uint16_t** kr = (const uint16_t**)malloc(sizeof(void*) * (size_t)S_kv);
    const uint16_t** vr = (const uint16_t**)malloc(sizeof(void*) * (size_t)S_kv);
    if (!qd || !scores || !kr || !vr) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 8)
      for (int64_t idx = 0; idx < count; ++idx) {
        const int64_t r = rows ? rows[idx] : idx;
        const int h = (int)(r % H_q);
        const int64_t bi = r / H_q;
        const int i = (int)(bi % S_q);
        const int b = (int)(bi / S_q);
        const int g = (int)(((int64_t)h * H_kv) / H_q); /* GQA kv head */

        const uint16_t* qrow = q + (((int64_t)b * S_q + i) * H_q + h) * D;
        for (int d = 0; d < D; ++d) qd[d] = g_h2d[qrow[d]];

        const int64_t n = causal ? (int64_t)i + 1 : (int64_t)S_kv; /* visible keys */
        for (int64_t j = 0; j < n; ++j) {
          const int64_t off = (((int64_t)b * S_kv + j) * H_kv + g) * D;
          kr[j] = k + off;
          vr[j] = v + off;
        }
        attend_row(qd, kr, vr, n, D, scores, out + idx * D, lse ? lse + idx : NULL);
      }
    }
    free(qd);
    free(scores);
    free((void*)kr);
    free((void*)vr);
  }
  return err ? -1 : 0;
}

/* ---- paged decode ------------------------------------------------------ */
/* q [num_seqs,H_q,D]; k_cache/v_cache [num_blocks,H_kv,block_size,D];
 * block_tables int32 [num_seqs,max_blocks_per_seq]; seq_lens int32 [num_seqs].
 * seqs: optional list of n_seqs sequence ids to compute; out is then
 *       [n_seqs,H_q,D], else [num_seqs,H_q,D].
 * Returns 0, -1 on invalid arguments, -2 if a table entry that a visible
 * token needs is outside [0, num_blocks) or a seq_len exceeds the table.     */
int oracle_decode_paged(const uint16_t* q, const uint16_t* k_cache,
                        const uint16_t* v_cache, const int32_t* block_tables,
                        const int32_t* seq_lens, double* out, int num_seqs,
                        int H_q, int H_kv, int D, int max_blocks_per_seq,
                        int block_size, int64_t num_blocks, const int64_t* seqs,
                        int64_t n_seqs, double* lse) {
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out) return -1;
  if (num_seqs <= 0 || H_q <= 0 || H_kv <= 0 || D <= 0 ||
      max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0)
    return -1;
  if (H_q % H_kv != 0) return -1;
  init_table();

  const int64_t count = seqs ? n_seqs : num_seqs;
  /* validate everything the rows below will touch */
  for (int64_t idx = 0; idx < count; ++idx) {
    const int64_t s = seqs ? seqs[idx] : idx;
    if (s < 0 || s >= num_seqs) return -1;
    const int64_t L = seq_lens[s];
    if (L > (int64_t)max_blocks_per_seq * block_size) return -2;
    const int64_t nb = L > 0 ? (L + block_size - 1) / block_size : 0;
    for (int64_t lb = 0; lb < nb; ++lb) {
      const int32_t phys = block_tables[s * (int64_t)max_blocks_per_seq + lb];
      if (phys < 0 || phys >= num_blocks) return -2;
    }
  }

  int64_t max_len = 1;
  for (int64_t idx = 0; idx < count; ++idx) {
    const int64_t s = seqs ? seqs[idx] : idx;
    if (seq_lens[s] > max_len) max_len = seq_lens[s];
  }

  int err = 0;
#pragma omp parallel
  {
    double* qd = (double*)malloc(sizeof(double) * D);
    double* scores = (double*)malloc(sizeof(double) * (size_t)max_len);
    const uint16_t** kr = (const uint16_t**)malloc(sizeof(void*) * (size_t)max_len);
    const uint16_t** vr = (const uint16_t**)malloc(sizeof(void*) * (size_t)max_len);
    if (!qd || !scores || !kr || !vr) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 1) collapse(2)
      for (int64_t idx = 0; idx < count; ++idx) {
        for (int h = 0; h < H_q; ++h) {
          const int64_t s = seqs ? seqs[idx] : idx;
          const int g = (int)(((int64_t)h * H_kv) / H_q); /* GQA kv head */
          const uint16_t* qrow = q + ((int64_t)s * H_q + h) * D;
          for (int d = 0; d < D; ++d) qd[d] = g_h2d[qrow[d]];

          const int64_t L = seq_lens[s] > 0 ? seq_lens[s] : 0;
          for (int64_t t = 0; t < L; ++t) {
            const int64_t phys =
                block_tables[s * (int64_t)max_blocks_per_seq + t / block_size];
            const int64_t off =
                ((phys * H_kv + g) * (int64_t)block_size + t % block_size) * D;
            kr[t] = k_cache + off;
            vr[t] = v_cache + off;
          }
          const int64_t o = idx * H_q + h;
          attend_row(qd, kr, vr, L, D, scores, out + o * D, lse ? lse + o : NULL);
        }
      }
    }
    free(qd);
    free(scores);
    free((void*)kr);
    free((void*)vr);
  }
  return err ? -1 : 0;
}

/* ---- paged KV append ---------------------------------------------------- */
/* The write side of the paged cache ("GRPO-CUDA Project Memory", "KV Cache
 * design" section: slot_mapping[token] = physical_block * block_size +
 * in-block offset, int64; "Known bugs fixed": padding tokens carry slot -1
 * and are skipped).  Token i's rows k_new[i, h, :] and v_new[i, h, :] (new
 * keys/values laid out [num_tokens, H_kv, D]) are copied to
 * cache[slot / block_size, h, slot % block_size, :] for every head h.
 * Readings: any slot outside [0, num_blocks * block_size) is skipped like -1;
 * tokens are applied in order, so a repeated slot keeps the last token's rows
 * (the GPU leaves repeated slots unspecified and no test uses them).
 * Returns the number of tokens written, or -1 on invalid arguments.          */
int64_t oracle_kv_append(const uint16_t* k_new, const uint16_t* v_new,
                         uint16_t* k_cache, uint16_t* v_cache,
                         const int64_t* slot_mapping, int64_t num_tokens,
                         int H_kv, int D, int block_size, int64_t num_blocks) {
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return -1;
  if (num_tokens < 0 || H_kv <= 0 || D <= 0 || block_size <= 0 || num_blocks <= 0)
    return -1;
  const int64_t capacity = num_blocks * (int64_t)block_size;
  int64_t written = 0;
  for (int64_t i = 0; i < num_tokens; ++i) {
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= capacity) continue;
    const int64_t block = slot / block_size;
    const int64_t off = slot % block_size;
    for (int h = 0; h < H_kv; ++h) {
      const uint16_t* ks = k_new + (i * H_kv + h) * (int64_t)D;
      const uint16_t* vs = v_new + (i * H_kv + h) * (int64_t)D;
      uint16_t* kd = k_cache + ((block * H_kv + h) * block_size + off) * (int64_t)D;
      uint16_t* vd = v_cache + ((block * H_kv + h) * block_size + off) * (int64_t)D;
      for (int d = 0; d < D; ++d) {
        kd[d] = ks[d];
        vd[d] = vs[d];
      }
    }
    ++written;
  }
  return written;
}

/* ---- RoPE table ------------------------------------------------------------ */
/* "GRPO-CUDA Project Memory", "RoPE design": a table of [max_seq_len, D/2]
 * entries precomputed once and read by the rotation.  Pair i of a head
 * turns by the angle pos * inv_freq[i], inv_freq[i] = theta^(-2i/D) (the
 * frequency the cross-attention trace spells 1/(base^(arange(0,D,2)/D))).
 * The pages do not give theta: it is a parameter (Qwen3 configurations use
 * 1e6; 1e4 is the classic value).  Here the angle, cosine and sine are fp64.
 * Returns 0, or -1 on invalid arguments.                                     */
int oracle_rope_table(double* cos_out, double* sin_out, int max_pos, int D, double theta) {
  if (!cos_out || !sin_out || max_pos <= 0 || D <= 0 || (D & 1) || !(theta > 0.0)) return -1;
  const int half = D / 2;
  for (int p = 0; p < max_pos; ++p) {
    for (int i = 0; i < half; ++i) {
      const double inv_freq = pow(theta, -2.0 * (double)i / (double)D);
      const double angle = (double)p * inv_freq;
      cos_out[(int64_t)p * half + i] = cos(angle);
      sin_out[(int64_t)p * half + i] = sin(angle);
    }
  }
  return 0;
}

/* ---- QK-norm + NeoX RoPE ------------------------------------------------- */
/* Qwen3 order ("GRPO-CUDA Project Memory", "Qwen3 key dims" and "Qwen3-
 * Specific Notes"): RMSNorm over each head's D values first, then the
 * rotary embedding.
 *   RMSNorm (per token and head, eps given; the pages' models use 1e-6):
 *     y_d = x_d / sqrt((1/D) * sum_e x_e^2 + eps) * w_d
 *   NeoX split-half rotation ("RoPE design"), for i in [0, D/2):
 *     out_i       = y_i * cos_i - y_{i+D/2} * sin_i
 *     out_{i+D/2} = y_{i+D/2} * cos_i + y_i * sin_i
 *   with cos_i, sin_i the table entries of the token's position.
 * x: [n_tokens, H, D] binary16; weight: [D] binary16, or NULL for rotation
 * only; positions: int32 [n_tokens]; tables: fp64 [max_pos, D/2].
 * Reading: a position outside [0, max_pos) has no table row; the token's
 * rows come out NaN (the GPU path does the same).  The norm and the rotation
 * are evaluated without intermediate rounding (the fused GPU kernel keeps
 * fp32 between them).
 * Returns 0, or -1 on invalid arguments.                                     */
int oracle_qk_norm_rope(const uint16_t* x, const uint16_t* weight, const int32_t* positions,
                        const double* cos_t, const double* sin_t, int64_t n_tokens, int H,
                        int D, int max_pos, double eps, double* out) {
  if (!x || !positions || !cos_t || !sin_t || !out) return -1;
  if (n_tokens < 0 || H <= 0 || D <= 0 || (D & 1) || max_pos <= 0 || eps < 0.0) return -1;
  const int half = D / 2;
  double* y = (double*)malloc(sizeof(double) * (size_t)D);
  if (!y) return -1;
  for (int64_t t = 0; t < n_tokens; ++t) {
    const int32_t pos = positions[t];
    for (int h = 0; h < H; ++h) {
      const uint16_t* xr = x + (t * H + h) * (int64_t)D;
      double* o = out + (t * H + h) * (int64_t)D;
      if (pos < 0 || pos >= max_pos) {
        for (int d = 0; d < D; ++d) o[d] = NAN;
        continue;
      }
      for (int d = 0; d < D; ++d) y[d] = half_bits_to_double(xr[d]);
      if (weight) {
        double ss = 0.0;
        for (int d = 0; d < D; ++d) ss += y[d] * y[d];
        const double r = sqrt(ss / (double)D + eps);
        for (int d = 0; d < D; ++d) y[d] = y[d] / r * half_bits_to_double(weight[d]);
      }
      const double* c = cos_t + (int64_t)pos * half;
      const double* s = sin_t + (int64_t)pos * half;
      for (int i = 0; i < half; ++i) {
        o[i] = y[i] * c[i] - y[i + half] * s[i];
        o[i + half] = y[i + half] * c[i] + y[i] * s[i];
      }
    }
  }
  free(y);
  return 0;
}

/* ---- interleaved-pair rotary embedding ---------------------------------- */
/* The rotation of the cross-attention trace (POPCORNBENCH "Kimi-K2.6" page,
 * its RoPE discussion): adjacent pairs (2j, 2j+1) of every head turn by the
 * angle pos * base^(-2j/D), pos being the row's index in its sequence:
 *     r_{2j}   = u_{2j} cos - u_{2j+1} sin
 *     r_{2j+1} = u_{2j} sin + u_{2j+1} cos
 * x: [B, T, H, D] binary16 (row t of every batch entry is at position t);
 * out: fp64 [B, T, H, D].  The non-causal cross-attention workload feeds Q
 * and K through this rotation (base 10000) before attention; the fp64
 * result is rounded to binary16 by the caller.
 * Returns 0, or -1 on invalid arguments.                                     */
int oracle_rope_interleaved(const uint16_t* x, int64_t B, int64_t T, int H, int D, double base,
                            double* out) {
  if (!x || !out || B < 0 || T < 0 || H <= 0 || D <= 0 || (D & 1) || !(base > 0.0)) return -1;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t = 0; t < T; ++t) {
      for (int h = 0; h < H; ++h) {
        const int64_t row = ((b * T + t) * H + h) * (int64_t)D;
        for (int j = 0; j < D / 2; ++j) {
          const double ang = (double)t * pow(base, -2.0 * (double)j / (double)D);
          const double c = cos(ang), sn = sin(ang);
          const double u0 = half_bits_to_double(x[row + 2 * j]);
          const double u1 = half_bits_to_double(x[row + 2 * j + 1]);
          out[row + 2 * j] = u0 * c - u1 * sn;
          out[row + 2 * j + 1] = u0 * sn + u1 * c;
        }
      }
    }
  }
  return 0;
}

/* ---- cross-attention module with RoPE --------------------------------------- */
/* The module of the cross-attention trace (POPCORNBENCH "Kimi-K2.6" page, the
 * problem statement and its nn.Linear notes): one layer of multi-head
 * cross-attention with rotary embeddings, no bias anywhere, dropout p = 0.
 *   Q = x_q W_q^T   [B, T_q, dim]     K = x_kv W_k^T, V = x_kv W_v^T [B, T_k, dim]
 *   head h is columns h*D .. h*D+D-1 (D = dim / H)
 *   RoPE on Q and K, adjacent pairs (2j, 2j+1) turned by pos * base^(-2j/D),
 *     pos = the row's index in its sequence (0..T-1):
 *       r_{2j}   = u_{2j} cos - u_{2j+1} sin
 *       r_{2j+1} = u_{2j} sin + u_{2j+1} cos
 *   A_h = softmax(Q_h K_h^T / sqrt(D)) V_h     (no mask)
 *   out = concat_h(A_h) W_o^T   [B, T_q, dim]
 * x_q, x_kv and the four [dim, dim] weights (nn.Linear layout [out, in]) are
 * binary16; every intermediate here is fp64.
 * Returns 0, or -1 on invalid arguments.                                     */
int oracle_cross_attention(const uint16_t* x_q, const uint16_t* x_kv, const uint16_t* w_q,
                           const uint16_t* w_k, const uint16_t* w_v, const uint16_t* w_o,
                           int B, int T_q, int T_k, int dim, int H, double base, double* out) {
  if (!x_q || !x_kv || !w_q || !w_k || !w_v || !w_o || !out) return -1;
  if (B <= 0 || T_q <= 0 || T_k <= 0 || dim <= 0 || H <= 0 || dim % H || ((dim / H) & 1) ||
      !(base > 0.0))
    return -1;
  const int D = dim / H;
  const int64_t nq = (int64_t)B * T_q, nk = (int64_t)B * T_k;
  double* Q = (double*)malloc(sizeof(double) * nq * dim);
  double* K = (double*)malloc(sizeof(double) * nk * dim);
  double* V = (double*)malloc(sizeof(double) * nk * dim);
  double* A = (double*)malloc(sizeof(double) * nq * dim);
  if (!Q || !K || !V || !A) {
    free(Q); free(K); free(V); free(A);
    return -1;
  }
  /* projections: y[r][c] = sum_e x[r][e] * W[c][e] */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nq + nk; ++r) {
    for (int c = 0; c < dim; ++c) {
      if (r < nq) {
        double s = 0.0;
        for (int e = 0; e < dim; ++e)
          s += half_bits_to_double(x_q[r * dim + e]) * half_bits_to_double(w_q[(int64_t)c * dim + e]);
        Q[r * dim + c] = s;
      } else {
        const int64_t rk = r - nq;
        double sk = 0.0, sv = 0.0;
        for (int e = 0; e < dim; ++e) {
          const double xe = half_bits_to_double(x_kv[rk * dim + e]);
          sk += xe * half_bits_to_double(w_k[(int64_t)c * dim + e]);
          sv += xe * half_bits_to_double(w_v[(int64_t)c * dim + e]);
        }
        K[rk * dim + c] = sk;
        V[rk * dim + c] = sv;
      }
    }
  }
  /* rotary embedding on Q (positions 0..T_q-1) and K (0..T_k-1) */
  for (int which = 0; which < 2; ++which) {
    double* X = which ? K : Q;
    const int T = which ? T_k : T_q;
    const int64_t rows = which ? nk : nq;
    for (int64_t r = 0; r < rows; ++r) {
      const double pos = (double)(r % T);
      for (int h = 0; h < H; ++h) {
        double* u = X + r * dim + (int64_t)h * D;
        for (int j = 0; j < D / 2; ++j) {
          const double ang = pos * pow(base, -2.0 * (double)j / (double)D);
          const double c = cos(ang), s = sin(ang);
          const double a = u[2 * j], b = u[2 * j + 1];
          u[2 * j] = a * c - b * s;
          u[2 * j + 1] = a * s + b * c;
        }
      }
    }
  }
  /* attention per (batch, head, query row), no mask */
  const double scale = pow((double)D, -0.5);
#pragma omp parallel for schedule(static)
  for (int64_t qi = 0; qi < nq * H; ++qi) {
    const int64_t r = qi / H;
    const int h = (int)(qi % H);
    const int64_t b = r / T_q;
    double* sc = (double*)malloc(sizeof(double) * T_k);
    const double* q = Q + r * dim + (int64_t)h * D;
    double m = -INFINITY;
    for (int j = 0; j < T_k; ++j) {
      const double* k = K + (b * T_k + j) * dim + (int64_t)h * D;
      double s = 0.0;
      for (int d = 0; d < D; ++d) s += q[d] * k[d];
      sc[j] = s * scale;
      if (sc[j] > m) m = sc[j];
    }
    double z = 0.0;
    for (int j = 0; j < T_k; ++j) {
      sc[j] = exp(sc[j] - m);
      z += sc[j];
    }
    double* a = A + r * dim + (int64_t)h * D;
    for (int d = 0; d < D; ++d) a[d] = 0.0;
    for (int j = 0; j < T_k; ++j) {
      const double* v = V + (b * T_k + j) * dim + (int64_t)h * D;
      const double p = sc[j] / z;
      for (int d = 0; d < D; ++d) a[d] += p * v[d];
    }
    free(sc);
  }
  /* output projection */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nq; ++r) {
    for (int c = 0; c < dim; ++c) {
      double s = 0.0;
      for (int e = 0; e < dim; ++e) s += A[r * dim + e] * half_bits_to_double(w_o[(int64_t)c * dim + e]);
      out[r * dim + c] = s;
    }
  }
  free(Q); free(K); free(V); free(A);
  return 0;
}
