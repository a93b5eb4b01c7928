/*
 * fa_oracle.c -- plain, slow, fp64 reference for exact softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library
 * and its Python binding) may link, load or call this file; only the tests,
 * the smoke check and the benchmark's CPU-baseline leg use it.  It shares
 * no code, header, table or conversion routine with the GPU path.
 *
 * What it computes (per batch b, head h, query row i):
 *   s_ij = scale * sum_k q_ik * k_jk                for every visible key j
 *   m_i  = max_j s_ij                                (pass 1)
 *   l_i  = sum_j exp(s_ij - m_i)                     (pass 2)
 *   o_i  = sum_j exp(s_ij - m_i) / l_i * v_j         (pass 3)
 *   lse_i = m_i + ln(l_i)
 * This is the "standard attention" definition the pages give: the scaled
 * dot products, a numerically safe softmax computed in three passes over a
 * row (max, sum of exponentials, normalise), and the weighted sum of value
 * rows.  Sources:
 *   - "FlashAttention dissected" (leren.llmnet.nl), section "The mathematical
 *     breakthrough": the softmax of a row, and the pseudocode's score
 *     S = Q K^T / sqrt(d);
 *   - "How Did I Write My First FlashAttention Kernel in CUDA?", the passage
 *     on why softmax normally needs three passes over the data;
 *   - "CUDA Flash Attention: Online Softmax with Shared Memory Tiling"
 *     (GitHub README), section "Kernel 1 -- Naive Attention": one score per
 *     (i, j), a row-wise max / exp / normalise, then O_i = sum_j P_ij V_j.
 * The visible set is every key j in [0, N), or j <= i when causal (key j > i
 * masked, the causal convention of the workload definitions; the pages
 * themselves do not define a causal mask).  A row with no visible key gets
 * o_i = 0 and lse_i = -inf.
 *
 * The general entry point also takes separate query and key lengths and
 * grouped K/V heads ("FlashAttention dissected", section "Interaction with
 * the KV cache during inference": a decoding step has N_q = 1 query against
 * N_kv cached keys, and several query heads may share one K/V head).  Query
 * head h reads K/V head h / (H / H_kv).  The pages fix no causal alignment
 * for N_q != N_kv; the reading taken is that query row i stands at key
 * position N_kv - N_q + i (the rows are the newest tokens), so key j is
 * visible when j <= i + N_kv - N_q.  For N_q = N_kv this is the mask above.
 *
 * oracle_bwd_f64 gives the gradients of L = sum(dO * O) with respect to Q, K
 * and V for a given upstream gradient dO (see that function).
 *
 * oracle_combine_f64 merges results computed over disjoint key ranges,
 * following the normalised update of "How Did I Write My First
 * FlashAttention Kernel in CUDA?", pseudo-algorithm steps 4 and 5, applied
 * to whole ranges (see that function).
 *
 * Inputs are read in their stored type and widened exactly to double:
 *   fp32  by a C cast;
 *   bf16  by placing the 16 stored bits above 16 zero bits of an fp32;
 *   fp16  by decoding sign / 5-bit exponent / 10-bit fraction (IEEE-754
 *         binary16) here, including subnormals, infinities and NaN.
 * All arithmetic after widening is double.  The N x N score matrix is never
 * formed: one row of scores (at most N doubles) lives per worker thread.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2 };

/* ---- exact widening of the stored element types ------------------------- */

static double widen_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double widen_f16(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int expo = (bits >> 10) & 0x1f;
  int frac = bits & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 * 2^-10 */
  } else if (expo == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp(1.0 + (double)frac / 1024.0, expo - 15);
  }
  return sign ? -mag : mag;
}

/* widen_f16 of every 16-bit pattern, filled once: the decode above costs an
 * ldexp per element, and the passes below widen each K/V element once per
 * query row. */
static double f16_table[1 << 16];
static pthread_once_t f16_once = PTHREAD_ONCE_INIT;

static void fill_f16_table(void) {
  for (uint32_t u = 0; u < (1u << 16); ++u) f16_table[u] = widen_f16((uint16_t)u);
}

static void widen_tables_ready(void) { pthread_once(&f16_once, fill_f16_table); }

static double load_elem(const void* base, int dtype, int64_t idx) {
  switch (dtype) {
    case ORACLE_F32: return (double)((const float*)base)[idx];
    case ORACLE_BF16: return widen_bf16(((const uint16_t*)base)[idx]);
    default: return f16_table[((const uint16_t*)base)[idx]];
  }
}

/* Exposed so that the tests can check the widening against independent
 * library conversions over every 16-bit pattern. */
double oracle_widen(int dtype, uint32_t bits) {
  if (dtype == ORACLE_BF16) return widen_bf16((uint16_t)bits);
  if (dtype == ORACLE_F16) return widen_f16((uint16_t)bits);
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* ---- one query row, three passes ---------------------------------------- */

typedef struct {
  const void *q, *k, *v;
  int dtype;
  int64_t H, Hkv, Nq, Nk, d;
  double scale;
  int causal;
  const int64_t* rows; /* flat (b*H + h)*Nq + i indices, or NULL for all */
  int64_t nrows;
  double *o, *lse;     /* o: [nrows, d], lse: [nrows] */
  int64_t first, last; /* this worker's slice of [0, nrows) */
} job_t;

static void one_row(const job_t* J, int64_t flat, double* o_out, double* lse_out,
                    double* s /* scratch, Nk doubles */, double* qi /* scratch, d doubles */) {
  const int64_t Nq = J->Nq, Nk = J->Nk, d = J->d;
  const int64_t bh = flat / Nq, i = flat % Nq;
  const int64_t b = bh / J->H, h = bh % J->H;
  const int64_t kvh = h / (J->H / J->Hkv);            /* K/V head of query head h */
  const int64_t qhead = bh * Nq * d;                  /* element offset of this (b, h) */
  const int64_t kvhead = (b * J->Hkv + kvh) * Nk * d; /* ... and of its K/V head */
  int64_t nvis = J->causal ? i + 1 + (Nk - Nq) : Nk;
  if (nvis < 0) nvis = 0;

  int64_t c;
  for (c = 0; c < d; ++c) o_out[c] = 0.0;
  if (nvis <= 0) {
    *lse_out = -INFINITY;
    return;
  }

  /* pass 1: scaled scores and their maximum */
  for (c = 0; c < d; ++c) qi[c] = load_elem(J->q, J->dtype, qhead + i * d + c);
  double m = -INFINITY;
  for (int64_t j = 0; j < nvis; ++j) {
    double dot = 0.0;
    for (c = 0; c < d; ++c) dot += qi[c] * load_elem(J->k, J->dtype, kvhead + j * d + c);
    s[j] = J->scale * dot;
    if (s[j] > m) m = s[j];
  }

  /* pass 2: sum of exponentials shifted by the maximum */
  double l = 0.0;
  for (int64_t j = 0; j < nvis; ++j) l += exp(s[j] - m);

  /* pass 3: normalised weights times value rows */
  for (int64_t j = 0; j < nvis; ++j) {
    double p = exp(s[j] - m) / l;
    for (c = 0; c < d; ++c) o_out[c] += p * load_elem(J->v, J->dtype, kvhead + j * d + c);
  }
  *lse_out = m + log(l);
}

static void* worker(void* arg) {
  const job_t* J = (const job_t*)arg;
  double* s = (double*)malloc(sizeof(double) * (size_t)((J->Nk > 0 ? J->Nk : 1) + J->d));
  if (!s) return (void*)1;
  for (int64_t r = J->first; r < J->last; ++r) {
    int64_t flat = J->rows ? J->rows[r] : r;
    one_row(J, flat, J->o + r * J->d, J->lse + r, s, s + (J->Nk > 0 ? J->Nk : 1));
  }
  free(s);
  return NULL;
}

/*
 * oracle_fwd_gqa_f64 -- q: contiguous [B, H, Nq, d], k and v: contiguous
 * [B, Hkv, Nk, d], all of `dtype`; Hkv divides H.
 * rows: optional list of flat row indices ((b*H + h)*Nq + i); NULL means all
 * B*H*Nq rows in order.  o: [nrows, d] doubles, lse: [nrows] doubles.
 * Returns 0 on success, -1 on a bad argument, -2 when out of memory.
 */
int oracle_fwd_gqa_f64(const void* q, const void* k, const void* v, int dtype, int64_t B,
                       int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, double scale,
                       int causal, const int64_t* rows, int64_t nrows, double* o, double* lse,
                       int nthreads) {
  widen_tables_ready();
  if (dtype < ORACLE_F32 || dtype > ORACLE_F16) return -1;
  if (B < 0 || H < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || d <= 0 || nrows < 0) return -1;
  if (Hkv == 0 ? H != 0 : H % Hkv != 0) return -1;
  if (!rows) nrows = B * H * Nq;
  if (nrows == 0) return 0;
  if (!q || !o || !lse || (Nk > 0 && (!k || !v))) return -1;
  if (rows) {
    for (int64_t r = 0; r < nrows; ++r)
      if (rows[r] < 0 || rows[r] >= B * H * Nq) return -1;
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nrows) nthreads = (int)nrows;

  job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !tids) {
    free(jobs);
    free(tids);
    return -2;
  }
  int rc = 0, started = 0;
  for (int t = 0; t < nthreads; ++t) {
    job_t* J = &jobs[t];
    J->q = q; J->k = k; J->v = v; J->dtype = dtype;
    J->H = H; J->Hkv = Hkv; J->Nq = Nq; J->Nk = Nk; J->d = d;
    J->scale = scale; J->causal = causal;
    J->rows = rows; J->nrows = nrows; J->o = o; J->lse = lse;
    J->first = nrows * t / nthreads;
    J->last = nrows * (t + 1) / nthreads;
    if (pthread_create(&tids[t], NULL, worker, J) != 0) {
      if (worker(J)) rc = -2; /* no thread: run this slice inline */
      continue;
    }
    tids[started++] = tids[t];
  }
  for (int t = 0; t < started; ++t) {
    void* ret = NULL;
    pthread_join(tids[t], &ret);
    if (ret) rc = -2;
  }
  free(jobs);
  free(tids);
  return rc;
}

/*
 * oracle_fwd_f64 -- the square multi-head case: q, k, v all contiguous
 * [B, H, N, d]; rows index ((b*H + h)*N + i).  Same returns.
 */
int oracle_fwd_f64(const void* q, const void* k, const void* v, int dtype, int64_t B,
                   int64_t H, int64_t N, int64_t d, double scale, int causal,
                   const int64_t* rows, int64_t nrows, double* o, double* lse,
                   int nthreads) {
  return oracle_fwd_gqa_f64(q, k, v, dtype, B, H, H, N, N, d, scale, causal, rows, nrows, o,
                            lse, nthreads);
}

/*
 * oracle_combine_f64 -- merge S results over disjoint key ranges.
 *
 * o_parts [S, rows, d]: range s's output for each row, already divided by
 * the range's own sum of exponentials; lse_parts [S, rows]: the natural log
 * of that sum (-inf for a range with no visible key).  Output: o [rows, d],
 * lse [rows].
 *
 * A range is the "new block" of the normalised online update (pseudo-algorithm
 * steps 4-5 of "How Did I Write My First FlashAttention Kernel in CUDA?"): a
 * block with local maximum m~, local sum l~ and normalised output O~ = P~V/l~
 * merges into the running (m, l, O) by
 *     m_new = max(m, m~)
 *     l_new = exp(m - m_new) l + exp(m~ - m_new) l~
 *     O     = (l exp(m - m_new) O + l~ exp(m~ - m_new) O~) / l_new.
 * The update only uses m~ and l~ through m~ + ln l~, so a range enters with
 * m~ = LSE_s and l~ = 1.  The running state starts empty (m = -inf, l = 0,
 * O = 0); a range with LSE_s = -inf has no keys and is skipped, so no
 * -inf - (-inf) is ever formed.  At the end lse = m + ln l (-inf if l = 0).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_combine_f64(const double* o_parts, const double* lse_parts, int64_t S, int64_t rows,
                       int64_t d, double* o, double* lse) {
  if (S < 1 || rows < 0 || d <= 0) return -1;
  if (rows == 0) return 0;
  if (!o_parts || !lse_parts || !o || !lse) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    double m = -INFINITY, l = 0.0;
    double* out = o + r * d;
    for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
    for (int64_t s = 0; s < S; ++s) {
      const double mt = lse_parts[s * rows + r], lt = 1.0;
      if (mt == -INFINITY) continue;
      const double* ot = o_parts + (s * rows + r) * d;
      const double m_new = mt > m ? mt : m;
      const double a_old = l * exp(m - m_new), a_new = lt * exp(mt - m_new);
      const double l_new = a_old + a_new;
      for (int64_t c = 0; c < d; ++c) out[c] = (a_old * out[c] + a_new * ot[c]) / l_new;
      m = m_new;
      l = l_new;
    }
    lse[r] = l > 0.0 ? m + log(l) : -INFINITY;
  }
  return 0;
}

/* ---- gradients ------------------------------------------------------------
 *
 * The pages only state that the backward pass recomputes the attention
 * weights from Q, K, V and the saved softmax statistics instead of storing
 * them ("FlashAttention dissected", section "Memory complexity: from O(N^2)
 * to O(N)").  The gradients themselves are the chain rule through the
 * definition above; per head, with P_ij = softmax_j(s_ij) over the visible
 * keys (P_ij = 0 for masked ones) and O = P V:
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij dP_ij  (= dO_i . O_i)
 *   dS_ij = P_ij (dP_ij - D_i)          (derivative of a softmax row)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 * Written out per row with the row's probabilities recomputed by the same
 * three passes as the forward oracle.
 *
 * With grouped K/V heads (query head h reads K/V head h / (H / H_kv)) the
 * same rules hold per query head, and K/V head g, being used by every query
 * head of its group, receives the sum of their contributions:
 *   dK_g = sum over h in group g of dK_h,   dV_g likewise.
 * With N_q != N_kv the visible keys of query row i are those of the forward
 * oracle (j <= i + N_kv - N_q when causal); a row with no visible key has no
 * weights and contributes nothing, and its dQ row is 0. */

typedef struct {
  const void *q, *k, *v, *dout;
  int dtype;
  int64_t H, Hkv, Nq, Nk, d;
  double scale;
  int causal;
  double *dq, *dk, *dv;  /* dq: [B*H, Nq, d]; dk, dv: [B*Hkv, Nk, d] */
  int64_t first, last;   /* this worker's K/V heads, b * Hkv + g */
  /* Query rows of this worker: i with i % row_parts == row_part.  With more
   * than one part, the worker adds its share of dK and dV of its single K/V
   * head into the private [Nk, d] arrays pdk, pdv (the caller sums the parts
   * in part order). */
  int64_t row_part, row_parts;
  double *pdk, *pdv;
} bjob_t;

/* Probabilities of query row i (q rows at element offset qhead) against the
 * keys at element offset kvhead, into p[0..nvis); returns nvis (0 when the
 * row sees no key). */
static int64_t row_probs(const double* qi /* query row i, widened */, const void* k, int dtype,
                         int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
                         int64_t kvhead, int64_t i, double* p) {
  const int64_t nvis = causal ? i + 1 + (Nk - Nq) : Nk;
  if (nvis <= 0) return 0;
  double m = -INFINITY;
  for (int64_t j = 0; j < nvis; ++j) {
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += qi[c] * load_elem(k, dtype, kvhead + j * d + c);
    p[j] = scale * dot;
    if (p[j] > m) m = p[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < nvis; ++j) l += exp(p[j] - m);
  for (int64_t j = 0; j < nvis; ++j) p[j] = exp(p[j] - m) / l;
  return nvis;
}

static void* bwd_worker(void* arg) {
  const bjob_t* J = (const bjob_t*)arg;
  const int64_t Nq = J->Nq, Nk = J->Nk, d = J->d;
  const int64_t grp = J->H / J->Hkv;
  double* p = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
  double* ds = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
  double* o = (double*)malloc(sizeof(double) * (size_t)d * 3);
  if (!p || !ds || !o) {
    free(p); free(ds); free(o);
    return (void*)1;
  }
  double* qi = o + d; /* query row i and its dO row, widened once per row */
  double* gi = o + 2 * d;
  for (int64_t bg = J->first; bg < J->last; ++bg) {
    const int64_t b = bg / J->Hkv, g = bg % J->Hkv;
    const int64_t kvhead = bg * Nk * d;
    double* dk = J->row_parts > 1 ? J->pdk : J->dk + kvhead;
    double* dv = J->row_parts > 1 ? J->pdv : J->dv + kvhead;
    for (int64_t e = 0; e < Nk * d; ++e) dk[e] = dv[e] = 0.0;
    for (int64_t hh = 0; hh < grp; ++hh) {
      const int64_t h = g * grp + hh;
      const int64_t qhead = (b * J->H + h) * Nq * d;
      double* dq = J->dq + qhead;
      for (int64_t i = J->row_part; i < Nq; i += J->row_parts) {
        for (int64_t c = 0; c < d; ++c) {
          dq[i * d + c] = 0.0;
          qi[c] = load_elem(J->q, J->dtype, qhead + i * d + c);
          gi[c] = load_elem(J->dout, J->dtype, qhead + i * d + c);
        }
        const int64_t nvis = row_probs(qi, J->k, J->dtype, Nq, Nk, d, J->scale, J->causal,
                                       kvhead, i, p);
        if (nvis == 0) continue;
        /* O_i and D_i = dO_i . O_i */
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        for (int64_t j = 0; j < nvis; ++j)
          for (int64_t c = 0; c < d; ++c)
            o[c] += p[j] * load_elem(J->v, J->dtype, kvhead + j * d + c);
        double D = 0.0;
        for (int64_t c = 0; c < d; ++c) D += gi[c] * o[c];
        /* dP_ij, dS_ij; dV_j += P_ij dO_i */
        for (int64_t j = 0; j < nvis; ++j) {
          double dp = 0.0;
          for (int64_t c = 0; c < d; ++c) {
            dp += gi[c] * load_elem(J->v, J->dtype, kvhead + j * d + c);
            dv[j * d + c] += p[j] * gi[c];
          }
          ds[j] = p[j] * (dp - D);
        }
        /* dQ_i = scale sum_j dS_ij k_j ; dK_j += scale dS_ij q_i */
        for (int64_t j = 0; j < nvis; ++j)
          for (int64_t c = 0; c < d; ++c) {
            dq[i * d + c] += J->scale * ds[j] * load_elem(J->k, J->dtype, kvhead + j * d + c);
            dk[j * d + c] += J->scale * ds[j] * qi[c];
          }
      }
    }
  }
  free(p); free(ds); free(o);
  return NULL;
}

/* One K/V head bg with its query rows split over nthreads workers: each
 * worker sums its rows' dK, dV contributions privately, then the parts are
 * added in part order (deterministic for a given thread count). */
static int bwd_rows_parallel(const void* q, const void* k, const void* v, const void* dout,
                             int dtype, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                             double scale, int causal, double* dq, double* dk, double* dv,
                             int64_t bg, int nthreads) {
  if (nthreads > Nq) nthreads = (int)Nq;
  const size_t n = (size_t)(Nk * d);
  bjob_t* jobs = (bjob_t*)calloc((size_t)nthreads, sizeof(bjob_t));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  double* priv = (double*)malloc(sizeof(double) * (n > 0 ? n : 1) * 2 * (size_t)nthreads);
  if (!jobs || !tids || !priv) {
    free(jobs); free(tids); free(priv);
    return -2;
  }
  int rc = 0;
  int* started = (int*)calloc((size_t)nthreads, sizeof(int));
  if (!started) {
    free(jobs); free(tids); free(priv);
    return -2;
  }
  for (int t = 0; t < nthreads; ++t) {
    bjob_t* J = &jobs[t];
    J->q = q; J->k = k; J->v = v; J->dout = dout; J->dtype = dtype;
    J->H = H; J->Hkv = Hkv; J->Nq = Nq; J->Nk = Nk; J->d = d;
    J->scale = scale; J->causal = causal;
    J->dq = dq; J->dk = dk; J->dv = dv;
    J->first = bg;
    J->last = bg + 1;
    J->row_part = t;
    J->row_parts = nthreads;
    J->pdk = priv + 2 * n * (size_t)t;
    J->pdv = J->pdk + n;
    if (pthread_create(&tids[t], NULL, bwd_worker, J) == 0) {
      started[t] = 1;
    } else if (bwd_worker(J)) {
      rc = -2;
    }
  }
  for (int t = 0; t < nthreads; ++t) {
    if (!started[t]) continue;
    void* ret = NULL;
    pthread_join(tids[t], &ret);
    if (ret) rc = -2;
  }
  if (rc == 0) {
    double *hk = dk + (size_t)bg * n, *hv = dv + (size_t)bg * n;
    for (size_t e = 0; e < n; ++e) hk[e] = hv[e] = 0.0;
    for (int t = 0; t < nthreads; ++t)
      for (size_t e = 0; e < n; ++e) {
        hk[e] += jobs[t].pdk[e];
        hv[e] += jobs[t].pdv[e];
      }
  }
  free(started); free(jobs); free(tids); free(priv);
  return rc;
}

/*
 * oracle_bwd_gqa_f64 -- q, dout: contiguous [B, H, Nq, d]; k, v: [B, Hkv,
 * Nk, d], all of `dtype`; H a multiple of Hkv.  dq: [B, H, Nq, d] and dk,
 * dv: [B, Hkv, Nk, d] doubles, written in full.  Threads work on whole K/V
 * heads (and so on whole groups of query heads), or, with fewer K/V heads
 * than threads, on the query rows of one head at a time.  Returns 0, -1 on a
 * bad argument, -2 when out of memory.
 */
int oracle_bwd_gqa_f64(const void* q, const void* k, const void* v, const void* dout, int dtype,
                       int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                       double scale, int causal, double* dq, double* dk, double* dv,
                       int nthreads) {
  widen_tables_ready();
  if (dtype < ORACLE_F32 || dtype > ORACLE_F16) return -1;
  if (B < 0 || H < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || d <= 0) return -1;
  if ((H == 0) != (Hkv == 0) || (Hkv > 0 && H % Hkv != 0)) return -1;
  const int64_t heads = B * Hkv;
  if (heads == 0 || (Nq == 0 && Nk == 0)) return 0;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
  if (nthreads < 1) nthreads = 1;
  /* Fewer K/V heads than threads: each head in turn, its query rows dealt
   * round-robin to the threads (same sums, in another order). */
  if (heads < nthreads && Nq > 1) {
    for (int64_t bg = 0; bg < heads; ++bg) {
      const int rc = bwd_rows_parallel(q, k, v, dout, dtype, H, Hkv, Nq, Nk, d, scale, causal,
                                       dq, dk, dv, bg, nthreads);
      if (rc) return rc;
    }
    return 0;
  }
  if (nthreads > heads) nthreads = (int)heads;
  bjob_t* jobs = (bjob_t*)calloc((size_t)nthreads, sizeof(bjob_t));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !tids) {
    free(jobs);
    free(tids);
    return -2;
  }
  int rc = 0, started = 0;
  for (int t = 0; t < nthreads; ++t) {
    bjob_t* J = &jobs[t];
    J->q = q; J->k = k; J->v = v; J->dout = dout; J->dtype = dtype;
    J->H = H; J->Hkv = Hkv; J->Nq = Nq; J->Nk = Nk; J->d = d;
    J->scale = scale; J->causal = causal;
    J->dq = dq; J->dk = dk; J->dv = dv;
    J->first = heads * t / nthreads;
    J->last = heads * (t + 1) / nthreads;
    J->row_part = 0;
    J->row_parts = 1;
    if (pthread_create(&tids[t], NULL, bwd_worker, J) != 0) {
      if (bwd_worker(J)) rc = -2;
      continue;
    }
    tids[started++] = tids[t];
  }
  for (int t = 0; t < started; ++t) {
    void* ret = NULL;
    pthread_join(tids[t], &ret);
    if (ret) rc = -2;
  }
  free(jobs);
  free(tids);
  return rc;
}

/* oracle_bwd_f64 -- the square case: q, k, v, dout, dq, dk, dv all [B, H, N, d]. */
int oracle_bwd_f64(const void* q, const void* k, const void* v, const void* dout, int dtype,
                   int64_t B, int64_t H, int64_t N, int64_t d, double scale, int causal,
                   double* dq, double* dk, double* dv, int nthreads) {
  return oracle_bwd_gqa_f64(q, k, v, dout, dtype, B, H, H, N, N, d, scale, causal, dq, dk, dv,
                            nthreads);
}

/*
 * oracle_bwd_dq_rows_gqa_f64 -- dQ for a list of flat query rows
 * ((b*H + h)*Nq + i) only: row i's gradient needs just row i's
 * probabilities, so sampled rows of a large problem cost O(Nk d) each.
 * Shapes as oracle_bwd_gqa_f64.  dq: [nrows, d] doubles.
 */
int oracle_bwd_dq_rows_gqa_f64(const void* q, const void* k, const void* v, const void* dout,
                               int dtype, int64_t B, int64_t H, int64_t Hkv, int64_t Nq,
                               int64_t Nk, int64_t d, double scale, int causal,
                               const int64_t* rows, int64_t nrows, double* dq) {
  widen_tables_ready();
  if (dtype < ORACLE_F32 || dtype > ORACLE_F16) return -1;
  if (B < 0 || H < 0 || Hkv <= 0 || Nq < 0 || Nk < 0 || d <= 0 || nrows < 0) return -1;
  if (H % Hkv != 0) return -1;
  if (nrows == 0) return 0;
  if (!q || !k || !v || !dout || !rows || !dq) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= B * H * Nq) return -1;
  double* p = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
  double* o = (double*)malloc(sizeof(double) * (size_t)d * 2);
  if (!p || !o) {
    free(p); free(o);
    return -2;
  }
  double* qi = o + d;
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t bh = rows[r] / Nq, i = rows[r] % Nq;
    const int64_t b = bh / H, h = bh % H;
    const int64_t qhead = bh * Nq * d, kvhead = (b * Hkv + h / (H / Hkv)) * Nk * d;
    double* out = dq + r * d;
    for (int64_t c = 0; c < d; ++c) {
      out[c] = 0.0;
      qi[c] = load_elem(q, dtype, qhead + i * d + c);
    }
    const int64_t nvis = row_probs(qi, k, dtype, Nq, Nk, d, scale, causal, kvhead, i, p);
    if (nvis == 0) continue;
    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < nvis; ++j)
      for (int64_t c = 0; c < d; ++c) o[c] += p[j] * load_elem(v, dtype, kvhead + j * d + c);
    double D = 0.0;
    for (int64_t c = 0; c < d; ++c) D += load_elem(dout, dtype, qhead + i * d + c) * o[c];
    for (int64_t j = 0; j < nvis; ++j) {
      double dp = 0.0;
      for (int64_t c = 0; c < d; ++c)
        dp += load_elem(dout, dtype, qhead + i * d + c) * load_elem(v, dtype, kvhead + j * d + c);
      const double ds = p[j] * (dp - D);
      for (int64_t c = 0; c < d; ++c)
        out[c] += scale * ds * load_elem(k, dtype, kvhead + j * d + c);
    }
  }
  free(p); free(o);
  return 0;
}

/* oracle_bwd_dq_rows_f64 -- the square case of oracle_bwd_dq_rows_gqa_f64. */
int oracle_bwd_dq_rows_f64(const void* q, const void* k, const void* v, const void* dout,
                           int dtype, int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                           int causal, const int64_t* rows, int64_t nrows, double* dq) {
  return oracle_bwd_dq_rows_gqa_f64(q, k, v, dout, dtype, B, H, H, N, N, d, scale, causal, rows,
                                    nrows, dq);
}
