/*
 * oracle.c -- plain, slow CPU reference for interval-mask flex attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this code.  The GPU library never
 * links, calls or includes it, and this file includes nothing from the GPU
 * library: the two implementations share no code.
 *
 * Everything here is the plain definition, written out with loops, in double
 * precision:
 *   - validate  : "Flex Attention Mask Plan Design" (cuDNN frontend docs),
 *                 §2 (endpoint order and bounds), §3.2 (Varlen prefix rules),
 *                 §4.3 (classifier validates every endpoint).
 *   - expand    : §2, visible(q) = [0,F0) U [F1,F2) U [F3,F4) U ...
 *   - classify  : §4.3, exactly one of empty / full / partial per (Q tile, K
 *                 tile); full needs the whole tile in bounds and every element
 *                 visible; a tile that sticks out past q_len or k_len is never
 *                 full.
 *   - pack      : §5, one bit per score element, 1 = keep, 0 = -inf.  This
 *                 library's consumer reads the predicate of row r, columns
 *                 [32w, 32w+32) of a tile from word r*W + w, bit (c mod 32),
 *                 W = T_KV/32; out-of-bounds elements are 0 bits.
 *   - CSR       : §4.5 / §4.6, exclusive offsets off[0]=0,
 *                 off[i+1]=off[i]+cnt[i]; partial and full lists independent,
 *                 sample-local K-tile indices in ascending order, rows
 *                 flattened head-major (flat = hm*rows_total + row).
 *   - attention : FlexAttention (Dong et al.), Eq. 1,
 *                 softmax(mod(Q K^T / sqrt(d))) V, with the mask as an additive
 *                 0 / -inf bias (Tessera paper, "masked attention" definition);
 *                 rows with nothing visible give O = 0 and LSE = -inf (mask
 *                 plan design §6.1).  LSE is the natural log of the sum of
 *                 exp(score) over visible keys, scores after score_mod.
 *   - Split-K   : Tessera page, "Split-K" (Figure 5): attention restricted to
 *                 a K range gives a partial state (normalized O and LSE of the
 *                 keys in the range); partial states merge by rescaling to a
 *                 common maximum (orc_attention_part, orc_merge).
 *   - K2Q view  : §4.4 / §4.7, the same pair classes read K-major, with a
 *                 K-major predicate per partial pair (see orc_k2q_build).
 *   - score_mod : softcap c*tanh(s/c) then ALiBi + slope_h*(k-q) with
 *                 sample-local positions (optionally ALiBi first); the scale is
 *                 applied before either.
 *   - backward  : the gradient of Eq. 1 for a given dO, by the chain rule
 *                 written out per row (see orc_attention_bwd); the softcap's
 *                 derivative is 1 - tanh^2, ALiBi's is 1 (FlexAttention,
 *                 "automatic backward of score_mod").
 *
 * Threads: independent rows are split over POSIX threads; each thread runs the
 * same plain loops on its own rows.  No -ffast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_ERR_SEQLENS = 1, ORC_ERR_RANGE = 2, ORC_ERR_ORDER = 4 };
enum { ORC_BSHD = 0, ORC_THD = 1 };

typedef struct {
  int32_t layout, batch, seqlen_q, seqlen_k, total_q, total_k;
  int32_t heads_q, heads_k, head_dim, mask_heads, nfunc;
  int32_t tile_q, tile_k;
} orc_problem;

/* ------------------------------------------------------------ geometry */

static void sample_of(const orc_problem* p, const int32_t* cu_q, const int32_t* cu_k, int b,
                      int64_t* q_off, int64_t* q_len, int64_t* k_off, int64_t* k_len) {
  if (p->layout == ORC_BSHD) {
    *q_off = (int64_t)b * p->seqlen_q;
    *q_len = p->seqlen_q;
    *k_off = (int64_t)b * p->seqlen_k;
    *k_len = p->seqlen_k;
  } else {
    *q_off = cu_q[b];
    *q_len = (int64_t)cu_q[b + 1] - cu_q[b];
    *k_off = cu_k[b];
    *k_len = (int64_t)cu_k[b + 1] - cu_k[b];
  }
}

/* Sample that owns Q token t (linear search; the prefix is validated). */
static int owner_of_token(const orc_problem* p, const int32_t* cu_q, int64_t t) {
  if (p->layout == ORC_BSHD) return (int)(t / p->seqlen_q);
  for (int b = 0; b < p->batch; ++b)
    if (t >= cu_q[b] && t < cu_q[b + 1]) return b;
  return -1;
}

static int32_t endpoint(const orc_problem* p, const int32_t* mf, int hm, int f, int64_t t) {
  return mf[((int64_t)hm * p->nfunc + f) * p->total_q + t];
}

/* ------------------------------------------------------------ validate */

/* Varlen prefix rules (§3.2): start at 0, end at the total, nondecreasing,
 * every length <= max_seqlen. */
static int prefix_ok(const int32_t* cu, int batch, int32_t total, int32_t max_len) {
  if (cu[0] != 0) return 0;
  if (cu[batch] != total) return 0;
  for (int b = 0; b < batch; ++b) {
    if (cu[b + 1] < cu[b]) return 0;
    if ((int64_t)cu[b + 1] - cu[b] > max_len) return 0;
  }
  return 1;
}

/* Returns the OR of ORC_ERR_* bits.  When the prefixes are invalid the sample
 * K lengths are undefined, so the per-endpoint checks are skipped. */
uint32_t orc_validate(const orc_problem* p, const int32_t* mf, const int32_t* cu_q,
                      const int32_t* cu_k) {
  uint32_t err = 0;
  if (p->layout == ORC_THD) {
    if (!prefix_ok(cu_q, p->batch, p->total_q, p->seqlen_q) ||
        !prefix_ok(cu_k, p->batch, p->total_k, p->seqlen_k))
      return ORC_ERR_SEQLENS;
  }
  for (int b = 0; b < p->batch; ++b) {
    int64_t q_off, q_len, k_off, k_len;
    sample_of(p, cu_q, cu_k, b, &q_off, &q_len, &k_off, &k_len);
    for (int hm = 0; hm < p->mask_heads; ++hm)
      for (int64_t q = 0; q < q_len; ++q)
        for (int f = 0; f < p->nfunc; ++f) {
          int32_t F = endpoint(p, mf, hm, f, q_off + q);
          if (F < 0 || F > k_len) err |= ORC_ERR_RANGE;
          if (f + 1 < p->nfunc && F > endpoint(p, mf, hm, f + 1, q_off + q)) err |= ORC_ERR_ORDER;
        }
  }
  return err;
}

/* ------------------------------------------------------------ expand */

/* visible[k] for k in [0, k_len): the union of [0,F0), [F1,F2), [F3,F4), ...
 * Each interval's members are marked one by one. */
void orc_expand_row(const int32_t* F, int64_t stride, int nfunc, int64_t k_len, uint8_t* vis) {
  for (int64_t k = 0; k < k_len; ++k) vis[k] = 0;
  for (int i = -1; i < nfunc; i += 2) {
    int64_t a = (i < 0) ? 0 : F[(int64_t)i * stride];
    int64_t b = F[(int64_t)(i + 1) * stride];
    for (int64_t k = a; k < b && k < k_len; ++k)
      if (k >= 0) vis[k] = 1;
  }
}

/* ------------------------------------------------------------ plan */

typedef struct {
  int64_t header[8];         /* rows, pnnz, fnnz, 0, 0, 0, 0, err */
  int32_t rows_total, nk_max, words;
  int32_t* cu_rows;          /* [B+1] */
  int32_t* seqdesc;          /* [B][8] */
  int32_t* p_off;            /* [Hmask*rows+1] */
  int32_t* f_off;
  int32_t* p_idx;            /* [pnnz] */
  int32_t* f_idx;            /* [fnnz] */
  uint32_t* p_masks;         /* [pnnz * tile_q * words] */
  uint8_t* cls;              /* [Hmask*rows*nk_max] 0 empty/nonexistent, 1 partial, 2 full */
} orc_plan;

typedef struct {
  const orc_problem* p;
  const int32_t* mf;
  const int32_t* cu_q;
  const int32_t* cu_k;
  orc_plan* plan;
  const int32_t* row_sample;
  int64_t item_begin, item_end;   /* flat (hm, row) items */
  int phase;                      /* 0 classify, 1 materialize */
} plan_job;

/* Expands rows [r0, r0+T_Q) of sample b (mask head hm) into vis[T_Q][k_len];
 * rows past q_len stay all-zero. */
static void expand_tile_rows(const orc_problem* p, const int32_t* mf, int hm, int64_t q_off,
                             int64_t q_len, int64_t r0, int64_t k_len, uint8_t* vis) {
  for (int r = 0; r < p->tile_q; ++r) {
    uint8_t* row = vis + (int64_t)r * (k_len > 0 ? k_len : 1);
    if (r0 + r < q_len) {
      const int32_t* F = mf + (int64_t)hm * p->nfunc * p->total_q + q_off + r0 + r;
      orc_expand_row(F, p->total_q, p->nfunc, k_len, row);
    } else {
      for (int64_t k = 0; k < k_len; ++k) row[k] = 0;
    }
  }
}

static void* plan_worker(void* arg) {
  plan_job* J = (plan_job*)arg;
  const orc_problem* p = J->p;
  orc_plan* P = J->plan;
  int64_t pitch = p->seqlen_k > 0 ? p->seqlen_k : 1;
  uint8_t* vis = (uint8_t*)malloc((size_t)p->tile_q * pitch);
  for (int64_t item = J->item_begin; item < J->item_end; ++item) {
    int hm = (int)(item / P->rows_total);
    int64_t row = item % P->rows_total;
    int b = J->row_sample[row];
    int64_t q_off, q_len, k_off, k_len;
    sample_of(p, J->cu_q, J->cu_k, b, &q_off, &q_len, &k_off, &k_len);
    int64_t i = row - P->cu_rows[b];
    int64_t r0 = i * p->tile_q;
    int64_t nk = (k_len + p->tile_k - 1) / p->tile_k;
    expand_tile_rows(p, J->mf, hm, q_off, q_len, r0, k_len, vis);
    uint8_t* cls = P->cls + item * P->nk_max;
    int64_t pw = P->p_off ? P->p_off[item] : 0, fw = P->f_off ? P->f_off[item] : 0;
    for (int64_t j = 0; j < nk; ++j) {
      int64_t c0 = j * p->tile_k;
      if (J->phase == 0) {
        int64_t count = 0;
        for (int r = 0; r < p->tile_q; ++r)
          for (int c = 0; c < p->tile_k; ++c)
            if (r0 + r < q_len && c0 + c < k_len && vis[(int64_t)r * k_len + c0 + c]) ++count;
        int in_bounds = (r0 + p->tile_q <= q_len) && (c0 + p->tile_k <= k_len);
        if (count == 0) cls[j] = 0;
        else if (in_bounds && count == (int64_t)p->tile_q * p->tile_k) cls[j] = 2;
        else cls[j] = 1;
      } else if (cls[j] == 1) {
        P->p_idx[pw] = (int32_t)j;
        uint32_t* words = P->p_masks + pw * (int64_t)p->tile_q * P->words;
        for (int r = 0; r < p->tile_q; ++r)
          for (int w = 0; w < P->words; ++w) {
            uint32_t word = 0;
            for (int bit = 0; bit < 32; ++bit) {
              int64_t c = c0 + 32 * w + bit;
              if (r0 + r < q_len && c < k_len && c < c0 + p->tile_k && vis[(int64_t)r * k_len + c])
                word |= 1u << bit;
            }
            words[r * P->words + w] = word;
          }
        ++pw;
      } else if (cls[j] == 2) {
        P->f_idx[fw++] = (int32_t)j;
      }
    }
  }
  free(vis);
  return NULL;
}

static void run_plan_phase(const orc_problem* p, const int32_t* mf, const int32_t* cu_q,
                           const int32_t* cu_k, orc_plan* P, const int32_t* row_sample, int phase,
                           int nthreads) {
  int64_t items = (int64_t)p->mask_heads * P->rows_total;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > items) nthreads = items > 0 ? (int)items : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  plan_job* jobs = (plan_job*)malloc(sizeof(plan_job) * nthreads);
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (plan_job){p, mf, cu_q, cu_k, P, row_sample, items * t / nthreads,
                         items * (t + 1) / nthreads, phase};
    pthread_create(&th[t], NULL, plan_worker, &jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
}

/* Builds the whole plan by brute force.  Returns NULL on allocation failure.
 * On a validation error the plan holds only the header (err != 0). */
orc_plan* orc_plan_build(const orc_problem* p, const int32_t* mf, const int32_t* cu_q,
                         const int32_t* cu_k, int nthreads) {
  orc_plan* P = (orc_plan*)calloc(1, sizeof(orc_plan));
  if (!P) return NULL;
  uint32_t err = orc_validate(p, mf, cu_q, cu_k);
  P->header[7] = err;
  if (err) return P;
  int B = p->batch;
  P->cu_rows = (int32_t*)calloc((size_t)B + 1, sizeof(int32_t));
  P->seqdesc = (int32_t*)calloc((size_t)B * 8 + 1, sizeof(int32_t));
  int64_t nk_max = 0;
  for (int b = 0; b < B; ++b) {
    int64_t q_off, q_len, k_off, k_len;
    sample_of(p, cu_q, cu_k, b, &q_off, &q_len, &k_off, &k_len);
    int64_t rows_b = (q_len + p->tile_q - 1) / p->tile_q;
    int64_t nk = (k_len + p->tile_k - 1) / p->tile_k;
    if (nk > nk_max) nk_max = nk;
    P->cu_rows[b + 1] = P->cu_rows[b] + (int32_t)rows_b;
    int32_t* sd = P->seqdesc + 8 * b;
    sd[0] = (int32_t)q_off; sd[1] = (int32_t)k_off; sd[2] = (int32_t)q_len; sd[3] = (int32_t)k_len;
    sd[4] = P->cu_rows[b]; sd[5] = (int32_t)rows_b; sd[6] = (int32_t)nk; sd[7] = 0;
  }
  P->rows_total = P->cu_rows[B];
  P->nk_max = (int32_t)(nk_max > 0 ? nk_max : 1);
  P->words = p->tile_k / 32;
  int32_t* row_sample = (int32_t*)calloc((size_t)P->rows_total + 1, sizeof(int32_t));
  for (int b = 0; b < B; ++b)
    for (int32_t r = P->cu_rows[b]; r < P->cu_rows[b + 1]; ++r) row_sample[r] = b;
  int64_t items = (int64_t)p->mask_heads * P->rows_total;
  P->cls = (uint8_t*)calloc((size_t)(items > 0 ? items : 1) * P->nk_max, 1);
  run_plan_phase(p, mf, cu_q, cu_k, P, row_sample, 0, nthreads);
  /* counts and exclusive offsets */
  P->p_off = (int32_t*)calloc((size_t)items + 1, sizeof(int32_t));
  P->f_off = (int32_t*)calloc((size_t)items + 1, sizeof(int32_t));
  for (int64_t it = 0; it < items; ++it) {
    int32_t pc = 0, fc = 0;
    for (int64_t j = 0; j < P->nk_max; ++j) {
      pc += P->cls[it * P->nk_max + j] == 1;
      fc += P->cls[it * P->nk_max + j] == 2;
    }
    P->p_off[it + 1] = P->p_off[it] + pc;
    P->f_off[it + 1] = P->f_off[it] + fc;
  }
  int64_t pnnz = P->p_off[items], fnnz = P->f_off[items];
  P->header[0] = P->rows_total;
  P->header[1] = pnnz;
  P->header[2] = fnnz;
  P->p_idx = (int32_t*)calloc((size_t)pnnz + 1, sizeof(int32_t));
  P->f_idx = (int32_t*)calloc((size_t)fnnz + 1, sizeof(int32_t));
  P->p_masks = (uint32_t*)calloc((size_t)pnnz * p->tile_q * P->words + 1, sizeof(uint32_t));
  run_plan_phase(p, mf, cu_q, cu_k, P, row_sample, 1, nthreads);
  free(row_sample);
  return P;
}

void orc_plan_sizes(const orc_plan* P, int64_t* header8, int32_t* rows_total, int32_t* nk_max) {
  for (int i = 0; i < 8; ++i) header8[i] = P->header[i];
  *rows_total = P->rows_total;
  *nk_max = P->nk_max;
}

/* Copies the plan out; any pointer may be NULL. */
void orc_plan_export(const orc_plan* P, const orc_problem* p, int32_t* cu_rows, int32_t* seqdesc,
                     int32_t* p_off, int32_t* p_idx, uint32_t* p_masks, int32_t* f_off,
                     int32_t* f_idx, uint8_t* cls) {
  int64_t items = (int64_t)p->mask_heads * P->rows_total;
  if (P->header[7]) return;
  if (cu_rows) memcpy(cu_rows, P->cu_rows, sizeof(int32_t) * (p->batch + 1));
  if (seqdesc) memcpy(seqdesc, P->seqdesc, sizeof(int32_t) * 8 * p->batch);
  if (p_off) memcpy(p_off, P->p_off, sizeof(int32_t) * (items + 1));
  if (f_off) memcpy(f_off, P->f_off, sizeof(int32_t) * (items + 1));
  if (p_idx) memcpy(p_idx, P->p_idx, sizeof(int32_t) * P->header[1]);
  if (f_idx) memcpy(f_idx, P->f_idx, sizeof(int32_t) * P->header[2]);
  if (p_masks) memcpy(p_masks, P->p_masks, sizeof(uint32_t) * P->header[1] * p->tile_q * P->words);
  if (cls) memcpy(cls, P->cls, (size_t)items * P->nk_max);
}

/* ------------------------------------------------------------ K2Q view */

/* Backward K-major view ("Flex Attention Mask Plan Design" §4.4 counting,
 * §4.7 materialization): for every mask head and K plan row (one K tile of
 * one sample; K rows flattened head-major, flat = hm*krows_total + krow,
 * krow = cu_krows[b] + j), the sample-local Q tiles i whose pair (i, j) is
 * partial and, independently, full -- the same three-way class as §4.3 --
 * in ascending i.  Each partial pair carries a K-major predicate:
 * word [r][c/32], bit c%32, is 1 iff score (Q row i*T_Q + c, K column
 * j*T_KV + r) is in bounds and visible.  Computed here from the dense
 * expansion of every Q tile, in two passes (classes and counts, then lists
 * and payload). */
typedef struct {
  int64_t header[4];          /* Q rows, K rows, partial nnz, full nnz */
  int32_t krows_total, qrows_total;
  int32_t* cu_krows;          /* [B+1] */
  int32_t* cu_qrows;          /* [B+1] */
  uint8_t* cls;               /* [Hmask][krows_total][max Q rows per sample] */
  int32_t qrows_max;
  int32_t* p_off;             /* [Hmask*krows+1] */
  int32_t* f_off;
  int32_t* p_idx;
  int32_t* f_idx;
  uint32_t* p_masks;          /* [pnnz][tile_k][tile_q/32] */
} orc_k2q;

typedef struct {
  const orc_problem* p;
  const int32_t* mf;
  const int32_t* cu_q;
  const int32_t* cu_k;
  orc_k2q* V;
  int64_t item_begin, item_end;   /* (hm, b, i) items, i over the sample's Q tiles */
  int64_t* item_tab;              /* [items][3] */
  int phase;
} k2q_job;

static void* k2q_worker(void* arg) {
  k2q_job* J = (k2q_job*)arg;
  const orc_problem* p = J->p;
  orc_k2q* V = J->V;
  int64_t pitch = p->seqlen_k > 0 ? p->seqlen_k : 1;
  uint8_t* vis = (uint8_t*)malloc((size_t)p->tile_q * pitch);
  int wq = p->tile_q / 32;
  for (int64_t it = J->item_begin; it < J->item_end; ++it) {
    int hm = (int)J->item_tab[3 * it], b = (int)J->item_tab[3 * it + 1];
    int64_t i = J->item_tab[3 * it + 2];
    int64_t q_off, q_len, k_off, k_len;
    sample_of(p, J->cu_q, J->cu_k, b, &q_off, &q_len, &k_off, &k_len);
    int64_t r0 = i * p->tile_q;
    int64_t nk = (k_len + p->tile_k - 1) / p->tile_k;
    expand_tile_rows(p, J->mf, hm, q_off, q_len, r0, k_len, vis);
    for (int64_t j = 0; j < nk; ++j) {
      int64_t c0 = j * p->tile_k;
      int64_t flat = (int64_t)hm * V->krows_total + V->cu_krows[b] + j;
      uint8_t* cls = V->cls + flat * V->qrows_max;
      if (J->phase == 0) {
        int64_t count = 0;
        for (int r = 0; r < p->tile_q; ++r)
          for (int c = 0; c < p->tile_k; ++c)
            if (r0 + r < q_len && c0 + c < k_len && vis[(int64_t)r * k_len + c0 + c]) ++count;
        int in_bounds = (r0 + p->tile_q <= q_len) && (c0 + p->tile_k <= k_len);
        if (count == 0) cls[i] = 0;
        else if (in_bounds && count == (int64_t)p->tile_q * p->tile_k) cls[i] = 2;
        else cls[i] = 1;
      } else if (cls[i] != 0) {
        /* rank of i among this K row's Q tiles of the same class */
        int64_t rank = 0;
        for (int64_t i2 = 0; i2 < i; ++i2) rank += cls[i2] == cls[i];
        if (cls[i] == 2) {
          V->f_idx[V->f_off[flat] + rank] = (int32_t)i;
          continue;
        }
        int64_t n = V->p_off[flat] + rank;
        V->p_idx[n] = (int32_t)i;
        uint32_t* words = V->p_masks + n * (int64_t)p->tile_k * wq;
        for (int r = 0; r < p->tile_k; ++r)          /* K row of the tile */
          for (int w = 0; w < wq; ++w) {
            uint32_t word = 0;
            for (int bit = 0; bit < 32; ++bit) {
              int64_t c = 32 * w + bit;                /* Q row of the tile */
              if (r0 + c < q_len && c0 + r < k_len && vis[c * k_len + c0 + r]) word |= 1u << bit;
            }
            words[r * wq + w] = word;
          }
      }
    }
  }
  free(vis);
  return NULL;
}

static void run_k2q_phase(const orc_problem* p, const int32_t* mf, const int32_t* cu_q,
                          const int32_t* cu_k, orc_k2q* V, int64_t* tab, int64_t items, int phase,
                          int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > items) nthreads = items > 0 ? (int)items : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  k2q_job* jobs = (k2q_job*)malloc(sizeof(k2q_job) * nthreads);
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (k2q_job){p, mf, cu_q, cu_k, V, items * t / nthreads, items * (t + 1) / nthreads, tab,
                        phase};
    pthread_create(&th[t], NULL, k2q_worker, &jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
}

/* Returns NULL on allocation failure or invalid input (the forward plan's
 * validation decides that). */
orc_k2q* orc_k2q_build(const orc_problem* p, const int32_t* mf, const int32_t* cu_q,
                       const int32_t* cu_k, int nthreads) {
  if (orc_validate(p, mf, cu_q, cu_k)) return NULL;
  orc_k2q* V = (orc_k2q*)calloc(1, sizeof(orc_k2q));
  if (!V) return NULL;
  int B = p->batch;
  V->cu_krows = (int32_t*)calloc((size_t)B + 1, sizeof(int32_t));
  V->cu_qrows = (int32_t*)calloc((size_t)B + 1, sizeof(int32_t));
  int64_t qmax = 1;
  for (int b = 0; b < B; ++b) {
    int64_t q_off, q_len, k_off, k_len;
    sample_of(p, cu_q, cu_k, b, &q_off, &q_len, &k_off, &k_len);
    int64_t qr = (q_len + p->tile_q - 1) / p->tile_q;
    if (qr > qmax) qmax = qr;
    V->cu_qrows[b + 1] = V->cu_qrows[b] + (int32_t)qr;
    V->cu_krows[b + 1] = V->cu_krows[b] + (int32_t)((k_len + p->tile_k - 1) / p->tile_k);
  }
  V->qrows_total = V->cu_qrows[B];
  V->krows_total = V->cu_krows[B];
  V->qrows_max = (int32_t)qmax;
  int64_t kitems = (int64_t)p->mask_heads * V->krows_total;
  V->cls = (uint8_t*)calloc((size_t)(kitems > 0 ? kitems : 1) * qmax, 1);
  int64_t items = (int64_t)p->mask_heads * V->qrows_total;
  int64_t* tab = (int64_t*)malloc(sizeof(int64_t) * 3 * (size_t)(items > 0 ? items : 1));
  int64_t n = 0;
  for (int hm = 0; hm < p->mask_heads; ++hm)
    for (int b = 0; b < B; ++b)
      for (int64_t i = 0; i < V->cu_qrows[b + 1] - V->cu_qrows[b]; ++i) {
        tab[3 * n] = hm; tab[3 * n + 1] = b; tab[3 * n + 2] = i; ++n;
      }
  run_k2q_phase(p, mf, cu_q, cu_k, V, tab, items, 0, nthreads);
  V->p_off = (int32_t*)calloc((size_t)kitems + 1, sizeof(int32_t));
  V->f_off = (int32_t*)calloc((size_t)kitems + 1, sizeof(int32_t));
  for (int64_t f = 0; f < kitems; ++f) {
    int32_t pc = 0, fc = 0;
    for (int64_t i = 0; i < qmax; ++i) {
      pc += V->cls[f * qmax + i] == 1;
      fc += V->cls[f * qmax + i] == 2;
    }
    V->p_off[f + 1] = V->p_off[f] + pc;
    V->f_off[f + 1] = V->f_off[f] + fc;
  }
  V->header[0] = V->qrows_total;
  V->header[1] = V->krows_total;
  V->header[2] = V->p_off[kitems];
  V->header[3] = V->f_off[kitems];
  V->p_idx = (int32_t*)calloc((size_t)V->header[2] + 1, sizeof(int32_t));
  V->f_idx = (int32_t*)calloc((size_t)V->header[3] + 1, sizeof(int32_t));
  V->p_masks = (uint32_t*)calloc((size_t)V->header[2] * p->tile_k * (p->tile_q / 32) + 1,
                                 sizeof(uint32_t));
  run_k2q_phase(p, mf, cu_q, cu_k, V, tab, items, 1, nthreads);
  free(tab);
  return V;
}

void orc_k2q_sizes(const orc_k2q* V, int64_t* header4) {
  for (int i = 0; i < 4; ++i) header4[i] = V->header[i];
}

void orc_k2q_export(const orc_k2q* V, const orc_problem* p, int32_t* cu_krows, int32_t* p_off,
                    int32_t* p_idx, uint32_t* p_masks, int32_t* f_off, int32_t* f_idx) {
  int64_t kitems = (int64_t)p->mask_heads * V->krows_total;
  if (cu_krows) memcpy(cu_krows, V->cu_krows, sizeof(int32_t) * (p->batch + 1));
  if (p_off) memcpy(p_off, V->p_off, sizeof(int32_t) * (kitems + 1));
  if (f_off) memcpy(f_off, V->f_off, sizeof(int32_t) * (kitems + 1));
  if (p_idx) memcpy(p_idx, V->p_idx, sizeof(int32_t) * V->header[2]);
  if (f_idx) memcpy(f_idx, V->f_idx, sizeof(int32_t) * V->header[3]);
  if (p_masks)
    memcpy(p_masks, V->p_masks, sizeof(uint32_t) * V->header[2] * p->tile_k * (p->tile_q / 32));
}

void orc_k2q_free(orc_k2q* V) {
  if (!V) return;
  free(V->cu_krows); free(V->cu_qrows); free(V->cls); free(V->p_off); free(V->f_off);
  free(V->p_idx); free(V->f_idx); free(V->p_masks);
  free(V);
}

void orc_plan_free(orc_plan* P) {
  if (!P) return;
  free(P->cu_rows); free(P->seqdesc); free(P->p_off); free(P->f_off);
  free(P->p_idx); free(P->f_idx); free(P->p_masks); free(P->cls);
  free(P);
}

/* ------------------------------------------------------------ attention */

typedef struct {
  int softcap_on;
  double softcap;
  int alibi_on;
  const float* slopes;   /* [heads_q] */
  int alibi_first;       /* 1: ALiBi before the softcap */
} orc_mod;

/* score_mod applied to one scaled score t of head h at sample-local (q, k). */
static double apply_mod(const orc_mod* m, double t, int h, int64_t q, int64_t k) {
  double bias = m->alibi_on ? (double)m->slopes[h] * (double)(k - q) : 0.0;
  if (m->alibi_on && m->alibi_first) t += bias;
  if (m->softcap_on) t = m->softcap * tanh(t / m->softcap);
  if (m->alibi_on && !m->alibi_first) t += bias;
  return t;
}

typedef struct {
  const orc_problem* p;
  const int32_t* mf;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const float *q, *k, *v;
  double scale;
  const orc_mod* mod;
  const int64_t* rows;   /* pairs (token, head); NULL = all rows */
  int64_t k_lo, k_hi;    /* only keys with k_lo <= k < k_hi (sample-local) count */
  int64_t begin, end;
  double* o;             /* [n][d] for selected rows; [total_q][Hq][d] for all */
  double* lse;           /* [n] ; [Hq][total_q] for all */
} attn_job;

static void* attn_worker(void* arg) {
  attn_job* J = (attn_job*)arg;
  const orc_problem* p = J->p;
  int d = p->head_dim;
  int64_t kmax = p->seqlen_k > 0 ? p->seqlen_k : 1;
  uint8_t* vis = (uint8_t*)malloc((size_t)kmax);
  double* s = (double*)malloc(sizeof(double) * (size_t)kmax);
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t n = J->begin; n < J->end; ++n) {
    int64_t t;
    int h;
    if (J->rows) {
      t = J->rows[2 * n];
      h = (int)J->rows[2 * n + 1];
    } else {
      t = n / p->heads_q;
      h = (int)(n % p->heads_q);
    }
    int b = owner_of_token(p, J->cu_q, t);
    int64_t q_off, q_len, k_off, k_len;
    sample_of(p, J->cu_q, J->cu_k, b, &q_off, &q_len, &k_off, &k_len);
    int64_t ql = t - q_off;
    int hm = p->mask_heads == 1 ? 0 : h;
    int g = h / (p->heads_q / p->heads_k);
    const int32_t* F = J->mf + (int64_t)hm * p->nfunc * p->total_q + t;
    orc_expand_row(F, p->total_q, p->nfunc, k_len, vis);
    const float* qrow = J->q + (t * p->heads_q + h) * (int64_t)d;
    double m = -INFINITY;
    int any = 0;
    for (int64_t kk = 0; kk < k_len; ++kk) {
      if (!vis[kk] || kk < J->k_lo || kk >= J->k_hi) continue;
      const float* krow = J->k + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
      double dot = 0.0;
      for (int i = 0; i < d; ++i) dot += (double)qrow[i] * (double)krow[i];
      s[kk] = apply_mod(J->mod, J->scale * dot, h, ql, kk);
      if (!any || s[kk] > m) m = s[kk];
      any = 1;
    }
    double* o = J->rows ? J->o + n * d : J->o + (t * p->heads_q + h) * (int64_t)d;
    double* lse = J->rows ? J->lse + n : J->lse + (int64_t)h * p->total_q + t;
    if (!any) {
      for (int i = 0; i < d; ++i) o[i] = 0.0;
      *lse = -INFINITY;
      continue;
    }
    double l = 0.0;
    for (int i = 0; i < d; ++i) acc[i] = 0.0;
    for (int64_t kk = 0; kk < k_len; ++kk) {
      if (!vis[kk] || kk < J->k_lo || kk >= J->k_hi) continue;
      double w = exp(s[kk] - m);
      l += w;
      const float* vrow = J->v + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
      for (int i = 0; i < d; ++i) acc[i] += w * (double)vrow[i];
    }
    for (int i = 0; i < d; ++i) o[i] = acc[i] / l;
    *lse = m + log(l);
  }
  free(vis);
  free(s);
  free(acc);
  return NULL;
}

static void attention_range(const orc_problem* p, const int32_t* mf, const int32_t* cu_q,
                            const int32_t* cu_k, const float* q, const float* k, const float* v,
                            double scale, const orc_mod* mod, int64_t k_lo, int64_t k_hi,
                            int64_t n, const int64_t* rows, double* o, double* lse,
                            int nthreads) {
  int64_t total = rows ? n : (int64_t)p->total_q * p->heads_q;
  if (nthreads < 1) nthreads = 1;
  if (total < nthreads) nthreads = total > 0 ? (int)total : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  attn_job* jobs = (attn_job*)malloc(sizeof(attn_job) * nthreads);
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (attn_job){p, mf, cu_q, cu_k, q, k, v, scale, mod, rows, k_lo, k_hi,
                         total * t / nthreads, total * (t + 1) / nthreads, o, lse};
    pthread_create(&th[t], NULL, attn_worker, &jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
}

/* Attention for selected rows (rows = n pairs (token, head)) or for every row
 * (rows = NULL, n ignored).  Inputs are float32 arrays holding the exact input
 * values ([tokens][heads][d]); everything is computed in double. */
void orc_attention(const orc_problem* p, const int32_t* mf, const int32_t* cu_q,
                   const int32_t* cu_k, const float* q, const float* k, const float* v,
                   double scale, int softcap_on, double softcap, int alibi_on,
                   const float* slopes, int alibi_first, int64_t n, const int64_t* rows,
                   double* o, double* lse, int nthreads) {
  orc_mod mod = {softcap_on, softcap, alibi_on, slopes, alibi_first};
  attention_range(p, mf, cu_q, cu_k, q, k, v, scale, &mod, 0, INT64_MAX, n, rows, o, lse,
                  nthreads);
}

/* Split-K partial state (Tessera page, "Split-K"): the same attention with the
 * visible set of every row cut to the sample-local keys k_lo <= k < k_hi.
 * O is normalized over those keys and LSE is the log of their sum of
 * exp(score); a row with none of its visible keys in the range gets O = 0 and
 * LSE = -inf.  Layouts as orc_attention. */
void orc_attention_part(const orc_problem* p, const int32_t* mf, const int32_t* cu_q,
                        const int32_t* cu_k, const float* q, const float* k, const float* v,
                        double scale, int softcap_on, double softcap, int alibi_on,
                        const float* slopes, int alibi_first, int64_t k_lo, int64_t k_hi,
                        int64_t n, const int64_t* rows, double* o, double* lse, int nthreads) {
  orc_mod mod = {softcap_on, softcap, alibi_on, slopes, alibi_first};
  attention_range(p, mf, cu_q, cu_k, q, k, v, scale, &mod, k_lo, k_hi, n, rows, o, lse,
                  nthreads);
}

/* Merge of Split-K partial states (Tessera page, "Split-K": partial states are
 * rescaled to a common maximum, summed and normalized).  Part s of row r has
 * O_s = o_parts[(s*nrows + r)*d ...] (normalized over its keys) and
 * L_s = lse_parts[s*nrows + r].  With M = max_s L_s:
 *   LSE = M + log(sum_s exp(L_s - M)),  O = sum_s exp(L_s - LSE) * O_s.
 * A part with L_s = -inf holds no keys and is not read; if every part is
 * empty the row gets O = 0 and LSE = -inf. */
void orc_merge(int nparts, int64_t nrows, int d, const double* o_parts,
               const double* lse_parts, double* o, double* lse) {
  for (int64_t r = 0; r < nrows; ++r) {
    double m = -INFINITY;
    for (int s = 0; s < nparts; ++s)
      if (lse_parts[s * nrows + r] > m) m = lse_parts[s * nrows + r];
    double* out = o + r * d;
    for (int i = 0; i < d; ++i) out[i] = 0.0;
    if (m == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double l = 0.0;
    for (int s = 0; s < nparts; ++s) {
      double ls = lse_parts[s * nrows + r];
      if (ls != -INFINITY) l += exp(ls - m);
    }
    double L = m + log(l);
    for (int s = 0; s < nparts; ++s) {
      double ls = lse_parts[s * nrows + r];
      if (ls == -INFINITY) continue;
      double w = exp(ls - L);
      const double* os = o_parts + (s * nrows + r) * d;
      for (int i = 0; i < d; ++i) out[i] += w * os[i];
    }
    lse[r] = L;
  }
}

/* ------------------------------------------------------------ backward */

/* d(score_mod)/d(scaled score) at scaled score t: the softcap's derivative at
 * its own input, 1 - tanh^2(u/c); ALiBi adds a constant. */
static double mod_slope(const orc_mod* m, double t, int h, int64_t q, int64_t k) {
  if (!m->softcap_on) return 1.0;
  double u = t;
  if (m->alibi_on && m->alibi_first) u += (double)m->slopes[h] * (double)(k - q);
  double th = tanh(u / m->softcap);
  return 1.0 - th * th;
}

typedef struct {
  const orc_problem* p;
  const int32_t* mf;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const float *q, *k, *v, *dout;
  double scale;
  const orc_mod* mod;
  int64_t begin, end;    /* items (sample, kv head) */
  double *dq, *dk, *dv;
} bwd_job;

/* One item = (sample b, kv head g): every Q row of b for every Q head of the
 * group.  For a row with visible keys k (scaled score x_k, modded t_k):
 *   P_k  = exp(t_k - LSE),              LSE = log sum_k exp(t_k)
 *   dP_k = dO . V_k
 *   dT_k = P_k (dP_k - sum_j P_j dP_j)  (softmax backward)
 *   dX_k = dT_k * dt/dx_k               (score_mod backward)
 *   dQ  += scale * dX_k * K_k,  dK_k += scale * dX_k * Q,  dV_k += P_k * dO.
 * dK and dV of the item's K rows receive only this item's contributions. */
static void* bwd_worker(void* arg) {
  bwd_job* J = (bwd_job*)arg;
  const orc_problem* p = J->p;
  int d = p->head_dim;
  int group = p->heads_q / p->heads_k;
  int64_t kmax = p->seqlen_k > 0 ? p->seqlen_k : 1;
  uint8_t* vis = (uint8_t*)malloc((size_t)kmax);
  double* x = (double*)malloc(sizeof(double) * (size_t)kmax);
  double* t = (double*)malloc(sizeof(double) * (size_t)kmax);
  double* P = (double*)malloc(sizeof(double) * (size_t)kmax);
  double* dP = (double*)malloc(sizeof(double) * (size_t)kmax);
  for (int64_t it = J->begin; it < J->end; ++it) {
    int b = (int)(it / p->heads_k);
    int g = (int)(it % p->heads_k);
    int64_t q_off, q_len, k_off, k_len;
    sample_of(p, J->cu_q, J->cu_k, b, &q_off, &q_len, &k_off, &k_len);
    for (int h = g * group; h < (g + 1) * group; ++h) {
      int hm = p->mask_heads == 1 ? 0 : h;
      for (int64_t ql = 0; ql < q_len; ++ql) {
        int64_t tok = q_off + ql;
        const int32_t* F = J->mf + (int64_t)hm * p->nfunc * p->total_q + tok;
        orc_expand_row(F, p->total_q, p->nfunc, k_len, vis);
        const float* qrow = J->q + (tok * p->heads_q + h) * (int64_t)d;
        const float* dorow = J->dout + (tok * p->heads_q + h) * (int64_t)d;
        double m = -INFINITY;
        int any = 0;
        for (int64_t kk = 0; kk < k_len; ++kk) {
          if (!vis[kk]) continue;
          const float* krow = J->k + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
          double dot = 0.0;
          for (int i = 0; i < d; ++i) dot += (double)qrow[i] * (double)krow[i];
          x[kk] = J->scale * dot;
          t[kk] = apply_mod(J->mod, x[kk], h, ql, kk);
          if (!any || t[kk] > m) m = t[kk];
          any = 1;
        }
        if (!any) continue;   /* nothing visible: no gradient flows */
        double l = 0.0;
        for (int64_t kk = 0; kk < k_len; ++kk)
          if (vis[kk]) l += exp(t[kk] - m);
        double lse = m + log(l);
        double Dsum = 0.0;
        for (int64_t kk = 0; kk < k_len; ++kk) {
          if (!vis[kk]) continue;
          const float* vrow = J->v + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
          P[kk] = exp(t[kk] - lse);
          double dot = 0.0;
          for (int i = 0; i < d; ++i) dot += (double)dorow[i] * (double)vrow[i];
          dP[kk] = dot;
          Dsum += P[kk] * dP[kk];
        }
        double* dqrow = J->dq + (tok * p->heads_q + h) * (int64_t)d;
        for (int64_t kk = 0; kk < k_len; ++kk) {
          if (!vis[kk]) continue;
          double dT = P[kk] * (dP[kk] - Dsum);
          double dX = dT * mod_slope(J->mod, x[kk], h, ql, kk);
          const float* krow = J->k + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
          double* dkrow = J->dk + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
          double* dvrow = J->dv + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
          for (int i = 0; i < d; ++i) {
            dqrow[i] += J->scale * dX * (double)krow[i];
            dkrow[i] += J->scale * dX * (double)qrow[i];
            dvrow[i] += P[kk] * (double)dorow[i];
          }
        }
      }
    }
  }
  free(vis);
  free(x);
  free(t);
  free(P);
  free(dP);
  return NULL;
}

/* Gradients of the attention output O with respect to Q, K and V for the
 * incoming gradient dout ([total_q][Hq][d]).  dq is [total_q][Hq][d], dk and
 * dv [total_k][Hk][d]; all three are overwritten.  Same inputs as
 * orc_attention; the forward quantities are recomputed here. */
void orc_attention_bwd(const orc_problem* p, const int32_t* mf, const int32_t* cu_q,
                       const int32_t* cu_k, const float* q, const float* k, const float* v,
                       const float* dout, double scale, int softcap_on, double softcap,
                       int alibi_on, const float* slopes, int alibi_first, double* dq,
                       double* dk, double* dv, int nthreads) {
  orc_mod mod = {softcap_on, softcap, alibi_on, slopes, alibi_first};
  int d = p->head_dim;
  memset(dq, 0, sizeof(double) * (size_t)p->total_q * p->heads_q * d);
  memset(dk, 0, sizeof(double) * (size_t)p->total_k * p->heads_k * d);
  memset(dv, 0, sizeof(double) * (size_t)p->total_k * p->heads_k * d);
  int64_t items = (int64_t)p->batch * p->heads_k;
  if (nthreads < 1) nthreads = 1;
  if (items < nthreads) nthreads = items > 0 ? (int)items : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  bwd_job* jobs = (bwd_job*)malloc(sizeof(bwd_job) * nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = (bwd_job){p, mf, cu_q, cu_k, q, k, v, dout, scale, &mod,
                        items * i / nthreads, items * (i + 1) / nthreads, dq, dk, dv};
    pthread_create(&th[i], NULL, bwd_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
}

typedef struct {
  const orc_problem* p;
  const int32_t* mf;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const float *q, *k, *v, *dout;
  double scale;
  const orc_mod* mod;
  const int64_t* rows;   /* pairs (token, head) */
  int64_t begin, end;
  double* dq;            /* [n][d] */
} bwd_rows_job;

/* dQ of selected rows only: the same per-row chain rule as bwd_worker (a
 * row's dQ depends on that row alone). */
static void* bwd_rows_worker(void* arg) {
  bwd_rows_job* J = (bwd_rows_job*)arg;
  const orc_problem* p = J->p;
  int d = p->head_dim;
  int group = p->heads_q / p->heads_k;
  int64_t kmax = p->seqlen_k > 0 ? p->seqlen_k : 1;
  uint8_t* vis = (uint8_t*)malloc((size_t)kmax);
  double* x = (double*)malloc(sizeof(double) * (size_t)kmax);
  double* t = (double*)malloc(sizeof(double) * (size_t)kmax);
  double* dP = (double*)malloc(sizeof(double) * (size_t)kmax);
  for (int64_t n = J->begin; n < J->end; ++n) {
    int64_t tok = J->rows[2 * n];
    int h = (int)J->rows[2 * n + 1];
    double* dqrow = J->dq + n * d;
    for (int i = 0; i < d; ++i) dqrow[i] = 0.0;
    int b = owner_of_token(p, J->cu_q, tok);
    int64_t q_off, q_len, k_off, k_len;
    sample_of(p, J->cu_q, J->cu_k, b, &q_off, &q_len, &k_off, &k_len);
    int64_t ql = tok - q_off;
    int hm = p->mask_heads == 1 ? 0 : h;
    int g = h / group;
    const int32_t* F = J->mf + (int64_t)hm * p->nfunc * p->total_q + tok;
    orc_expand_row(F, p->total_q, p->nfunc, k_len, vis);
    const float* qrow = J->q + (tok * p->heads_q + h) * (int64_t)d;
    const float* dorow = J->dout + (tok * p->heads_q + h) * (int64_t)d;
    double m = -INFINITY;
    int any = 0;
    for (int64_t kk = 0; kk < k_len; ++kk) {
      if (!vis[kk]) continue;
      const float* krow = J->k + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
      double dot = 0.0;
      for (int i = 0; i < d; ++i) dot += (double)qrow[i] * (double)krow[i];
      x[kk] = J->scale * dot;
      t[kk] = apply_mod(J->mod, x[kk], h, ql, kk);
      if (!any || t[kk] > m) m = t[kk];
      any = 1;
    }
    if (!any) continue;
    double l = 0.0;
    for (int64_t kk = 0; kk < k_len; ++kk)
      if (vis[kk]) l += exp(t[kk] - m);
    double lse = m + log(l);
    double Dsum = 0.0;
    for (int64_t kk = 0; kk < k_len; ++kk) {
      if (!vis[kk]) continue;
      const float* vrow = J->v + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
      double dot = 0.0;
      for (int i = 0; i < d; ++i) dot += (double)dorow[i] * (double)vrow[i];
      dP[kk] = dot;
      Dsum += exp(t[kk] - lse) * dot;
    }
    for (int64_t kk = 0; kk < k_len; ++kk) {
      if (!vis[kk]) continue;
      double P = exp(t[kk] - lse);
      double dX = P * (dP[kk] - Dsum) * mod_slope(J->mod, x[kk], h, ql, kk);
      const float* krow = J->k + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
      for (int i = 0; i < d; ++i) dqrow[i] += J->scale * dX * (double)krow[i];
    }
  }
  free(vis);
  free(x);
  free(t);
  free(dP);
  return NULL;
}

/* dQ [n][d] of the n selected (token, head) rows. */
void orc_attention_bwd_dq_rows(const orc_problem* p, const int32_t* mf, const int32_t* cu_q,
                               const int32_t* cu_k, const float* q, const float* k,
                               const float* v, const float* dout, double scale, int softcap_on,
                               double softcap, int alibi_on, const float* slopes,
                               int alibi_first, int64_t n, const int64_t* rows, double* dq,
                               int nthreads) {
  orc_mod mod = {softcap_on, softcap, alibi_on, slopes, alibi_first};
  if (nthreads < 1) nthreads = 1;
  if (n < nthreads) nthreads = n > 0 ? (int)n : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  bwd_rows_job* jobs = (bwd_rows_job*)malloc(sizeof(bwd_rows_job) * nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = (bwd_rows_job){p, mf, cu_q, cu_k, q, k, v, dout, scale, &mod, rows,
                             n * i / nthreads, n * (i + 1) / nthreads, dq};
    pthread_create(&th[i], NULL, bwd_rows_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
}

/* dK and dV of selected K rows: rows = n pairs (K token, KV head g).  The
 * same chain rule as bwd_worker, restricted to the keys asked for: for every
 * Q head h of g's group and every Q row q of the key's sample (in that
 * order, as bwd_worker adds them), the row's scores, log-sum-exp and
 * sum_j P_j dP_j are recomputed from that row alone, and a row that sees the
 * key adds scale * dX_qk * Q_q to its dK and P_qk * dO_q to its dV. */
typedef struct {
  const orc_problem* p;
  const int32_t* mf;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const float *q, *k, *v, *dout;
  double scale;
  const orc_mod* mod;
  const int64_t* rows;      /* pairs (k token, kv head) */
  const int64_t* item_of;   /* [n] item (sample * Hk + kv head) of each row */
  const int64_t* items;     /* distinct items, this job's share: items[begin..end) */
  int64_t n, begin, end;
  double *dk, *dv;          /* [n][d] */
} dkdv_rows_job;

static int owner_of_k_token(const orc_problem* p, const int32_t* cu_k, int64_t t) {
  if (p->layout == ORC_BSHD)
    return t >= 0 && t < (int64_t)p->batch * p->seqlen_k ? (int)(t / p->seqlen_k) : -1;
  for (int b = 0; b < p->batch; ++b)
    if (t >= cu_k[b] && t < cu_k[b + 1]) return b;
  return -1;
}

static void* dkdv_rows_worker(void* arg) {
  dkdv_rows_job* J = (dkdv_rows_job*)arg;
  const orc_problem* p = J->p;
  int d = p->head_dim;
  int group = p->heads_q / p->heads_k;
  int64_t kmax = p->seqlen_k > 0 ? p->seqlen_k : 1;
  uint8_t* vis = (uint8_t*)malloc((size_t)kmax);
  double* x = (double*)malloc(sizeof(double) * (size_t)kmax);
  double* t = (double*)malloc(sizeof(double) * (size_t)kmax);
  double* P = (double*)malloc(sizeof(double) * (size_t)kmax);
  double* dP = (double*)malloc(sizeof(double) * (size_t)kmax);
  for (int64_t it = J->begin; it < J->end; ++it) {
    int64_t item = J->items[it];
    int b = (int)(item / p->heads_k);
    int g = (int)(item % p->heads_k);
    int64_t q_off, q_len, k_off, k_len;
    sample_of(p, J->cu_q, J->cu_k, b, &q_off, &q_len, &k_off, &k_len);
    for (int h = g * group; h < (g + 1) * group; ++h) {
      int hm = p->mask_heads == 1 ? 0 : h;
      for (int64_t ql = 0; ql < q_len; ++ql) {
        int64_t tok = q_off + ql;
        const int32_t* F = J->mf + (int64_t)hm * p->nfunc * p->total_q + tok;
        orc_expand_row(F, p->total_q, p->nfunc, k_len, vis);
        const float* qrow = J->q + (tok * p->heads_q + h) * (int64_t)d;
        const float* dorow = J->dout + (tok * p->heads_q + h) * (int64_t)d;
        double m = -INFINITY;
        int any = 0;
        for (int64_t kk = 0; kk < k_len; ++kk) {
          if (!vis[kk]) continue;
          const float* krow = J->k + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
          double dot = 0.0;
          for (int i = 0; i < d; ++i) dot += (double)qrow[i] * (double)krow[i];
          x[kk] = J->scale * dot;
          t[kk] = apply_mod(J->mod, x[kk], h, ql, kk);
          if (!any || t[kk] > m) m = t[kk];
          any = 1;
        }
        if (!any) continue;   /* nothing visible: no gradient flows */
        double l = 0.0;
        for (int64_t kk = 0; kk < k_len; ++kk)
          if (vis[kk]) l += exp(t[kk] - m);
        double lse = m + log(l);
        double Dsum = 0.0;
        for (int64_t kk = 0; kk < k_len; ++kk) {
          if (!vis[kk]) continue;
          const float* vrow = J->v + ((k_off + kk) * p->heads_k + g) * (int64_t)d;
          P[kk] = exp(t[kk] - lse);
          double dot = 0.0;
          for (int i = 0; i < d; ++i) dot += (double)dorow[i] * (double)vrow[i];
          dP[kk] = dot;
          Dsum += P[kk] * dP[kk];
        }
        for (int64_t r = 0; r < J->n; ++r) {
          if (J->item_of[r] != item) continue;
          int64_t kk = J->rows[2 * r] - k_off;
          if (!vis[kk]) continue;
          double dT = P[kk] * (dP[kk] - Dsum);
          double dX = dT * mod_slope(J->mod, x[kk], h, ql, kk);
          double* dkrow = J->dk + r * d;
          double* dvrow = J->dv + r * d;
          for (int i = 0; i < d; ++i) {
            dkrow[i] += J->scale * dX * (double)qrow[i];
            dvrow[i] += P[kk] * (double)dorow[i];
          }
        }
      }
    }
  }
  free(vis);
  free(x);
  free(t);
  free(P);
  free(dP);
  return NULL;
}

/* dK, dV [n][d] of the n selected (K token, KV head) rows.  Returns 0, or -1
 * for a K token outside every sample. */
int orc_attention_bwd_dkdv_rows(const orc_problem* p, const int32_t* mf, const int32_t* cu_q,
                                const int32_t* cu_k, const float* q, const float* k,
                                const float* v, const float* dout, double scale, int softcap_on,
                                double softcap, int alibi_on, const float* slopes,
                                int alibi_first, int64_t n, const int64_t* rows, double* dk,
                                double* dv, int nthreads) {
  orc_mod mod = {softcap_on, softcap, alibi_on, slopes, alibi_first};
  int d = p->head_dim;
  memset(dk, 0, sizeof(double) * (size_t)(n > 0 ? n : 1) * d);
  memset(dv, 0, sizeof(double) * (size_t)(n > 0 ? n : 1) * d);
  if (n <= 0) return 0;
  int64_t* item_of = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
  int64_t* items = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
  int64_t nitems = 0;
  for (int64_t r = 0; r < n; ++r) {
    int b = owner_of_k_token(p, cu_k, rows[2 * r]);
    if (b < 0 || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= p->heads_k) {
      free(item_of);
      free(items);
      return -1;
    }
    item_of[r] = (int64_t)b * p->heads_k + rows[2 * r + 1];
    int seen = 0;
    for (int64_t i = 0; i < nitems; ++i) seen |= items[i] == item_of[r];
    if (!seen) items[nitems++] = item_of[r];
  }
  if (nthreads < 1) nthreads = 1;
  if (nitems < nthreads) nthreads = (int)nitems;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  dkdv_rows_job* jobs = (dkdv_rows_job*)malloc(sizeof(dkdv_rows_job) * nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = (dkdv_rows_job){p, mf, cu_q, cu_k, q, k, v, dout, scale, &mod, rows, item_of, items,
                              n, nitems * i / nthreads, nitems * (i + 1) / nthreads, dk, dv};
    pthread_create(&th[i], NULL, dkdv_rows_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  free(item_of);
  free(items);
  return 0;
}
