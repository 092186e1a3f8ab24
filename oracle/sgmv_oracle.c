/*
 * sgmv_oracle.c -- plain fp64 CPU oracle for SGMV expand-slice.
 *
 * TEST INFRASTRUCTURE ONLY (see sgmv_oracle.h).  Nothing here is tuned:
 * the computation is the definition written out as loops, split over output
 * rows only (rows are independent) with plain POSIX threads.  Build without
 * fast-math and with -ffp-contract=off.
 *
 * Definition followed (wiki page "Implementation: Predibase Lorax SGMV
 * Expand Slice Kernel"):
 *   - Description: for segment b and token m, row start_b + m of the output
 *     slice is updated with input[start_b + m] times lora_B[idx[b]].
 *   - I/O Contract, Inputs: lora_B is (lora_num, slice_size, rank), so the
 *     contraction runs over rank: y[n] = sum_k x[k] * B[a][n][k];
 *     b_seq_start_loc gives each segment's first row, seq_len_tensor its
 *     length; lora index -1 marks a segment without an adapter (rows
 *     untouched);
 *     add_inputs=false (default) overwrites, true accumulates.
 *   - Description / Signature (CAST_TYPE, the mixed-precision cast):
 *     float32 inputs are rounded to the 16-bit weight type before the
 *     products.
 * Readings where the page is silent are listed beside the code below.
 */
#define _GNU_SOURCE
#include "sgmv_oracle.h"

#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* IEEE 754 binary formats: exponent field width and trailing significand  */
/* width.  bfloat16 keeps binary32's exponent with a 7-bit significand.     */
/* ---------------------------------------------------------------------- */
static int format_of(int dtype, int* ebits, int* mbits) {
  switch (dtype) {
    case ORC_F16:  *ebits = 5; *mbits = 10; return 1;
    case ORC_BF16: *ebits = 8; *mbits = 7;  return 1;
    case ORC_F32:  *ebits = 8; *mbits = 23; return 1;
    default: return 0;
  }
}

double orc_decode(int dtype, uint32_t bits) {
  int eb, mb;
  if (!format_of(dtype, &eb, &mb)) return NAN;
  const int bias = (1 << (eb - 1)) - 1;
  const uint32_t emask = (1u << eb) - 1u;
  const uint32_t sign = (bits >> (eb + mb)) & 1u;
  const uint32_t e = (bits >> mb) & emask;
  const uint32_t m = bits & ((1u << mb) - 1u);
  double mag;
  if (e == emask) {
    mag = m ? NAN : INFINITY;
  } else if (e == 0) {
    /* subnormal: 0.m * 2^(1 - bias) */
    mag = ldexp((double)m, 1 - bias - mb);
  } else {
    /* normal: 1.m * 2^(e - bias) */
    mag = ldexp((double)((1u << mb) + m), (int)e - bias - mb);
  }
  return sign ? -mag : mag;
}

uint32_t orc_encode(int dtype, double v) {
  int eb, mb;
  if (!format_of(dtype, &eb, &mb)) return 0;
  const int bias = (1 << (eb - 1)) - 1;
  const uint32_t emask = (1u << eb) - 1u;
  const uint32_t sbit = (signbit(v) ? 1u : 0u) << (eb + mb);
  if (isnan(v)) return sbit | (emask << mb) | (1u << (mb - 1));
  const double a = fabs(v);
  if (isinf(a)) return sbit | (emask << mb);
  if (a == 0.0) return sbit;

  const int emin = 1 - bias;          /* exponent of the smallest normal   */
  int e2;
  (void)frexp(a, &e2);                /* a = f * 2^e2, 0.5 <= f < 1         */
  const int ea = e2 - 1;              /* floor(log2(a))                     */
  /* Spacing of the representable values around a: 2^(max(ea, emin) - mb). */
  const int qexp = (ea < emin ? emin : ea) - mb;
  const double scaled = ldexp(a, -qexp);   /* exact (power-of-two scaling)  */
  double r = floor(scaled);
  const double frac = scaled - r;          /* exact: scaled < 2^(mb + 1)    */
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;  /* ties to even */
  uint64_t ri = (uint64_t)r;

  uint32_t field, mant;
  if (ea < emin) {
    /* Subnormal range; rounding up to 2^mb reaches the smallest normal. */
    if (ri == (1ull << mb)) { field = 1; mant = 0; }
    else { field = 0; mant = (uint32_t)ri; }
  } else {
    int eu = ea;
    if (ri == (2ull << mb)) { eu += 1; ri = 1ull << mb; }   /* carry into next binade */
    if (eu > bias) return sbit | (emask << mb);            /* overflow -> infinity   */
    field = (uint32_t)(eu + bias);
    mant = (uint32_t)(ri - (1ull << mb));
  }
  return sbit | (field << mb) | mant;
}

void orc_decode_array(int dtype, const uint32_t* bits, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_decode(dtype, bits[i]);
}

void orc_encode_array(int dtype, const double* v, uint32_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_encode(dtype, v[i]);
}

static uint32_t load_bits(int dtype, const void* base, int64_t i) {
  if (dtype == ORC_F32) {
    uint32_t b;
    memcpy(&b, (const char*)base + 4 * i, 4);
    return b;
  }
  uint16_t h;
  memcpy(&h, (const char*)base + 2 * i, 2);
  return h;
}

static void store_bits(int dtype, void* base, int64_t i, uint32_t bits) {
  if (dtype == ORC_F32) {
    memcpy((char*)base + 4 * i, &bits, 4);
  } else {
    uint16_t h = (uint16_t)bits;
    memcpy((char*)base + 2 * i, &h, 2);
  }
}

int orc_threads(int threads) {
  if (threads > 0) return threads;
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof set, &set) == 0 && CPU_COUNT(&set) > 0) return CPU_COUNT(&set);
  return 1;
}

/* Run fn(ctx, worker, begin, end) over `workers` contiguous chunks of
 * [0, n); chunk 0 runs on the calling thread.  A chunk whose thread cannot
 * be started runs on the calling thread after the others are joined. */
typedef void (*chunk_fn)(void* ctx, int worker, int64_t begin, int64_t end);
typedef struct {
  chunk_fn fn;
  void* ctx;
  int worker;
  int64_t begin, end;
} chunk_job;

static void* chunk_main(void* p) {
  chunk_job* j = (chunk_job*)p;
  j->fn(j->ctx, j->worker, j->begin, j->end);
  return NULL;
}

static int run_chunks(int workers, int64_t n, chunk_fn fn, void* ctx) {
  chunk_job* jobs = (chunk_job*)malloc(sizeof(chunk_job) * (size_t)workers);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)workers);
  int* started = (int*)calloc((size_t)workers, sizeof(int));
  if (!jobs || !th || !started) {
    free(jobs); free(th); free(started);
    return ORC_NO_MEMORY;
  }
  for (int i = 0; i < workers; ++i) {
    jobs[i].fn = fn;
    jobs[i].ctx = ctx;
    jobs[i].worker = i;
    jobs[i].begin = n * i / workers;
    jobs[i].end = n * (i + 1) / workers;
  }
  for (int i = 1; i < workers; ++i)
    started[i] = pthread_create(&th[i], NULL, chunk_main, &jobs[i]) == 0;
  chunk_main(&jobs[0]);
  for (int i = 1; i < workers; ++i) {
    if (started[i]) pthread_join(th[i], NULL);
    else chunk_main(&jobs[i]);
  }
  free(jobs); free(th); free(started);
  return ORC_OK;
}

static int workers_for(int threads, int64_t n) {
  int w = orc_threads(threads);
  if (n < w) w = n > 0 ? (int)n : 1;
  return w;
}

/* ---------------------------------------------------------------------- */
/* Argument checks and the row -> segment map.                             */
/* ---------------------------------------------------------------------- */
static int check_args(const orc_slice* s, int ns, int64_t K, int64_t L, int out_dtype,
                      int64_t T, int64_t H, int64_t out_stride, int64_t batches) {
  int eb, mb;
  if (!s || ns < 1 || K < 1 || L < 0 || T < 0 || H < 0 || out_stride < H || batches < 0)
    return ORC_BAD_ARGUMENT;
  if (!format_of(out_dtype, &eb, &mb)) return ORC_BAD_ARGUMENT;
  for (int i = 0; i < ns; ++i) {
    /* Weights are float16 or bfloat16; inputs are the weight type or
     * float32 (I/O Contract, Inputs).  A 16-bit input of the other 16-bit
     * type is not a case the page describes and is rejected. */
    if (s[i].w_dtype != ORC_F16 && s[i].w_dtype != ORC_BF16) return ORC_BAD_ARGUMENT;
    if (s[i].x_dtype != s[i].w_dtype && s[i].x_dtype != ORC_F32) return ORC_BAD_ARGUMENT;
    if (s[i].N < 0 || s[i].offset < 0 || s[i].offset + s[i].N > H) return ORC_BAD_ARGUMENT;
    if (s[i].x_stride < K) return ORC_BAD_ARGUMENT;
    for (int j = 0; j < i; ++j) {
      if (s[i].N == 0 || s[j].N == 0) continue;
      if (s[i].offset < s[j].offset + s[j].N && s[j].offset < s[i].offset + s[i].N)
        return ORC_BAD_ARGUMENT;  /* overlapping column windows */
    }
  }
  return ORC_OK;
}

/* owner[t] = segment that writes row t, or -1.  A segment is active when its
 * adapter index is not -1 and its length is positive.  Active segments must
 * lie inside [0, T) and be pairwise disjoint. */
static int build_owner(int64_t T, int64_t L, const int64_t* start, const int64_t* lens,
                       const int64_t* idx, int64_t batches, int64_t** owner_out) {
  int64_t* owner = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
  if (!owner) return ORC_NO_MEMORY;
  for (int64_t t = 0; t < T; ++t) owner[t] = -1;
  for (int64_t b = 0; b < batches; ++b) {
    if (lens[b] < 0) { free(owner); return ORC_BAD_SEGMENT; }
    if (idx[b] < -1 || idx[b] >= L) { free(owner); return ORC_BAD_INDEX; }
    if (idx[b] == -1 || lens[b] == 0) continue;  /* no LoRA, or nothing to do */
    if (start[b] < 0 || start[b] > T - lens[b]) { free(owner); return ORC_BAD_SEGMENT; }
    for (int64_t m = 0; m < lens[b]; ++m) {
      if (owner[start[b] + m] != -1) { free(owner); return ORC_BAD_SEGMENT; }
      owner[start[b] + m] = b;
    }
  }
  *owner_out = owner;
  return ORC_OK;
}

/* Exact values of a whole (L, N, K) weight stack. */
static double* decode_stack(const orc_slice* s, int64_t K, int64_t L) {
  const int64_t n = L * s->N * K;
  double* w = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  if (!w) return NULL;
  for (int64_t i = 0; i < n; ++i) w[i] = orc_decode(s->w_dtype, load_bits(s->w_dtype, s->w, i));
  return w;
}

/* Value of input element x[t][k] as it enters the product: float32 inputs
 * are first rounded to the weight type (CAST_TYPE). */
static double input_value(const orc_slice* s, int64_t t, int64_t k) {
  const double v = orc_decode(s->x_dtype, load_bits(s->x_dtype, s->x, t * s->x_stride + k));
  if (s->x_dtype == ORC_F32) return orc_decode(s->w_dtype, orc_encode(s->w_dtype, v));
  return v;
}

/* Exact (fp64) slice value for row t, column n: the prior value when
 * accumulating, plus the dot product over rank.  Products of 16-bit values
 * are exact in fp64; the sum carries at most ~K ulp(fp64) of error. */
static double slice_value(const orc_slice* s, const double* wval, const double* xrow,
                          int64_t K, int64_t a, int64_t n, int add, double prior) {
  double r = add ? prior : 0.0;
  const double* wrow = wval + (a * s->N + n) * K;
  for (int64_t k = 0; k < K; ++k) r += xrow[k] * wrow[k];
  return r;
}

typedef struct {
  const orc_slice* s;
  const double* wval;
  int64_t K, out_stride, ref_base;
  void* out;
  int out_dtype, add;
  const int64_t* owner;
  const int64_t* idx;
  double* ref;
  int failed;
} expand_ctx;

/* Rows [begin, end) of one slice. */
static void expand_rows(void* p, int worker, int64_t begin, int64_t end) {
  (void)worker;
  expand_ctx* c = (expand_ctx*)p;
  const orc_slice* s = c->s;
  double* xrow = (double*)malloc(sizeof(double) * (size_t)c->K);
  if (!xrow) {
    __atomic_store_n(&c->failed, 1, __ATOMIC_RELAXED);
    return;
  }
  for (int64_t t = begin; t < end; ++t) {
    const int64_t b = c->owner[t];
    if (b < 0) continue;  /* not in an active segment: untouched */
    const int64_t a = c->idx[b];
    for (int64_t k = 0; k < c->K; ++k) xrow[k] = input_value(s, t, k);
    for (int64_t n = 0; n < s->N; ++n) {
      const int64_t o = t * c->out_stride + s->offset + n;
      const double prior =
          c->add ? orc_decode(c->out_dtype, load_bits(c->out_dtype, c->out, o)) : 0.0;
      const double r = slice_value(s, c->wval, xrow, c->K, a, n, c->add, prior);
      if (c->ref) c->ref[c->ref_base + t * s->N + n] = r;
      store_bits(c->out_dtype, c->out, o, orc_encode(c->out_dtype, r));
    }
  }
  free(xrow);
}

int orc_expand(const orc_slice* slices, int num_slices, int64_t K, int64_t L,
               void* out, int out_dtype, int64_t T, int64_t H, int64_t out_stride,
               const int64_t* start, const int64_t* lens, const int64_t* idx,
               int64_t batches, int add_inputs, double* ref, int threads) {
  int rc = check_args(slices, num_slices, K, L, out_dtype, T, H, out_stride, batches);
  if (rc != ORC_OK) return rc;
  int64_t* owner = NULL;
  rc = build_owner(T, L, start, lens, idx, batches, &owner);
  if (rc != ORC_OK) return rc;

  int64_t ref_base = 0;
  for (int si = 0; si < num_slices; ++si) {
    const orc_slice* s = &slices[si];
    double* wval = decode_stack(s, K, L);
    if (!wval) { free(owner); return ORC_NO_MEMORY; }
    expand_ctx c = {s, wval, K, out_stride, ref_base, out, out_dtype, add_inputs,
                    owner, idx, ref, 0};
    rc = run_chunks(workers_for(threads, T), T, expand_rows, &c);
    free(wval);
    if (rc != ORC_OK || c.failed) { free(owner); return ORC_NO_MEMORY; }
    ref_base += T * s->N;
  }
  free(owner);
  return ORC_OK;
}

/* ---------------------------------------------------------------------- */
/* Streaming comparator.                                                    */
/* ---------------------------------------------------------------------- */
static int is_nonfinite_bits(int dtype, uint32_t bits) {
  int eb = 0, mb = 0;
  if (!format_of(dtype, &eb, &mb)) return 1;
  const uint32_t emask = (1u << eb) - 1u;
  return ((bits >> mb) & emask) == emask;
}

static int is_nan_bits(int dtype, uint32_t bits) {
  int eb = 0, mb = 0;
  if (!format_of(dtype, &eb, &mb)) return 1;
  return is_nonfinite_bits(dtype, bits) && (bits & ((1u << mb) - 1u)) != 0;
}

static void note_bad(orc_report* r, int64_t row, int64_t col) {
  if (r->first_bad_row < 0 || row < r->first_bad_row ||
      (row == r->first_bad_row && col < r->first_bad_col)) {
    r->first_bad_row = row;
    r->first_bad_col = col;
  }
}

typedef struct {
  const orc_slice* slices;
  int num_slices;
  double** wval;
  int64_t K, H, out_stride;
  const void* prior;
  const void* cand;
  int out_dtype, add;
  double atol, rtol;
  const int64_t* owner;
  const int64_t* idx;
  const int64_t* rows;
  const int* col_slice;
  orc_report* part;  /* one per worker */
  int failed;
} check_ctx;

/* Compare rows [begin, end) of the row list (or of the output). */
static void check_rows(void* p, int worker, int64_t begin, int64_t end) {
  check_ctx* c = (check_ctx*)p;
  orc_report* mine = &c->part[worker];
  const int64_t K = c->K;
  const int od = c->out_dtype;
  double* xrows = (double*)malloc(sizeof(double) * (size_t)(K * c->num_slices));
  if (!xrows) {
    __atomic_store_n(&c->failed, 1, __ATOMIC_RELAXED);
    return;
  }
  for (int64_t i = begin; i < end; ++i) {
    const int64_t t = c->rows ? c->rows[i] : i;
    const int64_t b = c->owner[t];
    if (b >= 0)
      for (int si = 0; si < c->num_slices; ++si)
        for (int64_t k = 0; k < K; ++k) xrows[si * K + k] = input_value(&c->slices[si], t, k);
    for (int64_t col = 0; col < c->H; ++col) {
      const int64_t o = t * c->out_stride + col;
      const uint32_t cb = load_bits(od, c->cand, o);
      const uint32_t pb = load_bits(od, c->prior, o);
      const int si = c->col_slice[col];
      if (b < 0 || si < 0) {
        /* untouched region: bit-identical to the prior output */
        mine->checked_untouched++;
        if (cb != pb) { mine->bad_untouched++; note_bad(mine, t, col); }
        continue;
      }
      const orc_slice* s = &c->slices[si];
      const double r = slice_value(s, c->wval[si], xrows + si * K, K, c->idx[b],
                                   col - s->offset, c->add, orc_decode(od, pb));
      const uint32_t rb = orc_encode(od, r);
      mine->checked_values++;
      if (is_nonfinite_bits(od, rb)) {
        const int ok = is_nan_bits(od, rb) ? is_nan_bits(od, cb) : (cb == rb);
        if (!ok) { mine->bad_values++; note_bad(mine, t, col); }
        continue;
      }
      const double cv = orc_decode(od, cb);
      if (!isfinite(cv)) { mine->bad_values++; note_bad(mine, t, col); continue; }
      const double err = fabs(cv - r);
      const double allowed = c->atol + c->rtol * fabs(r);
      if (err > mine->max_abs_err) mine->max_abs_err = err;
      if (err / allowed > mine->max_tol_ratio) mine->max_tol_ratio = err / allowed;
      if (!(err <= allowed)) { mine->bad_values++; note_bad(mine, t, col); }
    }
  }
  free(xrows);
}

int orc_check(const orc_slice* slices, int num_slices, int64_t K, int64_t L,
              const void* prior, const void* cand, int out_dtype,
              int64_t T, int64_t H, int64_t out_stride,
              const int64_t* start, const int64_t* lens, const int64_t* idx,
              int64_t batches, int add_inputs, double atol, double rtol,
              const int64_t* rows, int64_t num_rows, int threads,
              orc_report* report) {
  if (!report) return ORC_BAD_ARGUMENT;
  int rc = check_args(slices, num_slices, K, L, out_dtype, T, H, out_stride, batches);
  if (rc != ORC_OK) return rc;
  if (rows) {
    for (int64_t i = 0; i < num_rows; ++i)
      if (rows[i] < 0 || rows[i] >= T) return ORC_BAD_ARGUMENT;
  }
  int64_t* owner = NULL;
  rc = build_owner(T, L, start, lens, idx, batches, &owner);
  if (rc != ORC_OK) return rc;

  const int64_t nrows = rows ? num_rows : T;
  const int workers = workers_for(threads, nrows);
  double** wval = (double**)calloc((size_t)num_slices, sizeof(double*));
  int* col_slice = (int*)malloc(sizeof(int) * (size_t)(H > 0 ? H : 1));
  orc_report* part = (orc_report*)calloc((size_t)workers, sizeof(orc_report));
  if (!wval || !col_slice || !part) rc = ORC_NO_MEMORY;
  for (int si = 0; rc == ORC_OK && si < num_slices; ++si) {
    wval[si] = decode_stack(&slices[si], K, L);
    if (!wval[si]) rc = ORC_NO_MEMORY;
  }
  if (rc == ORC_OK) {
    /* column -> slice map for one row (-1 = outside every slice) */
    for (int64_t col = 0; col < H; ++col) col_slice[col] = -1;
    for (int si = 0; si < num_slices; ++si)
      for (int64_t n = 0; n < slices[si].N; ++n) col_slice[slices[si].offset + n] = si;
    for (int w = 0; w < workers; ++w) part[w].first_bad_row = part[w].first_bad_col = -1;
    check_ctx c = {slices, num_slices, wval, K, H, out_stride, prior, cand, out_dtype,
                   add_inputs, atol, rtol, owner, idx, rows, col_slice, part, 0};
    rc = run_chunks(workers, nrows, check_rows, &c);
    if (rc == ORC_OK && c.failed) rc = ORC_NO_MEMORY;
  }
  if (rc == ORC_OK) {
    orc_report total;
    memset(&total, 0, sizeof total);
    total.first_bad_row = total.first_bad_col = -1;
    for (int w = 0; w < workers; ++w) {
      const orc_report* m = &part[w];
      total.checked_values += m->checked_values;
      total.checked_untouched += m->checked_untouched;
      total.bad_values += m->bad_values;
      total.bad_untouched += m->bad_untouched;
      if (m->max_abs_err > total.max_abs_err) total.max_abs_err = m->max_abs_err;
      if (m->max_tol_ratio > total.max_tol_ratio) total.max_tol_ratio = m->max_tol_ratio;
      if (m->first_bad_row >= 0) note_bad(&total, m->first_bad_row, m->first_bad_col);
    }
    *report = total;
  }
  if (wval)
    for (int si = 0; si < num_slices; ++si) free(wval[si]);
  free(wval);
  free(col_slice);
  free(part);
  free(owner);
  return rc;
}

/* ---------------------------------------------------------------------- */
/* LoRA-A projection (shrink), see sgmv_oracle.h.                           */
/* ---------------------------------------------------------------------- */
typedef struct {
  const void* x;
  int x_dtype, a_dtype, out_dtype;
  int64_t x_stride, H, K, T;
  const orc_shrink_slice* s;
  int ns;
  const double* a_tab;   /* exact value of every 16-bit weight pattern */
  const double* x_tab;   /* same for 16-bit inputs (NULL for float32)   */
  const int64_t* owner;
  const int64_t* idx;
  const int64_t* rows;
  double scale;
  double* ref;
  int failed;
} shrink_ctx;

/* Exact values of all 2^16 patterns of a 16-bit format (from orc_decode). */
static double* decode_table16(int dtype) {
  double* t = (double*)malloc(sizeof(double) * 65536);
  if (!t) return NULL;
  for (uint32_t b = 0; b < 65536; ++b) t[b] = orc_decode(dtype, b);
  return t;
}

static void shrink_rows(void* p, int worker, int64_t begin, int64_t end) {
  (void)worker;
  shrink_ctx* c = (shrink_ctx*)p;
  double* xrow = (double*)malloc(sizeof(double) * (size_t)c->H);
  if (!xrow) {
    __atomic_store_n(&c->failed, 1, __ATOMIC_RELAXED);
    return;
  }
  for (int64_t i = begin; i < end; ++i) {
    const int64_t t = c->rows ? c->rows[i] : i;
    const int64_t b = c->owner[t];
    if (b < 0) continue;  /* no active segment holds row t: untouched */
    const int64_t a = c->idx[b];
    /* Input row as it enters the products (float32 rounded to the weight
     * type, as in the expand). */
    for (int64_t h = 0; h < c->H; ++h) {
      const uint32_t bits = load_bits(c->x_dtype, c->x, t * c->x_stride + h);
      if (c->x_dtype == ORC_F32) {
        const double v = orc_decode(ORC_F32, bits);
        xrow[h] = c->a_tab[orc_encode(c->a_dtype, v)];
      } else {
        xrow[h] = c->x_tab[bits];
      }
    }
    for (int si = 0; si < c->ns; ++si) {
      const orc_shrink_slice* s = &c->s[si];
      for (int64_t k = 0; k < c->K; ++k) {
        const int64_t row_a = (a * c->K + k) * c->H;  /* A[a][k][:] */
        double r = 0.0;
        for (int64_t h = 0; h < c->H; ++h)
          r += xrow[h] * c->a_tab[load_bits(c->a_dtype, s->a, row_a + h)];
        r *= c->scale;
        if (c->ref) c->ref[(si * c->T + t) * c->K + k] = r;
        store_bits(c->out_dtype, s->out, t * s->out_stride + k, orc_encode(c->out_dtype, r));
      }
    }
  }
  free(xrow);
}

int orc_shrink(const void* x, int x_dtype, int64_t x_stride, int64_t T, int64_t H,
               const orc_shrink_slice* slices, int num_slices, int a_dtype, int64_t K,
               int64_t L, int out_dtype, const int64_t* start, const int64_t* lens,
               const int64_t* idx, int64_t batches, double scale, const int64_t* rows,
               int64_t num_rows, double* ref, int threads) {
  int eb, mb;
  if (!slices || num_slices < 1 || K < 1 || H < 1 || L < 0 || T < 0 || batches < 0 ||
      x_stride < H || num_rows < 0)
    return ORC_BAD_ARGUMENT;
  if (!format_of(out_dtype, &eb, &mb) || !format_of(x_dtype, &eb, &mb)) return ORC_BAD_ARGUMENT;
  /* Same dtype rules as the expand: 16-bit weights, inputs of the weight
   * type or float32. */
  if (a_dtype != ORC_F16 && a_dtype != ORC_BF16) return ORC_BAD_ARGUMENT;
  if (x_dtype != a_dtype && x_dtype != ORC_F32) return ORC_BAD_ARGUMENT;
  for (int si = 0; si < num_slices; ++si)
    if (slices[si].out_stride < K) return ORC_BAD_ARGUMENT;
  if (rows)
    for (int64_t i = 0; i < num_rows; ++i)
      if (rows[i] < 0 || rows[i] >= T) return ORC_BAD_ARGUMENT;
  int64_t* owner = NULL;
  int rc = build_owner(T, L, start, lens, idx, batches, &owner);
  if (rc != ORC_OK) return rc;
  double* a_tab = decode_table16(a_dtype);
  double* x_tab = x_dtype == ORC_F32 ? NULL : decode_table16(x_dtype);
  if (!a_tab || (x_dtype != ORC_F32 && !x_tab)) {
    free(a_tab); free(x_tab); free(owner);
    return ORC_NO_MEMORY;
  }
  const int64_t n = rows ? num_rows : T;
  shrink_ctx c = {x, x_dtype, a_dtype, out_dtype, x_stride, H, K, T, slices, num_slices,
                  a_tab, x_tab, owner, idx, rows, scale, ref, 0};
  rc = run_chunks(workers_for(threads, n), n, shrink_rows, &c);
  if (rc == ORC_OK && c.failed) rc = ORC_NO_MEMORY;
  free(a_tab);
  free(x_tab);
  free(owner);
  return rc;
}
