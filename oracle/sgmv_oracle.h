/*
 * sgmv_oracle.h -- CPU oracle for SGMV expand-slice.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and sgmv_oracle.c form a plain,
 * slow, fp64 reference of what the GPU library computes.  Only the tests,
 * the package's smoke entry and the benchmark's CPU-baseline leg may load
 * it.  It shares no code, header, table or helper with the GPU library.
 *
 * Source of the definition: the wiki page "Implementation: Predibase Lorax
 * SGMV Expand Slice Kernel" (Description; I/O Contract, Inputs and
 * Outputs).  For each segment b and each token m of that segment, the
 * slice out[start_b + m][slice_offset : slice_offset + N] receives
 * input[start_b + m] multiplied by the transpose of lora_B[idx[b]]
 * (lora_B is stored (lora_num, slice_size, rank), so the product is
 * y[n] = sum_k x[k] * B[idx[b]][n][k]); idx = -1 applies no LoRA;
 * add_inputs selects accumulate (true) or overwrite (false, the default).
 *
 * All arithmetic is fp64 with one final round-to-nearest-even into the
 * output dtype.  Encoders and decoders are written from the IEEE 754
 * binary interchange format definition (sign, biased exponent, trailing
 * significand) and cover binary16, bfloat16 (8-bit exponent, 7-bit
 * trailing significand) and binary32.
 */
#ifndef SGMV_ORACLE_H
#define SGMV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage types, as the I/O Contract lists them: float16 / bfloat16 for
 * weights, float16 / bfloat16 / float32 for inputs and outputs. */
enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_F32 = 2 };

/* Return codes. */
enum {
  ORC_OK = 0,
  ORC_BAD_ARGUMENT = 1,   /* shapes, dtypes, slice bounds, strides         */
  ORC_BAD_SEGMENT = 2,    /* segment outside [0, T) or overlapping another */
  ORC_BAD_INDEX = 3,      /* adapter index < -1 or >= lora_num             */
  ORC_NO_MEMORY = 4
};

/* Exact value of one stored element (bits in the low 16 or 32 bits). */
double orc_decode(int dtype, uint32_t bits);

/* Round-to-nearest, ties-to-even encoding of an fp64 value; overflow gives
 * +-infinity, NaN gives the canonical quiet NaN with the input's sign. */
uint32_t orc_encode(int dtype, double v);

/* Element-wise array forms of the two functions above. */
void orc_decode_array(int dtype, const uint32_t* bits, double* out, int64_t n);
void orc_encode_array(int dtype, const double* v, uint32_t* out, int64_t n);

/* One slice of the fused output (the multi-slice form applies each slice in
 * turn; column windows must not overlap). */
typedef struct {
  const void* x;      /* inputs, (T, K) rows of length >= K, row stride x_stride */
  int x_dtype;
  int64_t x_stride;   /* elements */
  const void* w;      /* lora_B, (L, N, K) contiguous                            */
  int w_dtype;
  int64_t N;          /* slice_size                                              */
  int64_t offset;     /* slice_offset                                            */
} orc_slice;

/*
 * Apply every slice to `out` (T rows of H elements, row stride out_stride)
 * in place.  `out` must hold the prior output O0 on entry.  If `ref` is not
 * NULL it receives, per slice in order, a (T, N_s) fp64 array of the exact
 * (pre-rounding) values for rows of active segments (other rows untouched).
 * `threads` <= 0 uses every CPU the process may run on.  Returns an ORC_* code; on error `out`
 * is unchanged.
 */
int orc_expand(const orc_slice* slices, int num_slices, int64_t K, int64_t L,
               void* out, int out_dtype, int64_t T, int64_t H, int64_t out_stride,
               const int64_t* start, const int64_t* lens, const int64_t* idx,
               int64_t batches, int add_inputs, double* ref, int threads);

/* Result of orc_check. */
typedef struct {
  int64_t checked_values;     /* slice elements compared against the fp64 value */
  int64_t checked_untouched;  /* elements compared bit for bit with O0          */
  int64_t bad_values;         /* slice elements outside tolerance / wrong class */
  int64_t bad_untouched;      /* untouched elements whose bits changed          */
  double max_abs_err;         /* max |c - r| over finite slice elements         */
  double max_tol_ratio;       /* max |c - r| / (atol + rtol*|r|); <= 1 passes  */
  int64_t first_bad_row, first_bad_col;  /* -1 if none */
} orc_report;

/*
 * Streaming comparator: recompute the exact value row by row and compare the
 * candidate output `cand` with it, without storing any fp64 array.  Slice
 * elements of active rows pass when |c - r| <= atol + rtol * |r| and c is
 * finite; where the correctly rounded value is not finite (overflow, NaN
 * inputs) the candidate must be the same kind of non-finite value.  Every
 * other element must equal O0 (`prior`) bit for bit.  If `rows` is not NULL
 * only those `num_rows` rows are checked.
 */
int orc_check(const orc_slice* slices, int num_slices, int64_t K, int64_t L,
              const void* prior, const void* cand, int out_dtype,
              int64_t T, int64_t H, int64_t out_stride,
              const int64_t* start, const int64_t* lens, const int64_t* idx,
              int64_t batches, int add_inputs, double atol, double rtol,
              const int64_t* rows, int64_t num_rows, int threads,
              orc_report* report);

/*
 * LoRA-A projection (shrink): the step that produces the expand's `inputs`.
 *
 * The wiki page "Implementation: Predibase Lorax SGMV Expand Slice Kernel"
 * (I/O Contract, Inputs; Usage Examples) describes `inputs` as the
 * rank-sized activations the A-side LoRA projection produces for every token
 * of every sequence, shape (total_tokens, rank).  The page does not print the projection itself;
 * this oracle takes the plainest reading consistent with it and with the
 * expand's conventions:
 *   - lora_A is stacked (lora_num, rank, hidden), out-by-in like lora_B;
 *   - for each segment b with adapter a = idx[b] != -1 and each row t of
 *     the segment, y[t][k] = scale * sum_h x[t][h] * A[a][k][h];
 *   - float32 inputs are rounded to the 16-bit weight type first (the same
 *     CAST_TYPE rule as the expand);
 *   - the result overwrites y (one rounding to the output dtype); rows of
 *     inactive segments, and rows outside every segment, are untouched.
 * Several slices (lora_A stacks with one output each, same rank) share the
 * input, as the fused QKV and gate/up layers do.
 */
typedef struct {
  const void* a;       /* lora_A stack, (L, K, H) contiguous, a_dtype      */
  void* out;           /* (T, K) rows, row stride out_stride elements      */
  int64_t out_stride;
} orc_shrink_slice;

/*
 * Project rows of x (T rows of H elements, row stride x_stride) into every
 * slice's output.  If `rows` is not NULL only those `num_rows` rows are
 * computed (each listed once).  If `ref` is not NULL it receives, per slice
 * in order, a (T, K) fp64 array of the exact pre-rounding values of the
 * computed active rows (other entries untouched).  Returns an ORC_* code;
 * after an argument, segment or index error no output is changed.
 */
int orc_shrink(const void* x, int x_dtype, int64_t x_stride, int64_t T, int64_t H,
               const orc_shrink_slice* slices, int num_slices, int a_dtype, int64_t K,
               int64_t L, int out_dtype, const int64_t* start, const int64_t* lens,
               const int64_t* idx, int64_t batches, double scale, const int64_t* rows,
               int64_t num_rows, double* ref, int threads);

/* Worker threads a call with `threads` uses at most (<= 0: the CPUs in the
 * process's affinity mask). */
int orc_threads(int threads);

#ifdef __cplusplus
}
#endif
#endif /* SGMV_ORACLE_H */
