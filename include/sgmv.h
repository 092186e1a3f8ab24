/*
 * sgmv.h -- C ABI of libsgmv: SGMV expand-slice on AMD Instinct MI355X (gfx950).
 *
 * Operation (wiki page "Implementation: Predibase Lorax SGMV Expand Slice
 * Kernel", Description and I/O Contract), and the LoRA-A projection that
 * produces its inputs (sgmv_shrink, below): for each segment b of a packed
 * batch and each token m of that segment, row t = b_seq_start_loc[b] + m of
 * the output gets, in its column window [slice_offset, slice_offset +
 * slice_size),
 *
 *     out[t][slice_offset + n] = (add_inputs ? out[t][slice_offset + n] : 0)
 *                                + sum_k inputs[t][k] * lora_b[a][n][k],
 *
 * with a = lora_indices[b].  lora_b is stored (lora_num, slice_size, rank),
 * so the product is inputs . lora_b[a]^T.  Index -1 means no LoRA: those rows
 * are left untouched, as is every column outside the window.  Products are
 * accumulated in fp32 and rounded once (nearest even) to the output dtype.
 * float32 inputs are first rounded to the 16-bit weight dtype (the page's
 * CAST_TYPE mixed-precision cast).
 *
 * Every call enqueues GPU work on `stream` and returns; nothing here
 * synchronises, copies device data to the host or allocates memory.  All
 * argument checks happen before any HIP call; on a non-OK status nothing has
 * been launched and sgmv_last_error() describes the problem.
 */
#ifndef SGMV_H
#define SGMV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGMV_ABI_VERSION 5
#define SGMV_MAX_SLICES 8      /* slices per multi-slice call                       */
#define SGMV_MAX_RANK 256      /* largest rank the register-tiled kernels take; larger
                                  ranks (any size) run on the generic kernel */
#define SGMV_MAX_FUSED_SLICES 3 /* slices per fused shrink-expand call (QKV, gate/up) */
#define SGMV_MAX_BATCHES 4000  /* segment table lives in on-chip memory (LDS, 64 KiB);
                                  also the most tokens of one per-token call */

/* Element types (I/O Contract: weights float16/bfloat16; inputs
 * float16/bfloat16/float32). */
typedef enum { SGMV_F16 = 0, SGMV_BF16 = 1, SGMV_F32 = 2 } sgmv_dtype;

typedef enum {
  SGMV_OK = 0,
  SGMV_ERR_INVALID_ARGUMENT = 1, /* shapes, strides, bounds, null pointers       */
  SGMV_ERR_UNSUPPORTED = 2,      /* valid but not implemented (dtype mix, rank)  */
  SGMV_ERR_HIP = 3               /* a HIP runtime call failed                    */
} sgmv_status;

/* A 2-D device matrix: `rows` x `cols` elements of `dtype`, rows
 * `row_stride` elements apart, unit column stride.  Borrowed. */
typedef struct {
  void* data;
  int32_t dtype;
  int64_t rows, cols, row_stride;
} sgmv_matrix;

/* A contiguous device stack of `num` matrices, each `rows` x `cols`
 * (lora_b: num = lora_num, rows = slice_size, cols = rank).  Borrowed. */
typedef struct {
  const void* data;
  int32_t dtype;
  int64_t num, rows, cols;
} sgmv_stack;

/* One slice of a fused output for sgmv_expand_multi_slice. */
typedef struct {
  sgmv_matrix inputs;     /* (total_tokens, rank)                         */
  sgmv_stack lora_b;      /* (lora_num, slice_size, rank)                 */
  int64_t slice_offset;   /* first output column of this slice            */
  int64_t slice_size;     /* must equal lora_b.rows                       */
} sgmv_slice;

/*
 * sgmv_expand_slice -- the page's sgmv_expand_slice (Signature; I/O Contract).
 *
 * inputs        device (total_tokens, rank) f16/bf16/f32; read only.
 * lora_b        device (lora_num, slice_size, rank) f16/bf16, contiguous; read only.
 *               inputs must be lora_b's dtype or f32.
 * out           device (total_tokens, full_hidden_size) f16/bf16/f32, modified in
 *               place only at rows of active segments x [slice_offset,
 *               slice_offset + slice_size).  row_stride >= cols.
 * b_seq_start_loc, seq_lens, lora_indices
 *               device int64[batches]; read only, never copied to the host.
 *               Segment b covers rows [b_seq_start_loc[b], +seq_lens[b]).
 * batches       number of segments, 0..SGMV_MAX_BATCHES.
 * max_seq_len   >= 0; a hint kept for signature parity (the device reads
 *               seq_lens itself and does not need it).
 * slice_offset, slice_size
 *               column window; slice_size must equal lora_b.rows and
 *               slice_offset + slice_size <= out.cols.
 * add_inputs    nonzero: accumulate onto out; zero: overwrite.
 * stream        HIP stream the work is enqueued on (0 = null stream).
 *
 * Device-side preconditions (not checkable without a sync): active segments
 * lie in [0, total_tokens) and are pairwise disjoint, and -1 <= index <
 * lora_num.  A segment that breaks the first or last of these is skipped
 * with no out-of-bounds access; overlapping segments give unspecified
 * values in the overlap.
 *
 * Returns SGMV_OK, or a status with nothing launched.  batches == 0,
 * slice_size == 0 or total_tokens == 0 return SGMV_OK without a launch.
 * SGMV_ERR_UNSUPPORTED for total_tokens >= 2^31 and for problems of more
 * than 2^31 - 1 work units of 16 rows x 256 columns (neither fits in
 * device memory).  The library keeps no device state between calls, so
 * calls on different streams may run concurrently.
 */
sgmv_status sgmv_expand_slice(sgmv_matrix inputs, sgmv_stack lora_b, sgmv_matrix out,
                              const int64_t* b_seq_start_loc, const int64_t* seq_lens,
                              const int64_t* lora_indices, int64_t batches,
                              int64_t max_seq_len, int64_t slice_offset, int64_t slice_size,
                              int add_inputs, hipStream_t stream);

/*
 * sgmv_expand_multi_slice -- several slices of one fused output in a single
 * launch (the page's Description: a future fused operator combining several
 * slice operations in one launch, for fused QKV or gate/up layouts).
 *
 * Equal, element for element and bit for bit, to calling sgmv_expand_slice
 * once per slice on the same `out`.  slices: host array of 1..SGMV_MAX_SLICES
 * descriptors, read during the call only.  All slices share `out`, the
 * segment metadata, the adapter indices, rank, dtypes, lora_num and
 * add_inputs; their column windows must not overlap.
 */
sgmv_status sgmv_expand_multi_slice(const sgmv_slice* slices, int num_slices, sgmv_matrix out,
                                    const int64_t* b_seq_start_loc, const int64_t* seq_lens,
                                    const int64_t* lora_indices, int64_t batches,
                                    int64_t max_seq_len, int add_inputs, hipStream_t stream);

/*
 * sgmv_bgmv_expand_slice -- the per-token counterpart (BGMV expand slice,
 * which the page names as the fixed-length counterpart of this operation):
 * every token carries its own adapter index,
 *
 *     out[t][slice_offset + n] = (add_inputs ? out[t][slice_offset + n] : 0)
 *                                + sum_k inputs[t][k] * lora_b[lora_indices[t]][n][k]
 *
 * for t in [0, total_tokens) with lora_indices[t] != -1; -1 leaves row t
 * untouched.  Identical to sgmv_expand_slice with batches = total_tokens,
 * b_seq_start_loc[t] = t and seq_lens[t] = 1, but reads no segment arrays.
 *
 * inputs, lora_b, out, slice_offset, slice_size, add_inputs, stream: as for
 *               sgmv_expand_slice.
 * lora_indices  device int64[total_tokens]; read only.  total_tokens =
 *               out.rows <= SGMV_MAX_BATCHES (else SGMV_ERR_UNSUPPORTED).
 *
 * Tokens are processed grouped by adapter (up to 16 per group, for up to
 * 1024 adapters), so tokens that share an adapter share its weight tiles.
 * Returns as sgmv_expand_slice.
 */
sgmv_status sgmv_bgmv_expand_slice(sgmv_matrix inputs, sgmv_stack lora_b, sgmv_matrix out,
                                   const int64_t* lora_indices, int64_t slice_offset,
                                   int64_t slice_size, int add_inputs, hipStream_t stream);

/* One slice of a fused LoRA-A projection for sgmv_shrink_multi_slice. */
typedef struct {
  sgmv_stack lora_a;      /* (lora_num, rank, hidden)                     */
  sgmv_matrix out;        /* (total_tokens, rank)                         */
} sgmv_shrink_slice;

/*
 * sgmv_shrink -- the LoRA-A projection that produces sgmv_expand_slice's
 * `inputs`.  The page (I/O Contract, Inputs; Usage Examples) describes those
 * inputs as the rank-sized activations the A-side LoRA projection produces
 * for every token of every sequence, (total_tokens, rank); it prints no
 * formula for the projection, so this takes the plainest reading consistent
 * with the expand:
 *
 *     out[t][k] = scale * sum_h inputs[t][h] * lora_a[a][k][h],   k < rank,
 *
 * for each segment b with a = lora_indices[b] != -1 and each row t of the
 * segment.  lora_a is stored (lora_num, rank, hidden) -- out-by-in, like
 * lora_b -- so the product is inputs . lora_a[a]^T.  Products are accumulated
 * in fp32, multiplied by `scale` and rounded once (nearest even) to the
 * output dtype; float32 inputs are first rounded to the 16-bit weight dtype.
 * The call overwrites: rows of index -1 segments and rows outside every
 * segment are left untouched.
 *
 * inputs        device (total_tokens, hidden) f16/bf16/f32; read only.
 * lora_a        device (lora_num, rank, hidden) f16/bf16, contiguous; read
 *               only.  inputs must be lora_a's dtype or f32.
 *               rank <= SGMV_MAX_RANK (else SGMV_ERR_UNSUPPORTED).
 * out           device (total_tokens, rank) f16/bf16/f32, row_stride >= rank;
 *               written only at rows of active segments.  Must not overlap
 *               inputs, lora_a or the metadata.
 * b_seq_start_loc, seq_lens, lora_indices, batches, max_seq_len, stream:
 *               as for sgmv_expand_slice, with the same device-side
 *               preconditions.
 * scale         fp32 factor applied to every sum (1 for the plain product).
 * workspace, workspace_bytes:
 *               NULL and 0, or a device buffer of at least
 *               sgmv_shrink_workspace_bytes() bytes, 16-byte aligned, whose
 *               contents are zero before its first use (hipMemset once);
 *               every call leaves the buffer ready for the next one.  With
 *               it, batches of 64-token units run balanced when there are
 *               more units than the device has compute units (at most twice
 *               as many: the units beyond one per compute unit are split)
 *               or at most half as many (every unit is split): units are
 *               split over the hidden size into parts whose fp32 partial
 *               sums go through the workspace and are added in a fixed
 *               order, so results are deterministic but may differ in
 *               rounding from a call without one (bit for bit equal on
 *               integer-valued data).
 *               Calls that may run at the same time (other streams) need
 *               workspaces of their own; it must not overlap any other
 *               argument.  A misaligned or short workspace returns
 *               SGMV_ERR_INVALID_ARGUMENT.
 *
 * Kernel choice (results are the same within tolerance, and bit for bit on
 * integer-valued data): the register-tiled kernels take rank % 8 == 0,
 * hidden % 8 == 0, 16-byte aligned rows, 64 rows of inputs and of each
 * output spanning < 2 GiB, and 16 * p rows of one adapter's lora_a block
 * spanning < 2 GiB, i.e. 32 * p * hidden < 2^31, where p is the next power
 * of two of ceil(rank / 16) (rank 256: hidden < 4 Mi); every other shape
 * runs on the generic kernel.
 *
 * Returns SGMV_OK, or a status with nothing launched; batches == 0 or
 * total_tokens == 0 return SGMV_OK without a launch.
 */
sgmv_status sgmv_shrink(sgmv_matrix inputs, sgmv_stack lora_a, sgmv_matrix out,
                        const int64_t* b_seq_start_loc, const int64_t* seq_lens,
                        const int64_t* lora_indices, int64_t batches, int64_t max_seq_len,
                        float scale, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * sgmv_shrink_multi_slice -- several LoRA-A projections of the same inputs
 * (the Q, K and V, or gate and up, adapters of a fused layer) in one call
 * that reads the inputs once.  Equal, bit for bit, to calling sgmv_shrink
 * once per slice (with the same workspace argument, null or not).  slices:
 * host array of 1..SGMV_MAX_SLICES descriptors,
 * read during the call only; all share rank, lora_num, the lora_a dtype and
 * the output dtype; outputs must not overlap each other.
 */
sgmv_status sgmv_shrink_multi_slice(sgmv_matrix inputs, const sgmv_shrink_slice* slices,
                                    int num_slices, const int64_t* b_seq_start_loc,
                                    const int64_t* seq_lens, const int64_t* lora_indices,
                                    int64_t batches, int64_t max_seq_len, float scale,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Bytes of the workspace sgmv_shrink and sgmv_shrink_multi_slice take on
 * the current device (16 MiB + 1 KiB on a 256-compute-unit MI355X). */
sgmv_status sgmv_shrink_workspace_bytes(size_t* bytes);

/*
 * sgmv_shrink_multi_slice_noalloc -- sgmv_shrink_multi_slice for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the workspace is a static
 * array inside the library (one copy per device, 20 MiB + 1280 bytes,
 * covering devices of up to 320 compute units, held until the process
 * ends) instead of an argument.  Each call first clears the array's part
 * counters with a small kernel on `stream`, then runs exactly what
 * sgmv_shrink_multi_slice with a workspace runs (same results, bit for
 * bit).  Calls that may overlap on one device (several streams, or host
 * threads) race on the shared array: serialise them.  Calls no allocating
 * routine.  Returns what sgmv_shrink_multi_slice returns, and
 * SGMV_ERR_UNSUPPORTED on a device with more than 320 compute units (the
 * array would be too small).
 */
sgmv_status sgmv_shrink_multi_slice_noalloc(sgmv_matrix inputs, const sgmv_shrink_slice* slices,
                                            int num_slices, const int64_t* b_seq_start_loc,
                                            const int64_t* seq_lens,
                                            const int64_t* lora_indices, int64_t batches,
                                            int64_t max_seq_len, float scale,
                                            hipStream_t stream);

/* One slice of a fused LoRA delta for sgmv_fused_shrink_expand. */
typedef struct {
  sgmv_stack lora_a;      /* (lora_num, rank, hidden)                     */
  sgmv_stack lora_b;      /* (lora_num, slice_size, rank)                 */
  int64_t slice_offset;   /* first output column of the slice's window    */
} sgmv_fused_slice;

/*
 * sgmv_fused_shrink_expand -- the LoRA-A projection (sgmv_shrink) and the
 * expand-slice of its result (sgmv_expand_multi_slice) for the slices of a
 * fused QKV or gate/up layer, in one launch, without storing the projected
 * rows.  The page motivates the slice kernel by a later operator that fuses
 * several slice operations into one launch (Description; Usage: fused QKV
 * and gate/up layers) and describes the expand's inputs as the A-side
 * projection's rank-sized activations (I/O Contract, Inputs).  For each
 * segment b with a = lora_indices[b] != -1, each row t of it and each slice
 * s:
 *
 *     y_s[t][k] = rne_w(scale * sum_h inputs[t][h] * lora_a_s[a][k][h]),
 *     out[t][off_s + n] = (add_inputs ? out[t][off_s + n] : 0)
 *                         + sum_k y_s[t][k] * lora_b_s[a][n][k],
 *
 * with rne_w the nearest-even rounding to the weights' 16-bit dtype -- the
 * result of sgmv_shrink_multi_slice into outputs of the weights' dtype
 * followed by sgmv_expand_multi_slice on those outputs, bit for bit equal
 * to them when the shrink runs without a workspace (with one, its parts
 * round differently); sums in fp32, each result rounded once (nearest
 * even) to the output dtype; float32 inputs rounded to the weight dtype
 * first.  Rows of index -1 segments, rows outside every segment and
 * columns outside the windows are left untouched.  The call takes the
 * shrink's two forms by the shrink's rule: from 64 units of 64 tokens
 * (129 for ranks up to 16), 64-row units that each expand over every column; below (short prefill
 * and decode batches), 16-row units, each expanded in column groups over
 * about one work item per compute unit.  Measured on MI355X, the call
 * beats the two calls for ranks up to 32 below 64 units of 64 tokens and
 * loses elsewhere (each unit reads its adapter's lora_B once per 16 or 64
 * rows, where the expand reuses it for up to 512): choose it there.
 *
 * inputs        device (total_tokens, hidden) f16/bf16/f32; read only.
 * slices        host array of 1..SGMV_MAX_FUSED_SLICES descriptors, read
 *               during the call only: lora_a (lora_num, rank, hidden) and
 *               lora_b (lora_num, slice_size, rank), contiguous, device,
 *               read only, all of one 16-bit dtype (inputs: that dtype or
 *               f32), one rank and one lora_num; windows must not overlap.
 * out           device (total_tokens, out_cols) f16/bf16/f32; written only
 *               at rows of active segments x the slices' windows; must not
 *               overlap the other buffers.
 * b_seq_start_loc, seq_lens, lora_indices, batches, max_seq_len, stream:
 *               as for sgmv_expand_slice, with the same device-side
 *               preconditions.
 * scale         fp32 factor applied to every projected sum before its
 *               rounding (1 for the plain product).
 * add_inputs    nonzero: accumulate onto out; zero: overwrite.
 *
 * Shapes: rank % 8 == 0 and rank <= 128 with 16 * p * num_slices <= 256
 * (p = next power of two of ceil(rank / 16)), hidden % 8 == 0, slice widths
 * % 8 == 0, 16-byte aligned data, rows and windows, and the shrink's lora_a
 * bound (32 * p * hidden < 2^31); other shapes return SGMV_ERR_UNSUPPORTED
 * (run sgmv_shrink_multi_slice and sgmv_expand_multi_slice instead).
 * Returns SGMV_OK, or a status with nothing launched; batches == 0,
 * total_tokens == 0 or all slice widths 0 return SGMV_OK without a launch.
 */
sgmv_status sgmv_fused_shrink_expand(sgmv_matrix inputs, const sgmv_fused_slice* slices,
                                     int num_slices, sgmv_matrix out,
                                     const int64_t* b_seq_start_loc, const int64_t* seq_lens,
                                     const int64_t* lora_indices, int64_t batches,
                                     int64_t max_seq_len, float scale, int add_inputs,
                                     hipStream_t stream);

/* Message for the last non-OK status returned on the calling thread ("" if
 * none).  The pointer stays valid until the thread's next libsgmv call. */
const char* sgmv_last_error(void);

/* SGMV_ABI_VERSION of the loaded library. */
int sgmv_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SGMV_H */
