/*
 * sp_csr.h -- unstructured-sparse CSR kernels for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels: CSR build, row swizzle, SpMM and
 * SDDMM.  What the operations compute follows the summary card of "Sparse GPU
 * Kernels for Deep Learning" (Gale, Zaharia, Young, Elsen; SC 2020); each entry
 * point names the passage it implements.  The card prints no formula; the
 * operations are the textbook definitions of the named kernels.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array argument is a DEVICE pointer (memory the caller got
 * from hipMalloc or an allocator on top of it, e.g. a torch tensor).  The
 * library never allocates, frees or retains caller memory and keeps no
 * mutable global state -- except the per-GPU scratch array that
 * sp_row_swizzle_noalloc sorts in, which that entry point describes -- and is
 * safe to call from several host threads at once.  Outputs must not overlap
 * inputs.
 *
 * Streams.  `stream` is a hipStream_t (NULL = the null stream).  Every call
 * only enqueues work on `stream` and returns without synchronising.  The
 * library records no hipMemsetAsync, so calls may be captured in HIP graphs.
 *
 * CSR.  Standard CSR with int32 indices and fp32 values (fp16/bf16 in the
 * mixed-precision entry points): an m x k matrix with
 * nnz entries has row_offsets[m+1] (row_offsets[0] = 0, non-decreasing,
 * row_offsets[m] = nnz), col_indices[nnz] (in [0, k), strictly increasing
 * within a row) and values[nnz].  These are preconditions, documented and not
 * checked on the device: a structure that violates them gives unspecified
 * results and may make the kernels read or write out of bounds.  Dense matrices are
 * row-major and contiguous.
 *
 * Row order.  `row_indices` (int32[m], a permutation of 0..m-1, or NULL for
 * the identity) gives the order in which rows are handed to the GPU's workers:
 * the r-th work slot handles row row_indices[r]; sp_row_swizzle computes the
 * balanced order.  It changes scheduling, not results, with one exception:
 * the balanced SpMM kernel (sp_spmm_balanced, and sp_spmm itself on wide B
 * when a row order is given) groups rows four at a time in that order, and a
 * group whose rows differ much in length splits its entries over four waves,
 * which changes rounding (deterministically for a given order).
 *
 * Errors.  Return codes only; nothing is thrown and nothing aborts.  Argument
 * checks happen on the host before any HIP call: a negative size, a NULL
 * pointer for a non-empty buffer, or a size beyond int32 indexing returns
 * SP_ERROR_INVALID_VALUE and enqueues nothing.  A problem outside what a
 * kernel supports (sizes beyond the launch limits, sp_sparse_attention's head
 * dimensions) returns SP_ERROR_NOT_SUPPORTED, also before any launch.  A
 * failed launch returns SP_ERROR_LAUNCH_FAILED.  Alignment is not required
 * unless an entry point says so: unaligned pointers or widths that are not
 * multiples of the vector width take a scalar-load variant of the same kernel.
 */
#ifndef SP_CSR_H
#define SP_CSR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sp_status {
    SP_SUCCESS = 0,
    SP_ERROR_INVALID_VALUE = 1,
    SP_ERROR_NOT_SUPPORTED = 2,
    SP_ERROR_LAUNCH_FAILED = 3
} sp_status_t;

/* A hipStream_t, passed as an opaque pointer so this header needs no HIP
 * header. */
typedef void *sp_stream_t;

/* Static English description of a status code (never NULL). */
const char *sp_status_string(sp_status_t status);

/* Library version as major*10000 + minor*100 + patch. */
int sp_version(void);

/* ------------------------------------------------------------------------
 * CSR build ("Summary" and "Interesting ideas" I5 of the card: the kernels
 * work on plain, standard CSR with no structural constraint).
 * ---------------------------------------------------------------------- */

/* row_offsets[0] = 0 and row_offsets[i+1] = lengths[0] + ... + lengths[i]
 * (the exclusive prefix sum of the row lengths).
 *   m            rows, >= 0
 *   lengths      int32[m], each >= 0, sum <= INT32_MAX (precondition)
 *   row_offsets  int32[m+1], output; must not overlap lengths
 * m == 0 writes row_offsets[0] = 0. */
sp_status_t sp_csr_offsets_from_lengths(int m, const int *lengths,
                                        int *row_offsets, sp_stream_t stream);

/* First half of building CSR from a dense m x k byte mask (row-major; a
 * nonzero byte marks a structural entry): writes row_offsets[m+1] for the
 * mask's rows.  The caller reads row_offsets[m] (= nnz) to size col_indices
 * and values, then calls sp_csr_fill_dense.
 *   mask         uint8[m*k]
 *   row_offsets  int32[m+1], output */
sp_status_t sp_csr_count_dense(int m, int k, const unsigned char *mask,
                               int *row_offsets, sp_stream_t stream);

/* Second half: col_indices/values of the mask's entries, rows ascending and
 * columns ascending within a row.  values[p] takes dense_values at the entry's
 * position; an explicit zero value at a set mask position stays an entry.
 *   row_offsets   int32[m+1] as written by sp_csr_count_dense for this mask
 *   dense_values  fp32[m*k] or NULL (then values is not written and may be NULL)
 *   col_indices   int32[nnz], output;  values fp32[nnz], output
 * Both outputs are written only at set mask positions; they must be non-NULL
 * whenever the mask has an entry (not checked: the host does not know nnz). */
sp_status_t sp_csr_fill_dense(int m, int k, const unsigned char *mask,
                              const float *dense_values, const int *row_offsets,
                              int *col_indices, float *values,
                              sp_stream_t stream);

/* ------------------------------------------------------------------------
 * Row swizzle ("Interesting ideas" I4 of the card: load balancing by
 * reordering rows, kept separate from how the kernels split their work).
 * ---------------------------------------------------------------------- */

/* row_indices[r] = the r-th row when rows are ordered by nonzero count,
 * longest first, rows of equal count by ascending row index (a unique,
 * deterministic order).
 *   row_offsets  int32[m+1] (CSR row offsets)
 *   row_indices  int32[m], output
 * Workspace-free: each row's slot is its rank among all rows' (length, index)
 * keys, m^2 comparisons -- a few microseconds up to ~16 K rows; above that
 * sp_row_swizzle_ws gives the same order in time linear in m. */
sp_status_t sp_row_swizzle(int m, const int *row_offsets, int *row_indices,
                           sp_stream_t stream);

/* *bytes = the device workspace sp_row_swizzle_ws needs for m rows: 0 up to
 * 16,384 rows, else 16 bytes per row plus 1 KiB per 4,096 rows (rounded up to
 * 256-byte multiples).  Host arithmetic only; m < 0 or bytes == NULL returns
 * SP_ERROR_INVALID_VALUE. */
sp_status_t sp_row_swizzle_workspace(int m, size_t *bytes);

/* sp_row_swizzle for structures of many rows ("Interesting ideas" I4 of the
 * card; the order is the same, bit for bit): above 16,384 rows a stable radix
 * sort of the rows by (k - length), 8 bits per pass, ceil(log2(k + 1) / 8)
 * passes, each three launches linear in m (two passes for k <= 65,535); at
 * most 16,384 rows, sp_row_swizzle's rank sort (no workspace used).
 *   k            columns of the matrix: every row holds at most k entries
 *                (true of any valid structure; a longer row is ordered as if
 *                it had k entries)
 *   row_offsets  int32[m+1];  row_indices  int32[m], output
 *   workspace    device memory of at least sp_row_swizzle_workspace(m) bytes,
 *                256-byte aligned, not overlapping the arguments (may be NULL
 *                when that size is 0); contents on entry do not matter and on
 *                return are unspecified; calls sharing one on overlapping
 *                streams race.
 * Errors: m < 0, k < 0, a NULL array that must exist, or a missing, short or
 * misaligned workspace returns SP_ERROR_INVALID_VALUE. */
sp_status_t sp_row_swizzle_ws(int m, int k, const int *row_offsets, int *row_indices,
                              void *workspace, size_t workspace_bytes, sp_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * sp_row_swizzle_ws without a workspace argument, the same order bit for bit.
 * Above 16,384 rows the radix sort runs in a 32 MiB scratch array the library
 * itself holds on each GPU it runs on (a device global, present from when the
 * library is first used there until the process ends); the call allocates and
 * frees nothing.  Every call on one GPU shares that GPU's array, so calls that
 * may overlap in time on one GPU (several streams, several host threads) race
 * and give unspecified orders; calls in one stream's order are safe.
 *   m            rows, at most SP_ROW_SWIZZLE_NOALLOC_MAX_ROWS
 *   k, row_offsets, row_indices   as sp_row_swizzle_ws
 * Errors: as sp_row_swizzle_ws, and m > SP_ROW_SWIZZLE_NOALLOC_MAX_ROWS returns
 * SP_ERROR_INVALID_VALUE before any HIP call. */
#define SP_ROW_SWIZZLE_NOALLOC_MAX_ROWS 2000000
sp_status_t sp_row_swizzle_noalloc(int m, int k, const int *row_offsets, int *row_indices,
                                   sp_stream_t stream);

/* CSR row offsets and the swizzled row order from row lengths in one launch
 * (the order depends on the lengths only): row_offsets as
 * sp_csr_offsets_from_lengths writes them and row_indices as sp_row_swizzle
 * writes them for those offsets.  For a structure given as per-row lists this
 * is the whole preparation before SpMM/SDDMM.
 *   lengths      int32[m], each >= 0, sum <= INT32_MAX (precondition)
 *   row_offsets  int32[m+1], output;  row_indices  int32[m], output */
sp_status_t sp_csr_build_from_lengths(int m, const int *lengths, int *row_offsets,
                                      int *row_indices, sp_stream_t stream);

/* ------------------------------------------------------------------------
 * SpMM ("Summary" of the card): C = A * B, A sparse in CSR, B dense.
 * ---------------------------------------------------------------------- */

/* C[i][j] = sum over entries p of row i of values[p] * B[col_indices[p]][j].
 * C is overwritten (an empty row gives a zero row).
 *   m, k, n      A is m x k, B is k x n, C is m x n;  nnz = row_offsets[m]
 *   row_indices  int32[m] row order, or NULL (identity)
 *   values, row_offsets, col_indices   the CSR of A
 *   b            fp32[k*n];  c  fp32[m*n], output
 * Sizes: m, k, n, nnz >= 0 and m*n, k*n < 2^62.  m == 0 or n == 0 enqueues
 * nothing.  Each output element is summed in an order fixed by the shapes
 * alone: in entry order (wide B, and B staged in LDS by row panels); per-lane
 * partial sums added by a fixed tree (B of at most 16 columns); four
 * consecutive parts of the row, each in entry order, added in order (few rows
 * averaging 256 entries or more).  With a row order given, B of more than 128
 * fp32 columns and one batch entry, the balanced kernel of sp_spmm_balanced
 * runs instead of the wide one (the card's I4: the swizzled order pairs long
 * rows with short ones in its groups), so rows of a skewed group are summed as
 * that entry point describes -- unless B is staged in LDS by row panels, which
 * takes precedence (fp32 one-batch problems whose panels fill every CU and
 * touch each staged B row at least 4 times on average).  sp_spmm_kernel_name
 * reports the choice.  Results are deterministic run to run. */
sp_status_t sp_spmm(int m, int k, int n, int nnz, const int *row_indices,
                    const float *values, const int *row_offsets,
                    const int *col_indices, const float *b, float *c,
                    sp_stream_t stream);

/* sp_spmm for row-length distributions with a heavy tail ("Interesting
 * ideas" I4 of the card: balancing kept separate from the kernels).  With
 * every wave of a launch resident at once, as on this GPU at these sizes, the
 * order rows are handed out in cannot balance anything by itself: the longest
 * row's chain of loads sets the duration.  Here, for B of more than 128 fp32
 * columns, workgroups of 4 waves take 4 rows in serpentine order over the
 * work slots (slots g, 2G-1-g, 2G+g, 4G-1-g of G groups: in the swizzled
 * order, long rows with short ones).  A group whose longest row holds at most
 * 1.5 times the group's mean runs one row per wave, summed in entry order as
 * sp_spmm's wide kernel sums it; any other group splits its entries (taken
 * row after row) into 4 equal parts, one per wave, and adds the parts'
 * partial sums of each row in order.  Results are deterministic for a given
 * row order and within rounding of sp_spmm.  sp_spmm runs this kernel by
 * itself when given a row order on one batch entry of such B (unless it stages
 * B by row panels); narrower B takes sp_spmm's kernels.  Arguments as
 * sp_spmm. */
sp_status_t sp_spmm_balanced(int m, int k, int n, int nnz, const int *row_indices,
                             const float *values, const int *row_offsets,
                             const int *col_indices, const float *b, float *c,
                             sp_stream_t stream);

/* `batch` independent SpMMs sharing one sparsity structure (row_offsets,
 * col_indices, row_indices): for z < batch,
 *   C_z = A_z * B_z, values_z = values + z*stride_values,
 *   b_z = b + z*stride_b, c_z = c + z*stride_c   (strides in elements).
 * stride_values or stride_b may be 0 (shared operand); stride_c must be
 * >= m*n when batch > 1 (outputs may not overlap). */
sp_status_t sp_spmm_batched(int m, int k, int n, int nnz,
                            const int *row_indices, const float *values,
                            const int *row_offsets, const int *col_indices,
                            const float *b, float *c, int batch,
                            long long stride_values, long long stride_b,
                            long long stride_c, sp_stream_t stream);

/* ------------------------------------------------------------------------
 * SDDMM ("Summary" and "Interesting ideas" I3 of the card): the dense product
 * X * Y^T evaluated only at the entries of a CSR mask, in the specialised form
 * gradients and sparse attention need -- no element-wise scaling by the
 * mask's values (the mask has no values here) and the second operand given
 * transposed, so both operands are read by contiguous rows.
 * ---------------------------------------------------------------------- */

/* out[p] = sum over l < d of X[i][l] * Y[col_indices[p]][l], for each entry p
 * of row i.  out is overwritten.  (A scale factor, such as sparse attention's
 * 1/sqrt(d), is the `alpha` of sp_sddmm_batched / sp_sddmm_ex; a power-of-two
 * scale may equally be applied to X first, with identical results.)
 *   m, k, d      mask is m x k, X is m x d, Y is k x d;  nnz = row_offsets[m]
 *   row_indices  int32[m] row order, or NULL (identity)
 *   row_offsets, col_indices   the mask's CSR structure
 *   x  fp32[m*d];  y  fp32[k*d];  out  fp32[nnz], output
 * d == 0 writes zeros.  Deterministic run to run. */
sp_status_t sp_sddmm(int m, int k, int d, int nnz, const int *row_indices,
                     const int *row_offsets, const int *col_indices,
                     const float *x, const float *y, float *out,
                     sp_stream_t stream);

/* sp_sddmm for row-length distributions with a heavy tail ("Interesting
 * ideas" I4 of the card: balancing kept separate from the kernels).  One wave
 * per row walks the row's windows of 64 entries in turn, so with every wave
 * resident at once the longest row's chain of windows would set the
 * duration.  Here each row slot gets a workgroup of 4 waves and wave j takes
 * windows j, j + 4, j + 8, ... of the row; entries need no combine step, so
 * outputs are bit-identical to the one-wave form.  Rows of at most 64 entries
 * leave three of their four waves idle (they exit at once), which costs about
 * nothing at these sizes.  sp_sddmm (and any SDDMM entry point on one batch
 * entry) takes this form by itself when the rows average 16 entries or more;
 * this entry point takes it always.  Arguments, errors and results as
 * sp_sddmm. */
sp_status_t sp_sddmm_balanced(int m, int k, int d, int nnz, const int *row_indices,
                              const int *row_offsets, const int *col_indices, const float *x,
                              const float *y, float *out, sp_stream_t stream);

/* `batch` SDDMMs sharing one mask: x_z = x + z*stride_x, y_z = y + z*stride_y,
 * out_z = out + z*stride_out (elements).  stride_out must be >= nnz when
 * batch > 1. */
sp_status_t sp_sddmm_batched(int m, int k, int d, int nnz,
                             const int *row_indices, const int *row_offsets,
                             const int *col_indices, const float *x,
                             const float *y, float alpha, float *out,
                             int batch, long long stride_x, long long stride_y,
                             long long stride_out, sp_stream_t stream);

/* Layout of SDDMM's second operand Y. */
typedef enum sp_y_layout {
    SP_Y_KD = 0, /* Y stored k x d: Yop(c, l) = y[c*d + l] (the transposed form) */
    SP_Y_DK = 1  /* Y stored d x k: Yop(c, l) = y[l*k + c] */
} sp_y_layout_t;

/* General SDDMM ("Interesting ideas" I3 of the card: the specialised form
 * above leaves out the element-wise scaling by the mask's values and assumes a
 * transposed operand; the card notes the general case is easy to add back).
 * For each batch entry z < batch and each entry p of row i:
 *   out_z[p] = alpha * v_z[p] * sum over l < d of X_z[i][l] * Yop_z(col_indices[p], l)
 *              + beta * out_z[p]
 * with v_z = mask_values + z*stride_values (v = 1 when mask_values is NULL),
 * x_z = x + z*stride_x, y_z = y + z*stride_y, out_z = out + z*stride_out.
 *   y_layout     SP_Y_KD or SP_Y_DK (anything else: SP_ERROR_INVALID_VALUE).
 *   mask_values  fp32[nnz] per batch entry, or NULL
 *   beta         0: out is overwritten and never read (it may hold NaN);
 *                otherwise out holds the prior values and is updated in place.
 *   workspace    device memory, used only with SP_Y_DK, else ignored; NULL or
 *                workspace_bytes >= sp_sddmm_general_workspace(k, d, batch,
 *                stride_y) and 256-byte aligned (otherwise
 *                SP_ERROR_INVALID_VALUE).  With a workspace, Y is first
 *                transposed into it (one k x d copy per batch entry, or one
 *                shared copy when stride_y = 0) and the SP_Y_KD kernels run on
 *                that copy: the same results bit for bit as SP_Y_KD on the
 *                caller's own transpose.  Without one, SP_Y_DK stages Y
 *                through LDS, transposed: for d <= 1024, masks of mean density
 *                1/20 or more by tiles of up to 64 columns (each output summed
 *                by 16 lanes, each in order over every 16th 4-element vector,
 *                then added pairwise across the lanes), sparser masks by the
 *                columns each panel of rows touches (each output summed in l
 *                order by one lane); beyond d = 1024 single elements are
 *                gathered along rows of Y (summed in l order).  The
 *                workspace is the caller's; its contents after the call are
 *                unspecified, and calls that share one on overlapping streams
 *                race.
 * Everything else as sp_sddmm_batched, which is this call with mask_values =
 * NULL, y_layout = SP_Y_KD, beta = 0 and no workspace.  Deterministic run to
 * run. */
sp_status_t sp_sddmm_general(int m, int k, int d, int nnz, const int *row_indices,
                             const int *row_offsets, const int *col_indices,
                             const float *mask_values, const float *x, const float *y,
                             int y_layout, float alpha, float beta, float *out, int batch,
                             long long stride_values, long long stride_x,
                             long long stride_y, long long stride_out, void *workspace,
                             size_t workspace_bytes, sp_stream_t stream);

/* Workspace bytes sp_sddmm_general needs to transpose a d x k Y:
 * k * d * 4 per batch entry, or once when stride_y = 0.  Host-only; negative
 * arguments or a NULL `bytes` return SP_ERROR_INVALID_VALUE. */
sp_status_t sp_sddmm_general_workspace(int k, int d, int batch, long long stride_y,
                                       size_t *bytes);

/* ------------------------------------------------------------------------
 * Mixed precision (fp16/bf16 operands, fp32 arithmetic).  The card's kernels
 * are fp32; 16-bit storage halves the bytes of the gathered operand, which
 * is what bounds these kernels.  Every 16-bit element is widened to fp32
 * exactly, a product of two 16-bit elements is exact in fp32, sums are fp32,
 * and outputs are fp32.  Summation orders are those of the fp32 entry points,
 * except that pairs of terms are added in one step: the bf16 vector SpMM adds
 * two consecutive entries' products per column, and the 16-bit vector SDDMM
 * (and attention scores) two consecutive elements' products, to the running
 * sum (v_dot2c_f32_bf16 / v_dot2c_f32_f16).
 * ---------------------------------------------------------------------- */

/* Element type of the 16-bit-capable operands. */
typedef enum sp_dtype {
    SP_DTYPE_F32 = 0,  /* IEEE binary32 */
    SP_DTYPE_F16 = 1,  /* IEEE binary16 */
    SP_DTYPE_BF16 = 2  /* bfloat16: the upper 16 bits of a binary32 */
} sp_dtype_t;

/* sp_spmm_batched with values and B of element type `dtype` (strides in
 * elements of that type); C is fp32.  SP_DTYPE_F32 is exactly
 * sp_spmm_batched.  16-bit B rows are read in 16-byte vectors of 8 elements
 * when n % 8 == 0 and B, C are 16-byte aligned, else element by element.
 * Narrow 16-bit B (up to 32 columns) with many entries per B element takes
 * the streaming kernel (B copied into LDS); it reads the values in whole
 * 4-byte words, so with an odd nnz it may read the 2 bytes after the value
 * array (the rest of the word holding the last value; never used).
 * An unknown dtype returns SP_ERROR_INVALID_VALUE. */
sp_status_t sp_spmm_ex(int m, int k, int n, int nnz, const int *row_indices, int dtype,
                       const void *values, const int *row_offsets, const int *col_indices,
                       const void *b, float *c, int batch, long long stride_values,
                       long long stride_b, long long stride_c, sp_stream_t stream);

/* Which kernel sp_spmm_ex (and so sp_spmm / sp_spmm_batched) would run for
 * these arguments: *name is set to a static string --
 *   "wide"      one wave per row strip, B rows gathered from L2;
 *   "balanced"  sp_spmm_balanced's kernel: wide B (more than 128 fp32
 *               columns), one batch entry and a row order given;
 *   "panel"     B staged in LDS and shared by a panel of 32 or 64 rows (fp32,
 *               one batch entry, n of at least one 128-column tile, enough
 *               panels to give every CU one, rows per panel times density at
 *               least 4);
 *   "panel_union" batches (n = 64, 128 or 256, k <= 65,536; 16-bit values and
 *               B widened to fp32 on load): per
 *               panel of 16 consecutive rows, the union of the rows' columns
 *               is formed once for 4 batch entries and C[panel] computed as
 *               matrix-core tiles over it; panels whose rows share few columns
 *               (or whose union rows of B hold a value that is not finite) run
 *               the wide kernel's accumulation, bit-identical to "wide";
 *   "narrow"    lanes over entries for B of at most 16 columns;
 *   "lds"       the streaming kernel, narrow B copied into LDS once per CU;
 *   "split"     few long rows cut into four parts per workgroup;
 *   "none"      nothing to launch (m, n or batch is 0);
 *   "unsupported" sizes beyond the launch limits.
 * The choice depends on the sizes, the element type, the batch and strides,
 * whether row_indices is NULL, and the alignment of values, col_indices, b and
 * c; no array is dereferenced (any pointers with the caller's alignment will
 * do; NULL is accepted where sp_spmm_ex would accept it).  It also reads the
 * current device's compute-unit count and LDS size.  Host-only; enqueues
 * nothing.  An unknown dtype, invalid sizes or NULL `name` return
 * SP_ERROR_INVALID_VALUE. */
sp_status_t sp_spmm_kernel_name(int m, int k, int n, int nnz, const int *row_indices, int dtype,
                                const void *values, const int *col_indices, const void *b,
                                const float *c, int batch, long long stride_values,
                                long long stride_b, long long stride_c, const char **name);

/* The name of the kernel sp_sddmm_general (and, for fp32 X and Y,
 * sp_sddmm_batched, sp_sddmm_ex) would run for these arguments:
 *   "panel_union" batches in the "multirow" domain with k <= 65,536: per
 *               panel of 16 consecutive rows, the union of the rows' columns
 *               is formed once for 4 batch entries and the scores computed as
 *               matrix-core tiles over it; panels whose rows share few columns
 *               run the multi-row walk (sp_sddmm_softmax, whose batches of
 *               the same shape take this kernel too: the row softmax body);
 *   "multirow"  several short rows per wave (16-byte-aligned X and Y, one
 *               16-byte vector per lane with 8 or 16 lanes per entry: fp32 d a
 *               multiple of 4 from 20 to 64, 16-bit d a multiple of 8 from 40
 *               to 128; row slots not split);
 *   "rows"      one wave per row slot;
 *   "split"     one batch entry whose rows average 16 entries or more: a
 *               row's 64-entry windows spread over a workgroup of 4 waves;
 *   "columns"   Y stored d x k, lanes over entries (no workspace);
 *   "dk_panel"  Y stored d x k, the touched columns staged per row panel;
 *   "dk_tile"   Y stored d x k, dense enough for X and Y tiles in LDS;
 *   "fill"      d = 0 with no mask values and beta = 0 (outputs set to 0);
 *   "none"      nothing to launch (m, nnz or batch is 0);
 *   "unsupported" sizes beyond the launch limits.
 * With a d x k Y and a workspace, the names are those of the k x d kernels
 * run after the transpose.  The choice depends on the sizes, the element
 * type, the batch and strides, whether mask_values and workspace are NULL,
 * beta == 0, y_layout and the alignment of x, y and the workspace; no array
 * is dereferenced (NULL is accepted where sp_sddmm_general would accept it).
 * It may read the current device's compute-unit count and LDS size.
 * Host-only; enqueues nothing.  An unknown dtype, invalid arguments or NULL
 * `name` return SP_ERROR_INVALID_VALUE. */
sp_status_t sp_sddmm_kernel_name(int m, int k, int d, int nnz, int dtype,
                                 const float *mask_values, const void *x, const void *y,
                                 int y_layout, float beta, int batch, long long stride_values,
                                 long long stride_x, long long stride_y, long long stride_out,
                                 void *workspace, size_t workspace_bytes, const char **name);

/* sp_sddmm_batched with X and Y of element type `dtype` (strides in elements
 * of that type); out is fp32.  SP_DTYPE_F32 is exactly sp_sddmm_batched.  An
 * unknown dtype returns SP_ERROR_INVALID_VALUE. */
sp_status_t sp_sddmm_ex(int m, int k, int d, int nnz, const int *row_indices,
                        const int *row_offsets, const int *col_indices, int dtype,
                        const void *x, const void *y, float alpha, float *out, int batch,
                        long long stride_x, long long stride_y, long long stride_out,
                        sp_stream_t stream);

/* ------------------------------------------------------------------------
 * SpMM and SDDMM together ("Summary" of the card: the two kernels of the
 * method).  Problems of DL sizes leave the GPU mostly idle in either kernel
 * alone; one launch that carries both keeps it busier and pays one launch.
 * ---------------------------------------------------------------------- */

/* The SpMM sp_spmm(m, k, n, nnz, row_indices, values, row_offsets,
 * col_indices, b, c) and the SDDMM sp_sddmm(s_m, s_k, d, s_nnz,
 * s_row_indices, s_row_offsets, s_col_indices, x, y, out) with its products
 * scaled by alpha (alpha = 1: exactly sp_sddmm) -- two independent problems,
 * whose sparsity structures may be the same arrays or different ones -- enqueued as one launch when both take their fp32 vector
 * paths (16-byte aligned operands, B and Y under 2 GiB, n % 4 == 0,
 * d % 4 == 0, d <= 256), otherwise as the two separate launches.  Results
 * are bit-identical to calling the two entry points, the SpMM with a NULL row
 * order (the pair sums every SpMM row in entry order; row_indices only
 * schedules).  Arguments are checked as those entry points check them; c and
 * out must not overlap each other or any input. */
sp_status_t sp_spmm_sddmm(int m, int k, int n, int nnz, const int *row_indices,
                          const float *values, const int *row_offsets, const int *col_indices,
                          const float *b, float *c, int s_m, int s_k, int d, int s_nnz,
                          const int *s_row_indices, const int *s_row_offsets,
                          const int *s_col_indices, const float *x, const float *y,
                          float alpha, float *out, sp_stream_t stream);

/* ------------------------------------------------------------------------
 * Transpose ("Summary" of the card: the kernels serve training; the input
 * gradient of C = A * B is dB = A^T * dC, an SpMM with the transposed sparse
 * operand).  sp_csr_transpose gives A^T in standard CSR; sp_row_swizzle and
 * sp_spmm on it then compute the product, entries of each output row summed in
 * ascending row order of A.
 * ---------------------------------------------------------------------- */

/* *bytes = the device workspace sp_csr_transpose needs for nnz entries
 * (about 20 bytes per entry plus 1 KiB per 4096 entries).  Pure host
 * arithmetic; enqueues nothing. */
sp_status_t sp_csr_transpose_workspace(int m, int k, int nnz, size_t *bytes);

/* The CSR of A^T (k x m) from the CSR of A (m x k): row j of A^T lists, in
 * ascending order, the rows i of A with an entry in column j, each with that
 * entry's value.  Identical on every run (no atomic operation decides an
 * order).
 *   row_offsets, col_indices, values   the CSR of A (values may be NULL when
 *                 t_values is NULL)
 *   t_row_offsets int32[k+1], output;  t_col_indices int32[nnz], output
 *   t_values      fp32[nnz], output, or NULL
 *   t_perm        int32[nnz], output, or NULL: t_perm[q] is the index in A's
 *                 arrays of A^T's entry q (for sp_csr_transpose_values)
 *   workspace     device memory of at least sp_csr_transpose_workspace bytes,
 *                 256-byte aligned, not overlapping any argument; its contents
 *                 on entry do not matter and on return are unspecified.
 * Errors: k == INT32_MAX, k == 0 with nnz > 0, a missing or short workspace,
 * or a NULL array that must exist returns SP_ERROR_INVALID_VALUE. */
sp_status_t sp_csr_transpose(int m, int k, int nnz, const int *row_offsets,
                             const int *col_indices, const float *values,
                             int *t_row_offsets, int *t_col_indices, float *t_values,
                             int *t_perm, void *workspace, size_t workspace_bytes,
                             sp_stream_t stream);

/* t_values[q] = values[t_perm[q]] for q < nnz: new values of A (same
 * structure) carried into the order of A^T without transposing again.
 * t_values must not overlap values. */
sp_status_t sp_csr_transpose_values(int nnz, const int *t_perm, const float *values,
                                    float *t_values, sp_stream_t stream);

/* ------------------------------------------------------------------------
 * Sparse attention ("Interesting ideas" I3 of the card: the SDDMM form sparse
 * attention needs).  Attention is scores (SDDMM), a softmax over each row's
 * entries, and their weighted sum (SpMM): the softmax alone, the scores with
 * their softmax in one pass, and the whole attention in one pass.
 * ---------------------------------------------------------------------- */

/* For each batch entry z < batch and each row i with entries p:
 *   out_z[p] = exp(in_z[p] - mx) / sum over the row's entries q of
 *              exp(in_z[q] - mx),   mx = the row's maximum of in_z,
 * computed in fp32 (expf); rows without entries are left untouched.
 * in_z = in + z*stride_in, out_z = out + z*stride_out (elements); the CSR
 * structure (row_offsets, row_indices) is shared by all batch entries.
 *   row_indices  int32[m] row order, or NULL (identity)
 *   in, out      fp32, nnz per batch entry; out may equal in (in place),
 *                otherwise they must not overlap.  stride_out >= nnz when
 *                batch > 1. */
sp_status_t sp_csr_row_softmax(int m, int nnz, const int *row_indices,
                               const int *row_offsets, const float *in, float *out,
                               int batch, long long stride_in, long long stride_out,
                               sp_stream_t stream);

/* Scores and their row softmax in one pass (sparse attention's first two
 * steps, "Interesting ideas" I3 of the card): for each batch entry z and each
 * row i with entries p,
 *   out_z[p] = exp(s_p - mx) / sum over the row's entries q of exp(s_q - mx),
 *   s_p = alpha * sum over l < d of X_z[i][l] * Y_z[col_indices[p]][l],
 *   mx = the row's maximum of s,
 * with X and Y of element type `dtype` (Y stored k x d), fp32 arithmetic and
 * expf; rows without entries are left untouched.  Equal, up to rounding, to
 * sp_sddmm_ex followed by sp_csr_row_softmax, without writing and re-reading
 * the scores in between.  Arguments as sp_sddmm_ex. */
sp_status_t sp_sddmm_softmax(int m, int k, int d, int nnz, const int *row_indices,
                             const int *row_offsets, const int *col_indices, int dtype,
                             const void *x, const void *y, float alpha, float *out, int batch,
                             long long stride_x, long long stride_y, long long stride_out,
                             sp_stream_t stream);

/* Sparse attention in one pass ("Interesting ideas" I3 of the card: the
 * SDDMM -> row softmax -> SpMM composition), without writing the scores or
 * the probabilities: for each batch entry z and each query row i with mask
 * entries p (columns j_p),
 *   out_z[i][:] = sum over p of P_p * V_z[j_p][:],
 *   P = the row softmax of s_p = alpha * sum over l < d of Q_z[i][l] * K_z[j_p][l]
 * (fp32 arithmetic, expf; the softmax in its running-maximum form, so rows of
 * any length take one pass).  A row without entries gives a zero row.
 *   m, k         query rows and key rows; the mask is m x k;  nnz = row_offsets[m]
 *   d            the head dimension of Q, K and V
 *   dtype        element type of Q, K and V (SP_DTYPE_*); out is fp32
 *   q            [m x d],  kmat, v  [k x d] per batch entry;  out  [m x d] fp32
 *   stride_*     elements between batch entries; stride_out >= m*d when batch > 1
 * Supported shapes: d = 32, 64, 128 or 256 for fp32 and 64, 128, 256 or 512
 * for 16-bit types; 16-byte aligned operands with strides that keep them so;
 * K and V under 2 GiB per batch entry.  Anything else returns
 * SP_ERROR_NOT_SUPPORTED (the three separate entry points handle it).
 * Batches (batch >= 2) of fp32 heads with d = 32 or 64, or of 16-bit heads
 * with d = 64 (widened to fp32), on at most 65,536 key rows take a kernel that
 * forms each 16-row panel's key union once for 4
 * batch entries and computes scores and the weighted sum of V as matrix-core
 * tiles over it (the softmax rescaled once per 16-key tile); panels whose rows
 * share few keys, and panels whose union rows of V hold a value that is not
 * finite, use the per-row walk, as do all other calls.  The results do not
 * depend on row_indices.
 * Deterministic run to run; equal up to rounding to sp_sddmm_softmax (or
 * sp_sddmm + sp_csr_row_softmax) followed by sp_spmm. */
sp_status_t sp_sparse_attention(int m, int k, int d, int nnz, const int *row_indices,
                                const int *row_offsets, const int *col_indices, int dtype,
                                const void *q, const void *kmat, const void *v, float alpha,
                                float *out, int batch, long long stride_q, long long stride_k,
                                long long stride_v, long long stride_out, sp_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SP_CSR_H */
