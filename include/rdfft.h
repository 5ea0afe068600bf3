/*
 * rdfft.h -- C ABI of the MI355X (gfx950) in-place real FFT and block-circulant
 * layer library (librdfft.so).
 *
 * Method: "Memory-Efficient Training with In-Place FFT Implementation"
 * (NeurIPS 2025, arXiv 2511.01385), as described on the Paper-Notes page
 * (zhaoyang97.github.io, section "方法详解") and the scime.ai summary page
 * (sections "Problem" and "Approach").
 *
 * Packed layout (Paper-Notes page, "Squeeze"): a real row x of length p (a
 * power of two) is replaced, in its own p-element buffer, by its DFT
 * y_k = sum_n x_n exp(-2 pi i k n / p) written as
 *     [0] = y_0,  [p/2] = y_{p/2},  [k] = Re y_k,  [p-k] = Im y_k  (0 < k < p/2).
 * y_0 and y_{p/2} are real and y_{p-k} = conj(y_k), so this is lossless.
 *
 * Common rules for every entry point
 *   - Pointers are DEVICE pointers owned by the caller: contiguous, row-major,
 *     16-byte aligned.  The library allocates no device memory, keeps no
 *     per-call state and is reentrant.  Its only device data is a read-only
 *     twiddle table compiled into the code object.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work and return; results are ready when the stream reaches that point.
 *   - Arguments are checked on the host before anything is enqueued.  On any
 *     error the call returns a nonzero status and neither reads nor writes
 *     device memory.  Size 0 (rows or batch) is a no-op returning RDFFT_OK;
 *     pointers are not checked then.
 *   - `dtype` selects the storage type of the row data (data, x, y, dy, dx,
 *     packed): RDFFT_F32 (float), RDFFT_BF16 (bfloat16) or RDFFT_F16 (IEEE
 *     half).  All arithmetic is fp32; 16-bit results are rounded to nearest
 *     even once, on store.  The circulant parameters c, their gradient dc and
 *     explicit complex spectra are always float.
 *   - Supported lengths: transforms and spectrum utilities p = 2, 4, 8, ...,
 *     32768 (a row is staged in one workgroup's LDS; the pages stop at 4096);
 *     circulant blocks p = 2, 4, ..., 4096, with d_in and d_out at most 2^24
 *     (RDFFT_ERR_SIZE beyond).
 *   - Non-finite inputs are propagated, not checked.
 */
#ifndef RDFFT_H
#define RDFFT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RDFFT_ABI_VERSION 6

/* storage types */
#define RDFFT_F32 0
#define RDFFT_BF16 1
#define RDFFT_F16 2

/* status codes */
#define RDFFT_OK 0
#define RDFFT_ERR_NULL 1   /* a required pointer is NULL */
#define RDFFT_ERR_SIZE 2   /* p not a supported power of two, or a negative / too large count */
#define RDFFT_ERR_SHAPE 3  /* d_in or d_out not a positive multiple of p */
#define RDFFT_ERR_DTYPE 4  /* dtype not RDFFT_F32 / RDFFT_BF16 / RDFFT_F16 */
#define RDFFT_ERR_ALIGN 5  /* a pointer is not 16-byte aligned */
#define RDFFT_ERR_ALIAS 6  /* an output buffer overlaps another buffer of the call */
#define RDFFT_ERR_LAUNCH 7 /* the HIP runtime refused a kernel launch */
#define RDFFT_ERR_SCRATCH 8 /* circulant_bwd_det_noalloc: the shape needs more than its 32 MiB workspace */

/* Version of this ABI (RDFFT_ABI_VERSION of the library that was built). */
int rdfft_abi_version(void);

/* Static string naming a status code ("ok", "null pointer", ...). */
const char* rdfft_status_string(int status);

/*
 * rdfft_forward -- in-place packed forward transform of `rows` rows.
 *   data  [rows, p] of dtype; on return each row holds its packed spectrum
 *         (layout above; unnormalised).  Decimation-in-time Cooley-Tukey whose
 *         every stage updates the four-element conjugate-symmetric groups
 *         {g+k, g+m/2-k, g+m/2+k, g+m-k} in place (Paper-Notes page,
 *         "四元素对称群 (Proposition 1)").  No buffer besides `data`.
 */
int rdfft_forward(void* data, int64_t rows, int64_t p, int dtype, void* stream);

/*
 * rdfft_inverse -- in-place inverse of rdfft_forward (carries the 1/p factor).
 *   data  [rows, p] of dtype holding packed spectra; on return the real rows.
 *   The butterfly graph of the forward run backwards, each group split into
 *   its symmetric and antisymmetric parts (Paper-Notes page, "原地 IFFT 设计";
 *   the per-stage 1/2 is applied once as 1/p, which is exact in binary).
 *   Any p reals are a valid packed spectrum.
 */
int rdfft_inverse(void* data, int64_t rows, int64_t p, int dtype, void* stream);

/*
 * circulant_fwd -- block-circulant layer forward (Paper-Notes page,
 * "循环矩阵训练适配"): for every token b and output block i,
 *     y[b, i*p:(i+1)*p] = IFFT( sum_j FFT(c[i, j, :]) * FFT(x[b, j*p:(j+1)*p]) ),
 * i.e. y = x W^T with W[i*p + a, j*p + t] = c[i, j, (a - t) mod p].
 *   x   [batch, d_in]   dtype, read only
 *   c   [q, k, p]       float (q = d_out/p, k = d_in/p), read only, time domain
 *   y   [batch, d_out]  dtype, written (must not overlap x or c)
 * Spectra live only on chip; nothing is written besides y.
 */
int circulant_fwd(const void* x, const float* c, void* y, int64_t batch, int64_t d_in, int64_t d_out,
                  int64_t p, int dtype, void* stream);

/*
 * circulant_bwd -- gradients of the layer above for an upstream gradient dy
 * (Paper-Notes page, section "循环矩阵训练适配": the gradients are again
 * products of packed spectra, which stay conjugate-symmetric):
 *     dx[b, j-block] = IFFT( sum_i conj(FFT(c[i, j])) * FFT(dy[b, i-block]) )   (= dy W)
 *     dc[i, j, :]    = IFFT( sum_b conj(FFT(x[b, j-block])) * FFT(dy[b, i-block]) )
 *   x   [batch, d_in]   dtype, read only
 *   c   [q, k, p]       float, read only
 *   dy  [batch, d_out]  dtype, read only
 *   dx  [batch, d_in]   dtype, overwritten; may be NULL to skip it
 *   dc  [q, k, p]       float, OVERWRITTEN (not accumulated) with the sum over
 *                       all tokens; may be NULL to skip it.  It is zeroed and
 *                       then serves as the accumulator of the token sum:
 *                       partial sums over token ranges are added atomically,
 *                       transformed back first or (for some p) as packed
 *                       spectra that an in-place inverse then transforms, so
 *                       the order of the fp32 token sum is not fixed (results
 *                       may differ in the last bits from call to call).
 * dx and dc must not both be NULL, and must not overlap each other or any
 * input.  When batch == 0, dc is set to zero (if given).
 */
int circulant_bwd(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch,
                  int64_t d_in, int64_t d_out, int64_t p, int dtype, void* stream);

/*
 * circulant_fwd_zero -- circulant_fwd that also sets dc[q, k, p] (float) to
 * zero, as a side job of the same launch where the forward runs its token-
 * persistent kernel (otherwise with one more small launch).  dc is meant to be
 * the gradient accumulator of c that circulant_bwd_acc adds into, so that a
 * training step of the layer (Paper-Notes page, "循环矩阵训练适配") needs no
 * separate clearing launch.  Arguments as circulant_fwd, plus
 *   dc  [q, k, p]  float, written with zeros; required even when batch == 0;
 *                  must not overlap x, c or y.
 */
int circulant_fwd_zero(const void* x, const float* c, void* y, float* dc, int64_t batch, int64_t d_in, int64_t d_out,
                       int64_t p, int dtype, void* stream);

/*
 * circulant_bwd_acc -- circulant_bwd that ADDS the token sum into dc instead
 * of overwriting it (dc += sum over tokens; dx is still overwritten).  The
 * arguments, their checks and the order-of-summation caveat are those of
 * circulant_bwd.  dc must hold finite values on entry.  Where the token sum
 * is gathered as packed spectra (p < 64; p = 64 and 128 when dx is NULL or the
 * one-launch backward does not fit), the old dc is transformed to packed
 * spectra first and returns to the time domain with the new sum, which is
 * exact up to the fp32 rounding of those two transforms.  When batch == 0
 * nothing is done.
 */
int circulant_bwd_acc(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch,
                      int64_t d_in, int64_t d_out, int64_t p, int dtype, void* stream);

/*
 * The layer with its weights given as packed spectra (Paper-Notes page,
 * "循环矩阵训练适配": the products above need FFT(c), never c itself).  A
 * caller that keeps cs = FFT(c) in a buffer of c's size, computed once per
 * value of c (once per optimizer step), saves the kernels from transforming
 * weight rows at every call: they read the weights' bins from cs.  c itself
 * is never overwritten (its spectra would not return it bitwise).
 *
 * circulant_weight_spectra -- cs[i, j, :] = packed FFT of c[i, j, :] (the
 * layout at the top of this file), for every block of the layer.
 *   c   [q, k, p]  float, read only
 *   cs  [q, k, p]  float, written; must not overlap c
 * p a power of two in [2, 4096]; d_in, d_out positive multiples of p with
 * q k p floats at most 2^31 - 1 - 4p bytes (RDFFT_ERR_SIZE otherwise).
 */
int circulant_weight_spectra(const float* c, float* cs, int64_t d_in, int64_t d_out, int64_t p, void* stream);

/*
 * circulant_fwd_step -- the forward of a training step from c: circulant_fwd
 * (circulant_fwd_zero when dc is not NULL) that also writes the weight
 * spectra cs, as circulant_weight_spectra would, for circulant_bwd_spec.
 * The forward transforms the weight rows anyway; where it runs its token-
 * persistent kernel, that launch stores them, otherwise one more launch
 * computes them.
 *   cs  [q, k, p]  float, written; must not overlap x, c, y or dc
 * Other arguments, checks and statuses as circulant_fwd and
 * circulant_fwd_zero, plus the size limit of circulant_weight_spectra; cs is
 * written when batch == 0 too.
 */
int circulant_fwd_step(const void* x, const float* c, void* y, float* dc, float* cs, int64_t batch, int64_t d_in,
                       int64_t d_out, int64_t p, int dtype, void* stream);

/*
 * circulant_fwd_spec -- circulant_fwd (or circulant_fwd_zero when dc is not
 * NULL) from the weight spectra cs that circulant_weight_spectra wrote.
 *   cs  [q, k, p]  float, read only, packed spectra of the weight rows
 *   dc  [q, k, p]  float or NULL: when given, set to zero as by
 *                  circulant_fwd_zero (also when batch == 0)
 * Other arguments, checks and statuses as circulant_fwd and
 * circulant_fwd_zero, with cs in the place of c, plus the size limit of
 * circulant_weight_spectra.
 */
int circulant_fwd_spec(const void* x, const float* cs, void* y, float* dc, int64_t batch, int64_t d_in, int64_t d_out,
                       int64_t p, int dtype, void* stream);

/*
 * circulant_bwd_spec -- circulant_bwd (accumulate == 0: dc overwritten) or
 * circulant_bwd_acc (accumulate != 0: the token sum added into dc) from the
 * weight spectra cs.  dx needs cs; dc is computed from x and dy alone, as in
 * those calls, with the same order-of-summation caveat.  Arguments, checks
 * and statuses as circulant_bwd, with cs in the place of c, plus the size
 * limit of circulant_weight_spectra.
 */
int circulant_bwd_spec(const void* x, const float* cs, const void* dy, void* dx, float* dc, int accumulate,
                       int64_t batch, int64_t d_in, int64_t d_out, int64_t p, int dtype, void* stream);

/*
 * circulant_bwd_det_workspace -- bytes of the workspace circulant_bwd_det
 * needs for this shape, with dx computed too (with_dx != 0) or not: one slice
 * of q k p floats per token range of the weight-gradient launch.  0 when
 * batch == 0.  The count depends on the shape only (not on dtype or device).
 *   bytes  out, the byte count; must not be NULL
 * Statuses as circulant_bwd's size and shape checks.
 */
int circulant_bwd_det_workspace(int64_t batch, int64_t d_in, int64_t d_out, int64_t p, int with_dx, int64_t* bytes);

/*
 * circulant_bwd_det -- circulant_bwd with a deterministic dc (same gradients,
 * Paper-Notes page, "循环矩阵训练适配"): each token range's partial sums are
 * stored into its own slice of the caller's workspace instead of added into dc
 * atomically, and one more launch sums the slices in a fixed order into dc.
 * dc is then bitwise the same from call to call for the same inputs, shape and
 * device model.  Arguments as circulant_bwd, plus
 *   ws        device workspace of ws_bytes bytes, 16-byte aligned, holding at
 *             least circulant_bwd_det_workspace(..., with_dx = dx != NULL)
 *             bytes (status RDFFT_ERR_SIZE otherwise); its contents on entry do
 *             not matter and are overwritten; it must not overlap any other
 *             argument.  May be NULL when that size is 0.
 * dc is required (not NULL) and overwritten; dx may be NULL.
 */
int circulant_bwd_det(const void* x, const float* c, const void* dy, void* dx, float* dc, float* ws, int64_t ws_bytes,
                      int64_t batch, int64_t d_in, int64_t d_out, int64_t p, int dtype, void* stream);

/*
 * circulant_bwd_det_noalloc -- circulant_bwd_det for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and the same bitwise
 * result, with the workspace taken from a 32 MiB array the library holds on
 * every GPU it runs on until the process ends.  Nothing is allocated: no
 * hipMalloc, hipFree or allocating library call.  Arguments as
 * circulant_bwd_det without ws / ws_bytes.
 *   - Returns RDFFT_ERR_SCRATCH, touching nothing, when the shape needs more
 *     than 32 MiB (circulant_bwd_det_workspace gives the need).
 *   - All calls on one GPU share that GPU's array, which keeps the last call's
 *     contents; no call needs it cleared (every slice a call reads, it wrote).
 *     Calls that overlap on one GPU (other streams, other threads) race on it:
 *     order them on one stream.
 *   - The array's device address is looked up on the first call on each device.
 */
int circulant_bwd_det_noalloc(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch,
                              int64_t d_in, int64_t d_out, int64_t p, int dtype, void* stream);

/*
 * rdfft_unpack -- packed spectra to explicit complex bins (the packed layout
 * above, Paper-Notes page "Squeeze", read out).
 *   packed [rows, p]          dtype, read only (e.g. the output of rdfft_forward)
 *   spec   [rows, p/2 + 1, 2] float, written: (Re y_f, Im y_f) for f = 0..p/2,
 *                             with Im y_0 = Im y_{p/2} = 0.  Must not overlap packed.
 * Exact (values are only moved, and widened for 16-bit dtypes).
 */
int rdfft_unpack(const void* packed, float* spec, int64_t rows, int64_t p, int dtype, void* stream);

/*
 * rdfft_pack -- explicit complex bins to packed spectra (inverse of rdfft_unpack).
 *   spec   [rows, p/2 + 1, 2] float, read only.  Im of bins 0 and p/2 is not
 *                             read (the spectrum of a real row has it zero).
 *   packed [rows, p]          dtype, written (16-bit dtypes: rounded to nearest
 *                             even); a valid input of rdfft_inverse.  Must not
 *                             overlap spec.
 */
int rdfft_pack(const float* spec, void* packed, int64_t rows, int64_t p, int dtype, void* stream);

/*
 * rdfft2d_forward -- in-place 2D forward transform of n real arrays of h x w
 * (the 2D extension the pages leave open, Paper-Notes page "局限与展望").
 *   data [n, h, w] of dtype; on return each array holds its 2D DFT
 *        Y[j, k] = sum_{a, b} x[a, b] exp(-2 pi i (j a / h + k b / w)) for
 *        k = 0..w/2 (the rest is conjugate), packed along each axis where the
 *        data is conjugate-symmetric:
 *          columns k = 0 and k = w/2: Y[., k] in the 1D packed layout along j
 *            ([0, k] = Y[0, k], [h/2, k] = Y[h/2, k], [j, k] = Re Y[j, k],
 *            [h-j, k] = Im Y[j, k] for 0 < j < h/2);
 *          0 < k < w/2: [j, k] = Re Y[j, k] and [j, w-k] = Im Y[j, k], every j.
 *   h: power of two in [2, 4096]; w: power of two in [2, 32768]; unnormalised.
 *   Three in-place passes over data (row transforms, column transforms, a
 *   combine of column pairs); 16-bit dtypes are rounded to storage after each.
 */
int rdfft2d_forward(void* data, int64_t n, int64_t h, int64_t w, int dtype, void* stream);

/*
 * rdfft2d_inverse -- in-place inverse of rdfft2d_forward (carries 1/(h w)).
 *   data [n, h, w] of dtype in the layout above; any h*w reals are a valid
 *   packed 2D spectrum.  The three passes run in reverse order.
 */
int rdfft2d_inverse(void* data, int64_t n, int64_t h, int64_t w, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RDFFT_H */
