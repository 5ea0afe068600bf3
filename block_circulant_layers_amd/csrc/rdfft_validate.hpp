// rdfft_validate.hpp -- host-side argument checks of the C ABI (no HIP calls).
//
// Every entry point runs these before enqueuing anything; on failure it
// returns the status and touches no device memory.
#pragma once

#include <stdint.h>

#include "rdfft.h"

namespace rdfft {

// row lengths: transforms and spectrum utilities up to 32768, circulant blocks up to 4096
inline bool valid_len(int64_t p, int64_t pmax = 32768) { return p >= 2 && p <= pmax && (p & (p - 1)) == 0; }
inline bool valid_dtype(int dtype) { return dtype == RDFFT_F32 || dtype == RDFFT_BF16 || dtype == RDFFT_F16; }
inline int64_t dtype_bytes(int dtype) { return dtype == RDFFT_F32 ? 4 : 2; }
inline bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// half-open byte ranges [a, a+na) and [b, b+nb) overlap
inline bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + static_cast<uintptr_t>(nb) && pb < pa + static_cast<uintptr_t>(na);
}

// largest element count any call accepts (keeps every byte offset in int64)
constexpr int64_t kMaxElems = int64_t(1) << 40;
// widest circulant activation row: the circulant kernels address a batch of
// up to 16 token rows through one buffer resource with 32-bit byte offsets
constexpr int64_t kMaxFeatures = int64_t(1) << 24;

inline int check_rdfft(const void* data, int64_t rows, int64_t p, int dtype) {
  if (!valid_dtype(dtype)) return RDFFT_ERR_DTYPE;
  if (!valid_len(p) || rows < 0 || rows > kMaxElems / p) return RDFFT_ERR_SIZE;
  if (rows == 0) return RDFFT_OK;
  if (data == nullptr) return RDFFT_ERR_NULL;
  if (!aligned16(data)) return RDFFT_ERR_ALIGN;
  return RDFFT_OK;
}

// packed rows [rows, p] of dtype and their complex bins [rows, p/2 + 1, 2] float
inline int check_spectrum(const void* packed, const float* spec, int64_t rows, int64_t p, int dtype) {
  if (!valid_dtype(dtype)) return RDFFT_ERR_DTYPE;
  if (!valid_len(p) || rows < 0 || rows > kMaxElems / (p + 2)) return RDFFT_ERR_SIZE;
  if (rows == 0) return RDFFT_OK;
  if (packed == nullptr || spec == nullptr) return RDFFT_ERR_NULL;
  if (!aligned16(packed) || !aligned16(spec)) return RDFFT_ERR_ALIGN;
  if (overlaps(packed, rows * p * dtype_bytes(dtype), spec, rows * (p + 2) * 4)) return RDFFT_ERR_ALIAS;
  return RDFFT_OK;
}

// n arrays of h x w (h <= 4096: the column transforms stage a column in LDS)
inline int check_rdfft2d(const void* data, int64_t n, int64_t h, int64_t w, int dtype) {
  if (!valid_dtype(dtype)) return RDFFT_ERR_DTYPE;
  if (!valid_len(h, 4096) || !valid_len(w) || n < 0 || n > kMaxElems / (h * w)) return RDFFT_ERR_SIZE;
  if (n == 0) return RDFFT_OK;
  if (data == nullptr) return RDFFT_ERR_NULL;
  if (!aligned16(data)) return RDFFT_ERR_ALIGN;
  return RDFFT_OK;
}

inline int check_circulant_dims(int64_t batch, int64_t d_in, int64_t d_out, int64_t p) {
  if (!valid_len(p, 4096) || batch < 0) return RDFFT_ERR_SIZE;
  if (d_in <= 0 || d_out <= 0 || d_in % p != 0 || d_out % p != 0) return RDFFT_ERR_SHAPE;
  if (d_in > kMaxFeatures || d_out > kMaxFeatures || batch > kMaxElems / d_in || batch > kMaxElems / d_out ||
      (d_in / p) > kMaxElems / d_out)
    return RDFFT_ERR_SIZE;
  return RDFFT_OK;
}

inline int check_circulant_fwd(const void* x, const float* c, const void* y, int64_t batch, int64_t d_in,
                               int64_t d_out, int64_t p, int dtype) {
  if (!valid_dtype(dtype)) return RDFFT_ERR_DTYPE;
  const int st = check_circulant_dims(batch, d_in, d_out, p);
  if (st != RDFFT_OK || batch == 0) return st;
  if (x == nullptr || c == nullptr || y == nullptr) return RDFFT_ERR_NULL;
  if (!aligned16(x) || !aligned16(c) || !aligned16(y)) return RDFFT_ERR_ALIGN;
  const int64_t eb = dtype_bytes(dtype);
  const int64_t cbytes = (d_out / p) * d_in * 4;
  if (overlaps(y, batch * d_out * eb, x, batch * d_in * eb) || overlaps(y, batch * d_out * eb, c, cbytes))
    return RDFFT_ERR_ALIAS;
  return RDFFT_OK;
}

// forward that also clears dc[q, k, p]: dc is required, even for an empty batch
inline int check_circulant_fwd_zero(const void* x, const float* c, const void* y, const float* dc, int64_t batch,
                                    int64_t d_in, int64_t d_out, int64_t p, int dtype) {
  const int st = check_circulant_fwd(x, c, y, batch, d_in, d_out, p, dtype);
  if (st != RDFFT_OK) return st;
  if (dc == nullptr) return RDFFT_ERR_NULL;
  if (!aligned16(dc)) return RDFFT_ERR_ALIGN;
  if (batch == 0) return RDFFT_OK;
  const int64_t eb = dtype_bytes(dtype);
  const int64_t cb = (d_out / p) * d_in * 4;
  if (overlaps(dc, cb, x, batch * d_in * eb) || overlaps(dc, cb, c, cb) || overlaps(dc, cb, y, batch * d_out * eb))
    return RDFFT_ERR_ALIAS;
  return RDFFT_OK;
}

inline int check_circulant_bwd(const void* x, const float* c, const void* dy, const void* dx, const float* dc,
                               int64_t batch, int64_t d_in, int64_t d_out, int64_t p, int dtype) {
  if (!valid_dtype(dtype)) return RDFFT_ERR_DTYPE;
  const int st = check_circulant_dims(batch, d_in, d_out, p);
  if (st != RDFFT_OK) return st;
  if (dx == nullptr && dc == nullptr) return RDFFT_ERR_NULL;
  if (batch == 0) {
    if (dc != nullptr && !aligned16(dc)) return RDFFT_ERR_ALIGN;
    return RDFFT_OK;
  }
  if (x == nullptr || c == nullptr || dy == nullptr) return RDFFT_ERR_NULL;
  if (!aligned16(x) || !aligned16(c) || !aligned16(dy) || (dx && !aligned16(dx)) || (dc && !aligned16(dc)))
    return RDFFT_ERR_ALIGN;
  const int64_t eb = dtype_bytes(dtype);
  const int64_t xb = batch * d_in * eb, yb = batch * d_out * eb, cb = (d_out / p) * d_in * 4;
  if (dx && (overlaps(dx, xb, x, xb) || overlaps(dx, xb, c, cb) || overlaps(dx, xb, dy, yb) ||
             overlaps(dx, xb, dc, cb)))
    return RDFFT_ERR_ALIAS;
  if (dc && (overlaps(dc, cb, x, xb) || overlaps(dc, cb, c, cb) || overlaps(dc, cb, dy, yb)))
    return RDFFT_ERR_ALIAS;
  return RDFFT_OK;
}

// the workspace of a deterministic dc (after check_circulant_bwd): dc is
// required; ws must hold `need` bytes (nothing when need == 0), be aligned and
// overlap no other argument
inline int check_det_workspace(const void* x, const float* c, const void* dy, const void* dx, const float* dc,
                               const float* ws, int64_t ws_bytes, int64_t need, int64_t batch, int64_t d_in,
                               int64_t d_out, int64_t p, int dtype) {
  if (dc == nullptr) return RDFFT_ERR_NULL;
  if (ws_bytes < 0 || ws_bytes < need) return RDFFT_ERR_SIZE;
  if (need == 0) return RDFFT_OK;
  if (ws == nullptr) return RDFFT_ERR_NULL;
  if (!aligned16(ws)) return RDFFT_ERR_ALIGN;
  const int64_t eb = dtype_bytes(dtype);
  const int64_t xb = batch * d_in * eb, yb = batch * d_out * eb, cb = (d_out / p) * d_in * 4;
  if (overlaps(ws, need, x, xb) || overlaps(ws, need, c, cb) || overlaps(ws, need, dy, yb) ||
      overlaps(ws, need, dc, cb) || (dx && overlaps(ws, need, dx, xb)))
    return RDFFT_ERR_ALIAS;
  return RDFFT_OK;
}

// weights given as packed spectra: the kernels read them through one buffer
// resource with 32-bit byte offsets, so the q k p floats of cs, plus one row
// of reads aimed past their end, stay below 2^31 bytes
inline int check_spec_size(int64_t d_in, int64_t d_out, int64_t p) {
  return (d_out / p) * d_in * 4 + 4 * p <= int64_t{0x7fffffff} ? RDFFT_OK : RDFFT_ERR_SIZE;
}

// circulant_weight_spectra: c and cs are separate [q, k, p] fp32 buffers
inline int check_weight_spectra(const float* c, const float* cs, int64_t d_in, int64_t d_out, int64_t p) {
  int st = check_circulant_dims(0, d_in, d_out, p);
  if (st == RDFFT_OK) st = check_spec_size(d_in, d_out, p);
  if (st != RDFFT_OK) return st;
  if (c == nullptr || cs == nullptr) return RDFFT_ERR_NULL;
  if (!aligned16(c) || !aligned16(cs)) return RDFFT_ERR_ALIGN;
  const int64_t cb = (d_out / p) * d_in * 4;
  return overlaps(cs, cb, c, cb) ? RDFFT_ERR_ALIAS : RDFFT_OK;
}

// circulant_fwd_step's output cs[q, k, p] (fp32): required, separate from
// every other buffer of the call (the other arguments checked before)
inline int check_fwd_step_spectra(const void* x, const float* c, const void* y, const float* dc, const float* cs,
                                  int64_t batch, int64_t d_in, int64_t d_out, int64_t p, int dtype) {
  const int st = check_spec_size(d_in, d_out, p);
  if (st != RDFFT_OK) return st;
  if (cs == nullptr || c == nullptr) return RDFFT_ERR_NULL;
  if (!aligned16(cs)) return RDFFT_ERR_ALIGN;
  const int64_t eb = dtype_bytes(dtype), cb = (d_out / p) * d_in * 4;
  if (overlaps(cs, cb, c, cb) || overlaps(cs, cb, dc, cb) || overlaps(cs, cb, x, batch * d_in * eb) ||
      overlaps(cs, cb, y, batch * d_out * eb))
    return RDFFT_ERR_ALIAS;
  return RDFFT_OK;
}

}  // namespace rdfft
