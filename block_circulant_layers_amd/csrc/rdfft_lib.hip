// rdfft_lib.hip -- C ABI of librdfft.so: argument checks, kernel selection, launches.
#include <hip/hip_runtime.h>

#include "rdfft.h"
#include "rdfft_kernels.hpp"
#include "circulant_kernels.hpp"
#include "rdfft_validate.hpp"
#include "spectrum_kernels.hpp"
#include "rdfft2d_kernels.hpp"

namespace rdfft {
namespace {

int launch_status() { return hipGetLastError() == hipSuccess ? RDFFT_OK : RDFFT_ERR_LAUNCH; }

// compute units of the current device (cached per device; 256 if the query fails)
int device_cus() {
  constexpr int kMaxDev = 64;
  static int cached[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int P, class Io, bool INV>
int launch_rdfft(void* data, int64_t rows, hipStream_t stream) {
  constexpr int E = standalone_elems(P, is_f32_io<Io>());
  constexpr int NT = wg_threads(P, E);
  constexpr int ROWS = NT / (P / E);
  const int64_t groups = (rows + ROWS - 1) / ROWS;
  const int64_t resident = static_cast<int64_t>(device_cus()) * wg_per_cu(P, is_f32_io<Io>());
  const int64_t grid = groups < resident ? groups : resident;
  auto* d = static_cast<typename Io::T*>(data);
  if (INV)
    rdfft_inv_kernel<P, Io><<<dim3(static_cast<unsigned>(grid)), dim3(NT), 0, stream>>>(d, rows);
  else
    rdfft_fwd_kernel<P, Io><<<dim3(static_cast<unsigned>(grid)), dim3(NT), 0, stream>>>(d, rows);
  return launch_status();
}

template <int P, class Io, bool INV>
int launch_rdfft_long(void* data, int64_t rows, hipStream_t stream) {
  constexpr int E = long_elems(P);
  const size_t lds = static_cast<size_t>(Row<P, E>::LDS) * sizeof(float);
  if (rows > 0x7fffffff) return RDFFT_ERR_SIZE;
  auto* d = static_cast<typename Io::T*>(data);
  if (INV)
    rdfft_inv_long_kernel<P, Io><<<dim3(static_cast<unsigned>(rows)), dim3(P / E), lds, stream>>>(d);
  else
    rdfft_fwd_long_kernel<P, Io><<<dim3(static_cast<unsigned>(rows)), dim3(P / E), lds, stream>>>(d);
  return launch_status();
}

template <class Io, bool INV>
int dispatch_rdfft(void* data, int64_t rows, int64_t p, hipStream_t s) {
  switch (p) {
    case 2: return launch_rdfft<2, Io, INV>(data, rows, s);
    case 4: return launch_rdfft<4, Io, INV>(data, rows, s);
    case 8: return launch_rdfft<8, Io, INV>(data, rows, s);
    case 16: return launch_rdfft<16, Io, INV>(data, rows, s);
    case 32: return launch_rdfft<32, Io, INV>(data, rows, s);
    case 64: return launch_rdfft<64, Io, INV>(data, rows, s);
    case 128: return launch_rdfft<128, Io, INV>(data, rows, s);
    case 256: return launch_rdfft<256, Io, INV>(data, rows, s);
    case 512: return launch_rdfft<512, Io, INV>(data, rows, s);
    case 1024: return launch_rdfft<1024, Io, INV>(data, rows, s);
    case 2048: return launch_rdfft<2048, Io, INV>(data, rows, s);
    case 4096: return launch_rdfft<4096, Io, INV>(data, rows, s);
    case 8192: return launch_rdfft<8192, Io, INV>(data, rows, s);  // the row (33 KB) fits static LDS
    case 16384: return launch_rdfft_long<16384, Io, INV>(data, rows, s);
    case 32768: return launch_rdfft_long<32768, Io, INV>(data, rows, s);
    default: return RDFFT_ERR_SIZE;
  }
}

// ---- block-circulant layer -------------------------------------------------

constexpr int kDcTargetWgs = 256;  // aim of the dc token split (workgroups in flight)

template <int P, class Io>
int launch_circ_mm(const void* in, const float* c, void* out, int64_t batch, int64_t nin, int64_t nout, bool trans,
                   hipStream_t s) {
  constexpr MmParams K = mm_params(P);
  const int64_t gx = (batch + K.tb - 1) / K.tb, gy = (nout + K.to - 1) / K.to;
  if (gx > 0x7fffffff || gy > 65535 || nin > 0x7fffffff || nout > 0x7fffffff) return RDFFT_ERR_SIZE;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
  const auto* pi = static_cast<const typename Io::T*>(in);
  auto* po = static_cast<typename Io::T*>(out);
  if (trans)
    circ_mm_kernel<P, true, Io><<<grid, dim3(K.nt), 0, s>>>(pi, c, po, batch, int(nin), int(nout));
  else
    circ_mm_kernel<P, false, Io><<<grid, dim3(K.nt), 0, s>>>(pi, c, po, batch, int(nin), int(nout));
  return launch_status();
}

int launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  fill_zero_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(p, n);
  return launch_status();
}

template <int P, class Io>
int launch_circ_dc(const void* x, const void* dy, float* dc, int64_t batch, int64_t k, int64_t q, hipStream_t s) {
  constexpr DcParams K = dc_params(P);
  const int64_t gy = (q + K.ti - 1) / K.ti, gz = (k + K.tj - 1) / K.tj;
  if (gy > 65535 || gz > 65535 || k > 0x7fffffff || q > 0x7fffffff) return RDFFT_ERR_SIZE;
  int64_t want_x = kDcTargetWgs / (gy * gz);
  if (want_x < 1) want_x = 1;
  int64_t tpw = (batch + want_x - 1) / want_x;
  tpw = (tpw + K.tb - 1) / K.tb * K.tb;
  const int64_t gx = (batch + tpw - 1) / tpw;
  if (gx > 0x7fffffff) return RDFFT_ERR_SIZE;
  int st = launch_fill_zero(dc, q * k * P, s);
  if (st != RDFFT_OK) return st;
  circ_dc_kernel<P, Io><<<dim3(unsigned(gx), unsigned(gy), unsigned(gz)), dim3(K.nt), 0, s>>>(
      static_cast<const typename Io::T*>(x), static_cast<const typename Io::T*>(dy), dc, batch, int(k), int(q), tpw);
  st = launch_status();
  if (st != RDFFT_OK) return st;
  return launch_rdfft<P, F32Io, true>(dc, q * k, s);
}

constexpr int64_t kMaxLds = 160 * 1024;
constexpr int64_t kTargetWgs = 256;  // workgroups per launch of the token-persistent kernels

// token split: about `target` workgroups over `tiles` weight tiles, tpw a multiple of tb
int64_t tokens_per_wg(int64_t batch, int64_t tiles, int tb, int64_t target = kTargetWgs) {
  int64_t gx = target / tiles;
  if (gx < 1) gx = 1;
  int64_t tpw = (batch + gx - 1) / gx;
  return (tpw + tb - 1) / tb * tb;
}

// y = circulant product of `in` (forward, or transposed for dx).  When the
// token-persistent kernel runs, it also clears zero[0..nzero) and sets
// *zeroed; otherwise zero is left alone.
template <int P, class Io>
int launch_circ_product(const void* in, const float* c, void* out, int64_t batch, int64_t nin, int64_t nout, bool trans,
                        hipStream_t s, float* zero = nullptr, int64_t nzero = 0, bool* zeroed = nullptr) {
  if constexpr (P >= 64) {
    using S = TpShape<P>;
    if (nin <= S::CR && S::fits(static_cast<int>(nin)) && S::lds_bytes(static_cast<int>(nin)) <= kMaxLds &&
        nout <= 0x7fffffff) {
      const int64_t gy = (nout + S::K.to - 1) / S::K.to;
      const int64_t tpw = tokens_per_wg(batch, gy, S::K.tb);
      const int64_t gx = (batch + tpw - 1) / tpw;
      if (gx > 0x7fffffff || gy > 65535) return RDFFT_ERR_SIZE;
      const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
      const size_t lds = static_cast<size_t>(S::lds_bytes(static_cast<int>(nin)));
      const auto* pi = static_cast<const typename Io::T*>(in);
      auto* po = static_cast<typename Io::T*>(out);
      if (!zero) nzero = 0;
      if (trans)
        circ_tp_kernel<P, true, Io><<<grid, dim3(S::K.nt), lds, s>>>(pi, c, po, batch, int(nin), int(nout), tpw, zero,
                                                                    nzero);
      else
        circ_tp_kernel<P, false, Io><<<grid, dim3(S::K.nt), lds, s>>>(pi, c, po, batch, int(nin), int(nout), tpw,
                                                                     zero, nzero);
      if (zeroed) *zeroed = nzero > 0;
      return launch_status();
    }
  }
  return launch_circ_mm<P, Io>(in, c, out, batch, nin, nout, trans, s);
}

template <int P, class Io>
int launch_circ_dc_any(const void* x, const void* dy, float* dc, int64_t batch, int64_t k, int64_t q, hipStream_t s,
                       bool zeroed) {
  if constexpr (P >= 64) {
    using S = DtpShape<P>;
    const int64_t gy = (q + S::K.ti - 1) / S::K.ti, gz = (k + S::K.tj - 1) / S::K.tj;
    if (gy > 65535 || gz > 65535 || k > 0x7fffffff || q > 0x7fffffff) return RDFFT_ERR_SIZE;
    const int64_t tpw = tokens_per_wg(batch, gy * gz, S::K.tb, S::K.wgs);
    const int64_t gx = (batch + tpw - 1) / tpw;
    if (gx > 0x7fffffff) return RDFFT_ERR_SIZE;
    int st = zeroed ? RDFFT_OK : launch_fill_zero(dc, q * k * P, s);
    if (st != RDFFT_OK) return st;
    circ_dctp_kernel<P, Io><<<dim3(unsigned(gx), unsigned(gy), unsigned(gz)), dim3(S::K.nt),
                              static_cast<size_t>(S::lds_bytes()), s>>>(
        static_cast<const typename Io::T*>(x), static_cast<const typename Io::T*>(dy), dc, batch, int(k), int(q), tpw);
    st = launch_status();
    if (st != RDFFT_OK || dc_time_domain(P, false)) return st;
    return launch_rdfft<P, F32Io, true>(dc, q * k, s);  // dc holds packed spectra
  } else {
    return launch_circ_dc<P, Io>(x, dy, dc, batch, k, q, s);
  }
}

// dx and dc in one launch (circ_bwd_kernel) where the row length allows it and
// the dx tiles fit; returns false when the caller must take the two-kernel path.
constexpr int64_t kBwdDxWgs = 256;  // dx workgroups the fused token split aims at

template <int P, class Io>
bool launch_circ_bwd_fused(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch,
                           int64_t k, int64_t q, hipStream_t s, int* status) {
  if constexpr (bwd_fusable<P>()) {
    using S = TpShape<P, true>;
    using D = DtpShape<P>;
    if (q > S::CR || !S::fits(static_cast<int>(q)) || S::lds_bytes(static_cast<int>(q)) > kMaxLds ||
        k > 0x7fffffff)
      return false;
    const int64_t gdy = (q + D::K.ti - 1) / D::K.ti, gdz = (k + D::K.tj - 1) / D::K.tj;
    const int64_t tpw_dc = tokens_per_wg(batch, gdy * gdz, D::K.tb, D::K.fwgs);
    const int64_t gdx = (batch + tpw_dc - 1) / tpw_dc;
    const int64_t gxy = (k + S::K.to - 1) / S::K.to;
    const int64_t tpw_dx = tokens_per_wg(batch, gxy, S::K.tb, kBwdDxWgs);
    const int64_t gxx = (batch + tpw_dx - 1) / tpw_dx;
    const int64_t ndc = gdx * gdy * gdz, nwg = ndc + gxx * gxy;
    if (nwg > 0x7fffffff || gdx > 0x7fffffff || gdy > 0x7fffffff || gxx > 0x7fffffff) return false;
    const int64_t lds_dx = S::lds_bytes(static_cast<int>(q)), lds_dc = D::lds_bytes();
    const int64_t lds = lds_dx > lds_dc ? lds_dx : lds_dc;
    int st = launch_fill_zero(dc, q * k * P, s);
    if (st == RDFFT_OK) {
      circ_bwd_kernel<P, Io><<<dim3(static_cast<unsigned>(nwg)), dim3(S::K.nt), static_cast<size_t>(lds), s>>>(
          static_cast<const typename Io::T*>(x), c, static_cast<const typename Io::T*>(dy),
          static_cast<typename Io::T*>(dx), dc, batch, int(k), int(q), tpw_dc, int(gdx), int(gdy), ndc, tpw_dx,
          int(gxx));
      st = launch_status();
    }
    *status = st;
    return true;
  } else {
    (void)x, (void)c, (void)dy, (void)dx, (void)dc, (void)batch, (void)k, (void)q, (void)s, (void)status;
    return false;
  }
}

template <int P, class Io>
int circ_fwd_p(const void* x, const float* c, void* y, int64_t batch, int64_t d_in, int64_t d_out, hipStream_t s) {
  return launch_circ_product<P, Io>(x, c, y, batch, d_in / P, d_out / P, false, s);
}

template <int P, class Io>
int circ_bwd_p(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch, int64_t d_in,
               int64_t d_out, hipStream_t s) {
  const int64_t k = d_in / P, q = d_out / P;
  if (batch == 0) return dc ? launch_fill_zero(dc, q * k * P, s) : RDFFT_OK;
  int fused_status = RDFFT_OK;
  if (dx && dc && launch_circ_bwd_fused<P, Io>(x, c, dy, dx, dc, batch, k, q, s, &fused_status)) return fused_status;
  bool zeroed = false;  // dc cleared by the dx kernel
  if (dx) {
    const int st = launch_circ_product<P, Io>(dy, c, dx, batch, q, k, true, s, dc, dc ? q * k * P : 0, &zeroed);
    if (st != RDFFT_OK) return st;
  }
  if (dc) return launch_circ_dc_any<P, Io>(x, dy, dc, batch, k, q, s, zeroed);
  return RDFFT_OK;
}

#define RDFFT_P_SWITCH(p, CALL)      \
  switch (p) {                       \
    case 2: return CALL(2);          \
    case 4: return CALL(4);          \
    case 8: return CALL(8);          \
    case 16: return CALL(16);        \
    case 32: return CALL(32);        \
    case 64: return CALL(64);        \
    case 128: return CALL(128);      \
    case 256: return CALL(256);      \
    case 512: return CALL(512);      \
    case 1024: return CALL(1024);    \
    case 2048: return CALL(2048);    \
    case 4096: return CALL(4096);    \
    default: return RDFFT_ERR_SIZE;  \
  }

template <class Io>
int circ_fwd_dispatch(const void* x, const float* c, void* y, int64_t batch, int64_t d_in, int64_t d_out, int64_t p,
                      hipStream_t s) {
#define CALL(P) circ_fwd_p<P, Io>(x, c, y, batch, d_in, d_out, s)
  RDFFT_P_SWITCH(p, CALL)
#undef CALL
}

template <class Io>
int circ_bwd_dispatch(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch, int64_t d_in,
                      int64_t d_out, int64_t p, hipStream_t s) {
#define CALL(P) circ_bwd_p<P, Io>(x, c, dy, dx, dc, batch, d_in, d_out, s)
  RDFFT_P_SWITCH(p, CALL)
#undef CALL
}

// call f(Io{}) with the storage type of dtype (validated before)
template <class F>
int by_dtype(int dtype, F f) {
  switch (dtype) {
    case RDFFT_BF16: return f(Bf16Io{});
    case RDFFT_F16: return f(F16Io{});
    default: return f(F32Io{});
  }
}

template <bool INV>
int rdfft_entry(void* data, int64_t rows, int64_t p, int dtype, void* stream) {
  const int st = check_rdfft(data, rows, p, dtype);
  if (st != RDFFT_OK || rows == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return by_dtype(dtype, [&](auto io) { return dispatch_rdfft<decltype(io), INV>(data, rows, p, s); });
}

// grid of the element-wise spectrum kernels: grid-stride over total elements
unsigned elementwise_grid(int64_t total) {
  const int64_t cap = static_cast<int64_t>(device_cus()) * 16;
  const int64_t want = (total + 255) / 256;
  return static_cast<unsigned>(want < cap ? want : cap);
}

// ---- 2D ----------------------------------------------------------------------

template <int H, class Io, bool INV>
int launch_cols(void* data, int64_t n, int64_t w, hipStream_t s) {
  using S = ColShape<H>;
  const int64_t ntiles = (w + S::CL - 1) / S::CL;
  if (n * ntiles > 0x7fffffff) return RDFFT_ERR_SIZE;
  col_kernel<H, INV, Io><<<dim3(static_cast<unsigned>(n * ntiles)), dim3(S::NT), static_cast<size_t>(S::lds_bytes()), s>>>(
      static_cast<typename Io::T*>(data), static_cast<int>(w), static_cast<int>(ntiles));
  return launch_status();
}

template <class Io, bool INV>
int dispatch_cols(void* data, int64_t n, int64_t h, int64_t w, hipStream_t s) {
  switch (h) {
    case 2: return launch_cols<2, Io, INV>(data, n, w, s);
    case 4: return launch_cols<4, Io, INV>(data, n, w, s);
    case 8: return launch_cols<8, Io, INV>(data, n, w, s);
    case 16: return launch_cols<16, Io, INV>(data, n, w, s);
    case 32: return launch_cols<32, Io, INV>(data, n, w, s);
    case 64: return launch_cols<64, Io, INV>(data, n, w, s);
    case 128: return launch_cols<128, Io, INV>(data, n, w, s);
    case 256: return launch_cols<256, Io, INV>(data, n, w, s);
    case 512: return launch_cols<512, Io, INV>(data, n, w, s);
    case 1024: return launch_cols<1024, Io, INV>(data, n, w, s);
    case 2048: return launch_cols<2048, Io, INV>(data, n, w, s);
    case 4096: return launch_cols<4096, Io, INV>(data, n, w, s);
    default: return RDFFT_ERR_SIZE;
  }
}

template <class Io, bool INV>
int launch_combine(void* data, int64_t n, int64_t h, int64_t w, hipStream_t s) {
  if (h < 4 || w < 4) return RDFFT_OK;  // no pair (j, k) with 0 < j < h/2 and 0 < k < w/2
  const int64_t total = n * (h / 2) * (w / 2);
  combine_kernel<INV, Io><<<dim3(elementwise_grid(total)), dim3(256), 0, s>>>(
      static_cast<typename Io::T*>(data), n, ilog2(static_cast<int>(h)), ilog2(static_cast<int>(w)));
  return launch_status();
}

template <bool INV>
int rdfft2d_entry(void* data, int64_t n, int64_t h, int64_t w, int dtype, void* stream) {
  const int st = check_rdfft2d(data, n, h, w, dtype);
  if (st != RDFFT_OK || n == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return by_dtype(dtype, [&](auto io) {
    using Io = decltype(io);
    int r;
    if (!INV) {
      if ((r = dispatch_rdfft<Io, false>(data, n * h, w, s)) != RDFFT_OK) return r;
      if ((r = dispatch_cols<Io, false>(data, n, h, w, s)) != RDFFT_OK) return r;
      return launch_combine<Io, false>(data, n, h, w, s);
    }
    if ((r = launch_combine<Io, true>(data, n, h, w, s)) != RDFFT_OK) return r;
    if ((r = dispatch_cols<Io, true>(data, n, h, w, s)) != RDFFT_OK) return r;
    return dispatch_rdfft<Io, true>(data, n * h, w, s);
  });
}

template <bool PACK>
int spectrum_entry(const void* packed, const float* spec, int64_t rows, int64_t p, int dtype, void* stream) {
  const int st = check_spectrum(packed, spec, rows, p, dtype);
  if (st != RDFFT_OK || rows == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int lp = ilog2(static_cast<int>(p));
  const unsigned grid = elementwise_grid(rows * (p / 2));  // one thread per bin below p/2
  return by_dtype(dtype, [&](auto io) {
    using Io = decltype(io);
    auto* z = static_cast<typename Io::T*>(const_cast<void*>(packed));
    if (PACK)
      pack_kernel<Io><<<dim3(grid), dim3(256), 0, s>>>(spec, z, rows, lp);
    else
      unpack_kernel<Io><<<dim3(grid), dim3(256), 0, s>>>(z, const_cast<float*>(spec), rows, lp);
    return launch_status();
  });
}

}  // namespace
}  // namespace rdfft

extern "C" {

int rdfft_abi_version(void) { return RDFFT_ABI_VERSION; }

const char* rdfft_status_string(int status) {
  switch (status) {
    case RDFFT_OK: return "ok";
    case RDFFT_ERR_NULL: return "null pointer";
    case RDFFT_ERR_SIZE:
      return "unsupported size (p a power of two in [2, 32768] for transforms and spectra, [2, 4096] for "
             "circulant layers; counts >= 0)";
    case RDFFT_ERR_SHAPE: return "d_in and d_out must be positive multiples of p";
    case RDFFT_ERR_DTYPE: return "unknown dtype (RDFFT_F32, RDFFT_BF16 or RDFFT_F16)";
    case RDFFT_ERR_ALIGN: return "pointer not 16-byte aligned";
    case RDFFT_ERR_ALIAS: return "output buffer overlaps another buffer";
    case RDFFT_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int rdfft_forward(void* data, int64_t rows, int64_t p, int dtype, void* stream) {
  return rdfft::rdfft_entry<false>(data, rows, p, dtype, stream);
}

int rdfft_inverse(void* data, int64_t rows, int64_t p, int dtype, void* stream) {
  return rdfft::rdfft_entry<true>(data, rows, p, dtype, stream);
}

int circulant_fwd(const void* x, const float* c, void* y, int64_t batch, int64_t d_in, int64_t d_out, int64_t p,
                  int dtype, void* stream) {
  const int st = rdfft::check_circulant_fwd(x, c, y, batch, d_in, d_out, p, dtype);
  if (st != RDFFT_OK || batch == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return rdfft::by_dtype(dtype, [&](auto io) {
    return rdfft::circ_fwd_dispatch<decltype(io)>(x, c, y, batch, d_in, d_out, p, s);
  });
}

int circulant_bwd(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch, int64_t d_in,
                  int64_t d_out, int64_t p, int dtype, void* stream) {
  const int st = rdfft::check_circulant_bwd(x, c, dy, dx, dc, batch, d_in, d_out, p, dtype);
  if (st != RDFFT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return rdfft::by_dtype(dtype, [&](auto io) {
    return rdfft::circ_bwd_dispatch<decltype(io)>(x, c, dy, dx, dc, batch, d_in, d_out, p, s);
  });
}

int rdfft_unpack(const void* packed, float* spec, int64_t rows, int64_t p, int dtype, void* stream) {
  return rdfft::spectrum_entry<false>(packed, spec, rows, p, dtype, stream);
}

int rdfft_pack(const float* spec, void* packed, int64_t rows, int64_t p, int dtype, void* stream) {
  return rdfft::spectrum_entry<true>(packed, spec, rows, p, dtype, stream);
}

int rdfft2d_forward(void* data, int64_t n, int64_t h, int64_t w, int dtype, void* stream) {
  return rdfft::rdfft2d_entry<false>(data, n, h, w, dtype, stream);
}

int rdfft2d_inverse(void* data, int64_t n, int64_t h, int64_t w, int dtype, void* stream) {
  return rdfft::rdfft2d_entry<true>(data, n, h, w, dtype, stream);
}

}  // extern "C"
