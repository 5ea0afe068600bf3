// rdfft_lib.hip -- C ABI of librdfft.so: argument checks, kernel selection, launches.
#include <hip/hip_runtime.h>

#include <atomic>

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
  const int64_t resident = static_cast<int64_t>(device_cus()) * wg_per_cu(P, is_f32_io<Io>(), INV);
  const int64_t grid = groups < resident ? groups : resident;
  auto* d = static_cast<typename Io::T*>(data);
  if (INV)
    hipLaunchKernelGGL((rdfft_inv_kernel<P, Io>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0, stream, d, rows);
  else
    hipLaunchKernelGGL((rdfft_fwd_kernel<P, Io>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0, stream, d, rows);
  return launch_status();
}

template <int P, class Io, bool INV>
int launch_rdfft_long(void* data, int64_t rows, hipStream_t stream) {
  constexpr int E = long_elems(P);
  const size_t lds = static_cast<size_t>(Row<P, E>::LDS) * sizeof(float);
  if (rows > 0x7fffffff) return RDFFT_ERR_SIZE;
  auto* d = static_cast<typename Io::T*>(data);
  if (INV)
    hipLaunchKernelGGL((rdfft_inv_long_kernel<P, Io>), dim3(static_cast<unsigned>(rows)), dim3(P / E), lds, stream, d);
  else
    hipLaunchKernelGGL((rdfft_fwd_long_kernel<P, Io>), dim3(static_cast<unsigned>(rows)), dim3(P / E), lds, stream, d);
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

// WSPEC: c holds the weights' packed spectra (every launcher below)
template <int P, class Io, bool WSPEC = false>
int launch_circ_mm(const void* in, const float* c, void* out, int64_t batch, int64_t nin, int64_t nout, bool trans,
                   hipStream_t s) {
  constexpr MmParams K = mm_params(P);
  const int64_t gx = (batch + K.tb - 1) / K.tb, gy = (nout + K.to - 1) / K.to;
  if (gx > 0x7fffffff || gy > 65535 || nin > 0x7fffffff || nout > 0x7fffffff) return RDFFT_ERR_SIZE;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
  const auto* pi = static_cast<const typename Io::T*>(in);
  auto* po = static_cast<typename Io::T*>(out);
  if (trans)
    hipLaunchKernelGGL((circ_mm_kernel<P, true, Io, WSPEC>), grid, dim3(K.nt), 0, s, pi, c, po, batch, int(nin),
                       int(nout));
  else
    hipLaunchKernelGGL((circ_mm_kernel<P, false, Io, WSPEC>), grid, dim3(K.nt), 0, s, pi, c, po, batch, int(nin),
                       int(nout));
  return launch_status();
}

int launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL((fill_zero_kernel), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, n);
  return launch_status();
}

// grid of a weight-gradient launch: gx token ranges of tpw tokens times gy x gz
// tiles of (i, j); ok = false when it exceeds the launch limits
struct DcSplit {
  int64_t gx, gy, gz, tpw;
  bool ok;
};

template <int P>
DcSplit dc_split_small(int64_t batch, int64_t k, int64_t q) {
  constexpr DcParams K = dc_params(P);
  DcSplit d{};
  d.gy = (q + K.ti - 1) / K.ti;
  d.gz = (k + K.tj - 1) / K.tj;
  if (d.gy > 65535 || d.gz > 65535 || k > 0x7fffffff || q > 0x7fffffff) return d;
  int64_t want_x = kDcTargetWgs / (d.gy * d.gz);
  if (want_x < 1) want_x = 1;
  int64_t tpw = (batch + want_x - 1) / want_x;
  d.tpw = (tpw + K.tb - 1) / K.tb * K.tb;
  d.gx = (batch + d.tpw - 1) / d.tpw;
  d.ok = d.gx <= 0x7fffffff;
  return d;
}

// the fixed-order sum of a deterministic dc (parts slices of the workspace ws),
// then the inverse where the slices hold packed spectra
template <int P>
int launch_dc_reduce(const float* ws, float* dc, int64_t n, int64_t parts, bool spectra, hipStream_t s) {
  const int64_t blocks = (n + kReduceEl - 1) / kReduceEl;
  if (parts > 0x7fffffff || blocks > 0x7fffffff) return RDFFT_ERR_SIZE;
  hipLaunchKernelGGL((dc_reduce_kernel), dim3(static_cast<unsigned>(blocks)), dim3(kReduceEl * kReduceGroups), 0, s,
                     ws, dc, n, static_cast<int>(parts));
  const int st = launch_status();
  if (st != RDFFT_OK || !spectra) return st;
  return launch_rdfft<P, F32Io, true>(dc, n / P, s);
}

// ws: deterministic mode, the partial sums stored into ws (one q k P slice per
// token range) and summed in order into dc; otherwise added into dc atomically
template <int P, class Io>
int launch_circ_dc(const void* x, const void* dy, float* dc, int64_t batch, int64_t k, int64_t q, hipStream_t s,
                   bool acc, float* ws) {
  constexpr DcParams K = dc_params(P);
  const DcSplit d = dc_split_small<P>(batch, k, q);
  if (!d.ok) return RDFFT_ERR_SIZE;
  const dim3 grid(unsigned(d.gx), unsigned(d.gy), unsigned(d.gz));
  const auto* px = static_cast<const typename Io::T*>(x);
  const auto* pdy = static_cast<const typename Io::T*>(dy);
  if (ws) {
    hipLaunchKernelGGL((circ_dc_kernel<P, Io, true>), grid, dim3(K.nt), 0, s, px, pdy, ws, batch, int(k), int(q),
                       d.tpw);
    const int st = launch_status();
    if (st != RDFFT_OK) return st;
    return launch_dc_reduce<P>(ws, dc, q * k * P, d.gx, true, s);
  }
  // the kernel adds packed spectra into dc, which the inverse at the end
  // transforms back: start from zero, or (accumulating) from the spectra of
  // what dc holds, so that the inverse returns old dc + the new sum
  int st = acc ? launch_rdfft<P, F32Io, false>(dc, q * k, s) : launch_fill_zero(dc, q * k * P, s);
  if (st != RDFFT_OK) return st;
  hipLaunchKernelGGL((circ_dc_kernel<P, Io>), grid, dim3(K.nt), 0, s, px, pdy, dc, batch, int(k), int(q), d.tpw);
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

// one-block layers (d_in = d_out = p) on circ_one_kernel, with the side jobs
// of the token-persistent kernel (clear zero[0..nzero); forward from c: store
// the weight spectrum into wout)
template <int P, class Io, bool WSPEC>
int launch_circ_one(const void* in, const float* c, void* out, int64_t batch, bool trans, hipStream_t s, float* zero,
                    int64_t nzero, bool* zeroed, float* wout, bool* wout_done) {
  constexpr int NT = P / elems_per_thread(P);
  const int64_t cap = static_cast<int64_t>(device_cus()) * kOneWgPerCu;
  const int64_t grid = batch < 1 ? 1 : batch < cap ? batch : cap;
  if (!zero) nzero = 0;
  const bool wo = wout != nullptr && !trans && !WSPEC && batch > 0;
  const auto* pi = static_cast<const typename Io::T*>(in);
  auto* po = static_cast<typename Io::T*>(out);
  if (trans)
    hipLaunchKernelGGL((circ_one_kernel<P, true, Io, WSPEC>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0, s, pi, c,
                       po, batch, zero, nzero, static_cast<float*>(nullptr));
  else
    hipLaunchKernelGGL((circ_one_kernel<P, false, Io, WSPEC>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0, s, pi,
                       c, po, batch, zero, nzero, wo ? wout : nullptr);
  if (zeroed) *zeroed = nzero > 0;
  if (wout_done) *wout_done = wo;
  return launch_status();
}

// row lengths whose one-block layers take circ_one_kernel
template <int P>
constexpr bool one_block_kernel() {
  return P == 4096;
}

// y = circulant product of `in` (forward, or transposed for dx).  When the
// token-persistent kernel (or the one-block kernel) runs, it also clears
// zero[0..nzero) and sets *zeroed, and (forward from c) stores the weight
// spectra into wout if given; otherwise zero and wout are left alone.
template <int P, class Io, bool WSPEC = false>
int launch_circ_product(const void* in, const float* c, void* out, int64_t batch, int64_t nin, int64_t nout, bool trans,
                        hipStream_t s, float* zero = nullptr, int64_t nzero = 0, bool* zeroed = nullptr,
                        float* wout = nullptr, bool* wout_done = nullptr) {
  if constexpr (one_block_kernel<P>()) {
    if (nin == 1 && nout == 1)
      return launch_circ_one<P, Io, WSPEC>(in, c, out, batch, trans, s, zero, nzero, zeroed, wout, wout_done);
  }
  if constexpr (P >= 64) {
    using S = TpShape<P, false, WSPEC>;
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
        hipLaunchKernelGGL((circ_tp_kernel<P, true, Io, WSPEC>), grid, dim3(S::K.nt), lds, s, pi, c, po, batch,
                           int(nin), int(nout), tpw, zero, nzero, static_cast<float*>(nullptr));
      else
        hipLaunchKernelGGL((circ_tp_kernel<P, false, Io, WSPEC>), grid, dim3(S::K.nt), lds, s, pi, c, po, batch,
                           int(nin), int(nout), tpw, zero, nzero, WSPEC ? nullptr : wout);
      if (zeroed) *zeroed = nzero > 0;
      if (wout_done) *wout_done = wout != nullptr && !trans && !WSPEC;
      return launch_status();
    }
  }
  return launch_circ_mm<P, Io, WSPEC>(in, c, out, batch, nin, nout, trans, s);
}

// split of the token-persistent weight-gradient tiles, `target` workgroups aimed at
template <int P>
DcSplit dc_split_tp(int64_t batch, int64_t k, int64_t q, int64_t target) {
  using S = DtpShape<P>;
  DcSplit d{};
  d.gy = (q + S::K.ti - 1) / S::K.ti;
  d.gz = (k + S::K.tj - 1) / S::K.tj;
  if (d.gy > 65535 || d.gz > 65535 || k > 0x7fffffff || q > 0x7fffffff) return d;
  d.tpw = tokens_per_wg(batch, d.gy * d.gz, S::K.tb, target);
  d.gx = (batch + d.tpw - 1) / d.tpw;
  d.ok = d.gx <= 0x7fffffff;
  return d;
}

template <int P, class Io>
int launch_circ_dc_any(const void* x, const void* dy, float* dc, int64_t batch, int64_t k, int64_t q, hipStream_t s,
                       bool zeroed, bool acc, float* ws) {
  if constexpr (P >= 64) {
    using S = DtpShape<P>;
    const DcSplit d = dc_split_tp<P>(batch, k, q, S::K.wgs);
    if (!d.ok) return RDFFT_ERR_SIZE;
    const int64_t gx = d.gx, gy = d.gy, gz = d.gz, tpw = d.tpw;
    if (ws) {
      hipLaunchKernelGGL((circ_dctp_kernel<P, Io, true>), dim3(unsigned(gx), unsigned(gy), unsigned(gz)),
                         dim3(S::K.nt), static_cast<size_t>(S::lds_bytes()), s, static_cast<const typename Io::T*>(x),
                         static_cast<const typename Io::T*>(dy), ws, batch, int(k), int(q), tpw);
      const int st = launch_status();
      if (st != RDFFT_OK) return st;
      return launch_dc_reduce<P>(ws, dc, q * k * P, gx, !dc_time_domain(P, false), s);
    }
    // accumulating into time-domain dc needs nothing first; into packed
    // spectra, dc is transformed forward (see launch_circ_dc)
    int st = RDFFT_OK;
    if (acc) {
      if (!dc_time_domain(P, false)) st = launch_rdfft<P, F32Io, false>(dc, q * k, s);
    } else if (!zeroed) {
      st = launch_fill_zero(dc, q * k * P, s);
    }
    if (st != RDFFT_OK) return st;
    hipLaunchKernelGGL((circ_dctp_kernel<P, Io>), dim3(unsigned(gx), unsigned(gy), unsigned(gz)), dim3(S::K.nt),
                       static_cast<size_t>(S::lds_bytes()), s, static_cast<const typename Io::T*>(x),
                       static_cast<const typename Io::T*>(dy), dc, batch, int(k), int(q), tpw);
    st = launch_status();
    if (st != RDFFT_OK || dc_time_domain(P, false)) return st;
    return launch_rdfft<P, F32Io, true>(dc, q * k, s);  // dc holds packed spectra
  } else {
    (void)zeroed;
    return launch_circ_dc<P, Io>(x, dy, dc, batch, k, q, s, acc, ws);
  }
}

// dx and dc in one launch (circ_bwd_kernel) where the row length allows it and
// the dx tiles fit; returns false when the caller must take the two-kernel path.
// dx workgroups the fused token split aims at: 128 beside the 128 dc
// workgroups fill the chip in one round of workgroups (D=4096 B=256 bf16
// training step, 256 -> 128: p=128 5.24 -> 5.61 M tokens/s, p=512 7.59 ->
// 8.58 M, p=4096 and the adapter shape unchanged; 64 and 96 slower everywhere)
constexpr int64_t kBwdDxWgs = 128;

// whether dx and dc of this shape run in one launch (circ_bwd_kernel)
template <int P, bool WSPEC = false>
bool bwd_fused_shape(int64_t k, int64_t q) {
  if constexpr (bwd_fusable<P>()) {
    using S = TpShape<P, true, WSPEC>;
    return q <= S::CR && S::fits(static_cast<int>(q)) && S::lds_bytes(static_cast<int>(q)) <= kMaxLds &&
           k <= 0x7fffffff;
  } else {
    (void)k, (void)q;
    return false;
  }
}

template <int P, class Io, bool WSPEC = false>
bool launch_circ_bwd_fused(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch,
                           int64_t k, int64_t q, bool acc, float* ws, hipStream_t s, int* status) {
  if constexpr (bwd_fusable<P>()) {
    using S = TpShape<P, true, WSPEC>;
    using D = DtpShape<P>;
    if (!bwd_fused_shape<P, WSPEC>(k, q) || (WSPEC && ws)) return false;
    const DcSplit d = dc_split_tp<P>(batch, k, q, D::K.fwgs);
    if (!d.ok) return false;
    const int64_t gdy = d.gy, gdz = d.gz, tpw_dc = d.tpw, gdx = d.gx;
    const int64_t gxy = (k + S::K.to - 1) / S::K.to;
    const int64_t tpw_dx = tokens_per_wg(batch, gxy, S::K.tb, kBwdDxWgs);
    const int64_t gxx = (batch + tpw_dx - 1) / tpw_dx;
    const int64_t ndc = gdx * gdy * gdz, nwg = ndc + gxx * gxy;
    if (nwg > 0x7fffffff || gdx > 0x7fffffff || gdy > 0x7fffffff || gxx > 0x7fffffff) return false;
    const int64_t lds_dx = S::lds_bytes(static_cast<int>(q)), lds_dc = D::lds_bytes();
    const int64_t lds = lds_dx > lds_dc ? lds_dx : lds_dc;
    const auto* px = static_cast<const typename Io::T*>(x);
    const auto* pdy = static_cast<const typename Io::T*>(dy);
    auto* pdx = static_cast<typename Io::T*>(dx);
    int st = RDFFT_OK;
    if (ws) {
      hipLaunchKernelGGL((circ_bwd_kernel<P, Io, true, WSPEC>), dim3(static_cast<unsigned>(nwg)), dim3(S::K.nt),
                         static_cast<size_t>(lds), s, px, c, pdy, pdx, ws, batch, int(k), int(q), tpw_dc, int(gdx),
                         int(gdy), ndc, tpw_dx, int(gxx));
      st = launch_status();
      if (st == RDFFT_OK) st = launch_dc_reduce<P>(ws, dc, q * k * P, gdx, false, s);  // time-domain slices
    } else {
      st = acc ? RDFFT_OK : launch_fill_zero(dc, q * k * P, s);  // dc is added into in the time domain
      if (st == RDFFT_OK) {
        hipLaunchKernelGGL((circ_bwd_kernel<P, Io, false, WSPEC>), dim3(static_cast<unsigned>(nwg)), dim3(S::K.nt),
                           static_cast<size_t>(lds), s, px, c, pdy, pdx, dc, batch, int(k), int(q), tpw_dc, int(gdx),
                           int(gdy), ndc, tpw_dx, int(gxx));
        st = launch_status();
      }
    }
    *status = st;
    return true;
  } else {
    (void)x, (void)c, (void)dy, (void)dx, (void)dc, (void)batch, (void)k, (void)q, (void)acc, (void)ws, (void)s,
        (void)status;
    return false;
  }
}

// cs[row] = packed spectrum of c[row], rows = q k (weights given as spectra)
template <int P>
int launch_weight_spectra(const float* c, float* cs, int64_t rows, hipStream_t s) {
  constexpr int CR = kSpecThreads / (P / elems_per_thread(P));
  const int64_t groups = (rows + CR - 1) / CR;
  const int64_t cap = static_cast<int64_t>(device_cus()) * 4;
  const int64_t grid = groups < cap ? groups : cap;
  if (grid <= 0) return RDFFT_OK;
  hipLaunchKernelGGL((weight_spectra_kernel<P>), dim3(static_cast<unsigned>(grid)), dim3(kSpecThreads), 0, s, c, cs,
                     rows);
  return launch_status();
}

// forward; a non-null zero[q k P] (a gradient accumulator of c) is cleared by
// the token-persistent kernel as a side job, or by a fill where another runs
template <int P, class Io, bool WSPEC = false>
int circ_fwd_p(const void* x, const float* c, void* y, int64_t batch, int64_t d_in, int64_t d_out, hipStream_t s,
               float* zero, float* wout = nullptr) {
  const int64_t k = d_in / P, q = d_out / P;
  bool zeroed = false, wrote = false;
  int st = launch_circ_product<P, Io, WSPEC>(x, c, y, batch, k, q, false, s, zero, zero ? q * k * P : 0, &zeroed,
                                             wout, &wrote);
  if (st == RDFFT_OK && wout && !wrote) st = launch_weight_spectra<P>(c, wout, q * k, s);
  if (st != RDFFT_OK || !zero || zeroed) return st;
  return launch_fill_zero(zero, q * k * P, s);
}

// token ranges of the weight-gradient launch a backward of this shape takes
// (with dx or without): the slices a deterministic dc needs in its workspace
template <int P>
int64_t dc_token_ranges(int64_t batch, int64_t k, int64_t q, bool with_dx) {
  if (batch == 0) return 0;
  DcSplit d{};
  if constexpr (P >= 64) {
    d = (with_dx && bwd_fused_shape<P>(k, q)) ? dc_split_tp<P>(batch, k, q, DtpShape<P>::K.fwgs)
                                              : dc_split_tp<P>(batch, k, q, DtpShape<P>::K.wgs);
  } else {
    (void)with_dx;
    d = dc_split_small<P>(batch, k, q);
  }
  return d.ok ? d.gx : -1;
}

// backward; acc: add the token sum into dc instead of overwriting it;
// ws: deterministic dc (see launch_circ_dc), overwritten, never with acc
template <int P, class Io, bool WSPEC = false>
int circ_bwd_p(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch, int64_t d_in,
               int64_t d_out, bool acc, hipStream_t s, float* ws = nullptr) {
  const int64_t k = d_in / P, q = d_out / P;
  if (batch == 0) return (dc && !acc) ? launch_fill_zero(dc, q * k * P, s) : RDFFT_OK;
  int fused_status = RDFFT_OK;
  if (dx && dc && launch_circ_bwd_fused<P, Io, WSPEC>(x, c, dy, dx, dc, batch, k, q, acc, ws, s, &fused_status))
    return fused_status;
  bool zeroed = false;  // dc cleared by the dx kernel
  if (dx) {
    float* zero = (acc || ws) ? nullptr : dc;
    const int st =
        launch_circ_product<P, Io, WSPEC>(dy, c, dx, batch, q, k, true, s, zero, zero ? q * k * P : 0, &zeroed);
    if (st != RDFFT_OK) return st;
  }
  if (dc) return launch_circ_dc_any<P, Io>(x, dy, dc, batch, k, q, s, zeroed, acc, ws);
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

template <class Io, bool WSPEC = false>
int circ_fwd_dispatch(const void* x, const float* c, void* y, int64_t batch, int64_t d_in, int64_t d_out, int64_t p,
                      hipStream_t s, float* zero, float* wout = nullptr) {
#define CALL(P) circ_fwd_p<P, Io, WSPEC>(x, c, y, batch, d_in, d_out, s, zero, wout)
  RDFFT_P_SWITCH(p, CALL)
#undef CALL
}

template <class Io, bool WSPEC = false>
int circ_bwd_dispatch(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch, int64_t d_in,
                      int64_t d_out, int64_t p, bool acc, hipStream_t s, float* ws = nullptr) {
#define CALL(P) circ_bwd_p<P, Io, WSPEC>(x, c, dy, dx, dc, batch, d_in, d_out, acc, s, ws)
  RDFFT_P_SWITCH(p, CALL)
#undef CALL
}

inline int weight_spectra_dispatch(const float* c, float* cs, int64_t rows, int64_t p, hipStream_t s) {
#define CALL(P) launch_weight_spectra<P>(c, cs, rows, s)
  RDFFT_P_SWITCH(p, CALL)
#undef CALL
}

// token ranges of the weight gradient (dims validated before); -1 past the launch limits
inline int64_t dc_token_ranges_dispatch(int64_t batch, int64_t d_in, int64_t d_out, int64_t p, bool with_dx) {
#define CALL(P) dc_token_ranges<P>(batch, d_in / P, d_out / P, with_dx)
  RDFFT_P_SWITCH(p, CALL)
#undef CALL
}

// ---- the allocation-free deterministic backward ---------------------------
// Workspace of circulant_bwd_det_noalloc: a file-scope device array, one copy
// on every GPU the library runs on, held until the process ends.  Host code
// never passes its name to a kernel (on the host the name stands for a host
// stand-in); it takes the array's device address once per device with
// hipGetSymbolAddress and passes that.
constexpr int64_t kScratchBytes = int64_t{32} << 20;  // 32 MiB
static __device__ __align__(256) float scratch[kScratchBytes / 4];

// device address of the current device's scratch, resolved on the first call
// on that device; nullptr when the runtime cannot resolve it
float* scratch_ptr() {
  constexpr int kMaxDev = 64;
  static std::atomic<float*> cached[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  float* p = cached[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
    p = static_cast<float*>(addr);
    cached[dev].store(p, std::memory_order_release);
  }
  return p;
}

// bytes of a deterministic dc's workspace: one q k p slice of floats per token range
inline int circ_det_workspace(int64_t batch, int64_t d_in, int64_t d_out, int64_t p, bool with_dx, int64_t* bytes) {
  const int64_t ranges = dc_token_ranges_dispatch(batch, d_in, d_out, p, with_dx);
  if (ranges < 0) return RDFFT_ERR_SIZE;
  const int64_t slice = (d_out / p) * d_in;  // q k p floats
  if (ranges > 0 && slice > (int64_t{1} << 62) / 4 / ranges) return RDFFT_ERR_SIZE;
  *bytes = ranges * slice * 4;
  return RDFFT_OK;
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
  hipLaunchKernelGGL((col_kernel<H, INV, Io>), dim3(static_cast<unsigned>(n * ntiles)), dim3(S::NT),
                     static_cast<size_t>(S::lds_bytes()), s, static_cast<typename Io::T*>(data), static_cast<int>(w),
                     static_cast<int>(ntiles));
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
  hipLaunchKernelGGL((combine_kernel<INV, Io>), dim3(elementwise_grid(total)), dim3(256), 0, s,
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
      hipLaunchKernelGGL((pack_kernel<Io>), dim3(grid), dim3(256), 0, s, spec, z, rows, lp);
    else
      hipLaunchKernelGGL((unpack_kernel<Io>), dim3(grid), dim3(256), 0, s, z, const_cast<float*>(spec), rows, lp);
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
    case RDFFT_ERR_SCRATCH:
      return "the deterministic dc of this shape needs more than the 32 MiB workspace of the allocation-free call "
             "(use circulant_bwd_det with a workspace)";
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
    return rdfft::circ_fwd_dispatch<decltype(io)>(x, c, y, batch, d_in, d_out, p, s, nullptr);
  });
}

int circulant_fwd_zero(const void* x, const float* c, void* y, float* dc, int64_t batch, int64_t d_in, int64_t d_out,
                       int64_t p, int dtype, void* stream) {
  const int st = rdfft::check_circulant_fwd_zero(x, c, y, dc, batch, d_in, d_out, p, dtype);
  if (st != RDFFT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch == 0) return rdfft::launch_fill_zero(dc, (d_out / p) * d_in, s);
  return rdfft::by_dtype(dtype, [&](auto io) {
    return rdfft::circ_fwd_dispatch<decltype(io)>(x, c, y, batch, d_in, d_out, p, s, dc);
  });
}

int circulant_bwd(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch, int64_t d_in,
                  int64_t d_out, int64_t p, int dtype, void* stream) {
  const int st = rdfft::check_circulant_bwd(x, c, dy, dx, dc, batch, d_in, d_out, p, dtype);
  if (st != RDFFT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return rdfft::by_dtype(dtype, [&](auto io) {
    return rdfft::circ_bwd_dispatch<decltype(io)>(x, c, dy, dx, dc, batch, d_in, d_out, p, false, s);
  });
}

int circulant_bwd_acc(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch,
                      int64_t d_in, int64_t d_out, int64_t p, int dtype, void* stream) {
  const int st = rdfft::check_circulant_bwd(x, c, dy, dx, dc, batch, d_in, d_out, p, dtype);
  if (st != RDFFT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return rdfft::by_dtype(dtype, [&](auto io) {
    return rdfft::circ_bwd_dispatch<decltype(io)>(x, c, dy, dx, dc, batch, d_in, d_out, p, true, s);
  });
}

int circulant_weight_spectra(const float* c, float* cs, int64_t d_in, int64_t d_out, int64_t p, void* stream) {
  const int st = rdfft::check_weight_spectra(c, cs, d_in, d_out, p);
  if (st != RDFFT_OK) return st;
  return rdfft::weight_spectra_dispatch(c, cs, (d_out / p) * (d_in / p), p, static_cast<hipStream_t>(stream));
}

int circulant_fwd_step(const void* x, const float* c, void* y, float* dc, float* cs, int64_t batch, int64_t d_in,
                       int64_t d_out, int64_t p, int dtype, void* stream) {
  int st = dc ? rdfft::check_circulant_fwd_zero(x, c, y, dc, batch, d_in, d_out, p, dtype)
              : rdfft::check_circulant_fwd(x, c, y, batch, d_in, d_out, p, dtype);
  if (st == RDFFT_OK) st = rdfft::check_fwd_step_spectra(x, c, y, dc, cs, batch, d_in, d_out, p, dtype);
  if (st != RDFFT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch == 0) {
    st = rdfft::weight_spectra_dispatch(c, cs, (d_out / p) * (d_in / p), p, s);
    return (st == RDFFT_OK && dc) ? rdfft::launch_fill_zero(dc, (d_out / p) * d_in, s) : st;
  }
  return rdfft::by_dtype(dtype, [&](auto io) {
    return rdfft::circ_fwd_dispatch<decltype(io)>(x, c, y, batch, d_in, d_out, p, s, dc, cs);
  });
}

int circulant_fwd_spec(const void* x, const float* cs, void* y, float* dc, int64_t batch, int64_t d_in, int64_t d_out,
                       int64_t p, int dtype, void* stream) {
  int st = dc ? rdfft::check_circulant_fwd_zero(x, cs, y, dc, batch, d_in, d_out, p, dtype)
              : rdfft::check_circulant_fwd(x, cs, y, batch, d_in, d_out, p, dtype);
  if (st == RDFFT_OK) st = rdfft::check_spec_size(d_in, d_out, p);
  if (st != RDFFT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch == 0) return dc ? rdfft::launch_fill_zero(dc, (d_out / p) * d_in, s) : RDFFT_OK;
  return rdfft::by_dtype(dtype, [&](auto io) {
    return rdfft::circ_fwd_dispatch<decltype(io), true>(x, cs, y, batch, d_in, d_out, p, s, dc);
  });
}

int circulant_bwd_spec(const void* x, const float* cs, const void* dy, void* dx, float* dc, int accumulate,
                       int64_t batch, int64_t d_in, int64_t d_out, int64_t p, int dtype, void* stream) {
  int st = rdfft::check_circulant_bwd(x, cs, dy, dx, dc, batch, d_in, d_out, p, dtype);
  if (st == RDFFT_OK) st = rdfft::check_spec_size(d_in, d_out, p);
  if (st != RDFFT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return rdfft::by_dtype(dtype, [&](auto io) {
    return rdfft::circ_bwd_dispatch<decltype(io), true>(x, cs, dy, dx, dc, batch, d_in, d_out, p, accumulate != 0, s);
  });
}

int circulant_bwd_det_workspace(int64_t batch, int64_t d_in, int64_t d_out, int64_t p, int with_dx, int64_t* bytes) {
  if (bytes == nullptr) return RDFFT_ERR_NULL;
  const int st = rdfft::check_circulant_dims(batch, d_in, d_out, p);
  if (st != RDFFT_OK) return st;
  return rdfft::circ_det_workspace(batch, d_in, d_out, p, with_dx != 0, bytes);
}

int circulant_bwd_det(const void* x, const float* c, const void* dy, void* dx, float* dc, float* ws, int64_t ws_bytes,
                      int64_t batch, int64_t d_in, int64_t d_out, int64_t p, int dtype, void* stream) {
  int st = rdfft::check_circulant_bwd(x, c, dy, dx, dc, batch, d_in, d_out, p, dtype);
  if (st != RDFFT_OK) return st;
  int64_t need = 0;
  st = rdfft::circ_det_workspace(batch, d_in, d_out, p, dx != nullptr, &need);
  if (st != RDFFT_OK) return st;
  st = rdfft::check_det_workspace(x, c, dy, dx, dc, ws, ws_bytes, need, batch, d_in, d_out, p, dtype);
  if (st != RDFFT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return rdfft::by_dtype(dtype, [&](auto io) {
    return rdfft::circ_bwd_dispatch<decltype(io)>(x, c, dy, dx, dc, batch, d_in, d_out, p, false, s, ws);
  });
}

int circulant_bwd_det_noalloc(const void* x, const float* c, const void* dy, void* dx, float* dc, int64_t batch,
                              int64_t d_in, int64_t d_out, int64_t p, int dtype, void* stream) {
  int st = rdfft::check_circulant_bwd(x, c, dy, dx, dc, batch, d_in, d_out, p, dtype);
  if (st != RDFFT_OK) return st;
  if (dc == nullptr) return RDFFT_ERR_NULL;
  int64_t need = 0;
  st = rdfft::circ_det_workspace(batch, d_in, d_out, p, dx != nullptr, &need);
  if (st != RDFFT_OK) return st;
  if (need > rdfft::kScratchBytes) return RDFFT_ERR_SCRATCH;
  float* ws = nullptr;
  if (need > 0) {
    ws = rdfft::scratch_ptr();
    if (ws == nullptr) return RDFFT_ERR_LAUNCH;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return rdfft::by_dtype(dtype, [&](auto io) {
    return rdfft::circ_bwd_dispatch<decltype(io)>(x, c, dy, dx, dc, batch, d_in, d_out, p, false, s, ws);
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
