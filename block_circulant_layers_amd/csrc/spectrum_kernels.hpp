// spectrum_kernels.hpp -- packed spectra <-> explicit complex bins.
//
// The packed layout (Paper-Notes page, "Squeeze") keeps a real row's DFT in
// its own p reals: [0] = y_0, [p/2] = y_{p/2}, [k] = Re y_k, [p-k] = Im y_k.
// These kernels convert to and from the p/2 + 1 complex bins y_0..y_{p/2}
// stored as (Re, Im) float pairs, for callers that want the spectrum
// explicitly.  Pure data movement (one pass over each buffer, coalesced along
// the packed row); one thread per packed element.
#pragma once

#include "rdfft_device.hpp"

namespace rdfft {

// element j of packed row r (lp = log2 p) goes to bin j (Re) for j <= p/2, to
// bin p - j (Im) above; bins 0 and p/2 get Im = 0 from the threads of j = 0, p/2
template <class Io>
__global__ void __launch_bounds__(256)
    unpack_kernel(const typename Io::T* __restrict__ z, float* __restrict__ spec, int64_t rows, int lp) {
  const int p = 1 << lp, h = p >> 1, nb = h + 1;
  const int64_t total = rows << lp;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t r = i >> lp;
    const int j = static_cast<int>(i & (p - 1));
    float* bins = spec + 2 * r * nb;
    const float v = Io::load(z + i);
    if (j <= h) {
      bins[2 * j] = v;
      if (j == 0 || j == h) bins[2 * j + 1] = 0.0f;
    } else {
      bins[2 * (p - j) + 1] = v;
    }
  }
}

// packed element j of row r takes Re of bin j (j <= p/2) or Im of bin p - j;
// Im of bins 0 and p/2 is never read
template <class Io>
__global__ void __launch_bounds__(256)
    pack_kernel(const float* __restrict__ spec, typename Io::T* __restrict__ z, int64_t rows, int lp) {
  const int p = 1 << lp, h = p >> 1, nb = h + 1;
  const int64_t total = rows << lp;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t r = i >> lp;
    const int j = static_cast<int>(i & (p - 1));
    const float* bins = spec + 2 * r * nb;
    Io::store(z + i, j <= h ? bins[2 * j] : bins[2 * (p - j) + 1]);
  }
}

}  // namespace rdfft
