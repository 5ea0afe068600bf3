// spectrum_kernels.hpp -- packed spectra <-> explicit complex bins.
//
// The packed layout (Paper-Notes page, "Squeeze") keeps a real row's DFT in
// its own p reals: [0] = y_0, [p/2] = y_{p/2}, [k] = Re y_k, [p-k] = Im y_k.
// These kernels convert to and from the p/2 + 1 complex bins y_0..y_{p/2}
// stored as (Re, Im) float pairs, for callers that want the spectrum
// explicitly.  Pure data movement (one pass over each buffer, coalesced), one
// thread per bin.
#pragma once

#include "rdfft_device.hpp"

namespace rdfft {

// One thread per bin f < p/2 of packed row r (lp = log2 p): bin f = (z[f],
// z[p-f]) written as one (Re, Im) pair, so each wavefront writes a contiguous
// run of pairs and reads an ascending and a descending run of the packed row;
// the thread of f = 0 also writes bin p/2 = (z[p/2], 0), and bin 0 gets Im 0.
template <class Io>
__global__ void __launch_bounds__(256)
    unpack_kernel(const typename Io::T* __restrict__ z, float* __restrict__ spec, int64_t rows, int lp) {
  const int p = 1 << lp, h = p >> 1, nb = h + 1;
  const int64_t total = rows << (lp - 1);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t r = i >> (lp - 1);
    const int f = static_cast<int>(i & (h - 1));
    const typename Io::T* row = z + (r << lp);
    float2* bins = reinterpret_cast<float2*>(spec + 2 * r * nb);
    const float re = Io::load(row + f);
    if (f == 0) {
      bins[0] = make_float2(re, 0.0f);
      bins[h] = make_float2(Io::load(row + h), 0.0f);
    } else {
      bins[f] = make_float2(re, Io::load(row + (p - f)));
    }
  }
}

// The inverse data movement, one thread per bin f < p/2: z[f] = Re bin f and
// z[p-f] = Im bin f; the thread of f = 0 also sets z[p/2] = Re bin p/2.  Im of
// bins 0 and p/2 is never read.
template <class Io>
__global__ void __launch_bounds__(256)
    pack_kernel(const float* __restrict__ spec, typename Io::T* __restrict__ z, int64_t rows, int lp) {
  const int p = 1 << lp, h = p >> 1, nb = h + 1;
  const int64_t total = rows << (lp - 1);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t r = i >> (lp - 1);
    const int f = static_cast<int>(i & (h - 1));
    typename Io::T* row = z + (r << lp);
    const float* bins = spec + 2 * r * nb;
    if (f == 0) {
      Io::store(row, bins[0]);
      Io::store(row + h, bins[2 * h]);
    } else {
      const float2 b = reinterpret_cast<const float2*>(bins)[f];
      Io::store(row + f, b.x);
      Io::store(row + (p - f), b.y);
    }
  }
}

}  // namespace rdfft
