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

typedef float f32x2 __attribute__((ext_vector_type(2)));

// the storage value of v (rounded to nearest even for 16-bit rows)
template <class Io>
__device__ __forceinline__ typename Io::T to_storage(float v) {
  if constexpr (sizeof(typename Io::T) == 4)
    return v;
  else
    return Io::narrow(v);
}

// Every element is touched once per call, so the accesses are non-temporal
// (measured: 4096x512 fp32 unpack 6.5 -> 5.7 us; 1024x4096 unpack 10.9 ->
// 9.1 us, pack 10.2 -> 9.3 us).

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
    f32x2* bins = reinterpret_cast<f32x2*>(spec + 2 * r * nb);
    const float re = Io::widen(__builtin_nontemporal_load(row + f));
    if (f == 0) {
      __builtin_nontemporal_store(f32x2{re, 0.0f}, bins);
      __builtin_nontemporal_store(f32x2{Io::widen(__builtin_nontemporal_load(row + h)), 0.0f}, bins + h);
    } else {
      __builtin_nontemporal_store(f32x2{re, Io::widen(__builtin_nontemporal_load(row + (p - f)))}, bins + f);
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
      __builtin_nontemporal_store(to_storage<Io>(__builtin_nontemporal_load(bins)), row);
      __builtin_nontemporal_store(to_storage<Io>(__builtin_nontemporal_load(bins + 2 * h)), row + h);
    } else {
      const f32x2 b = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(bins) + f);
      __builtin_nontemporal_store(to_storage<Io>(b.x), row + f);
      __builtin_nontemporal_store(to_storage<Io>(b.y), row + (p - f));
    }
  }
}

}  // namespace rdfft
