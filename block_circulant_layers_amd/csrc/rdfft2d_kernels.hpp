// rdfft2d_kernels.hpp -- the 2D extension of the in-place packed real FFT.
//
// The pages leave 2D open (Paper-Notes page, "局限与展望").  An H x W real
// array is replaced in place by its 2D DFT Y[j, k], k = 0..W/2, in the layout
// that packs each axis where the data is conjugate-symmetric (the 1D rule of
// the Paper-Notes page, "Squeeze"):
//   columns 0 and W/2 hold Y[., k] packed along j;
//   for 0 < k < W/2, [j, k] = Re Y[j, k] and [j, W-k] = Im Y[j, k], all j.
// Forward = packed transforms of the rows (the standalone 1D kernels), then
// packed transforms of every column (col_kernel: A = FFT of column k,
// B = FFT of column W-k), then the combine (combine_kernel) that turns the
// packed pair (A, B) into the complex column Y[., k] = A + i B in place.  The
// inverse undoes the three steps in reverse order.
#pragma once

#include "rdfft_kernels.hpp"

namespace rdfft {

// columns per workgroup of the column kernels: enough adjacent columns that a
// wavefront reads 64-byte runs of a row, within 1024 threads
__host__ __device__ constexpr int col_tile(int H) {
  return cmin(1024 / (H / elems_per_thread(H)), cmax(16, 256 / (H / elems_per_thread(H))));
}
// LDS floats per column (odd, so the same slot of adjacent columns falls in
// different banks)
template <int H>
__host__ __device__ constexpr int col_stride() {
  return Row<H, elems_per_thread(H)>::LDS | 1;
}

// Packed transforms of C = col_tile(H) adjacent columns of one image of
// [n, H, W]: workgroup b takes tile b % ntiles of image b / ntiles.  Columns
// past W are neither read nor written.  Each column is owned by T threads
// (t = thread / C; c = thread % C, adjacent lanes on adjacent columns).
template <int H, bool INV, class Io>
__global__ void __launch_bounds__(col_tile(H) * (H / elems_per_thread(H)))
    col_kernel(typename Io::T* __restrict__ data, int w, int ntiles) {
  constexpr int E = elems_per_thread(H);
  using Rw = Row<H, E>;
  constexpr int T = Rw::T;
  constexpr int C = col_tile(H);
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int c = tid % C, t = tid / C;
  const int col = static_cast<int>(blockIdx.x % ntiles) * C + c;
  const int64_t img = blockIdx.x / ntiles;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc<Io>(data + img * H * w, static_cast<int64_t>(H) * w);
  // element (row v + cst) of this column; columns past w aim past the image
  const int voff = col < w ? col : H * w;
  float* L = lds + c * col_stride<H>();
  if constexpr (!INV) {
    typename Rw::FwdTws tw;
    tw.load(t);
    row_fwd_to_lds<H>([rs, voff, w](int v, int cst) { return Io::widen(Io::braw(rs, v * w + voff, cst * w)); }, L, t,
                      tw);
    __syncthreads();  // the column is in L[0..H) in natural packed order
#pragma unroll
    for (int s = 0; s < E; ++s) Io::bstore(rs, (t + T * s) * w + voff, 0, L[t + T * s]);
  } else {
    typename Rw::InvTws tw;
    tw.load(t);
#pragma unroll
    for (int s = 0; s < E; ++s) L[t + T * s] = Io::widen(Io::braw(rs, (t + T * s) * w + voff, 0));
    __syncthreads();
    row_inv_from_lds<H>(
        L, [rs, voff, w](int v, int cst, float x) { Io::bstore(rs, v * w + voff, cst * w, x); }, t,
        1.0f / static_cast<float>(H), tw);
  }
}

// The combine of column k with column W-k, 0 < k < W/2, at rows j and H-j,
// 0 < j < H/2 (rows 0 and H/2 are already right): from the packed column
// spectra A (column k) and B (column W-k),
//   Y[j, k] = A_j + i B_j,  Y[H-j, k] = conj(A_j) + i conj(B_j).
// INV undoes it (the halves of the sums).  One thread per (image, j, k); the
// index runs over j < H/2, k < W/2 (powers of two) and skips j = 0, k = 0.
template <bool INV, class Io>
__global__ void __launch_bounds__(256)
    combine_kernel(typename Io::T* __restrict__ data, int64_t n, int lh, int lw) {
  const int h = 1 << lh, w = 1 << lw;
  const int64_t total = n << (lh - 1 + lw - 1);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int k = static_cast<int>(i & ((w >> 1) - 1));
    const int j = static_cast<int>((i >> (lw - 1)) & ((h >> 1) - 1));
    if (j == 0 || k == 0) continue;
    typename Io::T* img = data + (i >> (lh - 1 + lw - 1)) * h * w;
    typename Io::T* pa = img + static_cast<int64_t>(j) * w + k;             // [j, k]
    typename Io::T* pb = img + static_cast<int64_t>(h - j) * w + k;         // [H-j, k]
    typename Io::T* pc = img + static_cast<int64_t>(j) * w + (w - k);       // [j, W-k]
    typename Io::T* pd = img + static_cast<int64_t>(h - j) * w + (w - k);   // [H-j, W-k]
    const float a = Io::load(pa), b = Io::load(pb), c = Io::load(pc), d = Io::load(pd);
    if (!INV) {
      // a = Re A_j, b = Im A_j, c = Re B_j, d = Im B_j
      Io::store(pa, a - d);  // Re Y[j, k]
      Io::store(pb, a + d);  // Re Y[H-j, k]
      Io::store(pc, b + c);  // Im Y[j, k]
      Io::store(pd, c - b);  // Im Y[H-j, k]
    } else {
      Io::store(pa, 0.5f * (a + b));  // Re A_j
      Io::store(pb, 0.5f * (c - d));  // Im A_j
      Io::store(pc, 0.5f * (c + d));  // Re B_j
      Io::store(pd, 0.5f * (b - a));  // Im B_j
    }
  }
}

}  // namespace rdfft
