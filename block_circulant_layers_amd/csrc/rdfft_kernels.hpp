// rdfft_kernels.hpp -- row-level transforms and the standalone in-place rdFFT kernels.
//
// One row of P reals is transformed by T = P/E threads of one workgroup, the
// row staged through LDS between passes (see rdfft_device.hpp); a workgroup
// of NT threads carries NT/T rows.  The standalone kernels move each row
// through HBM exactly once each way (coalesced), in place, through a buffer
// resource that covers the workgroup's rows (rows past the end read 0 and
// drop their stores).
#pragma once

#include "rdfft_device.hpp"

namespace rdfft {

// elements per thread for row length P
__host__ __device__ constexpr int elems_per_thread(int P) { return P < 16 ? P : 16; }
// threads per workgroup of the standalone kernels: at least 256, or one whole row
__host__ __device__ constexpr int wg_threads(int P, int E) { return (P / E) > 256 ? (P / E) : 256; }

// Forward passes with input spectra of size B and all later ones.  The last
// pass either stores the natural packed row through st (global) or, when
// TO_LDS, scatters it to L[0..P) (layout P is the natural order).
template <int P, int E, int B, bool TO_LDS, class St>
__device__ __forceinline__ void fwd_rest(float (&a)[E], float* L, int t, St st) {
  using Rw = Row<P, E>;
  using PS = typename Rw::template Pass<B>;
  __syncthreads();  // the previous pass's scatter is visible
  Rw::template fwd_pass<B>(a, L, t);
  if constexpr (PS::BP == P && !TO_LDS) {
    Rw::template last_store<B>(a, t, st);
  } else {
    __syncthreads();  // every gather of this exchange is done
    Rw::template pass_scatter<B>(a, L, t);
    if constexpr (PS::BP != P) fwd_rest<P, E, PS::BP, TO_LDS>(a, L, t, st);
  }
}

// Inverse passes undoing forward passes B, B*R, ..., P.  The first one reads
// the natural packed row through ld (global) or, when FROM_LDS, from L[0..P).
// On return L holds the size-B spectra in layout B, synchronised.
template <int P, int E, int B, bool FROM_LDS, class Ld>
__device__ __forceinline__ void inv_rest(float (&a)[E], float* L, int t, Ld ld) {
  using Rw = Row<P, E>;
  using PS = typename Rw::template Pass<B>;
  auto from_lds = [L](int v, int c) { return L[v + c]; };
  if constexpr (PS::BP == P) {
    if constexpr (FROM_LDS) {
      Rw::template inv_pass<B>(a, from_lds, t);
      __syncthreads();
    } else {
      Rw::template inv_pass<B>(a, ld, t);
    }
  } else {
    inv_rest<P, E, PS::BP, FROM_LDS>(a, L, t, ld);
    Rw::template inv_pass<B>(a, from_lds, t);
    __syncthreads();  // every gather of this exchange is done
  }
  Rw::template inv_scatter<B>(a, L, t);
  __syncthreads();
}

// Forward transform of one row into L[0..P) (natural packed order).
// ld(var, cst) returns element var + cst (var = t, cst = T*s).  No barrier
// after the final write.  Every thread of the workgroup must call it.
template <int P, class Ld>
__device__ __forceinline__ void row_fwd_to_lds(Ld ld, float* L, int t) {
  constexpr int E = elems_per_thread(P);
  using Rw = Row<P, E>;
  float a[E];
  Rw::fwd_pass0(a, ld, t);
  if constexpr (P == E) {
#pragma unroll
    for (int s = 0; s < P; ++s) L[s] = a[s];
  } else {
    Rw::fwd_pass0_scatter(a, L, t);
    fwd_rest<P, E, E, true>(a, L, t, [](int, int, float) {});
  }
}

// Inverse transform of the natural packed row in L[0..P) (the caller has
// synchronised after writing it); st(var, cst, v) stores element var + cst.
// L is used as exchange space; no barrier after the last read of L.
// Every thread of the workgroup must call it.
template <int P, class St>
__device__ __forceinline__ void row_inv_from_lds(float* L, St st, int t, float scale) {
  constexpr int E = elems_per_thread(P);
  using Rw = Row<P, E>;
  float a[E];
  if constexpr (P == E) {
#pragma unroll
    for (int s = 0; s < P; ++s) a[s] = L[s];
    small_inv<P, 1>(a);
    constexpr int LP = ilog2(P);
#pragma unroll
    for (int s = 0; s < P; ++s) st(0, s, a[bitrev(s, LP)] * scale);
  } else {
    inv_rest<P, E, E, true>(a, L, t, [](int, int) { return 0.0f; });
    Rw::inv_pass0_store(a, L, t, scale, st);
  }
}

template <int P, class Io>
__global__ void __launch_bounds__(wg_threads(P, elems_per_thread(P)))
    rdfft_fwd_kernel(typename Io::T* __restrict__ data, int64_t rows) {
  constexpr int E = elems_per_thread(P);
  using Rw = Row<P, E>;
  constexpr int T = Rw::T;
  constexpr int NT = wg_threads(P, E);
  constexpr int ROWS = NT / T;
  __shared__ float lds[(P == E) ? 1 : ROWS * Rw::LDS];
  const int tid = threadIdx.x;
  const int rl = tid / T, t = tid % T;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * ROWS;
  const int64_t nrow = (rows - r0 < ROWS) ? rows - r0 : ROWS;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc<Io>(data + r0 * P, nrow * P);
  const int ro = rl * P;
  auto ld = [rs, ro](int v, int c) { return Io::bload(rs, ro + v, c); };
  auto st = [rs, ro](int v, int c, float x) { Io::bstore(rs, ro + v, c, x); };
  float a[E];
  Rw::fwd_pass0(a, ld, t);
  if constexpr (P == E) {
#pragma unroll
    for (int s = 0; s < P; ++s) st(0, s, a[s]);
  } else {
    float* L = lds + rl * Rw::LDS;
    Rw::fwd_pass0_scatter(a, L, t);
    fwd_rest<P, E, E, false>(a, L, t, st);
  }
}

template <int P, class Io>
__global__ void __launch_bounds__(wg_threads(P, elems_per_thread(P)))
    rdfft_inv_kernel(typename Io::T* __restrict__ data, int64_t rows) {
  constexpr int E = elems_per_thread(P);
  using Rw = Row<P, E>;
  constexpr int T = Rw::T;
  constexpr int NT = wg_threads(P, E);
  constexpr int ROWS = NT / T;
  constexpr float scale = 1.0f / static_cast<float>(P);
  __shared__ float lds[(P == E) ? 1 : ROWS * Rw::LDS];
  const int tid = threadIdx.x;
  const int rl = tid / T, t = tid % T;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * ROWS;
  const int64_t nrow = (rows - r0 < ROWS) ? rows - r0 : ROWS;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc<Io>(data + r0 * P, nrow * P);
  const int ro = rl * P;
  auto ld = [rs, ro](int v, int c) { return Io::bload(rs, ro + v, c); };
  auto st = [rs, ro](int v, int c, float x) { Io::bstore(rs, ro + v, c, x); };
  float a[E];
  if constexpr (P == E) {
#pragma unroll
    for (int s = 0; s < P; ++s) a[s] = ld(0, s);
    small_inv<P, 1>(a);
    constexpr int LP = ilog2(P);
#pragma unroll
    for (int s = 0; s < P; ++s) st(0, s, a[bitrev(s, LP)] * scale);
  } else {
    float* L = lds + rl * Rw::LDS;
    inv_rest<P, E, E, false>(a, L, t, ld);
    Rw::inv_pass0_store(a, L, t, scale, st);
  }
}

}  // namespace rdfft
