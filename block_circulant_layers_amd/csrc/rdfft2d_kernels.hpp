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

// Column pass.  A workgroup loads a tile of CL adjacent columns x all H rows
// into LDS (row runs of CL elements, coalesced), transforms the columns CP at
// a time (T = H/E threads per column, CP * T threads), and stores the tile
// back the same way.  CL is the widest power of two whose tile fits the LDS
// budget.  From H = 512 to 2048 the budget is 72 KB and the workgroup 512
// threads, so that two workgroups share a CU and one's loads overlap the
// other's transforms: fp32 forward / inverse, us, 144 KB and 1024 threads ->
// 72 KB and 512 threads: 512x2048 34.4 / 29.4 -> 31.6 / 26.6, 1024x1024
// 35.5 / 30.4 -> 31.9 / 27.2, 2048x2048 49.3 / 46.4 -> 46.3 / 43.2.  At
// H = 256 (23.8 / 21.9 -> 30.9 / 26.6) and H = 4096 (4096x4096: 114.5 / 100.5
// -> 123.6 / 102.3) the larger tile stays.
// LDS stride of a tile column.  In the load and store loops a 32-lane half
// wavefront covers 32/CL rows of the CL columns (CL < 32), or 32 columns of
// one row: the column stride must be 32/CL modulo the 32 banks in the first
// case, and odd in the second, for the half's addresses to fall in distinct
// banks.  (An odd stride at CL = 8 and 16 gave 4- and 2-way conflicts: 3072
// extra cycles per load or store loop of a 4096-row tile.)
__host__ __device__ constexpr int col_stride(int lds, int cl) {
  return cl >= 32 ? (lds | 1) : lds + ((32 / cl - lds % 32) + 32) % 32;
}

template <int H>
struct ColShape {
  static constexpr int E = elems_per_thread(H);
  static constexpr int T = H / E;
  static constexpr bool HALF = H >= 512 && H <= 2048;  // two workgroups per CU
  static constexpr int CL0 = ((HALF ? 72 : 144) * 1024) / ((Row<H, E>::LDS | 1) * 4);
  static constexpr int CL = CL0 >= 64 ? 64 : CL0 >= 32 ? 32 : CL0 >= 16 ? 16 : CL0 >= 8 ? 8 : 4;
  static constexpr int CS = col_stride(Row<H, E>::LDS, CL);
  static constexpr int CP = cmin(CL, (HALF ? 512 : 1024) / T);
  static constexpr int NT = CP * T;
  static constexpr int NP = CL / CP;
  static constexpr int64_t lds_bytes() { return static_cast<int64_t>(CL) * CS * 4; }
  static_assert(CL % CP == 0 && (H * CL) % NT == 0 && CL * CS * 4 <= 144 * 1024, "column tile");
};

// Workgroups are handed to the eight XCDs in turn (workgroup b to XCD b % 8),
// each with its own L2.  Tiles of adjacent columns share cache lines (a tile
// row is 32 or 64 bytes at H >= 2048), so tile ids are reordered to give each
// XCD a contiguous range: workgroups that run side by side on one XCD then
// share lines in its L2 instead of fetching them once per XCD.  A bijection
// of [0, total) for any total.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t total) {
  constexpr int64_t X = 8;
  const int64_t q = total / X, r = total % X, x = b % X, s = b / X;
  return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

// Columns of workgroup b: with tile = xcd_tile(b), tile % ntiles of image
// tile / ntiles of [n, H, W]; columns past W are neither read nor written.
template <int H, bool INV, class Io>
__global__ void __launch_bounds__(ColShape<H>::NT) col_kernel(typename Io::T* __restrict__ data, int w, int ntiles) {
  using S = ColShape<H>;
  constexpr int E = S::E, T = S::T, CS = S::CS, CL = S::CL, CP = S::CP, NT = S::NT;
  using Rw = Row<H, E>;
  RDFFT_DYNAMIC_LDS(lds);
  const int tid = threadIdx.x;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int c0 = static_cast<int>(tile % ntiles) * CL;
  const int64_t img = tile / ntiles;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc<Io>(data + img * H * w, static_cast<int64_t>(H) * w);
  // tile element e: row e / CL, column c0 + e % CL (adjacent lanes on adjacent columns)
  auto goff = [=](int e) {
    const int col = c0 + e % CL;
    return col < w ? (e / CL) * w + col : H * w;  // past the image: loads give 0, stores are dropped
  };
#pragma unroll 4
  for (int e = tid; e < H * CL; e += NT) lds[(e % CL) * CS + e / CL] = Io::widen(Io::braw(rs, goff(e), 0));
  __syncthreads();
  const int t = tid % T;
  if constexpr (!INV) {
    typename Rw::FwdTws tw;
    tw.load(t);
    for (int pass = 0; pass < S::NP; ++pass) {
      float* L = lds + (pass * CP + tid / T) * CS;
      if constexpr (H == E) {
        row_fwd_to_lds<H>([L](int v, int cst) { return L[v + cst]; }, L, t, tw);
      } else {
        float raw[E], a[E];
#pragma unroll
        for (int s = 0; s < E; ++s) raw[s] = L[t + T * s];
        __syncthreads();  // the column's values are in registers before L is reused
        Rw::fwd_pass0_from(a, raw, [](float v) { return v; });
        Rw::fwd_pass0_scatter(a, L, t);
        fwd_rest<H, E, E, true>(a, L, t, [](int, int, float) {}, tw);  // natural packed order in L
      }
      __syncthreads();
    }
  } else {
    typename Rw::InvTws tw;
    tw.load(t);
    constexpr float scale = 1.0f / static_cast<float>(H);
    for (int pass = 0; pass < S::NP; ++pass) {
      float* L = lds + (pass * CP + tid / T) * CS;
      if constexpr (H == E) {
        row_inv_from_lds<H>(L, [L](int v, int cst, float x) { L[v + cst] = x; }, t, scale, tw);
      } else {
        float a[E], o[E];
        inv_rest<H, E, E, true>(a, L, t, [](int, int) { return 0.0f; }, tw);
        Rw::inv_pass0_store(a, L, t, scale, [&o](int, int cst, float x) { o[cst / T] = x; });
        __syncthreads();  // every read of L is done
#pragma unroll
        for (int s = 0; s < E; ++s) L[t + T * s] = o[s];
      }
      __syncthreads();
    }
  }
  // default cache policy: the L2 merges the tile rows of neighbouring
  // workgroups into whole lines before they are written back
#pragma unroll 4
  for (int e = tid; e < H * CL; e += NT) Io::template bstore<0>(rs, goff(e), 0, lds[(e % CL) * CS + e / CL]);
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
