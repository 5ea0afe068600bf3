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
// threads per workgroup of the standalone kernels: one wavefront for rows of
// p <= 1024 (workgroups of one wave run their passes without waiting for
// other waves: 4096x512 fp32 forward 4.86 -> 4.46 us against 256 threads;
// at p = 1024, one row a workgroup against four: 4096x1024 fp32 forward +
// inverse 52.1-52.6% -> 55.2-56.1% of HBM over three runs, 16384x1024 +1
// point, bf16 +2%; at p = 2048 one row of 128 threads measured slower),
// else at least 256, or one whole row
__host__ __device__ constexpr int wg_threads(int P, int E) {
  return (P / E) > (P <= 1024 ? 64 : 256) ? (P / E) : (P <= 1024 ? 64 : 256);
}
// elements per thread of the standalone kernels (32, with one exchange fewer,
// measured slower: 4096x512 fp32 forward 7.2 us against 4.9 us, and 31.3
// against 28.9 us at p = 4096)
__host__ __device__ constexpr int standalone_elems(int P, bool /*f32*/) { return elems_per_thread(P); }
// resident workgroups per CU the standalone kernels are launched for (fp32
// rows of p >= 1024: two workgroups, each looping over more groups, measured
// faster than four; a second group of look-ahead measured slower; the fp32
// forward at p = 2048 and 4096 takes three (4096x2048 16.5 -> 14.5 us,
// 4096x4096 27.8 -> 26.5 us), and so does the inverse at p = 2048 (4096x2048
// 14.3 -> 13.7 us over three runs), while three slowed the inverse at p = 4096
// (25.4 -> 25.7 us) and four the forward at p = 2048 (14.3 -> 15.5 us), and
// three slowed both directions at p = 1024 with 256-thread workgroups; 16-bit rows of
// 2048 <= p <= 4096: four; p = 8192 (512 threads): two, as four would cap
// registers at 64 and spill; p <= 512: eight one-wave workgroups; p = 1024:
// eight one-wave workgroups for fp32, sixteen for 16-bit rows)
__host__ __device__ constexpr int wg_per_cu(int P, bool f32, bool inv) {
  return P == 1024 ? (f32 ? 8 : 16)
         : P > 1024 ? (f32 || P >= 8192 ? ((f32 && (P == 2048 || (!inv && P == 4096))) ? 3 : 2) : 4)
                    : 8;
}
// Forward kernels that stage the transformed row in LDS and store it in the
// aligned element order t + T*s, instead of storing the last pass's packed
// runs directly (their mirrored runs start one element past a line boundary,
// so every line is written in two parts).  Measured: 4096x512 fp32 5.36 ->
// 4.85 us, bf16 4.82 -> 4.27 us, 4096x4096 fp32 27.3 -> 26.8 us, 4096x256
// fp32 4.59 -> 4.04 us; slower for bf16 at p = 256 and 4096 and at p = 128.
__host__ __device__ constexpr bool fwd_staged_store(int P, bool f32) {
  return P >= 256 && (f32 || (P >= 512 && P <= 1024));
}
template <class Io>
constexpr bool is_f32_io() {
  return sizeof(typename Io::T) == 4;
}

// Forward passes with input spectra of size B and all later ones.  The last
// pass either stores the natural packed row through st (global) or, when
// TO_LDS, scatters it to L[0..P) (layout P is the natural order).
// on = false (uniform per wavefront): the wave only takes part in the
// barriers (a wave whose rows are all padding skips their arithmetic).
template <int P, int E, int B, bool TO_LDS, class St, class TW>
__device__ __forceinline__ void fwd_rest(float (&a)[E], float* L, int t, St st, const TW& tw, bool on = true) {
  using Rw = Row<P, E>;
  using PS = typename Rw::template Pass<B>;
  __syncthreads();  // the previous pass's scatter is visible
  if (on) Rw::template fwd_pass<B>(a, L, t, tw);
  if constexpr (PS::BP == P && !TO_LDS) {
    if (on) Rw::template last_store<B>(a, t, st);
  } else {
    __syncthreads();  // every gather of this exchange is done
    if (on) Rw::template pass_scatter<B>(a, L, t);
    if constexpr (PS::BP != P) fwd_rest<P, E, PS::BP, TO_LDS>(a, L, t, st, tw, on);
  }
}

// Inverse passes undoing forward passes B, B*R, ..., P.  The first one reads
// the natural packed row through ld (global) or, when FROM_LDS, from L[0..P).
// On return L holds the size-B spectra in layout B, synchronised.
template <int P, int E, int B, bool FROM_LDS, class Ld, class TW>
__device__ __forceinline__ void inv_rest(float (&a)[E], float* L, int t, Ld ld, const TW& tw, bool on = true) {
  using Rw = Row<P, E>;
  using PS = typename Rw::template Pass<B>;
  auto from_lds = [L](int v, int c) { return L[v + c]; };
  if constexpr (PS::BP == P) {
    if constexpr (FROM_LDS) {
      if (on) Rw::template inv_pass<B>(a, from_lds, t, tw);
      __syncthreads();
    } else {
      if (on) Rw::template inv_pass<B>(a, ld, t, tw);
    }
  } else {
    inv_rest<P, E, PS::BP, FROM_LDS>(a, L, t, ld, tw, on);
    if (on) Rw::template inv_pass<B>(a, from_lds, t, tw);
    __syncthreads();  // every gather of this exchange is done
  }
  if (on) Rw::template inv_scatter<B>(a, L, t);
  __syncthreads();
}

// Inverse passes below the first one: on entry L holds spectra of size Bout in
// layout Bout (synchronised); on return it holds the size-E spectra in layout E.
template <int P, int E, int Bout, class TW>
__device__ __forceinline__ void inv_down(float (&a)[E], float* L, int t, const TW& tw) {
  if constexpr (Bout > E) {
    using Rw = Row<P, E>;
    constexpr int B = Rw::pass_in_for(Bout);
    Rw::template inv_pass<B>(a, [L](int v, int c) { return L[v + c]; }, t, tw);
    __syncthreads();  // every gather of this exchange is done
    Rw::template inv_scatter<B>(a, L, t);
    __syncthreads();
    inv_down<P, E, B>(a, L, t, tw);
  }
}

// Forward transform of one row into L[0..P) (natural packed order).
// ld(var, cst) returns element var + cst (var = t, cst = T*s).  No barrier
// after the final write.  Every thread of the workgroup must call it.
// tw: the row's forward twiddles (Row<P, E>::FwdTws, loaded once by the caller).
template <int P, class Ld, class TW>
__device__ __forceinline__ void row_fwd_to_lds(Ld ld, float* L, int t, const TW& tw, bool on = true) {
  constexpr int E = elems_per_thread(P);
  using Rw = Row<P, E>;
  float a[E];
  if (on) Rw::fwd_pass0(a, ld, t);
  if constexpr (P == E) {
    if (on) {
#pragma unroll
      for (int s = 0; s < P; ++s) L[s] = a[s];
    }
  } else {
    if (on) Rw::fwd_pass0_scatter(a, L, t);
    fwd_rest<P, E, E, true>(a, L, t, [](int, int, float) {}, tw, on);
  }
}

// The same from values already loaded (raw[s] = element t + T*s, widened by
// widen): used where the loads were issued ahead of time.
template <int P, class V, class Wd, class TW>
__device__ __forceinline__ void row_fwd_raw_to_lds(const V (&raw)[elems_per_thread(P)], Wd widen, float* L, int t,
                                                   const TW& tw, bool on = true) {
  constexpr int E = elems_per_thread(P);
  using Rw = Row<P, E>;
  float a[E];
  if (on) Rw::fwd_pass0_from(a, raw, widen);
  if constexpr (P == E) {
    if (on) {
#pragma unroll
      for (int s = 0; s < P; ++s) L[s] = a[s];
    }
  } else {
    if (on) Rw::fwd_pass0_scatter(a, L, t);
    fwd_rest<P, E, E, true>(a, L, t, [](int, int, float) {}, tw, on);
  }
}

// Inverse transform of the natural packed row in L[0..P) (the caller has
// synchronised after writing it); st(var, cst, v) stores element var + cst.
// L is used as exchange space; no barrier after the last read of L.
// Every thread of the workgroup must call it.
// tw: the row's inverse twiddles (Row<P, E>::InvTws, loaded once by the caller).
template <int P, class St, class TW>
__device__ __forceinline__ void row_inv_from_lds(float* L, St st, int t, float scale, const TW& tw, bool on = true) {
  constexpr int E = elems_per_thread(P);
  using Rw = Row<P, E>;
  float a[E];
  if constexpr (P == E) {
    if (on) {
#pragma unroll
      for (int s = 0; s < P; ++s) a[s] = L[s];
      small_inv<P, 1>(a);
      constexpr int LP = ilog2(P);
#pragma unroll
      for (int s = 0; s < P; ++s) st(0, s, a[bitrev(s, LP)] * scale);
    }
  } else {
    inv_rest<P, E, E, true>(a, L, t, [](int, int) { return 0.0f; }, tw, on);
    if (on) Rw::inv_pass0_store(a, L, t, scale, st);
  }
}

// Standalone kernels whose rows are short: a wavefront access of one row
// covers T = P/16 consecutive elements, 16 to 64 bytes for 32 <= p <= 256.
// The rows of a workgroup's group are contiguous, so they move between HBM
// and LDS in 16-byte pieces instead (every wavefront access covers 1 KB), and
// the transform reads and writes its rows in LDS.  Measured (forward,
// element-wise path -> pieces): 16384x128 fp32 6.26 -> 4.23 us, bf16 5.05 ->
// 3.82 us; 8192x256 fp32 5.10 -> 4.55 us; 32768x64 fp32 6.95 -> 4.12 us;
// 65536x32 bf16 10.4 -> 3.5 us.  At p = 512 (64-byte bf16 accesses, 128-byte
// fp32) the pieces were slower for bf16 (3.98 -> 4.19 us).
__host__ __device__ constexpr bool block_io(int P, int /*elem*/) { return P >= 32 && P <= 256; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// The NT * E elements of a group (ROWS rows of P) as NT * CH pieces of 16
// bytes: piece j of thread tid is bytes [16 (j NT + tid), +16) of the group,
// elements e0 = (j NT + tid) VE .. e0 + VE - 1, all in row e0 / P.
template <int P, class Io, int NT>
struct BlockIo {
  static constexpr int ELEM = static_cast<int>(sizeof(typename Io::T));
  static constexpr int VE = 16 / ELEM;
  static constexpr int GROUP = NT * elems_per_thread(P);
  static constexpr int CH = GROUP / (VE * NT);
  static_assert(GROUP % (VE * NT) == 0 && P % VE == 0, "pieces");
  template <int AUX>
  static __device__ __forceinline__ void load(u32x4 (&v)[CH], __amdgpu_buffer_rsrc_t rs, int tid) {
#pragma unroll
    for (int j = 0; j < CH; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (j * NT + tid) * 16, 0, AUX);
  }
  // widen into LDS rows of stride LS floats
  static __device__ __forceinline__ void to_lds(const u32x4 (&v)[CH], float* lds, int LS, int tid) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int e0 = (j * NT + tid) * VE;
      float* d = lds + (e0 / P) * LS + e0 % P;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (ELEM == 4) {
          d[w] = __uint_as_float(v[j][w]);
        } else {
          d[2 * w] = Io::widen(static_cast<uint16_t>(v[j][w] & 0xffffu));
          d[2 * w + 1] = Io::widen(static_cast<uint16_t>(v[j][w] >> 16));
        }
      }
    }
  }
  // narrow from LDS rows of stride LS and store
  template <int AUX>
  static __device__ __forceinline__ void from_lds(const float* lds, int LS, __amdgpu_buffer_rsrc_t rs, int tid) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int e0 = (j * NT + tid) * VE;
      const float* d = lds + (e0 / P) * LS + e0 % P;
      u32x4 v;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (ELEM == 4)
          v[w] = __float_as_uint(d[w]);
        else
          v[w] = static_cast<uint32_t>(Io::narrow(d[2 * w])) | (static_cast<uint32_t>(Io::narrow(d[2 * w + 1])) << 16);
      }
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, (j * NT + tid) * 16, 0, AUX);
    }
  }
};
constexpr int kBlockLoadAux = 2, kBlockStoreAux = 2;  // streaming: every byte is touched once per launch

// forward / inverse loop of the standalone kernels with block I/O (see above)
template <int P, class Io, int NT>
__device__ __forceinline__ void fwd_block_loop(typename Io::T* __restrict__ data, int64_t rows, float* lds) {
  constexpr int E = elems_per_thread(P);
  using Rw = Row<P, E>;
  using BI = BlockIo<P, Io, NT>;
  constexpr int T = Rw::T, ROWS = NT / T;
  const int tid = threadIdx.x, t = tid % T;
  float* L = lds + (tid / T) * Rw::LDS;
  const int64_t ngroups = (rows + ROWS - 1) / ROWS, G = gridDim.x;
  int64_t g = blockIdx.x;
  if (g >= ngroups) return;
  auto rsrc = [data, rows](int64_t gg) {
    const int64_t r0 = gg * ROWS;
    return make_rsrc<Io>(data + r0 * P, ((rows - r0 < ROWS) ? rows - r0 : ROWS) * P);
  };
  u32x4 v[BI::CH];
  BI::template load<kBlockLoadAux>(v, rsrc(g), tid);
  typename Rw::FwdTws tw;
  tw.load(t);
  while (true) {
    BI::to_lds(v, lds, Rw::LDS, tid);
    __syncthreads();
    float a[E];
    Rw::fwd_pass0(a, [L](int var, int c) { return L[var + c]; }, t);
    if (g + G < ngroups) BI::template load<kBlockLoadAux>(v, rsrc(g + G), tid);
    __syncthreads();  // every pass-0 read is done before the scatter
    Rw::fwd_pass0_scatter(a, L, t);
    fwd_rest<P, E, E, true>(a, L, t, [](int, int, float) {}, tw);  // natural packed rows in LDS
    __syncthreads();
    BI::template from_lds<kBlockStoreAux>(lds, Rw::LDS, rsrc(g), tid);
    g += G;
    if (g >= ngroups) return;
    __syncthreads();  // the stores' LDS reads are done before the next group lands
  }
}

template <int P, class Io, int NT>
__device__ __forceinline__ void inv_block_loop(typename Io::T* __restrict__ data, int64_t rows, float* lds) {
  constexpr int E = elems_per_thread(P);
  using Rw = Row<P, E>;
  using BI = BlockIo<P, Io, NT>;
  constexpr int T = Rw::T, ROWS = NT / T, BL = Rw::pass_in_for(P);
  constexpr float scale = 1.0f / static_cast<float>(P);
  const int tid = threadIdx.x, t = tid % T;
  float* L = lds + (tid / T) * Rw::LDS;
  const int64_t ngroups = (rows + ROWS - 1) / ROWS, G = gridDim.x;
  int64_t g = blockIdx.x;
  if (g >= ngroups) return;
  auto rsrc = [data, rows](int64_t gg) {
    const int64_t r0 = gg * ROWS;
    return make_rsrc<Io>(data + r0 * P, ((rows - r0 < ROWS) ? rows - r0 : ROWS) * P);
  };
  u32x4 v[BI::CH];
  BI::template load<kBlockLoadAux>(v, rsrc(g), tid);
  typename Rw::InvTws tw;
  tw.load(t);
  while (true) {
    BI::to_lds(v, lds, Rw::LDS, tid);
    __syncthreads();
    float a[E], x[E];
    Rw::template inv_load_first<BL>(x, [L](int var, int c) { return L[var + c]; }, t);
    Rw::template inv_first_from<BL>(a, x, [](float y) { return y; }, t, tw);
    if (g + G < ngroups) BI::template load<kBlockLoadAux>(v, rsrc(g + G), tid);
    __syncthreads();  // every first-pass read is done before the scatter
    Rw::template inv_scatter<BL>(a, L, t);
    __syncthreads();
    inv_down<P, E, BL>(a, L, t, tw);
    Rw::inv_pass0_store(a, L, t, scale, [&x](int, int cst, float y) { x[cst / T] = y; });
    __syncthreads();  // every read of L is done
#pragma unroll
    for (int s2 = 0; s2 < E; ++s2) L[t + T * s2] = x[s2];
    __syncthreads();
    BI::template from_lds<kBlockStoreAux>(lds, Rw::LDS, rsrc(g), tid);
    g += G;
    if (g >= ngroups) return;
    __syncthreads();  // the stores' LDS reads are done before the next group lands
  }
}

// ---------------------------------------------------------------------------
// standalone kernels: persistent workgroups, each looping over groups of ROWS
// rows, with the next group's loads issued before the current group is
// transformed (its values wait in registers), so loads, arithmetic and stores
// of different groups overlap.  The twiddles depend only on the thread and
// stay in registers across the loop.
// ---------------------------------------------------------------------------
template <int P, class Io, int E = standalone_elems(P, is_f32_io<Io>()), int NT = wg_threads(P, E)>
__device__ __forceinline__ void rdfft_fwd_body(typename Io::T* __restrict__ data, int64_t rows) {
  using Rw = Row<P, E>;
  constexpr int T = Rw::T;
  constexpr int ROWS = NT / T;
  constexpr int SEG = cmin(T, 64) * static_cast<int>(sizeof(typename Io::T));  // bytes per row per wave access
  __shared__ float lds[(P == E) ? 1 : ROWS * Rw::LDS];
  if constexpr (block_io(P, sizeof(typename Io::T)) && E == elems_per_thread(P)) {
    fwd_block_loop<P, Io, NT>(data, rows, lds);
    return;
  }
  const int tid = threadIdx.x;
  const int rl = tid / T, t = tid % T;
  const int ro = rl * P;
  const int64_t ngroups = (rows + ROWS - 1) / ROWS;
  const int64_t G = gridDim.x;
  int64_t g = blockIdx.x;
  if (g >= ngroups) return;
  auto rsrc = [data, rows](int64_t gg) {
    const int64_t r0 = gg * ROWS;
    return make_rsrc<Io>(data + r0 * P, ((rows - r0 < ROWS) ? rows - r0 : ROWS) * P);
  };
  auto load = [=](typename Io::T(&raw)[E], int64_t gg) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(gg);
    Rw::fwd_load0(raw, [rs, ro](int v, int c) { return Io::template braw<row_load_aux(SEG)>(rs, ro + v, c); }, t);
  };
  typename Io::T raw[E];
  load(raw, g);
  typename Rw::FwdTws tw;
  tw.load(t);
  float* L = (P == E) ? lds : lds + rl * Rw::LDS;  // rows of P == E never touch LDS
  while (true) {
    float a[E];
    Rw::fwd_pass0_from(a, raw, [](typename Io::T v) { return Io::widen(v); });
    if (g + G < ngroups) load(raw, g + G);
    const __amdgpu_buffer_rsrc_t rs = rsrc(g);
    auto st = [rs, ro](int v, int c, float x) { Io::template bstore<row_store_aux(SEG)>(rs, ro + v, c, x); };
    if constexpr (P == E) {
#pragma unroll
      for (int s = 0; s < P; ++s) st(0, s, a[s]);
    } else if constexpr (fwd_staged_store(P, is_f32_io<Io>())) {
      Rw::fwd_pass0_scatter(a, L, t);
      fwd_rest<P, E, E, true>(a, L, t, st, tw);
      __syncthreads();  // the row is in L[0..P) in natural packed order
#pragma unroll
      for (int s = 0; s < E; ++s)
        Io::template bstore<row_store_aux_strided(SEG)>(rs, ro + t, T * s, L[t + T * s]);
    } else {
      Rw::fwd_pass0_scatter(a, L, t);
      fwd_rest<P, E, E, false>(a, L, t, st, tw);
    }
    g += G;
    if (g >= ngroups) return;
    if constexpr (P != E) __syncthreads();  // the last gathers are done before LDS is reused
  }
}

template <int P, class Io, int E = standalone_elems(P, is_f32_io<Io>()), int NT = wg_threads(P, E)>
__device__ __forceinline__ void rdfft_inv_body(typename Io::T* __restrict__ data, int64_t rows) {
  using Rw = Row<P, E>;
  constexpr int T = Rw::T;
  constexpr int ROWS = NT / T;
  constexpr int SEG = cmin(T, 64) * static_cast<int>(sizeof(typename Io::T));  // bytes per row per wave access
  constexpr float scale = 1.0f / static_cast<float>(P);
  __shared__ float lds[(P == E) ? 1 : ROWS * Rw::LDS];
  if constexpr (block_io(P, sizeof(typename Io::T)) && E == elems_per_thread(P)) {
    inv_block_loop<P, Io, NT>(data, rows, lds);
    return;
  }
  const int tid = threadIdx.x;
  const int rl = tid / T, t = tid % T;
  const int ro = rl * P;
  const int64_t ngroups = (rows + ROWS - 1) / ROWS;
  const int64_t G = gridDim.x;
  int64_t g = blockIdx.x;
  if (g >= ngroups) return;
  auto rsrc = [data, rows](int64_t gg) {
    const int64_t r0 = gg * ROWS;
    return make_rsrc<Io>(data + r0 * P, ((rows - r0 < ROWS) ? rows - r0 : ROWS) * P);
  };
  // loads of a group: the natural packed row as the first inverse pass wants it
  auto load = [=](typename Io::T(&raw)[E], int64_t gg) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(gg);
    auto ld = [rs, ro](int v, int c) { return Io::template braw<row_load_aux(SEG)>(rs, ro + v, c); };
    if constexpr (P == E) {
#pragma unroll
      for (int s = 0; s < P; ++s) raw[s] = ld(0, s);
    } else {
      Rw::template inv_load_first<Rw::pass_in_for(P)>(raw, ld, t);
    }
  };
  typename Io::T raw[E];
  load(raw, g);
  typename Rw::InvTws tw;
  tw.load(t);
  float* L = (P == E) ? lds : lds + rl * Rw::LDS;  // rows of P == E never touch LDS
  auto widen = [](typename Io::T v) { return Io::widen(v); };
  while (true) {
    float a[E];
    if constexpr (P == E) {
#pragma unroll
      for (int s = 0; s < P; ++s) a[s] = widen(raw[s]);
      small_inv<P, 1>(a);
    } else {
      constexpr int BL = Rw::pass_in_for(P);
      Rw::template inv_first_from<BL>(a, raw, widen, t, tw);
    }
    if (g + G < ngroups) load(raw, g + G);
    const __amdgpu_buffer_rsrc_t rs = rsrc(g);
    auto st = [rs, ro](int v, int c, float x) { Io::template bstore<row_store_aux_strided(SEG)>(rs, ro + v, c, x); };
    if constexpr (P == E) {
      constexpr int LP = ilog2(P);
#pragma unroll
      for (int s = 0; s < P; ++s) st(0, s, a[bitrev(s, LP)] * scale);
    } else {
      constexpr int BL = Rw::pass_in_for(P);
      Rw::template inv_scatter<BL>(a, L, t);
      __syncthreads();
      inv_down<P, E, BL>(a, L, t, tw);
      Rw::inv_pass0_store(a, L, t, scale, st);
    }
    g += G;
    if (g >= ngroups) return;
    if constexpr (P != E) __syncthreads();  // the last gathers are done before LDS is reused
  }
}

template <int P, class Io>
__global__ void __launch_bounds__(wg_threads(P, standalone_elems(P, is_f32_io<Io>())),
                                  wg_per_cu(P, is_f32_io<Io>(), false) *
                                      wg_threads(P, standalone_elems(P, is_f32_io<Io>())) / 256)
    rdfft_fwd_kernel(typename Io::T* __restrict__ data, int64_t rows) {
  rdfft_fwd_body<P, Io>(data, rows);
}

template <int P, class Io>
__global__ void __launch_bounds__(wg_threads(P, standalone_elems(P, is_f32_io<Io>())),
                                  wg_per_cu(P, is_f32_io<Io>(), true) *
                                      wg_threads(P, standalone_elems(P, is_f32_io<Io>())) / 256)
    rdfft_inv_kernel(typename Io::T* __restrict__ data, int64_t rows) {
  rdfft_inv_body<P, Io>(data, rows);
}

// ---------------------------------------------------------------------------
// rows longer than 8192 (16384 and 32768; fp32 32768 = 128 KB, in one CU's
// LDS; rows of 8192 run in the standalone kernels above, measured 2048x8192
// fp32 30.9 -> 27.5 us forward against these):
// one workgroup per row of P/E threads (E = 16, and 32 at 32768 to stay
// within 1024 threads), the row in dynamic LDS between passes, each pass's
// twiddles read from the per-pass tables as it runs.  The row is read and
// written once, like the standalone kernels above.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int long_elems(int P) { return P >= 32768 ? 32 : 16; }
constexpr int kMaxLongP = 32768;

// One pass's twiddles, read from its table ahead of the pass: the long-row
// kernels issue a pass's table reads before the barriers that precede it, so
// their latency overlaps the previous pass's scatter instead of following it.
template <int P, int E, int B, bool INV>
struct AheadTws {
  using Rw = Row<P, E>;
  using PS = typename Rw::template Pass<B>;
  using W = typename std::conditional<INV, Tw, TwF>::type;
  W w[PS::IPT][PS::R];
  // read through a buffer resource over the table: buffer loads are ordinary
  // memory reads that the barriers' fences keep where they are issued (plain
  // reads of the constant table may be sunk past a barrier to their first
  // use), and they count only against the vector memory counter
  __device__ __forceinline__ void load(int t) {
    static_assert(PS::R % 2 == 0 && sizeof(W) == 8, "16-byte reads of two twiddles");
    constexpr int NE = (B / 2) * PS::R;  // entries of the table: class k at [k R, k R + R)
    const W* tab;
    if constexpr (INV)
      tab = PassTw<B, PS::R>::inv();
    else
      tab = PassTw<B, PS::R>::fwd();
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<W*>(tab), 0, NE * static_cast<int>(sizeof(W)), kBufWord3);
#pragma unroll
    for (int n = 0; n < PS::IPT; ++n) {
      int rp, k;
      PS::item(t + Rw::T * n, rp, k);  // k = 0 reads the table's first entries, unused
#pragma unroll
      for (int j = 0; j < PS::R; j += 2) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (k * PS::R + j) * static_cast<int>(sizeof(W)), 0, 0);
        w[n][j] = W{__uint_as_float(v[0]), __uint_as_float(v[1])};
        w[n][j + 1] = W{__uint_as_float(v[2]), __uint_as_float(v[3])};
      }
    }
  }
  template <int B2, class WW, int RR>
  __device__ __forceinline__ void item(int n, int /*k*/, WW (&out)[RR]) const {
    static_assert(B2 == B && RR == PS::R, "the twiddles of one pass");
#pragma unroll
    for (int j = 0; j < RR; ++j) out[j] = w[n][j];
  }
};

// fwd_rest with each pass's twiddles issued ahead (tw: pass B's, already issued)
template <int P, int E, int B, bool TO_LDS, class St, class TW>
__device__ __forceinline__ void fwd_rest_ahead(float (&a)[E], float* L, int t, St st, const TW& tw) {
  using Rw = Row<P, E>;
  using PS = typename Rw::template Pass<B>;
  __syncthreads();  // the previous pass's scatter is visible
  Rw::template fwd_pass<B>(a, L, t, tw);
  if constexpr (PS::BP == P && !TO_LDS) {
    Rw::template last_store<B>(a, t, st);
  } else if constexpr (PS::BP == P) {
    __syncthreads();  // every gather of this exchange is done
    Rw::template pass_scatter<B>(a, L, t);
  } else {
    AheadTws<P, E, PS::BP, false> next;
    next.load(t);
    __syncthreads();  // every gather of this exchange is done
    Rw::template pass_scatter<B>(a, L, t);
    fwd_rest_ahead<P, E, PS::BP, TO_LDS>(a, L, t, st, next);
  }
}

// inv_down with each pass's twiddles issued ahead; on entry L holds the
// spectra of size Bout (the caller has issued tw, pass pass_in_for(Bout)'s
// twiddles, before its barrier)
template <int P, int E, int Bout, class TW>
__device__ __forceinline__ void inv_down_ahead(float (&a)[E], float* L, int t, const TW& tw) {
  using Rw = Row<P, E>;
  constexpr int B = Rw::pass_in_for(Bout);
  Rw::template inv_pass<B>(a, [L](int v, int c) { return L[v + c]; }, t, tw);
  __syncthreads();  // every gather of this exchange is done
  Rw::template inv_scatter<B>(a, L, t);
  if constexpr (B > E) {
    AheadTws<P, E, Rw::pass_in_for(B), true> next;
    next.load(t);
    __syncthreads();
    inv_down_ahead<P, E, B>(a, L, t, next);
  } else {
    __syncthreads();
  }
}

template <int P, class Io>
__global__ void __launch_bounds__(P / long_elems(P)) rdfft_fwd_long_kernel(typename Io::T* __restrict__ data) {
  constexpr int E = long_elems(P);
  using Rw = Row<P, E>;
  constexpr int T = Rw::T;
  constexpr int SEG = 64 * static_cast<int>(sizeof(typename Io::T));
  RDFFT_DYNAMIC_LDS(lds);
  const int t = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc<Io>(data + static_cast<int64_t>(blockIdx.x) * P, P);
  AheadTws<P, E, E, false> tw;
  tw.load(t);
  float a[E];
  Rw::fwd_pass0(a, [rs](int v, int c) { return Io::widen(Io::template braw<row_load_aux(SEG)>(rs, v, c)); }, t);
  Rw::fwd_pass0_scatter(a, lds, t);
  auto st = [rs](int v, int c, float x) { Io::template bstore<row_store_aux(SEG)>(rs, v, c, x); };
  if constexpr (fwd_staged_store(P, is_f32_io<Io>())) {
    fwd_rest_ahead<P, E, E, true>(a, lds, t, st, tw);
    __syncthreads();  // the row is in lds[0..P) in natural packed order
#pragma unroll
    for (int s = 0; s < E; ++s) Io::template bstore<row_store_aux_strided(SEG)>(rs, t, T * s, lds[t + T * s]);
  } else {
    fwd_rest_ahead<P, E, E, false>(a, lds, t, st, tw);
  }
}

template <int P, class Io>
__global__ void __launch_bounds__(P / long_elems(P)) rdfft_inv_long_kernel(typename Io::T* __restrict__ data) {
  constexpr int E = long_elems(P);
  using Rw = Row<P, E>;
  constexpr int SEG = 64 * static_cast<int>(sizeof(typename Io::T));
  constexpr int BL = Rw::pass_in_for(P);
  RDFFT_DYNAMIC_LDS(lds);
  const int t = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc<Io>(data + static_cast<int64_t>(blockIdx.x) * P, P);
  AheadTws<P, E, BL, true> tw;
  tw.load(t);
  float a[E];
  auto ld = [rs](int v, int c) { return Io::widen(Io::template braw<row_load_aux(SEG)>(rs, v, c)); };
  Rw::template inv_pass<BL>(a, ld, t, tw);  // the first pass reads the packed row from HBM
  AheadTws<P, E, Rw::pass_in_for(BL), true> next;
  next.load(t);
  Rw::template inv_scatter<BL>(a, lds, t);
  __syncthreads();
  inv_down_ahead<P, E, BL>(a, lds, t, next);
  auto st = [rs](int v, int c, float x) { Io::template bstore<row_store_aux_strided(SEG)>(rs, v, c, x); };
  Rw::inv_pass0_store(a, lds, t, 1.0f / static_cast<float>(P), st);
}

}  // namespace rdfft
