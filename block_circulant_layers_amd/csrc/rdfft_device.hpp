// rdfft_device.hpp -- gfx950 device building blocks of the in-place packed real FFT.
//
// Method: "Memory-Efficient Training with In-Place FFT Implementation"
// (Paper-Notes page, sections "Squeeze", "四元素对称群 (Proposition 1)",
// "原地 IFFT 设计").
//
// Packed layout of an r-point spectrum (r a power of two): slot 0 = y_0,
// slot r/2 = y_{r/2}, slot k = Re y_k, slot r-k = Im y_k (0 < k < r/2).
//
// Forward = radix-2 decimation in time on bit-reversed input.  Stage m merges,
// inside each m-block at g, the packed m/2-point spectra E (first half) and O
// (second half) in place:
//   DC pair      (g, g+m/2)                   (E0, O0) -> (E0+O0, E0-O0)
//   quarter pair (g+m/4, g+3m/4), m >= 4      slot g+3m/4 negated
//   group        {g+k, g+m/2-k, g+m/2+k, g+m-k}, 0 < k < m/4:
//                (ReE, ImE, ReO, ImO) -> (Re(E+t), Re(E-t), -Im(E-t), Im(E+t)),
//                t = W_m^k O, W_m = exp(-2 pi i / m)
// The inverse runs the same graph backwards; every inverse group returns
// (2E, 2O), so all per-stage halvings are applied once at the end as 1/r.
//
// GPU organisation (ours, not the pages'): a row of P reals is owned by
// T = P/E threads holding E values each.  Stages are grouped into passes.
//   * pass 0: thread t loads x[t + T*s] (s < E: coalesced across threads) and
//     runs stages 2..E in registers: the packed E-point spectrum of the
//     decimated subsequence with residue t mod T.
//   * pass with input spectra of size B and radix R (output size B*R): the
//     packed slots congruent to +-k mod B of the R sub-spectra that merge form
//     a set closed under stages 2B..B*R, so an "item" (output residue r',
//     class k) runs those log2(R) stages in registers.  Class k = 0 holds the
//     slots 0 and B/2 of each sub-spectrum (an R-point real transform plus a
//     half-bin-shifted one, all with constant twiddles).
//   * between passes the row goes through LDS in a padded residue-major
//     layout A(r, s) = r*(B + pad) + s; the paddings and the item-to-lane
//     order of every pass are chosen so that the 32-lane LDS accesses hit
//     distinct banks (checked against the bank-conflict counter).
//   * the last forward pass stores the natural packed layout directly; the
//     first inverse pass reads it directly (both coalesced).
// Twiddles: every item reads the R-1 twiddles of its groups from a per-pass
// table laid out [class][group], so a wave's lanes read one contiguous block
// with 16-byte loads.  The forward table holds (cos, tan): the group is
// evaluated as t = c (O_re + tan O_im, O_im - tan O_re), E +- t, which needs
// 6 instead of 8 VALU operations; the inverse table holds (cos, sin).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

// The workgroup's LDS block whose size the launch gives (dynamic shared
// memory).  A host build of these headers that runs the kernels on CPU
// threads (the LDS schedule checker among the tests) defines it beforehand.
#ifndef RDFFT_DYNAMIC_LDS
#define RDFFT_DYNAMIC_LDS(name) extern __shared__ float name[]
#endif

namespace rdfft {

struct Tw {
  float c, s;  // W = c - i s   (c = cos(theta), s = sin(theta), W = exp(-i theta))
};
struct TwF {
  float c, tn;  // W = c (1 - i tn), tn = tan(theta)
};

#include "twiddles.inc"

// ---------------------------------------------------------------------------
// compile-time helpers
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v >> 1); }
__host__ __device__ constexpr int bitrev(int v, int bits) {
  int r = 0;
  for (int i = 0; i < bits; ++i)
    if ((v >> i) & 1) r |= 1 << (bits - 1 - i);
  return r;
}
__host__ __device__ constexpr int cmin(int a, int b) { return a < b ? a : b; }
__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Twiddle of angle 2 pi * num / den, 0 <= num/den <= 1/4, from the table.
__device__ __forceinline__ Tw tw_const(int num, int den) { return kTw[num * (kTwN / den)]; }
__device__ __forceinline__ TwF twf_const(int num, int den) { return kTwF[num * (kTwN / den)]; }

// ---------------------------------------------------------------------------
// the pages' in-place operations on one four-element group
// slots (g+k, g+m/2-k, g+m/2+k, g+m-k) = (a1, a2, a3, a4)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void grp_fwd(float& a1, float& a2, float& a3, float& a4, TwF w) {
  // in: (Re E, Im E, Re O, Im O);  t = W O = c (u + i v), u = ReO + tan ImO, v = ImO - tan ReO
  const float u = __builtin_fmaf(w.tn, a4, a3);
  const float v = __builtin_fmaf(-w.tn, a3, a4);
  const float er = a1, ei = a2;
  a1 = __builtin_fmaf(w.c, u, er);   // Re y_k       = Re(E + t)
  a2 = __builtin_fmaf(-w.c, u, er);  // Re y_{m/2-k} = Re(E - t)
  a3 = __builtin_fmaf(w.c, v, -ei);  // Im y_{m/2-k} = -Im(E - t)
  a4 = __builtin_fmaf(w.c, v, ei);   // Im y_k       = Im(E + t)
}

__device__ __forceinline__ void grp_inv(float& a1, float& a2, float& a3, float& a4, Tw w) {
  // in: (Re y_k, Re y_{m/2-k}, Im y_{m/2-k}, Im y_k);  y_{m/2+k} = conj(y_{m/2-k})
  // out: (Re 2E, Im 2E, Re 2O, Im 2O),  2E = y_k + y_{m/2+k},  2O = (y_k - y_{m/2+k}) conj(W)
  const float er = a1 + a2, ei = a4 - a3;
  const float tr = a1 - a2, ti = a4 + a3;
  a1 = er;
  a2 = ei;
  a3 = tr * w.c - ti * w.s;
  a4 = tr * w.s + ti * w.c;
}

// ---------------------------------------------------------------------------
// complete packed R-point transform in registers on a[S*q], q < R, input in
// bit-reversed order (forward) / natural packed (inverse)
// ---------------------------------------------------------------------------
template <int R, int S>
__device__ __forceinline__ void small_fwd(float* a) {
#pragma unroll
  for (int m = 2; m <= R; m *= 2) {
#pragma unroll
    for (int g = 0; g < R; g += m) {
      const float e0 = a[S * g], o0 = a[S * (g + m / 2)];
      a[S * g] = e0 + o0;
      a[S * (g + m / 2)] = e0 - o0;
      if (m >= 4) a[S * (g + 3 * m / 4)] = -a[S * (g + 3 * m / 4)];
#pragma unroll
      for (int k = 1; k < m / 4; ++k)
        grp_fwd(a[S * (g + k)], a[S * (g + m / 2 - k)], a[S * (g + m / 2 + k)], a[S * (g + m - k)],
                twf_const(k, m));
    }
  }
}

template <int R, int S>
__device__ __forceinline__ void small_inv(float* a) {
#pragma unroll
  for (int m = R; m >= 2; m /= 2) {
#pragma unroll
    for (int g = 0; g < R; g += m) {
#pragma unroll
      for (int k = 1; k < m / 4; ++k)
        grp_inv(a[S * (g + k)], a[S * (g + m / 2 - k)], a[S * (g + m / 2 + k)], a[S * (g + m - k)],
                tw_const(k, m));
      if (m >= 4) {
        a[S * (g + m / 4)] = 2.0f * a[S * (g + m / 4)];
        a[S * (g + 3 * m / 4)] = -2.0f * a[S * (g + 3 * m / 4)];
      }
      const float y0 = a[S * g], yh = a[S * (g + m / 2)];
      a[S * g] = y0 + yh;
      a[S * (g + m / 2)] = y0 - yh;
    }
  }
}

// ---------------------------------------------------------------------------
// item of a pass (input spectra of size B, radix R), class 0 < k < B/2.
// a[2q] = slot qB + k, a[2q+1] = slot qB + B - k of the (B*R)-block, q < R.
// Stage s (m = 2B 2^s, h = 2^s) holds, per m-block (q in [base, base + 2h)),
// the groups kappa = k + B i ("type A") and kappa = B(i+1) - k ("type B"),
// i < h/2 (only kappa = k when s = 0):
//   type A slots (first q=base+i, mirror base+h-i-1, first base+h+i, mirror base+2h-i-1)
//   type B slots (mirror base+i, first base+h-i-1, mirror base+h+i, first base+2h-i-1)
// ---------------------------------------------------------------------------
// per-pass twiddle tables: the R-1 group twiddles of class k at [k*R, k*R + R-1)
template <int B, int R>
struct PassTw;
#define RDFFT_PASS_TW(B_, R_)                                                          \
  template <>                                                                          \
  struct PassTw<B_, R_> {                                                              \
    static __device__ __forceinline__ const TwF* fwd() { return kPassF_##B_##_##R_; } \
    static __device__ __forceinline__ const Tw* inv() { return kPassI_##B_##_##R_; }  \
  };
RDFFT_PASS_TW(16, 2)
RDFFT_PASS_TW(16, 4)
RDFFT_PASS_TW(16, 8)
RDFFT_PASS_TW(128, 2)
RDFFT_PASS_TW(128, 4)
RDFFT_PASS_TW(128, 8)
RDFFT_PASS_TW(1024, 2)
RDFFT_PASS_TW(1024, 4)
RDFFT_PASS_TW(1024, 8)
RDFFT_PASS_TW(8192, 2)
RDFFT_PASS_TW(8192, 4)
RDFFT_PASS_TW(32, 16)
RDFFT_PASS_TW(512, 16)
RDFFT_PASS_TW(8, 4)
RDFFT_PASS_TW(32, 4)
RDFFT_PASS_TW(512, 2)
RDFFT_PASS_TW(512, 4)
RDFFT_PASS_TW(2048, 2)
#undef RDFFT_PASS_TW

// the R-1 twiddles of an item, read as R/2 aligned 16-byte loads
template <class W, int R>
__device__ __forceinline__ void load_item_tw(const W* tab, int k, W (&w)[R]) {
  static_assert(sizeof(W) == 8 && R % 2 == 0, "twiddles are pairs of floats");
  __builtin_memcpy(w, tab + k * R, sizeof(w));
}

template <int B, int R>
__device__ __forceinline__ void item_fwd(float* a, const TwF (&w)[R]) {
  constexpr int NS = ilog2(R);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int h = 1 << s;
    const int j0 = h - 1;  // first twiddle of stage s
#pragma unroll
    for (int blk = 0; blk < (R >> (s + 1)); ++blk) {
      const int base = blk << (s + 1);
      if (s == 0) {
        grp_fwd(a[2 * base], a[2 * base + 1], a[2 * base + 2], a[2 * base + 3], w[0]);
      } else {
#pragma unroll
        for (int i = 0; i < h / 2; ++i) {
          // W_m^(k + B i) and W_m^(B(i+1) - k)
          grp_fwd(a[2 * (base + i)], a[2 * (base + h - i - 1) + 1], a[2 * (base + h + i)],
                  a[2 * (base + 2 * h - i - 1) + 1], w[j0 + 2 * i]);
          grp_fwd(a[2 * (base + i) + 1], a[2 * (base + h - i - 1)], a[2 * (base + h + i) + 1],
                  a[2 * (base + 2 * h - i - 1)], w[j0 + 2 * i + 1]);
        }
      }
    }
  }
}

template <int B, int R>
__device__ __forceinline__ void item_inv(float* a, const Tw (&w)[R]) {
  constexpr int NS = ilog2(R);
#pragma unroll
  for (int s = NS - 1; s >= 0; --s) {
    const int h = 1 << s;
    const int j0 = h - 1;
#pragma unroll
    for (int blk = 0; blk < (R >> (s + 1)); ++blk) {
      const int base = blk << (s + 1);
      if (s == 0) {
        grp_inv(a[2 * base], a[2 * base + 1], a[2 * base + 2], a[2 * base + 3], w[0]);
      } else {
#pragma unroll
        for (int i = 0; i < h / 2; ++i) {
          grp_inv(a[2 * (base + i)], a[2 * (base + h - i - 1) + 1], a[2 * (base + h + i)],
                  a[2 * (base + 2 * h - i - 1) + 1], w[j0 + 2 * i]);
          grp_inv(a[2 * (base + i) + 1], a[2 * (base + h - i - 1)], a[2 * (base + h + i) + 1],
                  a[2 * (base + 2 * h - i - 1)], w[j0 + 2 * i + 1]);
        }
      }
    }
  }
}

// class k = 0: a[2q] = slot qB (an R-point real transform, constant twiddles),
// a[2q+1] = slot qB + B/2 (half-bin shifted: groups kappa = B/2 + cB with
// W_m^kappa = W_(2^(s+2))^(2c+1); at s = 0 only the quarter-pair negation).
template <int R, bool INV>
__device__ __forceinline__ void item0_odd_stage(float* a, int s) {
  const int h = 1 << s;
#pragma unroll
  for (int blk = 0; blk < (R >> (s + 1)); ++blk) {
    const int base = blk << (s + 1);
    if (s == 0) {
      // quarter pair of stage 2B: slots g + B/2 (a[2 base + 1]) and g + 3B/2 (a[2 base + 3])
      if (INV) {
        a[2 * base + 1] = 2.0f * a[2 * base + 1];
        a[2 * base + 3] = -2.0f * a[2 * base + 3];
      } else {
        a[2 * base + 3] = -a[2 * base + 3];
      }
    } else {
#pragma unroll
      for (int c = 0; c < h / 2; ++c) {
        float& a1 = a[2 * (base + c) + 1];
        float& a2 = a[2 * (base + h - c - 1) + 1];
        float& a3 = a[2 * (base + h + c) + 1];
        float& a4 = a[2 * (base + 2 * h - c - 1) + 1];
        if (INV)
          grp_inv(a1, a2, a3, a4, tw_const(2 * c + 1, 4 * h));
        else
          grp_fwd(a1, a2, a3, a4, twf_const(2 * c + 1, 4 * h));
      }
    }
  }
}

template <int R>
__device__ __forceinline__ void item0_fwd(float* a) {
  small_fwd<R, 2>(a);
#pragma unroll
  for (int s = 0; s < ilog2(R); ++s) item0_odd_stage<R, false>(a, s);
}

template <int R>
__device__ __forceinline__ void item0_inv(float* a) {
#pragma unroll
  for (int s = ilog2(R) - 1; s >= 0; --s) item0_odd_stage<R, true>(a, s);
  small_inv<R, 2>(a);
}

// ---------------------------------------------------------------------------
// storage types and buffer-resource access
// ---------------------------------------------------------------------------
// A buffer resource covers [base, base + nbytes): loads past the end return
// 0 and stores past the end are dropped by the hardware, so rows beyond the
// last one need no branches.  voff is the lane-varying byte offset, soff a
// wave-uniform one.
constexpr int kBufWord3 = 0x00020000;
// Cache policies (aux bits of the buffer instructions: 2 = non-temporal,
// 16 = device scope) of row loads and stores that touch each element once per
// launch, by the bytes `seg` of one row that a wavefront access covers
// (min(T, 64) consecutive elements).  From 64-byte segments on, streaming
// both directions measured 10-20% faster than the default policy, and faster
// than streaming loads or stores alone; stores in the element order t + T*s
// (inverse outputs) are faster still at device scope, which slows the
// packed-order stores of the forward transform.  Shorter segments keep the
// default (streaming them measured slower for bf16), as do inputs that other
// workgroups read again (circulant kernels).
constexpr int kAuxDefault = 0;
__host__ __device__ constexpr int row_load_aux(int seg) { return seg >= 64 ? 2 : kAuxDefault; }
// natural packed order (forward outputs)
__host__ __device__ constexpr int row_store_aux(int seg) { return seg >= 64 ? 2 : kAuxDefault; }
// element order t + T*s (inverse outputs)
__host__ __device__ constexpr int row_store_aux_strided(int seg) { return seg >= 64 ? 18 : kAuxDefault; }

struct F32Io {
  using T = float;
  static __device__ __forceinline__ float widen(float v) { return v; }
  template <int AUX = kAuxDefault>
  static __device__ __forceinline__ float braw(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff * 4, soff * 4, AUX));
  }
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
  template <int AUX = kAuxDefault>
  static __device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, int voff, int soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff * 4, soff * 4, AUX);
  }
};
// 16-bit storage (bfloat16 or IEEE half): rows widened to fp32 on load and
// rounded to nearest even once on store.
struct Bf16Conv {
  static __device__ __forceinline__ float widen(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }
  static __device__ __forceinline__ uint16_t narrow(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
};
struct F16Conv {
  static __device__ __forceinline__ float widen(uint16_t h) { return static_cast<float>(__builtin_bit_cast(_Float16, h)); }
  static __device__ __forceinline__ uint16_t narrow(float v) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v)); }
};
template <class Conv>
struct Io16 {
  using T = uint16_t;
  static __device__ __forceinline__ float widen(uint16_t h) { return Conv::widen(h); }
  static __device__ __forceinline__ uint16_t narrow(float v) { return Conv::narrow(v); }
  template <int AUX = kAuxDefault>
  static __device__ __forceinline__ uint16_t braw(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff * 2, soff * 2, AUX);
  }
  static __device__ __forceinline__ float load(const uint16_t* p) { return widen(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = narrow(v); }
  template <int AUX = kAuxDefault>
  static __device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, int voff, int soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b16(narrow(v), r, voff * 2, soff * 2, AUX);
  }
};
struct Bf16Io : Io16<Bf16Conv> {};
struct F16Io : Io16<F16Conv> {};

template <class Io>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const typename Io::T* base, int64_t elems) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<typename Io::T*>(base), 0,
                                           static_cast<int>(elems * sizeof(typename Io::T)), kBufWord3);
}

// ---------------------------------------------------------------------------
// exchange layouts: padding of layout B and item order of the pass reading
// layout B, for rows of P with E = 16 per thread (E = 32 at P = 32768, whose
// layouts are 32, 512 and 8192).  Chosen by simulating the bank conflicts of
// every LDS access of the pass schedule: a wave's access is split into two
// halves of 32 lanes, and each half takes as many cycles as the largest number
// of distinct addresses that fall in one of 32 banks.  That count matches the
// SQ_LDS_BANK_CONFLICT counter of the long-row kernels exactly: 1024 extra
// cycles per row at 16384 (left as is: the conflict-free item order of its
// pass 1024 measured slower, 1024x16384 fp32 forward 39.1 -> 39.8 us) and 37888
// at 32768 with the layouts replaced here, which serialised the 64 lanes of
// every write into layout 512 (512x32768 fp32 forward 73.0 -> 50.6 us).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int lds_pad(int P, int B) {
  return B <= 16 || B == 32   ? 1
         : B == 128           ? (P <= 512 ? 8 : P == 1024 ? 4 : P == 2048 ? 2 : 1)
         : P == 32768 && B == 512 ? 1
                                  : 0;
}
// true: items of the pass with input size B are numbered class-fastest
// (k = item % (B/2)); false: residue-fastest (r' = item % NRES)
__host__ __device__ constexpr bool class_fast(int P, int B) {
  return (B == 128 && P >= 2048) || (P == 32768 && B == 512);
}

// ---------------------------------------------------------------------------
// one row of P reals, T = P/E threads (t = thread index within the row).
// Loaders are called as ld(var, cst) for element var + cst (var varies per
// lane, cst is a compile-time constant); storers as st(var, cst, value).
// ---------------------------------------------------------------------------
// twiddle placements of kernels that run both directions (Row::TwSet)
constexpr int kTwRegs = 0, kTwLds = 1, kTwRegsFwd = 2;

template <int P, int E>
struct Row {
  static_assert((P & (P - 1)) == 0 && P >= 2 && P <= 32768, "P must be a power of two in [2, 32768]");
  static_assert(E <= P && (E & (E - 1)) == 0 && E >= 2, "E must be a power of two <= P");
  static constexpr int T = P / E;

  template <int B>
  static constexpr int stride() { return B + lds_pad(P, B); }
  // layout of an exchange whose spectra have size B: residue r, slot s
  template <int B>
  static __device__ __forceinline__ int addr(int r, int s) { return r * stride<B>() + s; }

  // pass descriptors, input size B
  template <int B>
  struct Pass {
    static constexpr int R = cmin(P / B, E / 2);
    static constexpr int BP = B * R;
    static constexpr int NRES = P / BP;
    static constexpr int IPT = E / (2 * R);
    static constexpr bool KFAST = class_fast(P, B);
    static __device__ __forceinline__ void item(int it, int& rp, int& k) {
      if (KFAST) {
        k = it % (B / 2);
        rp = it / (B / 2);
      } else {
        rp = it % NRES;
        k = it / NRES;
      }
    }
  };

  // floats of LDS a row needs: the largest exchange layout
  template <int B>
  static constexpr int lds_from() {
    if constexpr (B >= P)
      return P;
    else
      return cmax((P / B) * stride<B>(), lds_from<Pass<B>::BP>());
  }
  static constexpr int LDS = (P == E) ? P : lds_from<E>();

  // Twiddles of this thread's items in every pass with input size >= B, read
  // once per kernel (they depend on the thread only) and kept in registers.
  template <int B, bool INV, bool END = (B >= P)>
  struct Tws {
    using PS = Pass<B>;
    using W = typename std::conditional<INV, Tw, TwF>::type;
    W w[PS::IPT][PS::R];
    Tws<PS::BP, INV> next;
    __device__ __forceinline__ void load(int t) {
#pragma unroll
      for (int n = 0; n < PS::IPT; ++n) {
        int rp, k;
        PS::item(t + T * n, rp, k);
        if constexpr (INV)
          load_item_tw(PassTw<B, PS::R>::inv(), k, w[n]);
        else
          load_item_tw(PassTw<B, PS::R>::fwd(), k, w[n]);
      }
      next.load(t);
    }
    // the twiddles of the pass with input size B2 >= B
    template <int B2>
    __device__ __forceinline__ const auto& at() const {
      if constexpr (B2 == B)
        return w;
      else
        return next.template at<B2>();
    }
    // twiddle provider interface: the R twiddles of item n (class k) of pass B2
    template <int B2, class WW, int RR>
    __device__ __forceinline__ void item(int n, int /*k*/, WW (&out)[RR]) const {
      const auto& src = at<B2>()[n];
#pragma unroll
      for (int j = 0; j < RR; ++j) out[j] = src[j];
    }
  };
  template <int B, bool INV>
  struct Tws<B, INV, true> {
    __device__ __forceinline__ void load(int) {}
  };
  using FwdTws = Tws<E, false>;
  using InvTws = Tws<E, true>;

  // Twiddle provider reading the per-pass (cos, tan) tables from an LDS copy
  // (for kernels that cannot keep them in registers); inverse twiddles take
  // sin = cos * tan.
  struct LdsTws {
    const TwF* base;
    template <int B>
    static constexpr int offset() {
      if constexpr (B == E)
        return 0;
      else
        return offset<pass_in_for(B)>() + (pass_in_for(B) / 2) * Pass<pass_in_for(B)>::R;
    }
    static constexpr int entries() { return (P == E) ? 0 : offset<P>(); }
    // cooperative copy of the global tables into dst (entries() values)
    template <int B = E>
    static __device__ __forceinline__ void fill(TwF* dst, int tid, int nt) {
      if constexpr (B < P) {
        constexpr int R = Pass<B>::R, N = (B / 2) * R;
        const TwF* src = PassTw<B, R>::fwd();
        for (int i = tid; i < N; i += nt) dst[offset<B>() + i] = src[i];
        fill<Pass<B>::BP>(dst, tid, nt);
      }
    }
    template <int B, class WW, int RR>
    __device__ __forceinline__ void item(int /*n*/, int k, WW (&out)[RR]) const {
      TwF f[RR];
      __builtin_memcpy(f, base + offset<B>() + k * RR, sizeof(f));
#pragma unroll
      for (int j = 0; j < RR; ++j) {
        if constexpr (std::is_same<WW, TwF>::value)
          out[j] = f[j];
        else
          out[j] = Tw{f[j].c, f[j].c * f[j].tn};
      }
    }
  };

  // Twiddle provider reading each item's twiddles from the per-pass tables
  // when the pass runs (kernels with too many passes or threads to keep them
  // in registers).
  struct GlobalTws {
    template <int B, class WW, int RR>
    __device__ __forceinline__ void item(int /*n*/, int k, WW (&out)[RR]) const {
      if constexpr (std::is_same<WW, TwF>::value)
        load_item_tw(PassTw<B, RR>::fwd(), k, out);
      else
        load_item_tw(PassTw<B, RR>::inv(), k, out);
    }
  };

  // Both directions' twiddles for a kernel that runs forward and inverse
  // transforms, by placement: kTwRegs (register copies of both tables),
  // kTwLds (one LDS table of lds_floats() floats that init() fills
  // cooperatively; a barrier must follow before the first transform) or
  // kTwRegsFwd (registers for the forward (cos, tan) only; the inverse takes
  // sin = cos * tan from them, half the registers of kTwRegs).
  template <int MODE, int D = 0>
  struct TwSet {
    FwdTws f;
    InvTws i;
    static constexpr int lds_floats() { return 0; }
    __device__ __forceinline__ void init(TwF*, int, int, int t) {
      f.load(t);
      i.load(t);
    }
    __device__ __forceinline__ const FwdTws& fwd() const { return f; }
    __device__ __forceinline__ const InvTws& inv() const { return i; }
  };
  template <int D>
  struct TwSet<kTwLds, D> {
    LdsTws l;
    static constexpr int lds_floats() { return (2 * LdsTws::entries() + 3) / 4 * 4; }
    __device__ __forceinline__ void init(TwF* dst, int tid, int nt, int) {
      LdsTws::fill(dst, tid, nt);
      l.base = dst;
    }
    __device__ __forceinline__ const LdsTws& fwd() const { return l; }
    __device__ __forceinline__ const LdsTws& inv() const { return l; }
  };
  struct InvFromFwd {
    const FwdTws& f;
    template <int B, class WW, int RR>
    __device__ __forceinline__ void item(int n, int k, WW (&out)[RR]) const {
      TwF src[RR];
      f.template item<B>(n, k, src);
#pragma unroll
      for (int j = 0; j < RR; ++j) out[j] = Tw{src[j].c, src[j].c * src[j].tn};
    }
  };
  template <int D>
  struct TwSet<kTwRegsFwd, D> {
    FwdTws f;
    static constexpr int lds_floats() { return 0; }
    __device__ __forceinline__ void init(TwF*, int, int, int t) { f.load(t); }
    __device__ __forceinline__ const FwdTws& fwd() const { return f; }
    __device__ __forceinline__ InvFromFwd inv() const { return InvFromFwd{f}; }
  };

  // ---- forward ----------------------------------------------------------
  // pass 0: thread t reads elements t + T*s (coalesced across threads)
  template <class Ld>
  static __device__ __forceinline__ void fwd_pass0(float (&a)[E], Ld ld, int t) {
    constexpr int LE = ilog2(E);
#pragma unroll
    for (int s = 0; s < E; ++s) a[bitrev(s, LE)] = ld(t, T * s);
    small_fwd<E, 1>(a);
  }
  // the same split in two: the loads (raw values, possibly a row ahead) ...
  template <class V, class Ld>
  static __device__ __forceinline__ void fwd_load0(V (&raw)[E], Ld ld, int t) {
#pragma unroll
    for (int s = 0; s < E; ++s) raw[s] = ld(t, T * s);
  }
  // ... and the stages
  template <class V, class Wd>
  static __device__ __forceinline__ void fwd_pass0_from(float (&a)[E], const V (&raw)[E], Wd widen) {
    constexpr int LE = ilog2(E);
#pragma unroll
    for (int s = 0; s < E; ++s) a[bitrev(s, LE)] = widen(raw[s]);
    small_fwd<E, 1>(a);
  }

  static __device__ __forceinline__ void fwd_pass0_scatter(const float (&a)[E], float* L, int t) {
#pragma unroll
    for (int s = 0; s < E; ++s) L[addr<E>(t, s)] = a[s];
  }

  // gather items of the pass with input size B from LDS (layout B) and run it
  template <int B, class W>
  static __device__ __forceinline__ void fwd_pass(float (&a)[E], const float* L, int t, const W& tw) {
    using PS = Pass<B>;
    constexpr int R = PS::R, LR = ilog2(R);
#pragma unroll
    for (int n = 0; n < PS::IPT; ++n) {
      int rp, k;
      PS::item(t + T * n, rp, k);
      const int k2 = (k == 0) ? (B / 2) : (B - k);
      float* v = a + 2 * R * n;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        const int r = rp + PS::NRES * bitrev(q, LR);
        v[2 * q] = L[addr<B>(r, k)];
        v[2 * q + 1] = L[addr<B>(r, k2)];
      }
      if (k == 0) {
        item0_fwd<R>(v);
      } else {
        TwF w[R];
        tw.template item<B>(n, k, w);
        item_fwd<B, R>(v, w);
      }
    }
  }

  // write the items of pass B to LDS in layout B*R (natural order when B*R == P)
  template <int B>
  static __device__ __forceinline__ void pass_scatter(const float (&a)[E], float* L, int t) {
    using PS = Pass<B>;
    constexpr int R = PS::R;
#pragma unroll
    for (int n = 0; n < PS::IPT; ++n) {
      int rp, k;
      PS::item(t + T * n, rp, k);
      const int k2 = (k == 0) ? (B / 2) : (B - k);
      const float* v = a + 2 * R * n;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        L[addr<PS::BP>(rp, q * B + k)] = v[2 * q];
        L[addr<PS::BP>(rp, q * B + k2)] = v[2 * q + 1];
      }
    }
  }

  // store the items of the last pass (B*R == P) in natural packed order
  template <int B, class St>
  static __device__ __forceinline__ void last_store(const float (&a)[E], int t, St st) {
    using PS = Pass<B>;
    static_assert(PS::BP == P, "not the last pass");
    constexpr int R = PS::R;
#pragma unroll
    for (int n = 0; n < PS::IPT; ++n) {
      const int k = t + T * n;
      const int k2 = (k == 0) ? (B / 2) : (B - k);
      const float* v = a + 2 * R * n;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        st(k, q * B, v[2 * q]);
        st(k2, q * B, v[2 * q + 1]);
      }
    }
  }

  // ---- inverse -----------------------------------------------------------
  // gather items of inverse pass B (input spectra of size B*R) through
  // src(var, cst) -- LDS in layout B*R, or the natural packed row when
  // B*R == P -- and run it
  template <int B, class Src, class W>
  static __device__ __forceinline__ void inv_pass(float (&a)[E], Src src, int t, const W& tw) {
    using PS = Pass<B>;
    constexpr int R = PS::R;
#pragma unroll
    for (int n = 0; n < PS::IPT; ++n) {
      int rp, k;
      PS::item(t + T * n, rp, k);
      const int k2 = (k == 0) ? (B / 2) : (B - k);
      float* v = a + 2 * R * n;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        v[2 * q] = src(addr<PS::BP>(rp, k), q * B);
        v[2 * q + 1] = src(addr<PS::BP>(rp, k2), q * B);
      }
      if (k == 0) {
        item0_inv<R>(v);
      } else {
        Tw w[R];
        tw.template item<B>(n, k, w);
        item_inv<B, R>(v, w);
      }
    }
  }

  // the first inverse pass (B*R == P) split in two: the loads of the natural
  // packed row (raw values, possibly a row ahead) ...
  template <int B, class V, class Ld>
  static __device__ __forceinline__ void inv_load_first(V (&raw)[E], Ld ld, int t) {
    using PS = Pass<B>;
    static_assert(PS::BP == P, "not the first inverse pass");
    constexpr int R = PS::R;
#pragma unroll
    for (int n = 0; n < PS::IPT; ++n) {
      const int k = t + T * n;
      const int k2 = (k == 0) ? (B / 2) : (B - k);
#pragma unroll
      for (int q = 0; q < R; ++q) {
        raw[2 * R * n + 2 * q] = ld(k, q * B);
        raw[2 * R * n + 2 * q + 1] = ld(k2, q * B);
      }
    }
  }
  // ... and its stages
  template <int B, class V, class Wd, class W>
  static __device__ __forceinline__ void inv_first_from(float (&a)[E], const V (&raw)[E], Wd widen, int t,
                                                        const W& tw) {
    using PS = Pass<B>;
    constexpr int R = PS::R;
#pragma unroll
    for (int n = 0; n < PS::IPT; ++n) {
      const int k = t + T * n;
      float* v = a + 2 * R * n;
#pragma unroll
      for (int j = 0; j < 2 * R; ++j) v[j] = widen(raw[2 * R * n + j]);
      if (k == 0) {
        item0_inv<R>(v);
      } else {
        Tw w[R];
        tw.template item<B>(n, k, w);
        item_inv<B, R>(v, w);
      }
    }
  }

  // input size of the pass whose output size is Bout (Bout > E)
  static constexpr int pass_in_for(int Bout) {
    int b = E;
    while (b * cmin(P / b, E / 2) != Bout) b *= cmin(P / b, E / 2);
    return b;
  }

  // write the items of inverse pass B to LDS in layout B
  template <int B>
  static __device__ __forceinline__ void inv_scatter(const float (&a)[E], float* L, int t) {
    using PS = Pass<B>;
    constexpr int R = PS::R, LR = ilog2(R);
#pragma unroll
    for (int n = 0; n < PS::IPT; ++n) {
      int rp, k;
      PS::item(t + T * n, rp, k);
      const int k2 = (k == 0) ? (B / 2) : (B - k);
      const float* v = a + 2 * R * n;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        const int r = rp + PS::NRES * bitrev(q, LR);
        L[addr<B>(r, k)] = v[2 * q];
        L[addr<B>(r, k2)] = v[2 * q + 1];
      }
    }
  }

  // inverse pass 0: gather residue t's E-point spectrum from LDS (layout E),
  // invert, store element t + T s = value * scale through st(var, cst, v)
  template <class St>
  static __device__ __forceinline__ void inv_pass0_store(float (&a)[E], const float* L, int t, float scale, St st) {
    constexpr int LE = ilog2(E);
#pragma unroll
    for (int s = 0; s < E; ++s) a[s] = L[addr<E>(t, s)];
    small_inv<E, 1>(a);
#pragma unroll
    for (int s = 0; s < E; ++s) st(t, T * s, a[bitrev(s, LE)] * scale);
  }
};

}  // namespace rdfft
