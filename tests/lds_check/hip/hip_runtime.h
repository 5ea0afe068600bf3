// hip/hip_runtime.h stand-in for running the library's kernels on CPU threads.
//
// Test infrastructure only: the LDS schedule checker builds rdfft_lib.hip for
// the host against this header (g++/clang++, C++20, ThreadSanitizer), so the
// C ABI, its dispatch logic and the kernel templates run unchanged, with
//   * one host thread per GPU thread of a workgroup; workgroups one after
//     another;
//   * __syncthreads() a pthread barrier of the workgroup's threads (the
//     sanitizer knows its ordering, so any two threads touching one LDS slot
//     between two barriers, at least one of them writing, is reported);
//   * __shared__ arrays static (one copy, reused by consecutive workgroups)
//     and the launch's dynamic LDS a fresh NaN-filled block per workgroup;
//   * buffer-resource loads and stores with the hardware's range rule (a raw
//     buffer checks the lane offset against its size; loads past it read 0,
//     stores past it are dropped), and an abort when the lane offset is in
//     range but the scalar offset carries the access past the buffer;
//   * readfirstlane the identity (the kernels apply it to values that are
//     uniform across the wavefront);
//   * global float atomics as compare-exchange loops.
#pragma once

#include <pthread.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <vector>

#define __global__
#define __device__
#define __host__
#define __align__(x) __attribute__((aligned(x)))
#define HIP_SYMBOL(X) X
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static
#define __restrict__ __restrict

struct dim3 {
  unsigned x = 1, y = 1, z = 1;
  constexpr dim3() = default;
  constexpr dim3(unsigned a, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};

typedef int hipError_t;
typedef void* hipStream_t;
constexpr hipError_t hipSuccess = 0;
enum hipDeviceAttribute_t { hipDeviceAttributeMultiprocessorCount = 0 };

namespace emu {

struct Ctx {
  dim3 tid, bid, bdim, gdim;
  pthread_barrier_t* bar = nullptr;
};
inline thread_local Ctx ctx;
inline float* dyn_lds = nullptr;
// compute units the library's launch logic sizes its persistent grids for
inline int num_cus() {
  const char* s = std::getenv("EMU_CUS");
  return s ? std::atoi(s) : 2;
}
inline long launches = 0, workgroups = 0;

inline void fail(const char* what) {
  std::fprintf(stderr, "EMU ERROR: %s\n", what);
  std::abort();
}

struct WorkItem {
  std::function<void()>* body;
  Ctx c;
};
inline void* run_item(void* p) {
  auto* w = static_cast<WorkItem*>(p);
  ctx = w->c;
  (*w->body)();
  return nullptr;
}

// Runs body() as the kernel's workgroups, one after another, each as
// block.x * block.y * block.z host threads.
inline void launch(dim3 grid, dim3 block, size_t dyn_bytes, std::function<void()> body) {
  const unsigned nt = block.x * block.y * block.z;
  if (nt == 0 || nt > 1024) fail("workgroup size");
  std::vector<float> dyn(dyn_bytes / sizeof(float) + 4);
  dyn_lds = dyn.data();
  std::vector<pthread_t> th(nt);
  std::vector<WorkItem> items(nt);
  pthread_attr_t attr;
  pthread_attr_init(&attr);
  pthread_attr_setstacksize(&attr, 1 << 20);
  ++launches;
  for (unsigned bz = 0; bz < grid.z; ++bz)
    for (unsigned by = 0; by < grid.y; ++by)
      for (unsigned bx = 0; bx < grid.x; ++bx) {
        for (auto& v : dyn) v = std::nanf("");
        pthread_barrier_t bar;
        pthread_barrier_init(&bar, nullptr, nt);
        for (unsigned t = 0; t < nt; ++t) {
          items[t].body = &body;
          items[t].c = Ctx{dim3(t % block.x, (t / block.x) % block.y, t / (block.x * block.y)), dim3(bx, by, bz),
                           block, grid, &bar};
          if (pthread_create(&th[t], &attr, run_item, &items[t]) != 0) fail("pthread_create");
        }
        for (unsigned t = 0; t < nt; ++t) pthread_join(th[t], nullptr);
        pthread_barrier_destroy(&bar);
        ++workgroups;
      }
  pthread_attr_destroy(&attr);
}

struct Rsrc {
  char* base;
  int64_t nbytes;
};

inline bool in_range(const Rsrc& r, int voff, int soff, int size) {
  if (voff < 0 || static_cast<int64_t>(voff) + size > r.nbytes) return false;
  if (static_cast<int64_t>(voff) + soff + size > r.nbytes || soff < 0)
    fail("buffer access whose lane offset is in range but whose scalar offset leaves the buffer");
  return true;
}
template <class T>
inline T bload(Rsrc r, int voff, int soff) {
  T v{};
  if (in_range(r, voff, soff, sizeof(T))) std::memcpy(&v, r.base + voff + soff, sizeof(T));
  return v;
}
template <class T>
inline void bstore(T v, Rsrc r, int voff, int soff) {
  if (in_range(r, voff, soff, sizeof(T))) std::memcpy(r.base + voff + soff, &v, sizeof(T));
}

}  // namespace emu

typedef emu::Rsrc __amdgpu_buffer_rsrc_t;
typedef unsigned int emu_u32x4 __attribute__((ext_vector_type(4)));

#define threadIdx (emu::ctx.tid)
#define blockIdx (emu::ctx.bid)
#define blockDim (emu::ctx.bdim)
#define gridDim (emu::ctx.gdim)
#define RDFFT_DYNAMIC_LDS(name) float* name = emu::dyn_lds

inline void __syncthreads() { pthread_barrier_wait(emu::ctx.bar); }

#define __builtin_amdgcn_readfirstlane(v) (v)
inline emu::Rsrc emu_make_rsrc(void* p, int /*stride*/, int nbytes, int /*flags*/) {
  return emu::Rsrc{static_cast<char*>(p), nbytes};
}
#define __builtin_amdgcn_make_buffer_rsrc emu_make_rsrc
#define __builtin_amdgcn_raw_buffer_load_b16(r, v, s, a) emu::bload<uint16_t>(r, v, s)
#define __builtin_amdgcn_raw_buffer_load_b32(r, v, s, a) emu::bload<uint32_t>(r, v, s)
#define __builtin_amdgcn_raw_buffer_load_b128(r, v, s, a) emu::bload<emu_u32x4>(r, v, s)
#define __builtin_amdgcn_raw_buffer_store_b16(x, r, v, s, a) emu::bstore<uint16_t>(x, r, v, s)
#define __builtin_amdgcn_raw_buffer_store_b32(x, r, v, s, a) emu::bstore<uint32_t>(x, r, v, s)
#define __builtin_amdgcn_raw_buffer_store_b128(x, r, v, s, a) emu::bstore<emu_u32x4>(x, r, v, s)

inline float __uint_as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
inline uint32_t __float_as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }

inline float unsafeAtomicAdd(float* p, float v) {
  uint32_t* u = reinterpret_cast<uint32_t*>(p);
  uint32_t old = __atomic_load_n(u, __ATOMIC_RELAXED);
  while (true) {
    const uint32_t nv = __float_as_uint(__uint_as_float(old) + v);
    if (__atomic_compare_exchange_n(u, &old, nv, false, __ATOMIC_RELAXED, __ATOMIC_RELAXED)) break;
  }
  return __uint_as_float(old);
}

inline hipError_t hipGetLastError() { return hipSuccess; }
// a __device__ variable is a host variable here: its address is the symbol's
template <class T>
inline hipError_t hipGetSymbolAddress(void** p, const T& symbol) {
  *p = const_cast<void*>(static_cast<const void*>(&symbol));
  return hipSuccess;
}
inline hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
inline hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = emu::num_cus();
  return hipSuccess;
}

#define hipLaunchKernelGGL(kernel, grid, block, lds, stream, ...) \
  emu::launch(grid, block, lds, [=]() { kernel(__VA_ARGS__); })
