// stream_probe.hip -- the measurement reference for the in-place transforms
// (libstreamprobe.so, loaded by bench.py only; not part of the rdFFT ABI).
//
// An in-place pass that reads every float of a buffer once and writes it back
// once, scaled, with nothing in between: the HBM traffic of an in-place
// transform (each row read once and written once) with none of its
// arithmetic.  Its time over a buffer of some size is what any in-place
// kernel of that size can approach on this part (launch ramp, memory latency
// and the drain of the last stores included).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;
constexpr int64_t kChunk = static_cast<int64_t>(kThreads) * kPerThread;  // floats per workgroup iteration

// NT: non-temporal loads and stores (every byte is touched once per launch)
template <bool NT>
__global__ void __launch_bounds__(kThreads) stream_inplace_kernel(float* __restrict__ d, int64_t n, float scale) {
  const int64_t full = n / kChunk;
  for (int64_t c = blockIdx.x; c < full; c += gridDim.x) {
    float* base = d + c * kChunk + threadIdx.x;
    float v[kPerThread];
#pragma unroll
    for (int s = 0; s < kPerThread; ++s) v[s] = NT ? __builtin_nontemporal_load(base + kThreads * s) : base[kThreads * s];
#pragma unroll
    for (int s = 0; s < kPerThread; ++s) {
      if (NT)
        __builtin_nontemporal_store(v[s] * scale, base + kThreads * s);
      else
        base[kThreads * s] = v[s] * scale;
    }
  }
  // the last partial chunk, one float per thread
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = full * kChunk + static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride)
    d[i] = d[i] * scale;
}

}  // namespace

extern "C" {

// In place: data[i] *= scale for 0 <= i < n (fp32, device memory, caller-owned),
// on `grid` workgroups of 256 threads (grid >= 1) looping over 16 KB chunks;
// policy 0 = default cache policy, 1 = non-temporal loads and stores.
// Returns 0, or -1 on a bad argument or a failed launch.
int stream_probe(float* data, int64_t n, int grid, int policy, float scale, void* stream) {
  if (!data || n < 0 || grid < 1 || (policy != 0 && policy != 1)) return -1;
  if (n == 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (policy)
    stream_inplace_kernel<true><<<dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s>>>(data, n, scale);
  else
    stream_inplace_kernel<false><<<dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s>>>(data, n, scale);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
