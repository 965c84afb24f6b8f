// Device ceilings measured on the device itself, reported beside the
// published MI355X figures that the roofline fractions use:
//   - the rate at which plain 16-byte streaming loads read a buffer far
//     larger than the caches (HBM read bandwidth);
//   - the rate of v_mfma_f32_32x32x16_f16 -- the instruction of the prefill
//     GEMMs -- with operands already in registers (fp16 dense matrix peak).
// A separate library (libmoepeaks.so); the layer does not use it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr int kMfmaThreads = 256;
constexpr int kMfmaChains = 4;  // independent accumulators per wave

// A workgroup reads a contiguous chunk of kReadUnroll * kReadThreads
// 16-byte vectors per step (all of its loads in flight at once; DRAM sees
// whole 32 KiB runs), chunks grid-strided; a partial last chunk is read
// vector by vector.  The words fold into one that is stored only if it
// equals a value the data cannot produce by chance, so the loads stay and
// nothing is written.
__global__ __launch_bounds__(kReadThreads) void k_read(const u32x4* __restrict__ p, size_t n16, uint32_t* sink) {
  constexpr size_t kChunk = (size_t)kReadUnroll * kReadThreads;
  const size_t full = n16 / kChunk;
  uint32_t acc = 0;
  for (size_t c = blockIdx.x; c < full; c += gridDim.x) {
    const u32x4* q = p + c * kChunk + threadIdx.x;
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(q + u * kReadThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (blockIdx.x == 0)
    for (size_t i = full * kChunk + threadIdx.x; i < n16; i += kReadThreads) {
      const u32x4 v = __builtin_nontemporal_load(p + i);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// kMfmaChains independent 32x32x16 fp16 products per wave and iteration,
// operands from the thread index (so they are not constants); the sum of the
// accumulators is stored only if it is NaN, which the small operands cannot
// produce.
__global__ __launch_bounds__(kMfmaThreads) void k_mfma(int iters, float* sink) {
  half8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(((threadIdx.x + i) & 7) * 0.0009765625f);
    b[i] = (_Float16)(((threadIdx.x * 3 + i) & 7) * 0.0009765625f);
  }
  floatx16 c[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[k][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[k][i];
  if (s != s) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" {

// One read pass over `bytes` (a multiple of 16) of device memory at `buf`
// (16-byte aligned), on `stream`.  `sink`: one device word that is (in
// practice) never written.  Returns a hipError_t.
int moe_peaks_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!buf || !sink || bytes % 16 || ((uintptr_t)buf & 15) || blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read, dim3(blocks), dim3(kReadThreads), 0, (hipStream_t)stream, (const u32x4*)buf, bytes / 16,
                     sink);
  return (int)hipGetLastError();
}

// `blocks` workgroups of 4 waves, each wave issuing iters * kMfmaChains
// MFMAs; flops of the launch = blocks * 4 * iters * kMfmaChains * 32768.
// `sink`: `blocks` device floats, written only on NaN.
int moe_peaks_mfma(int blocks, int iters, float* sink, void* stream) {
  if (!sink || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma, dim3(blocks), dim3(kMfmaThreads), 0, (hipStream_t)stream, iters, sink);
  return (int)hipGetLastError();
}

// MFMA instructions per wave and iteration, threads per workgroup.
int moe_peaks_mfma_chains(void) { return kMfmaChains; }
int moe_peaks_mfma_threads(void) { return kMfmaThreads; }

}  // extern "C"
