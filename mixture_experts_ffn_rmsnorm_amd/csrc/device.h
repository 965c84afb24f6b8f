// Device helpers shared by the kernels: bf16/fp16 conversion, wave64
// reductions, and the routing routine used both by the full layer and by the
// stand-alone routing entry point.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"
#include "moe_ffn.h"

namespace moe {

constexpr int kWave = 64;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// bf16 bits -> f32 (exact: bf16 is the upper half of binary32)
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Eight bf16 weights packed in a uint4 -> eight floats.
__device__ __forceinline__ void unpack8(const uint4& q, float* f) {
  f[0] = bf16lo(q.x); f[1] = bf16hi(q.x);
  f[2] = bf16lo(q.y); f[3] = bf16hi(q.y);
  f[4] = bf16lo(q.z); f[5] = bf16hi(q.z);
  f[6] = bf16lo(q.w); f[7] = bf16hi(q.w);
}

// Streaming 16-byte load of data read once (expert weights): non-temporal
// so it does not evict reusable lines from the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

// Accurate SwiGLU for the f32 decode path: silu(g) * u with expf.
__device__ __forceinline__ float swiglu_f32(float g, float u) { return g / (1.0f + expf(-g)) * u; }

__device__ __forceinline__ double sigmoid_f64(float logit) {
  return 1.0 / (1.0 + exp(-(double)logit));
}

// "a ranks before b": larger key first, equal keys to the lower expert id.
__device__ __forceinline__ bool ranks_before(double ka, int ea, double kb, int eb) {
  return ka > kb || (ka == kb && ea < eb);
}

struct RowRoute {
  int idx[kMaxTopK];
  float w[kMaxTopK];
  bool valid[kMaxTopK];
  uint32_t flags;
};

// Routes one row with one wavefront; every lane returns the same result.
//   score layer: top-K experts by key sigmoid(logit) + bias (float64),
//     descending, equal keys to the lower index; weights are the unbiased
//     sigmoids of the chosen experts over their sum.
//   hash layer: the table row of the token id in column order, weighted by
//     the renormalised sigmoids of those experts; a token id outside
//     [0, table_rows) masks the whole row, a table entry outside
//     [0, E) masks its slot.
// `logits` is the row's f32 logits [E] (global memory).
__device__ __forceinline__ RowRoute route_row(const float* __restrict__ logits, int E, int K, int layer_kind,
                                              const float* __restrict__ bias, const int32_t* __restrict__ table,
                                              int64_t table_rows, int32_t token) {
  const int lane = threadIdx.x & (kWave - 1);
  RowRoute rr;
  rr.flags = 0;
  if (layer_kind == 1) {  // hash
    const bool tok_ok = token >= 0 && (int64_t)token < table_rows;
    double s[kMaxTopK];
    double tot = 0.0;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
      if (k >= K) { rr.idx[k] = -1; rr.valid[k] = false; s[k] = 0.0; continue; }
      int e = tok_ok ? table[(int64_t)token * K + k] : -1;
      bool ok = tok_ok && e >= 0 && e < E;
      rr.idx[k] = e;
      rr.valid[k] = ok;
      s[k] = ok ? sigmoid_f64(logits[e]) : 0.0;
      tot += s[k];
      if (tok_ok && !ok) rr.flags |= MOE_FLAG_BAD_TABLE_ENTRY;
    }
    if (!tok_ok) rr.flags |= MOE_FLAG_BAD_TOKEN;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) rr.w[k] = (rr.valid[k] && tot > 0.0) ? (float)(s[k] / tot) : 0.0f;
    return rr;
  }
  // score layer: each lane owns experts lane, lane+64, lane+128, lane+192
  double key[4], sg[4];
  bool taken[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = lane + kWave * j;
    taken[j] = e >= E;
    sg[j] = (e < E) ? sigmoid_f64(logits[e]) : 0.0;
    key[j] = (e < E) ? sg[j] + (double)bias[e] : 0.0;
  }
  double tot = 0.0;
  double s[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k >= K) { rr.idx[k] = -1; rr.valid[k] = false; s[k] = 0.0; continue; }
    double bk = 0.0, bsg = 0.0;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = lane + kWave * j;
      if (!taken[j] && (be == 0x7fffffff || ranks_before(key[j], e, bk, be))) {
        bk = key[j];
        be = e;
        bsg = sg[j];
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      double ok_ = __shfl_xor(bk, o, kWave);
      int oe = __shfl_xor(be, o, kWave);
      double osg = __shfl_xor(bsg, o, kWave);
      bool take = (oe != 0x7fffffff) && (be == 0x7fffffff || ranks_before(ok_, oe, bk, be));
      if (take) {
        bk = ok_;
        be = oe;
        bsg = osg;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + kWave * j == be) taken[j] = true;
    rr.idx[k] = be;
    rr.valid[k] = true;
    s[k] = bsg;
    tot += bsg;
  }
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) rr.w[k] = (k < K) ? (float)(s[k] / tot) : 0.0f;
  return rr;
}

}  // namespace moe
