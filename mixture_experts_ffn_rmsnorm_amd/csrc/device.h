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

// Write-through (agent-scope) store / load of one float: data that another
// workgroup reads -- of the same kernel after a flag or counter says so (the
// writer waits for these stores to complete, sync_stores, before raising
// it), or of a later launch, on any XCD.  The reader's loads bypass stale
// cache lines.
__device__ __forceinline__ void store_wt(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_wt(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Checked build (MOE_CHECKED): an index produced by an earlier step of the
// call is tested where it is used; a failed test sets MOE_FLAG_CHECK in the
// status word, and the caller clamps the index as the default build does
// (so nothing reads or writes out of bounds either way).  The default build
// compiles the tests away.
__device__ __forceinline__ void check_index(uint32_t* status, bool ok) {
#ifdef MOE_CHECKED
  if (!ok) atomicOr(status, (uint32_t)MOE_FLAG_CHECK);
#else
  (void)status;
  (void)ok;
#endif
}

// Every store this thread issued has completed.
__device__ __forceinline__ void sync_stores() { __builtin_amdgcn_s_waitcnt(0); }

// v moved across lanes inside each 16-lane row by a DPP control (every
// lane of the wave active): quad_perm [1,0,3,2] (0xB1) and [2,3,0,1] (0x4E)
// swap lane bit 0 / bit 1, row_half_mirror (0x141) and row_mirror (0x140)
// reverse 8 / 16 lanes, row_ror:n (0x120 + n) rotates the row by n lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Lane c (0..15) of each 16-lane row, in every lane of that row (DPP
// row_newbcast:c).  c must fold to a constant (an unrolled loop index).
__device__ __forceinline__ uint32_t row_bcast(uint32_t v, int c) {
#define MOE_ROW_BCAST(n) \
  case n: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + n, 0xF, 0xF, false);
  switch (c) {
    MOE_ROW_BCAST(0) MOE_ROW_BCAST(1) MOE_ROW_BCAST(2) MOE_ROW_BCAST(3) MOE_ROW_BCAST(4) MOE_ROW_BCAST(5)
    MOE_ROW_BCAST(6) MOE_ROW_BCAST(7) MOE_ROW_BCAST(8) MOE_ROW_BCAST(9) MOE_ROW_BCAST(10) MOE_ROW_BCAST(11)
    MOE_ROW_BCAST(12) MOE_ROW_BCAST(13) MOE_ROW_BCAST(14) default: break;
  }
#undef MOE_ROW_BCAST
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x15F, 0xF, 0xF, false);
}
// Sum over the 16 lanes of each row, in every lane of the row: after the
// two quad swaps every lane holds its quad's sum, the half mirror adds the
// other quad of its 8, the mirror the other 8 of its row.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  return v + dpp_f32<0x140>(v);
}
// Sum over the wave (every lane active), the same in every lane: the rows'
// sums read out and added in row order.  DPP moves and lane reads instead
// of LDS-crossbar shuffles: a handful of cycles each.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const int b = __float_as_int(v);
  return ((__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
          __int_as_float(__builtin_amdgcn_readlane(b, 32))) + __int_as_float(__builtin_amdgcn_readlane(b, 48));
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

// Selection key of the score route: sigmoid(logit) + bias, in float64.
__device__ __forceinline__ double score_key(float logit, float bias) { return sigmoid_f64(logit) + (double)bias; }

// Order-preserving map of a float64 key onto uint64 (larger key -> larger
// integer); finite keys map to values >= 1, so 0 can mark "no candidate".
__device__ __forceinline__ uint64_t ordered_key(double k) {
  const uint64_t b = (uint64_t)__double_as_longlong(k);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// max(v, v from the lane `CTRL` selects within its 16-lane row), 0 for lanes
// whose source falls outside the row.
template <int CTRL>
__device__ __forceinline__ uint64_t umax_dpp(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, true);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, true);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

// Maximum of a uint64 over the wavefront, returned to every lane: shifts by
// 1, 2, 4, 8 lanes inside each 16-lane row leave the row maximum in its lane
// 15; the four row maxima are read back as scalars.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax_dpp<0x111>(v);  // row_shr:1
  v = umax_dpp<0x112>(v);  // row_shr:2
  v = umax_dpp<0x114>(v);  // row_shr:4
  v = umax_dpp<0x118>(v);  // row_shr:8
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r + 15);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r + 15);
    const uint64_t x = ((uint64_t)hi << 32) | lo;
    m = x > m ? x : m;
  }
  return m;
}

// Top-K of one row's keys with one wavefront: lane l holds the keys of
// experts l, l+64, l+128, l+192 (key[j]; experts >= E absent).  Larger key
// first; equal keys go to the lower expert id.  Every lane gets the same K
// indices in idx and, in lg_sel, the f32 logit lg[j] of each chosen expert.
__device__ __forceinline__ void select_topk(const double (&key)[4], const float (&lg)[4], int E, int K,
                                            int (&idx)[kMaxTopK], float (&lg_sel)[kMaxTopK]) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = (lane + kWave * j < E) ? ordered_key(key[j]) : 0ull;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    idx[k] = -1;
    lg_sel[k] = 0.f;
    if (k >= K) continue;
    uint64_t lm = u[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) lm = u[j] > lm ? u[j] : lm;
    const uint64_t m = wave_max_u64(lm);
    // the lowest expert id holding the maximum: experts are ordered by
    // (j, lane), so scan j upwards and take the lowest lane
    int e = 0;
    float l = lg[0];
    bool found = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (found) continue;
      const uint64_t mask = __ballot(u[j] == m && m != 0ull);
      if (mask) {
        const int wl = __ffsll((unsigned long long)mask) - 1;
        e = wl + kWave * j;
        l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lg[j]), wl));
        if (lane == wl) u[j] = 0ull;
        found = true;
      }
    }
    idx[k] = found ? e : 0;
    lg_sel[k] = l;
  }
}

// Score route of one row given its keys and logits (lane layout of
// select_topk): indices by select_topk, weights the unbiased sigmoids of the
// chosen logits over their sum.
__device__ __forceinline__ RowRoute score_route_keys(const double (&key)[4], const float (&lg)[4], int E, int K) {
  RowRoute rr;
  rr.flags = 0;
  float ls[kMaxTopK];
  select_topk(key, lg, E, K, rr.idx, ls);
  double s[kMaxTopK], tot = 0.0;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    s[k] = (k < K) ? sigmoid_f64(ls[k]) : 0.0;
    tot += s[k];
  }
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    rr.valid[k] = k < K;
    rr.w[k] = (k < K) ? (float)(s[k] / tot) : 0.0f;
  }
  return rr;
}

// Hash route of one row: the table row of the token id in column order,
// weighted by the renormalised sigmoids of those experts' logits.  A token
// id outside [0, table_rows) masks the whole row (indices -1); an entry
// outside [0, E) masks its slot (raw entry kept).
__device__ __forceinline__ RowRoute hash_route_row(const float* __restrict__ logits, int E, int K,
                                                   const int32_t* __restrict__ table, int64_t table_rows,
                                                   int32_t token) {
  RowRoute rr;
  rr.flags = 0;
  const bool tok_ok = token >= 0 && (int64_t)token < table_rows;
  double s[kMaxTopK];
  double tot = 0.0;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k >= K) {
      rr.idx[k] = -1;
      rr.valid[k] = false;
      s[k] = 0.0;
      continue;
    }
    const int e = tok_ok ? table[(int64_t)token * K + k] : -1;
    const bool ok = tok_ok && e >= 0 && e < E;
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

// Hash route of one row whose logits are held in the select_topk lane
// layout (lane l: experts l, l+64, l+128, l+192); same result as
// hash_route_row.
__device__ __forceinline__ RowRoute hash_route_lanes(const float (&lg)[4], int E, int K,
                                                     const int32_t* __restrict__ table, int64_t table_rows,
                                                     int32_t token) {
  RowRoute rr;
  rr.flags = 0;
  const bool tok_ok = token >= 0 && (int64_t)token < table_rows;
  double s[kMaxTopK];
  double tot = 0.0;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k >= K) {
      rr.idx[k] = -1;
      rr.valid[k] = false;
      s[k] = 0.0;
      continue;
    }
    const int e = tok_ok ? table[(int64_t)token * K + k] : -1;
    const bool ok = tok_ok && e >= 0 && e < E;
    rr.idx[k] = e;
    rr.valid[k] = ok;
    float l = 0.f;
    if (ok) {
      const int j = e / kWave, src = e % kWave;
      const float v = j == 0 ? lg[0] : j == 1 ? lg[1] : j == 2 ? lg[2] : lg[3];
      l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
    }
    s[k] = ok ? sigmoid_f64(l) : 0.0;
    tot += s[k];
    if (tok_ok && !ok) rr.flags |= MOE_FLAG_BAD_TABLE_ENTRY;
  }
  if (!tok_ok) rr.flags |= MOE_FLAG_BAD_TOKEN;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) rr.w[k] = (rr.valid[k] && tot > 0.0) ? (float)(s[k] / tot) : 0.0f;
  return rr;
}

// Routes one row with one wavefront from its f32 logits (keys computed here);
// every lane returns the same result.
__device__ __forceinline__ RowRoute route_row(const float* __restrict__ logits, int E, int K, int layer_kind,
                                              const float* __restrict__ bias, const int32_t* __restrict__ table,
                                              int64_t table_rows, int32_t token) {
  if (layer_kind == MOE_LAYER_HASH) return hash_route_row(logits, E, K, table, table_rows, token);
  const int lane = threadIdx.x & (kWave - 1);
  double key[4];
  float lg[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    lg[j] = (e < E) ? logits[e] : 0.f;
    key[j] = (e < E) ? score_key(lg[j], bias[e]) : 0.0;
  }
  return score_route_keys(key, lg, E, K);
}

}  // namespace moe
