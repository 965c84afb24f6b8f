// Hyper-connection wrapper around the FFN layer.  forward_ffn_rows on the
// hf2q ffn_forward.rs page keeps the residual as hc streams, F32
// [rows, hc, hidden]; before the FFN it normalises each row's flattened
// state without a scale (rms_norm_no_scale_f32), multiplies it by
// hc_ffn_fn into (2 + hc) * hc mixes, splits those into pre / post / comb
// maps (dispatch_hc_split_sinkhorn) and mixes the streams into the FFN
// input (dispatch_hc_pre); after it, dispatch_hc_post builds the new state.
// The split, pre and post arithmetic is the reading stated in moe_ffn.h.
//
//   k_hc_mix   1-4 rows: one block per slice of 1024 flattened inputs: the
//              slice's dot products with every hc_fn row and its sum of
//              squares on the vector ALUs, then wave-wide sums; the decode
//              head adds the slices and splits (decode.hip)
//   k_hc_mix_mfma  more rows: one block per (32-row tile, slice): the same
//              dot products as one 32 x 32 tile of bf16 MFMAs, the state
//              split exactly into three bf16 terms
//   k_hc_pre   (more than 4 rows) per (row, hidden chunk): the row's slices
//              added in order, normalised and split (hc_split.h), then FFN
//              input = sum_i pre_i * state_i
//   k_hc_post  new_j = post_j * ffn_output + sum_i comb[j][i] * state_i
//              (more than 4 rows; with 1-4 the decode reduce does it)
//
// Everything is f32 with sums in a fixed order (bitwise reproducible).
#include "device.h"
#include "hc_split.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kHcThreads = 256;
constexpr int kHcWaves = kHcThreads / kWave;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// FFN input of row r (maps in LDS) for hidden values h .. h+3
template <int HC>
__device__ __forceinline__ void pre_mix(const HcArgs& a, int64_t r, const float* map, int h) {
  const float* st = a.state + r * HC * a.H + h;
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < HC; ++i) {
    const float p = map[i];
    const float4 s = *(const float4*)(st + (int64_t)i * a.H);
    x.x = fmaf(p, s.x, x.x); x.y = fmaf(p, s.y, x.y); x.z = fmaf(p, s.z, x.z); x.w = fmaf(p, s.w, x.w);
  }
  *(float4*)(a.ffn_in + r * a.H + h) = x;
}

template <int HC>
__global__ __launch_bounds__(kHcThreads) void k_hc_mix(const HcArgs a) {
  constexpr int MW = (2 + HC) * HC, V = MW + 1;  // mixes, then the sum of squares
  const int tile = blockIdx.x, sl = blockIdx.y;
  const int t = threadIdx.x, wv = t / kWave, lane = t % kWave;
  const int64_t r0 = (int64_t)tile * kHcRows;
  const int nr = a.R - r0 < kHcRows ? (int)(a.R - r0) : kHcRows;
  const int K = HC * a.H;
  const int kend = (sl + 1) * a.slice_k < K ? (sl + 1) * a.slice_k : K;

  float acc[kHcRows][V];
#pragma unroll
  for (int r = 0; r < kHcRows; ++r)
#pragma unroll
    for (int m = 0; m < V; ++m) acc[r][m] = 0.f;
  // the thread's pieces k, k + 4 * threads, ... of the slice, in order
#pragma unroll 1
  for (int k = sl * a.slice_k + 4 * t; k < kend; k += 4 * kHcThreads) {  // K is a multiple of 4
    float w[MW][4];
#pragma unroll
    for (int m = 0; m < MW; ++m) {
      const uint2 q = *(const uint2*)(a.fn + (int64_t)m * K + k);
      w[m][0] = bf16lo(q.x); w[m][1] = bf16hi(q.x); w[m][2] = bf16lo(q.y); w[m][3] = bf16hi(q.y);
    }
#pragma unroll
    for (int r = 0; r < kHcRows; ++r) {
      if (r < nr) {
        const float4 s = *(const float4*)(a.state + (r0 + r) * K + k);
        acc[r][MW] = fmaf(s.x, s.x, fmaf(s.y, s.y, fmaf(s.z, s.z, fmaf(s.w, s.w, acc[r][MW]))));
#pragma unroll
        for (int m = 0; m < MW; ++m)
          acc[r][m] = fmaf(s.x, w[m][0], fmaf(s.y, w[m][1], fmaf(s.z, w[m][2], fmaf(s.w, w[m][3], acc[r][m]))));
      }
    }
  }
  // block sums: each 16-lane row of each wave by DPP moves (no lane reads),
  // then the block's rows in order
  constexpr int kRows16 = kHcWaves * (kWave / 16);
  __shared__ float s_part[kRows16][kHcRows * V];
#pragma unroll
  for (int r = 0; r < kHcRows; ++r) {
    if (r < nr) {  // block-uniform
#pragma unroll
      for (int m = 0; m < V; ++m) {
        const float v = row16_sum(acc[r][m]);
        if ((lane & 15) == 0) s_part[wv * (kWave / 16) + lane / 16][r * V + m] = v;
      }
    }
  }
  __syncthreads();
  float* part = a.partial + ((int64_t)tile * a.slices + sl) * (kHcRows * V);
  for (int q = t; q < nr * V; q += kHcThreads) {
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kRows16; ++w2) v += s_part[w2][q];
    part[q] = v;  // read by the next launch
  }
}

// More than 4 rows, on the matrix cores: one block per (32-row tile, slice
// of slice_k flattened inputs), its 4 waves taking every 4th 16-input k-step
// of the slice.  The slice's dot products are one 32 x 32 tile of
// v_mfma_f32_32x32x16_bf16 (mix columns past (2+hc)*hc are zero): the f32
// state is split exactly into three bf16 terms, hi + mid + lo (24
// significant bits; each difference is exact in f32), each multiplied by
// the bf16 hc_fn values as they are, f32 accumulation.  Lane l carries row
// l % 32 of the state and mix l % 32 of hc_fn, inputs 8 * (l / 32) .. +7
// of each k-step (the operand layout of the instruction); the sum of
// squares comes from the same loads on the vector ALUs.  The block adds its
// waves in order and leaves one partial per row; rows past the batch read
// its last row and are never read back.
template <int HC>
__global__ __launch_bounds__(kHcThreads) void k_hc_mix_mfma(const HcArgs a) {
  constexpr int MW = (2 + HC) * HC, V = MW + 1;
  static_assert(MW <= 32, "the mixes fit one 32-column tile");
  const int tile = blockIdx.x, sl = blockIdx.y;
  const int t = threadIdx.x, wv = t / kWave, lane = t % kWave;
  const int K = HC * a.H;
  const int rl = lane % 32, half = lane / 32;
  const int64_t r0 = (int64_t)tile * kHcMfmaRows;
  const int64_t rg = r0 + rl < a.R ? r0 + rl : a.R - 1;
  const float* srow = a.state + rg * K + 8 * half;
  const bool mcol = rl < MW;
  const uint16_t* frow = a.fn + (int64_t)(mcol ? rl : 0) * K + 8 * half;
  const int kbeg = sl * a.slice_k;
  const int kend = kbeg + a.slice_k < K ? kbeg + a.slice_k : K;
  floatx16 acc = {};
  float ss = 0.f;
#pragma unroll 4
  for (int k0 = kbeg + wv * 16; k0 + 16 <= kend; k0 += kHcWaves * 16) {
    const float4 x0 = *(const float4*)(srow + k0), x1 = *(const float4*)(srow + k0 + 4);
    const uint4 wq = mcol ? *(const uint4*)(frow + k0) : make_uint4(0u, 0u, 0u, 0u);
    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    bf16x8 hi, mid, lo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 h = (__bf16)x[i];
      const float d1 = x[i] - (float)h;
      const __bf16 m = (__bf16)d1;
      hi[i] = h;
      mid[i] = m;
      lo[i] = (__bf16)(d1 - (float)m);
      ss = fmaf(x[i], x[i], ss);
    }
    const bf16x8 w = __builtin_bit_cast(bf16x8, wq);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, w, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mid, w, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, w, acc, 0, 0, 0);
  }
  // lane l holds mix l % 32 of rows 8 (v / 4) + 4 (l / 32) + v % 4
  __shared__ float s_acc[kHcWaves][kHcMfmaRows][MW];
  __shared__ float s_ss[kHcWaves][2][kHcMfmaRows];
  if (mcol)
#pragma unroll
    for (int v = 0; v < 16; ++v) s_acc[wv][8 * (v / 4) + 4 * half + (v % 4)][rl] = acc[v];
  s_ss[wv][half][rl] = ss;
  __syncthreads();
  float* part = a.partial + ((int64_t)tile * a.slices + sl) * (kHcMfmaRows * V);
  for (int q = t; q < kHcMfmaRows * V; q += kHcThreads) {
    const int rr = q / V, m = q % V;
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kHcWaves; ++w2) v += m < MW ? s_acc[w2][rr][m] : s_ss[w2][0][rr] + s_ss[w2][1][rr];
    part[q] = v;  // read by the next launch
  }
}

// More than 4 rows: one row's split, then its FFN input for 4 hidden values
// per thread.  Lane m of wave 0 adds mix m over the row's slices in order;
// every hidden chunk of a row repeats the split; chunk 0 stores the mixes
// and maps.
template <int HC>
__global__ __launch_bounds__(kHcThreads) void k_hc_pre(const HcArgs a) {
  constexpr int MW = (2 + HC) * HC, V = MW + 1;
  const int64_t r = blockIdx.x;
  const int t = threadIdx.x;
  __shared__ float s_map[1][MW];
  __shared__ float s_sum[1][V];
  if (t < V) {  // mix t (t = MW: the sum of squares) over the slices, in order
    const int tr = a.tile_rows;
    const float* part = a.partial + (r / tr) * a.slices * (tr * V) + (r % tr) * V + t;
    float v = 0.f;
#pragma unroll 8
    for (int64_t s2 = 0; s2 < a.slices; ++s2) v += part[s2 * (tr * V)];
    s_sum[0][t] = v;
  }
  __syncthreads();
  if (t < kWave)
    hc_split_rows<HC>(&s_sum[0][0], V, 1, (float)(HC * a.H), a.eps, a.scale, a.base, a.iters, &s_map[0][0], MW,
                      blockIdx.y == 0 ? a.mixes + r * MW : nullptr);
  __syncthreads();
  if (blockIdx.y == 0)
    for (int m = t; m < MW; m += kHcThreads) a.maps[r * MW + m] = s_map[0][m];
  const int h = (blockIdx.y * kHcThreads + t) * 4;
  if (h < a.H) pre_mix<HC>(a, r, s_map[0], h);
}

// new state: 4 hidden values of every stream per thread
template <int HC>
__global__ __launch_bounds__(kHcThreads) void k_hc_post(const HcArgs a) {
  constexpr int MW = (2 + HC) * HC;
  const int64_t r = blockIdx.x;
  const int h = (blockIdx.y * kHcThreads + threadIdx.x) * 4;
  if (h >= a.H) return;
  const float* mp = a.maps + r * MW;
  float4 s[HC];
#pragma unroll
  for (int i = 0; i < HC; ++i) s[i] = *(const float4*)(a.state + (r * HC + i) * a.H + h);
  const float4 f = *(const float4*)(a.ffn_out + r * a.H + h);
#pragma unroll
  for (int j = 0; j < HC; ++j) {
    const float p = mp[HC + j];
    float4 o = make_float4(p * f.x, p * f.y, p * f.z, p * f.w);
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      const float c = mp[2 * HC + j * HC + i];
      o.x = fmaf(c, s[i].x, o.x); o.y = fmaf(c, s[i].y, o.y); o.z = fmaf(c, s[i].z, o.z); o.w = fmaf(c, s[i].w, o.w);
    }
    *(float4*)(a.out + (r * HC + j) * a.H + h) = o;
  }
}

template <int HC>
hipError_t run_hc_pre_t(const HcArgs& a, hipStream_t s) {
  HcArgs args = a;
  const bool small = a.R <= kHcRows;  // 1-4 rows: one tile on the vector ALUs; the decode head splits
  hipError_t err = launch("hc_mix", small ? (const void*)k_hc_mix<HC> : (const void*)k_hc_mix_mfma<HC>,
                          dim3((unsigned)((a.R + a.tile_rows - 1) / a.tile_rows), (unsigned)a.slices),
                          dim3(kHcThreads), 0, s, &args);
  if (err != hipSuccess || small) return err;
  return launch("hc_pre", (const void*)k_hc_pre<HC>, dim3(a.R, (a.H / 4 + kHcThreads - 1) / kHcThreads),
                dim3(kHcThreads), 0, s, &args);
}

template <int HC>
hipError_t run_hc_post_t(const HcArgs& a, hipStream_t s) {
  HcArgs args = a;
  return launch("hc_post", (const void*)k_hc_post<HC>, dim3(a.R, (a.H / 4 + kHcThreads - 1) / kHcThreads),
                dim3(kHcThreads), 0, s, &args);
}

}  // namespace

hipError_t run_hc_pre(const HcArgs& a, hipStream_t s) {
  switch (a.hc) {
    case 1: return run_hc_pre_t<1>(a, s);
    case 2: return run_hc_pre_t<2>(a, s);
    case 3: return run_hc_pre_t<3>(a, s);
    case 4: return run_hc_pre_t<4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t run_hc_post(const HcArgs& a, hipStream_t s) {
  switch (a.hc) {
    case 1: return run_hc_post_t<1>(a, s);
    case 2: return run_hc_post_t<2>(a, s);
    case 3: return run_hc_post_t<3>(a, s);
    case 4: return run_hc_post_t<4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
