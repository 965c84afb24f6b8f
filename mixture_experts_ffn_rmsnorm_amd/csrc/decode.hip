// Decode path (1..4 rows): the layer is a stream of expert weights read once
// from HBM, so every projection is a wavefront GEMV with f32 activations
// held in LDS and bf16 weights widened in registers.
//
//   k_dec_router_shared  RMSNorm + router logits (one expert per wave) and,
//                        in the same grid, the shared expert's gate/up +
//                        SwiGLU (it needs no routing)
//   k_dec_gateup         routing prologue (top-k or hash, distinct experts
//                        of the batch), then gate/up + SwiGLU of the routed
//                        experts, one (expert, 16 inter rows) tile per block
//   k_dec_down           down projections of routed + shared experts with
//                        the weighted reduce fused: each block owns 16 output
//                        columns and sums every expert's contribution in a
//                        fixed order, so no atomics and bitwise-stable output
//
// Stage order follows forward_ffn_rows on the hf2q ffn_forward.rs page
// (rms_norm -> MoE gate -> route -> sanitize -> routed/shared gate, up ->
// swiglu -> routed/shared down -> weighted reduce).
#include "device.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 16;  // weight rows per block for gate/up (per matrix) and down

// Per-lane partial dot products of NW bf16 weight rows against up to 4
// activation rows (f32, LDS or global).  Lane l covers 8 consecutive
// columns of every 512-column chunk; when LEN is not a multiple of 512 the
// lanes past the end of the last chunk sit it out.
template <int NW, int LEN>
__device__ __forceinline__ void wave_gemv(const uint16_t* const (&w)[NW], const float* const (&xr)[4], int nr,
                                          float (&acc)[NW][4]) {
  static_assert(LEN % 256 == 0, "row length must be a multiple of 256");
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int c = 0; c < LEN; c += 512) {
    if (LEN % 512 != 0 && c + lane * 8 >= LEN) break;
    uint4 q[NW];
#pragma unroll
    for (int n = 0; n < NW; ++n) q[n] = load_stream(w[n] + c + lane * 8);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < nr) {
        const float4* xp = (const float4*)(xr[r] + c + lane * 8);
        const float4 a = xp[0], b = xp[1];
#pragma unroll
        for (int n = 0; n < NW; ++n) {
          float f[8];
          unpack8(q[n], f);
          float s = acc[n][r];
          s = fmaf(f[0], a.x, s); s = fmaf(f[1], a.y, s);
          s = fmaf(f[2], a.z, s); s = fmaf(f[3], a.w, s);
          s = fmaf(f[4], b.x, s); s = fmaf(f[5], b.y, s);
          s = fmaf(f[6], b.z, s); s = fmaf(f[7], b.w, s);
          acc[n][r] = s;
        }
      }
    }
  }
}

// RMSNorm of R (<= 4) rows into LDS: xs[r*H + j] = x[r,j] * (mean x^2 + eps)^-1/2 * g[j].
// The first floats of xs double as the cross-wave reduction scratch.
template <int H>
__device__ __forceinline__ void norm_rows_to_lds(const float* __restrict__ x, const float* __restrict__ g, int R,
                                                 float eps, float* xs) {
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  constexpr int V = H / 4;  // float4 per row
  for (int r = 0; r < R; ++r) {
    float ss = 0.f;
    for (int i = t; i < V; i += kThreads) {
      float4 v = ((const float4*)(x + (int64_t)r * H))[i];
      ss = fmaf(v.x, v.x, ss); ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss); ss = fmaf(v.w, v.w, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) xs[wv * kDecodeMaxRows + r] = ss;
  }
  __syncthreads();
  float rs[kDecodeMaxRows];
#pragma unroll
  for (int r = 0; r < kDecodeMaxRows; ++r) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) tot += xs[w * kDecodeMaxRows + r];
    rs[r] = 1.0f / sqrtf(tot / (float)H + eps);
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kDecodeMaxRows; ++r) {
    if (r >= R) break;
    for (int i = t; i < V; i += kThreads) {
      float4 v = ((const float4*)(x + (int64_t)r * H))[i];
      float4 gg = ((const float4*)g)[i];
      float4 o;
      o.x = v.x * rs[r] * gg.x; o.y = v.y * rs[r] * gg.y; o.z = v.z * rs[r] * gg.z; o.w = v.w * rs[r] * gg.w;
      ((float4*)(xs + r * H))[i] = o;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Router logits + shared-expert gate/up.  Blocks [0, nrb) compute logits for
// 4 experts each (one per wave); blocks [nrb, nrb + I/16) compute 16 rows of
// the shared expert's SwiGLU output for every batch row.
template <int H, int I>
__global__ __launch_bounds__(kThreads) void k_dec_router_shared(const FwdArgs a) {
  extern __shared__ float xs[];  // [R][H]
  const int R = a.R;
  norm_rows_to_lds<H>(a.x, a.norm_w, R, a.eps, xs);
  const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int nrb = (a.E + 3) / 4;
  if (blockIdx.x == 0) {  // publish xn for the routed gate/up kernel
    for (int i = threadIdx.x; i < R * H / 4; i += kThreads) ((float4*)a.xn32)[i] = ((const float4*)xs)[i];
  }
  const float* xr[4] = {xs, xs + (R > 1 ? H : 0), xs + (R > 2 ? 2 * H : 0), xs + (R > 3 ? 3 * H : 0)};
  if ((int)blockIdx.x < nrb) {
    const int e = blockIdx.x * 4 + wv;
    if (e >= a.E) return;
    const uint16_t* w[1] = {a.router + (int64_t)e * H};
    float acc[1][4] = {};
    wave_gemv<1, H>(w, xr, R, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < R) {
        float v = wave_sum(acc[0][r]);
        if (lane == 0) a.logits[(int64_t)r * a.E + e] = v;
      }
    }
    return;
  }
  const int i0 = (blockIdx.x - nrb) * kTileRows + wv * 4;
  const uint16_t* w[8];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    w[n] = a.gate_sh + (int64_t)(i0 + n) * H;
    w[4 + n] = a.up_sh + (int64_t)(i0 + n) * H;
  }
  float acc[8][4] = {};
  wave_gemv<8, H>(w, xr, R, acc);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r < R) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        float g = wave_sum(acc[n][r]);
        float u = wave_sum(acc[4 + n][r]);
        if (lane == 0) a.h32[(int64_t)(kDecodeMaxSlots + r) * I + i0 + n] = swiglu_f32(g, u);
      }
    }
  }
}

// Distinct (expert, row) pairs of the batch, grouped by expert (ascending),
// rows ascending inside a group; duplicate slots of one row (possible only
// with a malformed hash table) merge by summing their weights.  Runs on
// wave 0; inputs in LDS.
__device__ void build_plan(const int* s_idx, const float* s_w, const unsigned char* s_valid, int R, int K, int E,
                           DecodePlan* P) {
  const int lane = threadIdx.x & (kWave - 1);
  const int S = R * K;
  int e = -1, r = 0;
  float w = 0.f;
  bool v = false;
  if (lane < S) {
    r = lane / K;
    e = s_idx[lane];
    w = s_w[lane];
    v = s_valid[lane] && e >= 0 && e < E;
  }
  const int kNone = 0x7fffffff;
  const int key = v ? e * 8 + r : kNone;
  bool first = v;
  float wsum = 0.f;
  for (int t = 0; t < S; ++t) {
    int kt = __shfl(key, t, kWave);
    float wt = __shfl(w, t, kWave);
    if (v && kt == key) {
      wsum += wt;
      if (t < lane) first = false;
    }
  }
  int pos = 0, gidx = 0;
  bool efirst = first;
  for (int t = 0; t < S; ++t) {
    int ft = __shfl((int)first, t, kWave);
    int kt = __shfl(key, t, kWave);
    if (ft && kt < key) ++pos;
    if (ft && (kt >> 3) == (key >> 3) && kt < key) efirst = false;
  }
  for (int t = 0; t < S; ++t) {
    int eft = __shfl((int)efirst, t, kWave);
    int kt = __shfl(key, t, kWave);
    if (eft && (kt >> 3) < (key >> 3)) ++gidx;
  }
  const int ngroups = __popcll(__ballot(efirst));
  const int nentries = __popcll(__ballot(first));
  if (first) {
    P->entry_row[pos] = r;
    P->entry_w[pos] = wsum;
  }
  if (efirst) {
    P->group_expert[gidx] = e;
    P->group_begin[gidx] = pos;
  }
  if (lane == 0) {
    P->ngroups = ngroups;
    P->nentries = nentries;
    P->group_begin[ngroups] = nentries;
  }
}

// ---------------------------------------------------------------------------
// Routing prologue + routed gate/up + SwiGLU.  grid = (I/16, max groups).
template <int H, int I>
__global__ __launch_bounds__(kThreads) void k_dec_gateup(const FwdArgs a) {
  __shared__ int s_idx[kDecodeMaxSlots];
  __shared__ float s_w[kDecodeMaxSlots];
  __shared__ unsigned char s_valid[kDecodeMaxSlots];
  __shared__ uint32_t s_flags[kDecodeMaxRows];
  __shared__ DecodePlan P;
  const int R = a.R, K = a.K;
  const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  if (wv < R) {
    const int32_t tok = (a.layer_kind == MOE_LAYER_HASH) ? a.token_ids[wv] : 0;
    RowRoute rr = route_row(a.logits + (int64_t)wv * a.E, a.E, K, a.layer_kind, a.bias, a.table, a.table_rows, tok);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k) {
        if (k < K) {
          s_idx[wv * K + k] = rr.idx[k];
          s_w[wv * K + k] = rr.w[k];
          s_valid[wv * K + k] = rr.valid[k];
        }
      }
      s_flags[wv] = rr.flags;
    }
  }
  __syncthreads();
  if (wv == 0) build_plan(s_idx, s_w, s_valid, R, K, a.E, &P);
  __syncthreads();
  const int u = blockIdx.y;
  if (blockIdx.x == 0 && u == 0) {  // publish routing, plan and status once
    for (int s = threadIdx.x; s < R * K; s += kThreads) {
      a.idx[s] = s_idx[s];
      a.wts[s] = s_w[s];
    }
    if (threadIdx.x < R) a.rowflags[threadIdx.x] = s_flags[threadIdx.x];
    if (threadIdx.x == 0) {
      uint32_t f = 0;
      for (int r = 0; r < R; ++r) f |= s_flags[r];
      a.status[0] = f;
    }
    const int* src = (const int*)&P;
    int* dst = (int*)a.plan;
    for (int i = threadIdx.x; i < (int)(sizeof(DecodePlan) / 4); i += kThreads) dst[i] = src[i];
  }
  if (u >= P.ngroups) return;
  const int e = P.group_expert[u];
  const int b = P.group_begin[u], nr = P.group_begin[u + 1] - b;
  // activations of this group's rows straight from xn32 (L2-resident)
  const float* xr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) xr[j] = a.xn32 + (int64_t)P.entry_row[b + (j < nr ? j : 0)] * H;
  const int i0 = blockIdx.x * kTileRows + wv * 4;
  const uint16_t* w[8];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    w[n] = a.gate + ((int64_t)e * I + i0 + n) * H;
    w[4 + n] = a.up + ((int64_t)e * I + i0 + n) * H;
  }
  float acc[8][4] = {};
  wave_gemv<8, H>(w, xr, nr, acc);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < nr) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        float g = wave_sum(acc[n][j]);
        float uu = wave_sum(acc[4 + n][j]);
        if (lane == 0) a.h32[(int64_t)(b + j) * I + i0 + n] = swiglu_f32(g, uu);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Down projections + weighted reduce.  grid = H/16; each wave owns 4 output
// columns and, per lane, accumulates weight * partial dot over every group
// (routed experts in ascending id, then the shared expert with weight 1),
// reducing across the wave once at the end.
template <int H, int I>
__global__ __launch_bounds__(kThreads) void k_dec_down(const FwdArgs a) {
  __shared__ DecodePlan P;
  {
    const int* src = (const int*)a.plan;
    int* dst = (int*)&P;
    for (int i = threadIdx.x; i < (int)(sizeof(DecodePlan) / 4); i += kThreads) dst[i] = src[i];
  }
  __syncthreads();
  const int R = a.R;
  const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int h0 = blockIdx.x * kTileRows + wv * 4;
  float acc[4][4] = {};
  const int ng = P.ngroups;
  for (int g = 0; g <= ng; ++g) {
    const bool shared = g == ng;
    const uint16_t* wbase = shared ? a.down_sh : a.down + (int64_t)P.group_expert[g] * H * I;
    const int b = shared ? 0 : P.group_begin[g];
    const int nr = shared ? R : P.group_begin[g + 1] - b;
    const uint16_t* w[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) w[n] = wbase + (int64_t)(h0 + n) * I;
    const float* xr[4];
    int rowj[4];
    float wj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int jj = j < nr ? j : 0;
      xr[j] = a.h32 + (int64_t)(shared ? kDecodeMaxSlots + jj : b + jj) * I;
      rowj[j] = shared ? jj : P.entry_row[b + jj];
      wj[j] = shared ? 1.0f : P.entry_w[b + jj];
    }
    float p[4][4] = {};
    wave_gemv<4, I>(w, xr, nr, p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < nr) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float sc = (rr == rowj[j]) ? wj[j] : 0.0f;
#pragma unroll
          for (int n = 0; n < 4; ++n) acc[n][rr] = fmaf(sc, p[n][j], acc[n][rr]);
        }
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    if (rr < R) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        float v = wave_sum(acc[n][rr]);
        if (lane == 0) a.out[(int64_t)rr * H + h0 + n] = v;
      }
    }
  }
}

template <int H, int I>
hipError_t run_decode_t(const FwdArgs& a, hipStream_t s) {
  FwdArgs args = a;
  const int nrb = (a.E + 3) / 4;
  hipError_t err = launch("dec_router_shared", (const void*)k_dec_router_shared<H, I>,
                          dim3(nrb + I / kTileRows), dim3(kThreads), (size_t)a.R * H * 4, s, &args);
  if (err != hipSuccess) return err;
  const int gmax = a.R * a.K < a.E ? a.R * a.K : a.E;
  err = launch("dec_gateup", (const void*)k_dec_gateup<H, I>, dim3(I / kTileRows, gmax), dim3(kThreads), 0, s,
               &args);
  if (err != hipSuccess) return err;
  return launch("dec_down_reduce", (const void*)k_dec_down<H, I>, dim3(H / kTileRows), dim3(kThreads), 0, s,
                &args);
}

}  // namespace

hipError_t run_decode(const FwdArgs& a, hipStream_t s) {
  if (a.H == 4096 && a.I == 2048) return run_decode_t<4096, 2048>(a, s);
  if (a.H == 512 && a.I == 256) return run_decode_t<512, 256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
