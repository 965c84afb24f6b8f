// Decode path (1..4 rows).  The layer is a stream of expert weights read
// once from HBM: every projection is a wavefront GEMV whose f32 activations
// sit in LDS while bf16 weight rows stream through registers, each row read
// front to back with the next rows already requested (activation reads use
// the LDS counter, so they never wait behind the weight loads).
//
//   k_dec_head     router logits (+ float64 selection keys), the routing
//                  plan of distinct (expert, row) pairs, and the shared
//                  expert's gate/up + SwiGLU, whose streaming covers the
//                  router's latency
//   k_dec_gateup   the shared expert's down projection (first blocks), then
//                  routed gate/up + SwiGLU, one (expert, 16 inter rows) tile
//                  per block
//   k_dec_down     routed down projections for 16 or 32 hidden rows per block
//   k_dec_reduce   out = sum of weight * down + shared in a fixed order
//
// With one row the launches divide the work differently, and no workgroup
// ever waits for another:
//   k_dec_head<true>  router only; each router wave also stores its expert's
//                     selection key and float64 sigmoid
//   k_dec1_gateup     shared gate/up blocks, and routed gate/up blocks that
//                     each route the row from those keys before streaming
//   k_dec1_down       output-stationary down: each block streams 8 hidden
//                     rows of every matrix (the routed experts', then the
//                     shared one's) and forms those outputs itself
//
// Inside the hyper-connection wrapper (hc > 0) every head block also adds
// the mix launch's partial sums and splits them, forms each row from the
// streams while staging it, and the block forming the output writes the new
// streams.
//
// Stage order follows forward_ffn_rows on the hf2q ffn_forward.rs page
// (rms_norm -> MoE gate -> route -> sanitize -> routed/shared gate, up ->
// swiglu -> routed/shared down -> weighted reduce); the page's rows*top_k
// one-expert matvecs become one pass over the batch's distinct experts.
#include <type_traits>

#include "device.h"
#include "hc_split.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kGuRows = 16;     // inter rows per routed gate/up block (x2 matrices): 4 waves x 4
constexpr int kShRows = 8;      // inter rows per shared gate/up block: 4 waves x 2
// hidden rows per down block of two to four rows: 4 waves x 4 (bf16,
// 8-bit), 4 waves x 8 (4-bit, whose rows are a quarter of bf16's).  Four-row
// down launch, 16 / 32 / 8 rows per block: bf16 60.4 / 62.7 / 63.6 us,
// 8-bit 40.1 / 41.2 / 43.8 us, 4-bit 31.4 / 30.4 / 36.1 us.
template <int MX> constexpr int kDnRows = MX == 2 ? 32 : 16;
// hidden rows per shared-down block of the gate/up launch (4 waves x 4): its
// H/16 blocks give every compute unit one of them besides its routed blocks
constexpr int kSdRows = 16;
// Weight rows in flight per wave: two, multiplied as a pair (one LDS read
// of an activation value serves both weight rows).  Measured against one
// row at a time: bf16 one row 71.5-72.1 vs 72.9-73.9 us, four rows 209.6
// vs 213.6-216.0 us; 8-bit weights four rows 172.9 us with two rows in
// flight vs 177.7 us with four (four in flight without pairs: 83 us at one
// row).
template <int MX> constexpr int kNbuf = 2;
template <int MX> constexpr bool kPair = true;
// The one-row down launch keeps four rows (two pairs) in flight per wave
// through a fully unrolled stream: it has half as many waves per compute
// unit as the other launches (two blocks of 74 KB of LDS each).  Measured
// against two rows: down 21.0 vs 22.5 us (bf16), 14.5-15.2 vs 15.1-15.4 us
// (8-bit), 12.3-12.6 vs 12.7-12.9 us (4-bit).
constexpr int kNbuf1Down = 4;

// An expert matrix [out][LEN] in one of the weight formats MX: 0 bf16
// values; 1 block-scaled 8-bit values (E4M3 codes [out][LEN], one E8M0
// scale per 32 columns, [out][LEN/32]); 2 block-scaled 4-bit values (E2M1
// codes packed two per byte, [out][LEN/2], the same scales).  WRow is one
// row of it.
struct WMat {
  const void* w;
  const uint8_t* s;  // MX only
};
struct WRow {
  const void* w;
  const uint8_t* s;
};
template <int MX, int LEN>
__device__ __forceinline__ WRow wrow(const WMat& m, int64_t i) {
  if constexpr (MX) return WRow{(const uint8_t*)m.w + i * (MX == 2 ? LEN / 2 : LEN), m.s + i * (LEN / 32)};
  else return WRow{(const uint16_t*)m.w + i * LEN, nullptr};
}
// Expert e's matrix of `elems` values from the forward's arguments.
template <int MX>
__device__ __forceinline__ WMat expert_mat(const uint16_t* bf, const uint8_t* q, const uint8_t* s, int64_t e,
                                           int64_t elems) {
  if constexpr (MX) return WMat{q + e * (MX == 2 ? elems / 2 : elems), s + e * (elems / 32)};
  else return WMat{bf + e * elems, nullptr};
}

// E8M0 scale code -> f32: 2^(c-127) (the f32 exponent field itself for c in
// 1..254; 2^-127, a subnormal, for 0; NaN for 255).
__device__ __forceinline__ float e8m0_f32(uint32_t c) {
  return c == 0 ? __uint_as_float(0x00400000u) : (c == 255 ? __uint_as_float(0x7fc00000u) : __uint_as_float(c << 23));
}
// Eight E4M3 codes (little-endian bytes of q) -> eight floats, exactly.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void unpack8_e4m3(const uint2& q, float* f) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, true);
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y; f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}
// Eight E2M1 codes (the nibbles of q, lowest first) -> eight floats,
// exactly (v_cvt_scalef32_pk_f32_fp4 with scale 1 converts the two codes
// of one byte; each result pair is taken as one 64-bit value).
__device__ __forceinline__ void unpack8_e2m1(uint32_t q, float* f) {
  const uint64_t v0 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0));
  const uint64_t v1 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1));
  const uint64_t v2 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2));
  const uint64_t v3 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3));
  f[0] = __uint_as_float((uint32_t)v0); f[1] = __uint_as_float((uint32_t)(v0 >> 32));
  f[2] = __uint_as_float((uint32_t)v1); f[3] = __uint_as_float((uint32_t)(v1 >> 32));
  f[4] = __uint_as_float((uint32_t)v2); f[5] = __uint_as_float((uint32_t)(v2 >> 32));
  f[6] = __uint_as_float((uint32_t)v3); f[7] = __uint_as_float((uint32_t)(v3 >> 32));
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 load_stream8(const void* p) {
  const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t load_stream4(const void* p) { return __builtin_nontemporal_load((const uint32_t*)p); }

// f(std::integral_constant<int, K>{}) for K = B .. E-1, in order.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// One wavefront walks a sequence of whole weight rows (global) and dots each
// with up to 4 f32 activation rows in LDS (row r at act + r*LEN).  Each row
// is read front to back as contiguous wave loads (1 KiB for bf16, 512 B for
// 8-bit codes); NBUF rows are in flight (the next ones load while the
// current one is multiplied), which keeps the DRAM streams long.  Lane l
// covers 8 consecutive columns of every 512-column chunk; lanes past the end
// of a partial chunk (LEN not a multiple of 512) neither load nor add.  With
// MX the row's scale bytes come with one 4-byte load per lane, and chunk c's
// lane takes the scale of its 32-column block from the lane holding it
// (columns c*512 + 8l.. lie in block 16c + l/4, in scale dword 4c + r for
// the lanes of 16-lane row r = l/16): lane 16r + p loads scale dword 4p + r,
// so the dword a row needs for chunk c sits in its own lane c, broadcast
// within the row by a DPP move; the lane's 8-term partial of the chunk is
// multiplied by the scale (a power of two: exact) and added.
// rowsrc(j) gives row j (WRow); pre() runs once after the first NBUF rows
// are requested (staging the activations there overlaps it with the first
// weight fetch; it must end with a barrier if it fills LDS); sink(j, part)
// receives each lane's partial sums part[0..nr) of row j (reduce them with
// wave_sum); it must not store to global memory: loads and stores share one
// wait counter, and a store among the weight loads makes every later wait
// drain them all.
// With PAIR rows are multiplied two at a time, so each activation value read
// from LDS serves both (with several activation rows and half-size 8-bit
// weight rows the LDS reads, not the weight stream, bound the loop
// otherwise).  actof(j) gives row j's activations (stream_rows: the same for
// every row); with PAIR rows 2i and 2i + 1 must share them.
// MAXROWS 0: a rolled loop over groups of NBUF rows, nrows a positive
// multiple of NBUF.  MAXROWS > 0: nrows is any positive multiple of the
// pair size up to MAXROWS, each count its own fully unrolled stream.
template <int LEN, int NBUF, int MX, bool PAIR, int MAXROWS, class RowSrc, class ActOf, class Pre, class Sink>
__device__ __forceinline__ void stream_rows_by(int nrows, RowSrc rowsrc, ActOf actof, int nr, Pre pre, Sink sink) {
  constexpr bool TAIL = MAXROWS > 0;
  static_assert(LEN % 256 == 0, "row length must be a multiple of 256");
  static_assert(!PAIR || NBUF % 2 == 0, "pairs of rows in flight");
  constexpr int NCH = (LEN + 511) / 512;
  const int lane = threadIdx.x & (kWave - 1);
  const bool full = LEN % 512 == 0 || lane * 8 < LEN % 512;  // active in the last chunk
  using Chunk = typename std::conditional<MX == 2, uint32_t, typename std::conditional<MX == 1, uint2, uint4>::type>::type;
  Chunk q[NBUF][NCH];
  uint32_t sw[NBUF];  // MX: this lane's 4 scale bytes of the row (dword sdw)
  static_assert(!MX || NCH <= 16, "one scale dword per lane of a 16-lane row and chunk");
  const int sdw = 4 * (lane & 15) + (lane >> 4);
  auto load_row = [&](int b, int j) {
    const WRow src = rowsrc(j);
    if constexpr (MX == 2) {  // 4-bit codes: 4 bytes per lane and chunk
      const uint8_t* p = (const uint8_t*)src.w + lane * 4;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        if (c < NCH - 1 || full) q[b][c] = load_stream4(p + c * 256);
      sw[b] = sdw * 4 < LEN / 32 ? *(const uint32_t*)(src.s + sdw * 4) : 0u;
    } else if constexpr (MX) {
      const uint8_t* p = (const uint8_t*)src.w + lane * 8;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        if (c < NCH - 1 || full) q[b][c] = load_stream8(p + c * 512);
      sw[b] = sdw * 4 < LEN / 32 ? *(const uint32_t*)(src.s + sdw * 4) : 0u;
    } else {
      const uint16_t* p = (const uint16_t*)src.w + lane * 8;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        if (c < NCH - 1 || full) q[b][c] = load_stream(p + c * 512);
    }
  };
  // rows b .. b+NR-1 (NR = 1, or 2 with PAIR) against the activations
  auto dot_rows = [&](int b, int j, auto nr_c, float (&part)[2][4]) {
    constexpr int NR = decltype(nr_c)::value;
    const float* act = actof(j);
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[i][r] = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float sc[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        sc[i] = 1.f;
        if constexpr (MX) {  // every lane takes part in the broadcast
          const uint32_t w = row_bcast(sw[b + i], c);
          sc[i] = e8m0_f32((w >> (8 * ((lane >> 2) & 3))) & 255u);
        }
      }
      if (c < NCH - 1 || full) {
        float f[NR][8];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          if constexpr (MX == 2) unpack8_e2m1(q[b + i][c], f[i]);
          else if constexpr (MX) unpack8_e4m3(q[b + i][c], f[i]);
          else unpack8(q[b + i][c], f[i]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (r < nr) {
            const float4* xp = (const float4*)(act + r * LEN + c * 512 + lane * 8);
            const float4 u = xp[0], v = xp[1];
#pragma unroll
            for (int i = 0; i < NR; ++i) {
              float s = MX ? 0.f : part[i][r];
              s = fmaf(f[i][0], u.x, s); s = fmaf(f[i][1], u.y, s); s = fmaf(f[i][2], u.z, s); s = fmaf(f[i][3], u.w, s);
              s = fmaf(f[i][4], v.x, s); s = fmaf(f[i][5], v.y, s); s = fmaf(f[i][6], v.z, s); s = fmaf(f[i][7], v.w, s);
              part[i][r] = MX ? fmaf(sc[i], s, part[i][r]) : s;
            }
          }
        }
      }
    }
  };
  constexpr int STEP = PAIR ? 2 : 1;
  using StepC = std::integral_constant<int, STEP>;
#pragma unroll
  for (int b = 0; b < NBUF; ++b) load_row(b, TAIL && b >= nrows ? nrows - 1 : b);
  pre();
  if constexpr (!TAIL) {
    // Steady state: every row of the group has a successor NBUF rows on,
    // whose loads go out as soon as the row is multiplied.  The loads are
    // unconditional, so the compiler's wait for each chunk counts exactly
    // the loads issued after it, and NBUF rows stay in flight (a conditional
    // refill makes every wait assume it did not happen, and each wave then
    // also waits for the row it has just requested).
#pragma unroll 1
    for (int j0 = 0; j0 + NBUF < nrows; j0 += NBUF) {
#pragma unroll
      for (int b = 0; b < NBUF; b += STEP) {
        float part[2][4];
        dot_rows(b, j0 + b, StepC{}, part);
#pragma unroll
        for (int i = 0; i < STEP; ++i) load_row(b + i, j0 + b + i + NBUF);
#pragma unroll
        for (int i = 0; i < STEP; ++i) sink(j0 + b + i, part[i]);
      }
    }
    // last group: no further loads
#pragma unroll
    for (int b = 0; b < NBUF; b += STEP) {
      float part[2][4];
      dot_rows(b, nrows - NBUF + b, StepC{}, part);
#pragma unroll
      for (int i = 0; i < STEP; ++i) sink(nrows - NBUF + b + i, part[i]);
    }
  } else {
    // nrows (a multiple of STEP, at most MAXROWS) is dispatched to a fully
    // unrolled stream: every slot is a fixed set of registers, so no value
    // is copied between slots (a copy waits for every load in flight) and
    // each wait counts exactly the rows requested after its own; NBUF rows
    // stay in flight to the end.  The slots past nrows hold copies of its
    // last row, unused.
    static_for<1, MAXROWS / STEP + 1>([&](auto n_c) {
      constexpr int NROWS = decltype(n_c)::value * STEP;
      if (nrows != NROWS) return;
#pragma unroll
      for (int j = 0; j < NROWS; j += STEP) {
        float part[2][4];
        dot_rows(j % NBUF, j, StepC{}, part);
        // the refill may not move above the products, whose registers it reuses
        __builtin_amdgcn_sched_barrier(0);
        if (j + NBUF < NROWS)
#pragma unroll
          for (int i = 0; i < STEP; ++i) load_row((j + i) % NBUF, j + i + NBUF);
#pragma unroll
        for (int i = 0; i < STEP; ++i) sink(j + i, part[i]);
      }
    });
  }
}
template <int LEN, int NBUF, int MX, bool PAIR, class RowSrc, class Pre, class Sink>
__device__ __forceinline__ void stream_rows(int nrows, RowSrc rowsrc, const float* act, int nr, Pre pre, Sink sink) {
  stream_rows_by<LEN, NBUF, MX, PAIR, 0>(nrows, rowsrc, [act](int) { return act; }, nr, pre, sink);
}

// RMSNorm of R (<= 4) rows into LDS: xs[r*H + j] = x[r,j] * (mean x^2 + eps)^-1/2 * g[j].
// Every row's loads go out before the first reduction (one memory round
// trip for the batch, not one per row), and the values stay in registers
// for the scaled write.  The first floats of xs double as the cross-wave
// reduction scratch.  With the hyper-connection wrapper folded in (a.hc >
// 0) wave 0 first adds the mix launch's slice partials of each (row, mix)
// in slice order and splits them (hc_split.h); with `store_x` (block 0) the
// mixes and maps are stored.  Each row is then formed from the streams,
// x[r] = sum_i pre[r][i] * state[r][i] (i in order, from 0), and `store_x`
// stores it to a.hc_x.  With MAXR = 1 (the one-row head) the streams'
// values are requested with the partials, before the split, and wait in
// registers; with more rows they are requested after it.
template <int H, int MAXR = kDecodeMaxRows>
__device__ __forceinline__ void norm_rows_to_lds(const FwdArgs& a, bool store_x, float* xs) {
  const float* __restrict__ x = a.x;
  const float* __restrict__ g = a.norm_w;
  const int R = a.R;
  const float eps = a.eps;
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  constexpr int V = H / 4;                            // float4 per row
  constexpr int NPT = (V + kThreads - 1) / kThreads;  // float4 per thread and row
  float4 v[kDecodeMaxRows][NPT];
  float4 gg[NPT];  // the norm weight, requested with the rows
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int i = t + k * kThreads;
    gg[k] = i < V ? ((const float4*)g)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (a.hc > 0) {
    constexpr int MWX = (2 + kHcMax) * kHcMax;
    __shared__ float s_hsum[kHcRows][MWX + 1];
    __shared__ float s_hmap[kHcRows][MWX];
    const int hc = a.hc, mw = (2 + hc) * hc, mv = mw + 1;
    float4 sv[MAXR == 1 ? kHcMax : 1][NPT];  // one row: its streams, requested now
    if constexpr (MAXR == 1) {
#pragma unroll
      for (int i = 0; i < kHcMax; ++i)
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
          const int idx = t + k * kThreads;
          sv[i][k] = (i < hc && idx < V) ? ((const float4*)(a.hc_state + (int64_t)i * H))[idx]
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    if (wv == 0) {
      // (row, value) pair q = r * mv + m over the slices, in slice order
#pragma unroll
      for (int u = 0; u < 2; ++u) {  // R * mv <= 100 pairs
        const int q = lane + kWave * u;
        if (q < R * mv) {
          float sum = 0.f;
#pragma unroll 8
          for (int64_t s2 = 0; s2 < a.hc_slices; ++s2) sum += a.hc_partial[s2 * (kHcRows * mv) + q];
          s_hsum[q / mv][q % mv] = sum;
        }
      }
      __builtin_amdgcn_wave_barrier();
      hc_split_rows_n(hc, &s_hsum[0][0], MWX + 1, R, (float)(hc * H), eps, a.hc_scale, a.hc_base, a.hc_iters,
                      &s_hmap[0][0], MWX, store_x ? a.hc_mixes : nullptr);
    }
    __syncthreads();
    if (store_x)
      for (int q = t; q < R * mw; q += kThreads) a.hc_maps[q] = s_hmap[q / mw][q % mw];
    float p[kDecodeMaxRows][kHcMax];
#pragma unroll
    for (int r = 0; r < kDecodeMaxRows; ++r)
#pragma unroll
      for (int i = 0; i < kHcMax; ++i) p[r][i] = (r < R && i < hc) ? s_hmap[r][i] : 0.f;
#pragma unroll
    for (int r = 0; r < MAXR; ++r)
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        const int idx = t + k * kThreads;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < R && idx < V) {
#pragma unroll
          for (int i = 0; i < kHcMax; ++i) {
            if (i < hc) {
              const float4 s = MAXR == 1 ? sv[MAXR == 1 ? i : 0][k]
                                         : ((const float4*)(a.hc_state + ((int64_t)r * hc + i) * H))[idx];
              o.x = fmaf(p[r][i], s.x, o.x); o.y = fmaf(p[r][i], s.y, o.y);
              o.z = fmaf(p[r][i], s.z, o.z); o.w = fmaf(p[r][i], s.w, o.w);
            }
          }
          if (store_x) ((float4*)(a.hc_x + (int64_t)r * H))[idx] = o;
        }
        v[r][k] = o;
      }
#pragma unroll
    for (int r = MAXR; r < kDecodeMaxRows; ++r)
#pragma unroll
      for (int k = 0; k < NPT; ++k) v[r][k] = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
#pragma unroll
    for (int r = 0; r < kDecodeMaxRows; ++r)
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        const int i = t + k * kThreads;
        v[r][k] = (r < R && i < V) ? ((const float4*)(x + (int64_t)r * H))[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
  }
#pragma unroll
  for (int r = 0; r < kDecodeMaxRows; ++r) {
    if (r < R) {
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        ss = fmaf(v[r][k].x, v[r][k].x, ss); ss = fmaf(v[r][k].y, v[r][k].y, ss);
        ss = fmaf(v[r][k].z, v[r][k].z, ss); ss = fmaf(v[r][k].w, v[r][k].w, ss);
      }
      ss = wave_sum(ss);
      if (lane == 0) xs[wv * kDecodeMaxRows + r] = ss;
    }
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
  for (int k = 0; k < NPT; ++k) {
    const int i = t + k * kThreads;
    if (i < V) {
#pragma unroll
      for (int r = 0; r < kDecodeMaxRows; ++r) {
        if (r < R) {
          float4 o;
          o.x = v[r][k].x * rs[r] * gg[k].x; o.y = v[r][k].y * rs[r] * gg[k].y;
          o.z = v[r][k].z * rs[r] * gg[k].z; o.w = v[r][k].w * rs[r] * gg[k].w;
          ((float4*)(xs + r * H))[i] = o;
        }
      }
    }
  }
  __syncthreads();
}

// Copy `nr` rows of LEN floats (global rows src[j]) into LDS rows dst + j*LEN,
// two rows per memory round trip (both rows' loads issued before their
// stores).
template <int LEN>
__device__ __forceinline__ void stage_rows(float* dst, const float* const (&src)[4], int nr) {
  constexpr int V = LEN / 4;
  constexpr int NPT = (V + kThreads - 1) / kThreads;
#pragma unroll
  for (int j0 = 0; j0 < kDecodeMaxRows; j0 += 2) {
    if (j0 >= nr) break;
    float4 v[2][NPT];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        const int i = threadIdx.x + k * kThreads;
        v[j][k] = (j0 + j < nr && i < V) ? ((const float4*)src[j0 + j])[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        const int i = threadIdx.x + k * kThreads;
        if (j0 + j < nr && i < V) ((float4*)(dst + (j0 + j) * LEN))[i] = v[j][k];
      }
  }
  __syncthreads();
}

// Gate/up + SwiGLU of PAIRS inter rows of one expert for the `nr` activation
// rows in LDS: tile x of `tiles` takes rows x, x + tiles, x + 2*tiles, ...,
// so the blocks working on one expert at the same time read neighbouring
// rows; wave w streams gate_i then up_i for every fourth of them.  h32 rows
// hout..hout+nr-1 receive silu(gate . x) * (up . x).
template <int H, int I, int PAIRS, int NBUF, int MX, bool PAIR, class Pre>
__device__ __forceinline__ void gateup_tile(const WMat& gm, const WMat& um, const float* xs, int nr, int x, int tiles,
                                            float* h32, int hout, Pre pre) {
  constexpr int W = kThreads / kWave, PPW = PAIRS / W;  // pairs per wave
  static_assert(PPW * 4 <= kWave, "one lane per result");
  __shared__ float s_res[W * PPW * 4];  // results wait here until the stream ends
  const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  float* res = s_res + wv * PPW * 4;
  float g[4];
  auto row_of = [&](int j) { return x + (wv + (j >> 1) * W) * tiles; };
  auto rowsrc = [&](int j) { return wrow<MX, H>((j & 1) ? um : gm, row_of(j)); };
  auto sink = [&](int j, const float (&part)[4]) {
    if (!(j & 1)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) g[r] = part[r];
      return;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < nr) {
        const float gs = wave_sum(g[r]);
        const float us = wave_sum(part[r]);
        if (lane == 0) res[(j >> 1) * 4 + r] = swiglu_f32(gs, us);
      }
    }
  };
  static_assert((2 * PPW) % NBUF == 0, "whole groups of rows in flight");
  stream_rows<H, NBUF, MX, PAIR>(2 * PPW, rowsrc, xs, nr, pre, sink);
  const int p = lane >> 2, r = lane & 3;
  if (p < PPW && r < nr) store_wt(&h32[(int64_t)(hout + r) * I + row_of(2 * p)], res[lane]);
}

// Distinct (expert, row) pairs of the batch, grouped by expert (ascending),
// rows ascending inside a group; duplicate slots of one row (possible only
// with a malformed hash table) merge by summing their weights in slot order.
// Runs on wave 0 with lane s holding slot s: the slots' keys and weights go
// through LDS once, and every lane then walks them 8 at a time (same-address
// broadcast reads) comparing in registers.  Loops, not straight-line code:
// this runs once per call, on a cold instruction cache.
__device__ __forceinline__ void build_plan(const int* s_idx, const float* s_w, const unsigned char* s_valid,
                                           int R, int K, int E, DecodePlan* P) {
  __shared__ __attribute__((aligned(16))) int s_key[kDecodeMaxSlots];
  __shared__ __attribute__((aligned(16))) float s_kw[kDecodeMaxSlots];
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
  if (lane < kDecodeMaxSlots) {
    s_key[lane] = key;
    s_kw[lane] = w;
  }
  __builtin_amdgcn_wave_barrier();
  auto keys8 = [&](int t0, int (&kk)[8]) {
    const int4 a = *(const int4*)(s_key + t0), b = *(const int4*)(s_key + t0 + 4);
    kk[0] = a.x; kk[1] = a.y; kk[2] = a.z; kk[3] = a.w; kk[4] = b.x; kk[5] = b.y; kk[6] = b.z; kk[7] = b.w;
  };
  bool first = v;
  float wsum = 0.f;
#pragma unroll 1
  for (int t0 = 0; t0 < S; t0 += 8) {
    int kk[8];
    keys8(t0, kk);
    const float4 a = *(const float4*)(s_kw + t0), b = *(const float4*)(s_kw + t0 + 4);
    const float kw[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool eq = v && kk[i] == key;
      if (eq) wsum += kw[i];
      first = first && !(eq && t0 + i < lane);
    }
  }
  const uint64_t fmask = __ballot(first);
  int pos = 0;
  bool efirst = first;
#pragma unroll 1
  for (int t0 = 0; t0 < S; t0 += 8) {
    int kk[8];
    keys8(t0, kk);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ft = (fmask >> (t0 + i)) & 1;
      pos += (ft && kk[i] < key) ? 1 : 0;
      efirst = efirst && !(ft && (kk[i] >> 3) == (key >> 3) && kk[i] < key);
    }
  }
  const uint64_t emask = __ballot(efirst);
  int gidx = 0;
#pragma unroll 1
  for (int t0 = 0; t0 < S; t0 += 8) {
    int kk[8];
    keys8(t0, kk);
#pragma unroll
    for (int i = 0; i < 8; ++i) gidx += (((emask >> (t0 + i)) & 1) && (kk[i] >> 3) < (key >> 3)) ? 1 : 0;
  }
  const int ngroups = __popcll(emask);
  const int nentries = __popcll(fmask);
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

// The plan of one row, in slot order: group g is the g-th valid slot (its
// expert, one entry for row 0 with the slot's weight).  Two slots that name
// one expert (only from a malformed hash table) stay two groups, each adding
// its weight times that expert's output -- the sum over slots as defined.
// A handful of wave-wide operations on wave 0 (lane k = slot k), no loops:
// the routed gate/up blocks run it before their streams start.
__device__ __forceinline__ void build_plan_one_row(const int* s_idx, const float* s_w, const unsigned char* s_valid,
                                                   int K, int E, DecodePlan* P) {
  const int lane = threadIdx.x & (kWave - 1);
  int e = -1;
  float w = 0.f;
  bool v = false;
  if (lane < K) {
    e = s_idx[lane];
    w = s_w[lane];
    v = s_valid[lane] && e >= 0 && e < E;
  }
  const uint64_t vm = __ballot(v);
  const int gidx = __popcll(vm & ((1ull << lane) - 1ull));
  const int n = __popcll(vm);
  if (v) {
    P->group_expert[gidx] = e;
    P->group_begin[gidx] = gidx;
    P->entry_row[gidx] = 0;
    P->entry_w[gidx] = w;
  }
  if (lane == 0) {
    P->ngroups = n;
    P->nentries = n;
    P->group_begin[n] = n;
  }
}

// Route of one row by one wavefront, slot-parallel: lane k < K returns
// slot k (index, weight, valid); flags (the row's status bits) are the same
// in every lane.  lg holds the logits in the select_topk lane layout (lane
// l: experts l, l+64, l+128, l+192).  Score layers: the K largest keys
// sigmoid(logit) + bias (bias bs0..bs3 in the same layout), larger first,
// equal keys to the lower expert id;
// hash layers: `ent`, lane k's entry of the token's table row (tok_ok false
// for a token id outside the table).  Weights are the chosen experts'
// sigmoids over their sum, summed in slot order.  Same results, in the same
// order of operations, as select_topk + score_route_keys and
// hash_route_entries; written with one copy of each step (keys, selection,
// weights), which keeps the kernel small.
struct SlotRoute {
  int idx;
  float w;
  bool valid;
  uint32_t flags;
};
__device__ __forceinline__ SlotRoute route_slots(float lg0, float lg1, float lg2, float lg3, float bs0, float bs1,
                                                 float bs2, float bs3, int E, int K, bool hash, bool tok_ok, int ent) {
  const int lane = threadIdx.x & (kWave - 1);
  SlotRoute o;
  o.flags = 0;
  float lsel = 0.f;  // this lane's slot: the logit its weight comes from
  bool use = false;  // ... and whether the slot is valid
  if (!hash) {
    uint64_t u0 = 0, u1 = 0, u2 = 0, u3 = 0;
#pragma unroll 1
    for (int j = 0; j < 4; ++j) {
      const int e = lane + kWave * j;
      const float l = j == 0 ? lg0 : j == 1 ? lg1 : j == 2 ? lg2 : lg3;
      const float bj = j == 0 ? bs0 : j == 1 ? bs1 : j == 2 ? bs2 : bs3;
      const uint64_t k = e < E ? ordered_key(score_key(l, bj)) : 0ull;
      u0 = j == 0 ? k : u0;
      u1 = j == 1 ? k : u1;
      u2 = j == 2 ? k : u2;
      u3 = j == 3 ? k : u3;
    }
    o.idx = -1;
#pragma unroll 1
    for (int k = 0; k < K; ++k) {
      uint64_t lm = u0 > u1 ? u0 : u1;
      lm = u2 > lm ? u2 : lm;
      lm = u3 > lm ? u3 : lm;
      const uint64_t m = wave_max_u64(lm);
      // the lowest expert id holding the maximum: experts are ordered by
      // (j, lane), so take the lowest j, then the lowest lane
      const uint64_t b0 = __ballot(u0 == m && m != 0ull), b1 = __ballot(u1 == m && m != 0ull);
      const uint64_t b2 = __ballot(u2 == m && m != 0ull), b3 = __ballot(u3 == m && m != 0ull);
      const int j = b0 ? 0 : b1 ? 1 : b2 ? 2 : b3 ? 3 : -1;
      const uint64_t bm = j == 0 ? b0 : j == 1 ? b1 : j == 2 ? b2 : b3;
      int e = 0;
      float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lg0), 0));
      if (j >= 0) {
        const int wl = __ffsll((unsigned long long)bm) - 1;
        e = wl + kWave * j;
        const float lj = j == 0 ? lg0 : j == 1 ? lg1 : j == 2 ? lg2 : lg3;
        l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lj), wl));
        if (lane == wl) {
          u0 = j == 0 ? 0ull : u0;
          u1 = j == 1 ? 0ull : u1;
          u2 = j == 2 ? 0ull : u2;
          u3 = j == 3 ? 0ull : u3;
        }
      }
      if (lane == k) {
        o.idx = e;
        lsel = l;
      }
    }
    use = lane < K;
  } else {
    const int e = (tok_ok && lane < K) ? ent : -1;
    use = tok_ok && lane < K && e >= 0 && e < E;
    const int src = use ? (e & (kWave - 1)) : 0, j = use ? e / kWave : 0;
    const float v0 = __shfl(lg0, src), v1 = __shfl(lg1, src), v2 = __shfl(lg2, src), v3 = __shfl(lg3, src);
    lsel = j == 0 ? v0 : j == 1 ? v1 : j == 2 ? v2 : v3;
    o.idx = lane < K ? e : -1;
    if (__ballot(tok_ok && lane < K && !use)) o.flags |= MOE_FLAG_BAD_TABLE_ENTRY;
    if (!tok_ok) o.flags |= MOE_FLAG_BAD_TOKEN;
  }
  const double sg = use ? sigmoid_f64(lsel) : 0.0;
  double tot = 0.0;
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    const int lo = __builtin_amdgcn_readlane((int)(uint32_t)__double_as_longlong(sg), k);
    const int hi = __builtin_amdgcn_readlane((int)(uint32_t)(__double_as_longlong(sg) >> 32), k);
    tot += __longlong_as_double(((long long)(uint32_t)hi << 32) | (uint32_t)lo);
  }
  o.valid = use;
  o.w = (use && (!hash || tot > 0.0)) ? (float)(sg / tot) : 0.0f;
  return o;
}

// route_slots for one row from per-expert values the router launch stored:
// key[j] = ordered_key(score_key(logit, bias)) and sig[j] = sigmoid_f64(logit)
// of expert lane + 64j (the same functions route_slots applies to the
// logits, so the same bits).  The selection loop, its tie-break and the
// weights are route_slots'; the sigmoid of a chosen expert is read from its
// lane instead of recomputed.
__device__ __forceinline__ double lane_f64(double v, int src) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(uint32_t)b, src);
  const int hi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
  return __longlong_as_double(((long long)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ SlotRoute route_slots_keyed(const uint64_t (&key)[4], const double (&sig)[4], int E, int K,
                                                       bool hash, bool tok_ok, int ent) {
  const int lane = threadIdx.x & (kWave - 1);
  SlotRoute o;
  o.flags = 0;
  double sg = 0.0;
  bool use = false;
  if (!hash) {
    uint64_t u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = lane + kWave * j < E ? key[j] : 0ull;
    o.idx = -1;
#pragma unroll 1
    for (int k = 0; k < K; ++k) {
      uint64_t lm = u[0] > u[1] ? u[0] : u[1];
      lm = u[2] > lm ? u[2] : lm;
      lm = u[3] > lm ? u[3] : lm;
      const uint64_t m = wave_max_u64(lm);
      const uint64_t b0 = __ballot(u[0] == m && m != 0ull), b1 = __ballot(u[1] == m && m != 0ull);
      const uint64_t b2 = __ballot(u[2] == m && m != 0ull), b3 = __ballot(u[3] == m && m != 0ull);
      const int j = b0 ? 0 : b1 ? 1 : b2 ? 2 : b3 ? 3 : -1;
      const uint64_t bm = j == 0 ? b0 : j == 1 ? b1 : j == 2 ? b2 : b3;
      int e = 0;
      double v = lane_f64(sig[0], 0);
      if (j >= 0) {
        const int wl = __ffsll((unsigned long long)bm) - 1;
        e = wl + kWave * j;
        v = lane_f64(j == 0 ? sig[0] : j == 1 ? sig[1] : j == 2 ? sig[2] : sig[3], wl);
        if (lane == wl) {
          u[0] = j == 0 ? 0ull : u[0];
          u[1] = j == 1 ? 0ull : u[1];
          u[2] = j == 2 ? 0ull : u[2];
          u[3] = j == 3 ? 0ull : u[3];
        }
      }
      if (lane == k) {
        o.idx = e;
        sg = v;
      }
    }
    use = lane < K;
  } else {
    const int e = (tok_ok && lane < K) ? ent : -1;
    use = tok_ok && lane < K && e >= 0 && e < E;
    const int src = use ? (e & (kWave - 1)) : 0, j = use ? e / kWave : 0;
    double v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const long long b = __double_as_longlong(sig[q]);
      const int lo = __shfl((int)(uint32_t)b, src), hi = __shfl((int)(uint32_t)(b >> 32), src);
      v[q] = __longlong_as_double(((long long)(uint32_t)hi << 32) | (uint32_t)lo);
    }
    sg = use ? (j == 0 ? v[0] : j == 1 ? v[1] : j == 2 ? v[2] : v[3]) : 0.0;
    o.idx = lane < K ? e : -1;
    if (__ballot(tok_ok && lane < K && !use)) o.flags |= MOE_FLAG_BAD_TABLE_ENTRY;
    if (!tok_ok) o.flags |= MOE_FLAG_BAD_TOKEN;
  }
  if (!use) sg = 0.0;
  double tot = 0.0;
#pragma unroll 1
  for (int k = 0; k < K; ++k) tot += lane_f64(sg, k);
  o.valid = use;
  o.w = (use && (!hash || tot > 0.0)) ? (float)(sg / tot) : 0.0f;
  return o;
}

// Routing of the one row by wave 0 of a one-row gate/up block, from the
// selection keys and float64 sigmoids the router launch stored (plain loads:
// written by the launch before).
__device__ void route_one_row(const FwdArgs& a, int* s_idx, float* s_w, unsigned char* s_valid, uint32_t* s_flags) {
  const int K = a.K, E = a.E;
  const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  if (wv != 0) return;
  const bool hash = a.layer_kind == MOE_LAYER_HASH;
  int ent = -1;
  bool tok_ok = false;
  if (hash) {
    const int32_t tok = a.token_ids[0];
    tok_ok = tok >= 0 && (int64_t)tok < a.table_rows;
    if (tok_ok && lane < K) ent = a.table[(int64_t)tok * K + lane];
  }
  uint64_t key[4];
  double sig[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    key[j] = e < E ? a.sync->route_key[e] : 0ull;
    sig[j] = e < E ? a.sync->route_sig[e] : 0.0;
  }
  const SlotRoute sr = route_slots_keyed(key, sig, E, K, hash, tok_ok, ent);
  if (lane < K) {
    s_idx[lane] = sr.idx;
    s_w[lane] = sr.w;
    s_valid[lane] = sr.valid;
  }
  if (lane == 0) s_flags[0] = sr.flags;
}

// Routing of the batch by the router launch's last block: wave r < R
// routes row r from the logits the router blocks published (read past any
// stale cache line: other workgroups wrote them) into LDS.  It first reads
// what the route needs besides the logits (bias, or the token's table row).
__device__ void route_batch(const FwdArgs& a, int* s_idx, float* s_w, unsigned char* s_valid, uint32_t* s_flags) {
  const int R = a.R, K = a.K, E = a.E;
  const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  if (wv >= R) return;
  const bool hash = a.layer_kind == MOE_LAYER_HASH;
  int ent = -1;
  bool tok_ok = false;
  float bias[4] = {0.f, 0.f, 0.f, 0.f};
  if (hash) {
    const int32_t tok = a.token_ids[wv];
    tok_ok = tok >= 0 && (int64_t)tok < a.table_rows;
    if (tok_ok && lane < K) ent = a.table[(int64_t)tok * K + lane];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) bias[j] = (lane + kWave * j < E) ? a.bias[lane + kWave * j] : 0.f;
  }
  float lg[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    lg[j] = e < E ? load_wt(&a.logits[(int64_t)wv * E + e]) : 0.f;
  }
  const SlotRoute sr = route_slots(lg[0], lg[1], lg[2], lg[3], bias[0], bias[1], bias[2], bias[3], E, K, hash, tok_ok,
                                   ent);
  if (lane < K) {
    s_idx[wv * K + lane] = sr.idx;
    s_w[wv * K + lane] = sr.w;
    s_valid[wv * K + lane] = sr.valid;
  }
  if (lane == 0) s_flags[wv] = sr.flags;
}

// Writes the block's routing (indices, weights, row flags, status word) and
// the plan (from LDS) to the workspace for the later launches and the
// caller.
__device__ void publish_routing(const FwdArgs& a, const int* s_idx, const float* s_w, const uint32_t* s_flags,
                                const DecodePlan* P) {
  const int R = a.R;
  for (int s = threadIdx.x; s < R * a.K; s += kThreads) {
    a.idx[s] = s_idx[s];
    a.wts[s] = s_w[s];
  }
  if ((int)threadIdx.x < R) a.rowflags[threadIdx.x] = s_flags[threadIdx.x];
  if (threadIdx.x == 0) {
    uint32_t f = 0;
    for (int r = 0; r < R; ++r) f |= s_flags[r];
    a.status[0] = f;
  }
  const int* ps = (const int*)P;
  int* pd = (int*)a.plan;
  for (int i = threadIdx.x; i < (int)(sizeof(DecodePlan) / 4); i += kThreads) pd[i] = ps[i];
}

// The plan as read by the tail kernel, every field clamped to its range so
// that no value can index outside the buffers.
struct PlanGroup {
  int expert, begin, nr;
};
__device__ __forceinline__ int plan_ngroups(const DecodePlan* P) {
  const int n = P->ngroups;
  return n < 0 ? 0 : (n > kDecodeMaxSlots ? kDecodeMaxSlots : n);
}
__device__ __forceinline__ PlanGroup plan_group(const DecodePlan* P, int u, int E, uint32_t* status) {
  PlanGroup g;
  const int e = P->group_expert[u];
  g.expert = e < 0 ? 0 : (e >= E ? E - 1 : e);
  int b = P->group_begin[u], n = P->group_begin[u + 1];
  check_index(status, e >= 0 && e < E && b >= 0 && n > b && n - b <= kDecodeMaxRows && n <= kDecodeMaxSlots);
  b = b < 0 ? 0 : (b > kDecodeMaxSlots - 1 ? kDecodeMaxSlots - 1 : b);
  n = n - b;  // n <= 0 (only from a corrupt plan) just means no rows
  n = n > kDecodeMaxRows ? kDecodeMaxRows : n;
  if (b + n > kDecodeMaxSlots) n = kDecodeMaxSlots - b;
  g.begin = b;
  g.nr = n;
  return g;
}
__device__ __forceinline__ int plan_row(const DecodePlan* P, int j, int R, uint32_t* status) {
  const int r = P->entry_row[j];
  check_index(status, r >= 0 && r < R);
  return r < 0 ? 0 : (r >= R ? R - 1 : r);
}

// Down projection of ROWS hidden rows of one expert (wbase [H][I]) for the
// nr activation rows staged in hs: the block's i-th row (i = wave + 4j) is
// x + i * stride, so concurrent blocks read neighbouring rows.  d32 rows
// ent..ent+nr-1 receive the results (written through).
template <int H, int I, int ROWS, int NBUF, int MX, bool PAIR, class Pre>
__device__ __forceinline__ void down_tile(const WMat& wm, const float* hs, int nr, int x, int stride, float* d32,
                                          int ent, Pre pre) {
  constexpr int W = kThreads / kWave, RPW = ROWS / W;  // rows per wave
  static_assert(RPW * 4 <= kWave && RPW % NBUF == 0, "one lane per result; whole row groups in flight");
  __shared__ float s_res[ROWS * 4];  // results wait here until the stream ends
  const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  float* res = s_res + wv * RPW * 4;
  auto row_of = [&](int j) { return x + (wv + j * W) * stride; };
  auto rowsrc = [&](int j) { return wrow<MX, I>(wm, row_of(j)); };
  auto sink = [&](int j, const float (&part)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < nr) {
        const float v = wave_sum(part[r]);
        if (lane == 0) res[j * 4 + r] = v;
      }
    }
  };
  stream_rows<I, NBUF, MX, PAIR>(RPW, rowsrc, hs, nr, pre, sink);
  const int j = lane >> 2, r = lane & 3;
  if (j < RPW && r < nr) store_wt(&d32[(int64_t)(ent + r) * H + row_of(j)], res[lane]);
}

// ---------------------------------------------------------------------------
// Head kernel: router, routing plan and the shared expert's gate/up.
// grid = E/4 router blocks, then I/8 shared gate/up blocks.
//   Router block (experts 4b .. 4b+3, one per wave): requests its router
//   rows, normalises the batch rows into LDS, forms logit[r,e] = sum_j
//   W[e,j] xn[r,j] and writes it through.  Then it counts itself in; the
//   block that completes the count -- every logit is written by then --
//   routes the batch (wave r row r), builds the plan
//   of distinct (expert, row) pairs, publishes indices, weights, row flags,
//   status and the plan, and resets the count for the next call.  No
//   workgroup waits for another.
//   Shared gate/up block: RMSNorm into LDS, then 8 inter rows of the shared
//   expert's SwiGLU output for every row; its streaming covers the router's
//   latency and the routing.  The first of these blocks publishes xn.
// kRouterOnly (one row): the router blocks alone, each wave also storing
// its expert's selection key and sigmoid; without the wrapper every lane
// dots its own columns in registers and the norm is applied to the sum.
template <int H, int I, bool kRouterOnly, int MX>
__global__ __launch_bounds__(kThreads) void k_dec_head(const FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) float xs[];  // [R][H]
  __shared__ int s_idx[kDecodeMaxSlots];
  __shared__ float s_w[kDecodeMaxSlots];
  __shared__ unsigned char s_valid[kDecodeMaxSlots];
  __shared__ uint32_t s_flags[kDecodeMaxRows];
  __shared__ DecodePlan P;
  __shared__ int s_last;
  const int R = a.R, E = a.E, K = a.K;
  const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  DecodeSync* sy = a.sync;
  const int nrb = (E + 3) / 4, nsh = I / kShRows;
  const int b = blockIdx.x;
  if (!kRouterOnly && b >= nrb) {  // shared gate/up block
    const int x = b - nrb;
    auto stage = [&]() {
      norm_rows_to_lds<H>(a, false, xs);
      if (x == 0)
        for (int i = threadIdx.x; i < R * H / 4; i += kThreads) ((float4*)a.xn32)[i] = ((const float4*)xs)[i];
    };
    stage();
    gateup_tile<H, I, kShRows, kNbuf<MX>, MX, kPair<MX>>(expert_mat<MX>(a.gate_sh, a.gate_sh_q, a.gate_sh_s, 0, (int64_t)I * H),
                                      expert_mat<MX>(a.up_sh, a.up_sh_q, a.up_sh_s, 0, (int64_t)I * H), xs, R, x, nsh,
                                      a.h32, kDecodeMaxSlots, [] {});
    return;
  }
  // router block: expert e = 4b + w per wave.  The weight row's loads go out
  // first; the block then normalises its rows into LDS (one round trip for
  // the batch) and each wave dots its row with them.
  const int e = b * 4 + wv;
  constexpr int NCH = (H + 511) / 512;
  const bool full = H % 512 == 0 || lane * 8 < H % 512;
  uint4 q[NCH];
  // one row: the expert's selection bias, requested with its router row
  const float bias_e = (kRouterOnly && e < E && lane == 0 && a.layer_kind != MOE_LAYER_HASH) ? a.bias[e] : 0.f;
  if (e < E) {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (c < NCH - 1 || full) q[c] = load_stream(a.router + (int64_t)e * H + c * 512 + lane * 8);
  }
  if constexpr (kRouterOnly) {
    if (a.hc == 0) {
      // One row without the wrapper: logit = (sum_j W[e,j] x_j g_j) / rms(x).
      // Every wave loads the row and the norm weight at its own lanes'
      // columns (those of its router row), so the dot needs no LDS and no
      // barrier; the sum of squares comes from the same values.  Block 0's
      // wave 0 also stores xn = x / rms(x) * g for the later launches.
      float xv[NCH][8], gv[NCH][8];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int col = c * 512 + lane * 8;
        if (c < NCH - 1 || full) {
          const float4 x0 = *(const float4*)(a.x + col), x1 = *(const float4*)(a.x + col + 4);
          const float4 g0 = *(const float4*)(a.norm_w + col), g1 = *(const float4*)(a.norm_w + col + 4);
          xv[c][0] = x0.x; xv[c][1] = x0.y; xv[c][2] = x0.z; xv[c][3] = x0.w;
          xv[c][4] = x1.x; xv[c][5] = x1.y; xv[c][6] = x1.z; xv[c][7] = x1.w;
          gv[c][0] = g0.x; gv[c][1] = g0.y; gv[c][2] = g0.z; gv[c][3] = g0.w;
          gv[c][4] = g1.x; gv[c][5] = g1.y; gv[c][6] = g1.z; gv[c][7] = g1.w;
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) xv[c][i] = gv[c][i] = 0.f;
        }
      }
      float ss = 0.f, dot = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        float f[8];
        unpack8(e < E && (c < NCH - 1 || full) ? q[c] : make_uint4(0u, 0u, 0u, 0u), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ss = fmaf(xv[c][i], xv[c][i], ss);
          dot = fmaf(f[i], xv[c][i] * gv[c][i], dot);
        }
      }
      ss = wave_sum(ss);
      dot = wave_sum(dot);
      const float rs = 1.0f / sqrtf(ss / (float)H + a.eps);
      if (b == 0 && wv == 0) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          if (c < NCH - 1 || full) {
            float4 o0, o1;
            o0.x = xv[c][0] * rs * gv[c][0]; o0.y = xv[c][1] * rs * gv[c][1];
            o0.z = xv[c][2] * rs * gv[c][2]; o0.w = xv[c][3] * rs * gv[c][3];
            o1.x = xv[c][4] * rs * gv[c][4]; o1.y = xv[c][5] * rs * gv[c][5];
            o1.z = xv[c][6] * rs * gv[c][6]; o1.w = xv[c][7] * rs * gv[c][7];
            *(float4*)(a.xn32 + c * 512 + lane * 8) = o0;
            *(float4*)(a.xn32 + c * 512 + lane * 8 + 4) = o1;
          }
        }
      }
      if (e < E && lane == 0) {
        const float v = dot * rs;
        a.logits[e] = v;
        sy->route_sig[e] = sigmoid_f64(v);
        sy->route_key[e] = a.layer_kind == MOE_LAYER_HASH ? 0ull : ordered_key(score_key(v, bias_e));
      }
      return;
    }
  }
  norm_rows_to_lds<H, kRouterOnly ? 1 : kDecodeMaxRows>(a, b == 0, xs);
  if (kRouterOnly && b == 0)  // the later launches stage the normalised row from xn
    for (int i = threadIdx.x; i < R * H / 4; i += kThreads) ((float4*)a.xn32)[i] = ((const float4*)xs)[i];
  if (e < E) {
    float dot[kDecodeMaxRows] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c < NCH - 1 || full) {
        const int col = c * 512 + lane * 8;
        float f[8];
        unpack8(q[c], f);
#pragma unroll
        for (int r = 0; r < kDecodeMaxRows; ++r) {
          if (r < R) {
            const float4 x0 = *(const float4*)(xs + r * H + col), x1 = *(const float4*)(xs + r * H + col + 4);
            const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) dot[r] = fmaf(f[i], xv[i], dot[r]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kDecodeMaxRows; ++r) {
      if (r < R) {
        const float v = wave_sum(dot[r]);
        if (lane == 0) {
          if (kRouterOnly) {  // one row: what the gate/up blocks' routing needs of this expert
            a.logits[e] = v;
            sy->route_sig[e] = sigmoid_f64(v);
            sy->route_key[e] = a.layer_kind == MOE_LAYER_HASH ? 0ull : ordered_key(score_key(v, bias_e));
          } else {
            store_wt(&a.logits[(int64_t)r * E + e], v);
          }
        }
      }
    }
  }
  if (kRouterOnly) return;
  // count in once the logits are written through (a wait for the block's
  // own stores, no cache-wide fence); the last router block routes, reading
  // them with write-through loads
  sync_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&sy->arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == (uint32_t)nrb;
  __syncthreads();
  if (!s_last) return;
  route_batch(a, s_idx, s_w, s_valid, s_flags);
  __syncthreads();
  if (wv == 0) build_plan(s_idx, s_w, s_valid, R, K, E, &P);
  __syncthreads();
  publish_routing(a, s_idx, s_w, s_flags, &P);
  if (threadIdx.x == 0) sy->arrive = 0;  // every router block of this call has counted in
}

// ---------------------------------------------------------------------------
// Shared down + routed gate/up.  grid = H/16 shared-down blocks (dispatched
// first: the shared h is complete, and their streaming covers the routed
// blocks' plan read and staging), then G * I/16 routed gate/up blocks (G =
// max distinct routed experts); with one row, 256 + 6 * 128 blocks put one
// shared-down and three routed blocks on every compute unit, so no unit
// has more to stream than another.  Shared-down block x: hidden rows x,
// x + H/16, ... of the shared expert's down projection -> d32 shared rows.
// Gate/up block (u, x): inter rows x, x + I/16, ... of the plan's u-th
// expert -> h32.
template <int H, int I, int MX>
__global__ __launch_bounds__(kThreads) void k_dec_gateup(const FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) float xs[];  // [nr][H] activations, or [R][I] shared h
  constexpr int nsd = H / kSdRows, gut = I / kGuRows;
  const int b = blockIdx.x;
  if (b < nsd) {
    const float* src[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) src[j] = a.h32 + (int64_t)(kDecodeMaxSlots + (j < a.R ? j : 0)) * I;
    down_tile<H, I, kSdRows, kNbuf<MX>, MX, kPair<MX>>(expert_mat<MX>(a.down_sh, a.down_sh_q, a.down_sh_s, 0, (int64_t)H * I), xs, a.R, b,
                                 H / kSdRows, a.d32, kDecodeMaxSlots,
                             [&]() { stage_rows<I>(xs, src, a.R); });
    return;
  }
  const DecodePlan* P = a.plan;
  const int u = (b - nsd) / gut, x = (b - nsd) % gut;
  if (u >= plan_ngroups(P)) return;
  const PlanGroup g = plan_group(P, u, a.E, a.status);
  const float* src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) src[j] = a.xn32 + (int64_t)plan_row(P, g.begin + (j < g.nr ? j : 0), a.R, a.status) * H;
  gateup_tile<H, I, kGuRows, kNbuf<MX>, MX, kPair<MX>>(expert_mat<MX>(a.gate, a.gate_q, a.gate_s, g.expert, (int64_t)I * H),
                                    expert_mat<MX>(a.up, a.up_q, a.up_s, g.expert, (int64_t)I * H), xs, g.nr, x, gut,
                             a.h32, g.begin, [&]() { stage_rows<H>(xs, src, g.nr); });
}

// ---------------------------------------------------------------------------
// One-row gate/up launch: grid = I/8 shared gate/up blocks, then
// G * I/16 routed gate/up blocks (G = top_k).  The router launch before it
// has written the logits, each expert's selection key and sigmoid, and xn.
// A routed block routes the row itself -- wave 0 reads the keys and
// sigmoids and picks the slots with the head plan block's selection, then
// builds the slot-order plan in LDS -- and streams the rows of the plan's
// u-th expert;
// the u = 0, x = 0 block also publishes the routing and the plan.  No block waits for another: with one row the routing is a few
// microseconds of work that every block repeats, against the
// cross-workgroup round trips of a shared plan.  At full size this is 256 +
// 6 * 128 blocks, one shared and three routed per compute unit.
template <int H, int I, int MX>
__global__ __launch_bounds__(kThreads) void k_dec1_gateup(const FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) float xs[];  // [H] normalised row
  __shared__ int s_idx[kDecodeMaxSlots];
  __shared__ float s_w[kDecodeMaxSlots];
  __shared__ unsigned char s_valid[kDecodeMaxSlots];
  __shared__ uint32_t s_flags[kDecodeMaxRows];
  __shared__ DecodePlan P;
  constexpr int nsh = I / kShRows, gut = I / kGuRows;
  const int b = blockIdx.x;
  const float* src[4] = {a.xn32, a.xn32, a.xn32, a.xn32};
  if (b < nsh) {  // shared gate/up block
    // the row count stays a run-time value (a.R = 1 here): with a constant 1
    // the compiler keeps the whole activation row in registers
    gateup_tile<H, I, kShRows, kNbuf<MX>, MX, kPair<MX>>(expert_mat<MX>(a.gate_sh, a.gate_sh_q, a.gate_sh_s, 0, (int64_t)I * H),
                                      expert_mat<MX>(a.up_sh, a.up_sh_q, a.up_sh_s, 0, (int64_t)I * H), xs, a.R, b, nsh,
                                      a.h32, kDecodeMaxSlots,
                                  [&]() { stage_rows<H>(xs, src, a.R); });
    return;
  }
  const int u = (b - nsh) / gut, x = (b - nsh) % gut;
  route_one_row(a, s_idx, s_w, s_valid, s_flags);  // wave 0 (the row)
  __syncthreads();
  if (threadIdx.x < kWave) build_plan_one_row(s_idx, s_w, s_valid, a.K, a.E, &P);
  __syncthreads();
  if (u == 0 && x == 0) publish_routing(a, s_idx, s_w, s_flags, &P);
  if (u >= plan_ngroups(&P)) return;
  const PlanGroup g = plan_group(&P, u, a.E, a.status);
  const int nr = g.nr < a.R ? g.nr : a.R;  // LDS holds a.R rows
  gateup_tile<H, I, kGuRows, kNbuf<MX>, MX, kPair<MX>>(expert_mat<MX>(a.gate, a.gate_q, a.gate_s, g.expert, (int64_t)I * H),
                                    expert_mat<MX>(a.up, a.up_q, a.up_s, g.expert, (int64_t)I * H), xs, nr, x, gut,
                                a.h32, g.begin, [&]() { stage_rows<H>(xs, src, nr); });
}

// ---------------------------------------------------------------------------
// Routed down (2-4 rows).  grid = (H/D, G) with D = kDnRows and G the most
// distinct routed experts.  Block (x, u) computes hidden rows x, x + H/D,
// ... of the plan's u-th expert's down projection for its rows and writes
// them to d32 (the entries' rows); blocks past the plan's groups return at
// once.  The weighted reduce is the next launch: a block here ends with its
// stream, with no wait for its stores and no count.
template <int H, int I, int MX>
__global__ __launch_bounds__(kThreads) void k_dec_down(const FwdArgs a) {
  __shared__ float hs[kDecodeMaxRows * I];
  const DecodePlan* P = a.plan;
  const int u = blockIdx.y;
  if (u >= plan_ngroups(P)) return;
  const PlanGroup g = plan_group(P, u, a.E, a.status);
  const float* src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) src[j] = a.h32 + (int64_t)(g.begin + (j < g.nr ? j : 0)) * I;
  down_tile<H, I, kDnRows<MX>, kNbuf<MX>, MX, kPair<MX>>(expert_mat<MX>(a.down, a.down_q, a.down_s, g.expert, (int64_t)H * I), hs,
                                                         g.nr, blockIdx.x, H / kDnRows<MX>, a.d32, g.begin,
                                                     [&]() { stage_rows<I>(hs, src, g.nr); });  // ends with a barrier
}

// Weighted reduce + shared (2-4 rows).  grid = R*H/256, thread -> (row r,
// hidden h).  out[r][h] = sum over r's (expert, row) pairs in plan order
// (experts ascending) of weight * down, then + the shared down written by
// the gate/up launch -- a fixed order, so the output is bitwise
// reproducible; with no valid routed expert, out = shared down.  The
// hyper-connection post-mix follows.
template <int H>
__global__ __launch_bounds__(kThreads) void k_dec_reduce(const FwdArgs a) {
  static_assert(H % kThreads == 0, "a block covers part of one row");
  __shared__ int s_er[kDecodeMaxSlots];  // the plan's entry rows and weights
  __shared__ float s_ew[kDecodeMaxSlots];
  const DecodePlan* P = a.plan;
  const int ng = plan_ngroups(P);
  int ne = P->nentries;
  ne = ne < 0 ? 0 : (ne > kDecodeMaxSlots ? kDecodeMaxSlots : ne);
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int r = (int)(t / H), h = (int)(t % H);
  // hyper-connection post-mix: the row's old streams at h, requested first
  float st[kHcMax];
  if (a.hc > 0) {
#pragma unroll
    for (int i = 0; i < kHcMax; ++i)
      if (i < a.hc) st[i] = a.hc_state[((int64_t)r * a.hc + i) * H + h];
  }
  // the down launch's partials and the shared expert's down rows were
  // written by blocks on every XCD: read past any stale cache line
  const float sh = load_wt(&a.d32[(int64_t)(kDecodeMaxSlots + r) * H + h]);
  // every entry's partial is requested at once (one memory round trip; the
  // index is clamped, so the loads past ne re-read a valid row)
  float v[kDecodeMaxSlots];
#pragma unroll
  for (int j = 0; j < kDecodeMaxSlots; ++j) v[j] = load_wt(&a.d32[(int64_t)(j < ne ? j : (ne > 0 ? ne - 1 : 0)) * H + h]);
  if (threadIdx.x < kDecodeMaxSlots) {
    s_er[threadIdx.x] = P->entry_row[threadIdx.x];
    s_ew[threadIdx.x] = P->entry_w[threadIdx.x];
  }
  __syncthreads();
  float o = 0.f;
  if (ng > 0) {
    // the row's own entries, in plan order
#pragma unroll
    for (int j = 0; j < kDecodeMaxSlots; ++j)
      if (j < ne && s_er[j] == r) o = fmaf(s_ew[j], v[j], o);
  }
  o += sh;
  a.out[(int64_t)r * H + h] = o;
  if (a.hc > 0) {  // new[r][j] = post_j * out + sum_i comb[j][i] * state_i, i in order
    const int hc = a.hc, mw = (2 + hc) * hc;
    const float* mp = a.hc_maps + (int64_t)r * mw;
#pragma unroll
    for (int j = 0; j < kHcMax; ++j) {
      if (j < hc) {
        float w = mp[hc + j] * o;
#pragma unroll
        for (int i = 0; i < kHcMax; ++i)
          if (i < hc) w = fmaf(mp[2 * hc + j * hc + i], st[i], w);
        a.hc_out[((int64_t)r * hc + j) * H + h] = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One-row down + reduce, output-stationary: grid = H/8 blocks.  Block x owns
// the hidden rows x + i*H/8, i = 0..7 (wave w: i = w and w + 4, so the
// blocks running together read neighbouring rows of each matrix).  Every
// wave reads the plan itself (its groups' experts and weights; with one row
// group u holds entry u), the block stages group u's h vector (u in plan
// order) and the shared expert's into LDS, and each wave then streams its
// two rows of every matrix -- the plan's experts in order, then the shared
// one; the two rows share the activation -- keeping the dot products in
// LDS.  Thread i < 8 then forms out = sum over u of w_u * down_u, then +
// shared down -- the order of the reduce launch of two to four rows -- and
// the hyper-connection post-mix follows (its state and maps staged with
// the h vectors).  No block waits for another and nothing goes through the
// workspace.  At full size: 512
// blocks, two per compute unit, each streaming 8 rows of every matrix.
template <int H, int I, int MX>
__global__ __launch_bounds__(kThreads) void k_dec1_down(const FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) float hs[];  // [ng + 1][I]
  constexpr int W = kThreads / kWave, ROWS = 2 * W, stride = H / ROWS;
  static_assert(H % ROWS == 0, "whole row groups");
  __shared__ float s_res[(kMaxTopK + 1) * ROWS];
  __shared__ float s_st[kHcMax * ROWS];
  __shared__ float s_map[(2 + kHcMax) * kHcMax];
  const DecodePlan* P = a.plan;
  const int cap = a.K < a.E ? a.K : a.E;  // hs holds cap + 1 vectors
  int ng = plan_ngroups(P);
  check_index(a.status, ng <= cap);
  ng = ng > cap ? cap : ng;  // <= kMaxTopK
  // lane u < kMaxTopK of every wave holds group u's expert, entry and
  // weight (clamped; read for every u, the plan's arrays being whole)
  const int x = blockIdx.x, wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int ul = lane < kMaxTopK ? lane : 0;
  int exv = P->group_expert[ul], ebv = P->group_begin[ul];
  check_index(a.status, ul >= ng || (exv >= 0 && exv < a.E && ebv == ul && P->group_begin[ul + 1] == ul + 1));
  exv = exv < 0 ? 0 : (exv >= a.E ? a.E - 1 : exv);
  ebv = ebv < 0 ? 0 : (ebv >= kDecodeMaxSlots ? kDecodeMaxSlots - 1 : ebv);
  const float ewv = P->entry_w[ebv];
  const int64_t msz = (int64_t)H * I;
  const WMat shm = expert_mat<MX>(a.down_sh, a.down_sh_q, a.down_sh_s, 0, msz);
  auto rowsrc = [&](int j) {
    const int m = j >> 1;
    const int e = __builtin_amdgcn_readlane(exv, m < kMaxTopK ? m : 0);
    const WMat wm = m < ng ? expert_mat<MX>(a.down, a.down_q, a.down_s, e, msz) : shm;
    return wrow<MX, I>(wm, x + (wv + W * (j & 1)) * stride);
  };
  auto actof = [&](int j) { return (const float*)hs + (j >> 1) * I; };
  auto sink = [&](int j, const float (&part)[4]) {
    const float v = wave_sum(part[0]);
    if (lane == 0) s_res[(j >> 1) * ROWS + wv + W * (j & 1)] = v;
  };
  const int hc = a.hc > kHcMax ? kHcMax : a.hc;
  auto pre = [&]() {
    // h vectors, global -> LDS directly (no registers held): group u's from
    // its entry's row, then the shared expert's
    constexpr int V = I / 4;  // float4 per vector
    static_assert(V % kWave == 0, "whole waves per vector");
    for (int m = 0; m <= ng; ++m) {
      const int row = m < ng ? __builtin_amdgcn_readlane(ebv, m < kMaxTopK ? m : 0) : kDecodeMaxSlots;
      const float* src = a.h32 + (int64_t)row * I;
#pragma unroll
      for (int k = 0; k < (V + kThreads - 1) / kThreads; ++k) {
        const int i = threadIdx.x + k * kThreads;  // float4 index; i - lane: the wave's first
        if (V % kThreads == 0 || i < V)
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + 4 * i),
                                           (__attribute__((address_space(3))) void*)(hs + m * I + 4 * (i - lane)), 16, 0, 0);
      }
    }
    const int t = threadIdx.x;
    if (hc > 0 && t < hc * ROWS) s_st[t] = a.hc_state[(int64_t)(t / ROWS) * H + x + (t % ROWS) * stride];
    if (hc > 0 && t < (2 + hc) * hc) s_map[t] = a.hc_maps[t];
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
    __syncthreads();
  };
  stream_rows_by<I, kNbuf1Down, MX, true, 2 * (kMaxTopK + 1)>(2 * (ng + 1), rowsrc, actof, 1, pre, sink);
  __syncthreads();
  const int t = threadIdx.x;
  if (t >= ROWS) return;
  const int h = x + t * stride;
  float o = 0.f;
#pragma unroll
  for (int u = 0; u < kMaxTopK; ++u)
    if (u < ng) o = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ewv), u)), s_res[u * ROWS + t], o);
  o += s_res[ng * ROWS + t];
  a.out[h] = o;
  if (hc > 0) {  // new[j] = post_j * out + sum_i comb[j][i] * state_i, i in order
#pragma unroll
    for (int j = 0; j < kHcMax; ++j) {
      if (j < hc) {
        float v = s_map[hc + j] * o;
#pragma unroll
        for (int i = 0; i < kHcMax; ++i)
          if (i < hc) v = fmaf(s_map[2 * hc + j * hc + i], s_st[i * ROWS + t], v);
        a.hc_out[(int64_t)j * H + h] = v;
      }
    }
  }
}

template <int H, int I, int MX>
hipError_t run_decode_t(const FwdArgs& a, hipStream_t s) {
  FwdArgs args = a;
  const int gmax = a.R * a.K < a.E ? a.R * a.K : a.E;
  hipError_t err;
  if (a.R == 1) {
    // one row: router launch, then gate/up blocks that route for
    // themselves, then the output-stationary down
    err = launch(MX == 2 ? "dec1_router_mx4" : MX ? "dec1_router_mx" : "dec1_router", (const void*)k_dec_head<H, I, true, MX>, dim3((a.E + 3) / 4),
                 dim3(kThreads), (size_t)H * 4, s, &args);
    if (err != hipSuccess) return err;
    err = launch(MX == 2 ? "dec1_gateup_mx4" : MX ? "dec1_gateup_mx" : "dec1_gateup", (const void*)k_dec1_gateup<H, I, MX>,
                 dim3(I / kShRows + gmax * (I / kGuRows)), dim3(kThreads), (size_t)H * 4, s, &args);
    if (err != hipSuccess) return err;
    return launch(MX == 2 ? "dec1_down_reduce_mx4" : MX ? "dec1_down_reduce_mx" : "dec1_down_reduce", (const void*)k_dec1_down<H, I, MX>,
                  dim3(H / 8), dim3(kThreads), (size_t)(gmax + 1) * I * 4, s, &args);
  }
  err = launch(MX == 2 ? "dec_head_mx4" : MX ? "dec_head_mx" : "dec_head", (const void*)k_dec_head<H, I, false, MX>,
               dim3((a.E + 3) / 4 + I / kShRows), dim3(kThreads), (size_t)a.R * H * 4, s, &args);
  if (err != hipSuccess) return err;
  err = launch(MX == 2 ? "dec_gateup_mx4" : MX ? "dec_gateup_mx" : "dec_gateup", (const void*)k_dec_gateup<H, I, MX>,
               dim3(H / kSdRows + gmax * (I / kGuRows)), dim3(kThreads), (size_t)a.R * H * 4, s, &args);
  if (err != hipSuccess) return err;
  err = launch(MX == 2 ? "dec_down_mx4" : MX ? "dec_down_mx" : "dec_down", (const void*)k_dec_down<H, I, MX>,
               dim3(H / kDnRows<MX>, gmax), dim3(kThreads), 0, s, &args);
  if (err != hipSuccess) return err;
  return launch("dec_reduce", (const void*)k_dec_reduce<H>, dim3(a.R * H / kThreads), dim3(kThreads), 0, s, &args);
}

}  // namespace

hipError_t run_decode(const FwdArgs& a, hipStream_t s) {
  if (a.H == 4096 && a.I == 2048)
    return a.mx == 2 ? run_decode_t<4096, 2048, 2>(a, s)
           : a.mx    ? run_decode_t<4096, 2048, 1>(a, s)
                     : run_decode_t<4096, 2048, 0>(a, s);
  if (a.H == 512 && a.I == 256)
    return a.mx == 2 ? run_decode_t<512, 256, 2>(a, s) : a.mx ? run_decode_t<512, 256, 1>(a, s) : run_decode_t<512, 256, 0>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
