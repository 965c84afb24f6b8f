// Prefill path (more than 4 rows): routed rows are grouped by expert and
// every projection is a grouped GEMM on the fp16 matrix cores.
//
//   k_pre_router   RMSNorm (f32) -> xn16 (fp16 GEMM operand); router logits
//                  on f32 activations; routing of each row (score top-k or
//                  hash) in the same block
//   k_pre_sort     counting sort of the (row, expert) pairs: per expert the
//                  ascending list of rows that chose it, plus each slot's
//                  rank in that list (one block per expert, stable)
//   k_gemm<0>      gate/up GEMM of every (expert, row-tile, column-tile),
//                  the shared expert being one more group, with SwiGLU in
//                  the epilogue -> h16
//   k_gemm<1>      down GEMM -> per-(expert,row) outputs in f32
//   k_pre_reduce   out[r] = sum_k w[r,k] * down_k + shared, slots in k order
//
// Steps and their order follow forward_ffn_rows on the hf2q ffn_forward.rs
// page; its "slotted" indexed matmul over [rows, top_k] becomes the sort +
// grouped GEMM here.
//
// Matrix-core precision: weights are bf16; activations (xn, and the SwiGLU
// output h) are rounded to fp16 and multiplied by the bf16 weights converted
// to fp16 (exact for |w| >= 2^-14, nearly so below), accumulating in f32 on
// v_mfma_f32_32x32x16_f16.  fp16 keeps 3 more mantissa bits than bf16 at the
// same matrix-core rate.
#include "device.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// ===========================================================================
// Router: 16 rows per block.
constexpr int kRB = 16;  // rows per block
constexpr int kKT = 32;  // router k-tile

template <int H>
__global__ __launch_bounds__(kThreads) void k_pre_router(const FwdArgs a) {
  __shared__ float s_rs[kRB];
  __shared__ float As[kKT][kRB];
  __shared__ float Bs[kKT * kMaxExperts];  // [kKT][E]; reused as logits [kRB][E]
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  const int E = a.E, K = a.K;
  const int64_t r0 = (int64_t)blockIdx.x * kRB;
  const int nrows = (int)((a.R - r0) < kRB ? (a.R - r0) : kRB);

  // 1. RMSNorm factors, and xn16 for the matrix-core GEMM
  for (int j = wv; j < kRB; j += kThreads / kWave) {
    if (j >= nrows) break;
    const float4* xr = (const float4*)(a.x + (r0 + j) * H);
    float ss = 0.f;
    for (int i = lane; i < H / 4; i += kWave) {
      float4 v = xr[i];
      ss = fmaf(v.x, v.x, ss); ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss); ss = fmaf(v.w, v.w, ss);
    }
    ss = wave_sum(ss);
    const float rs = 1.0f / sqrtf(ss / (float)H + a.eps);
    if (lane == 0) s_rs[j] = rs;
    half4* dst = (half4*)(a.xn16 + (r0 + j) * H);
    for (int i = lane; i < H / 4; i += kWave) {
      float4 v = xr[i];
      float4 g = ((const float4*)a.norm_w)[i];
      half4 o;
      o.x = (_Float16)(v.x * rs * g.x); o.y = (_Float16)(v.y * rs * g.y);
      o.z = (_Float16)(v.z * rs * g.z); o.w = (_Float16)(v.w * rs * g.w);
      dst[i] = o;
    }
  }
  __syncthreads();

  // 2. logits[16][E] = xn[16][H] . Wr[E][H]^T on f32 FMA.  Thread t owns
  //    rows 4*(t/64)..+4 and experts 4*(t%64)..+4.
  const int rg = (t / 64) * 4, eg = (t % 64) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += kKT) {
    {  // A tile: 16 rows x 32 k, normalised on the fly
      const int row = t / 16, kk = (t % 16) * 2;
      float v0 = 0.f, v1 = 0.f;
      if (row < nrows) {
        const float2 xv = *(const float2*)(a.x + (r0 + row) * H + k0 + kk);
        const float2 gv = *(const float2*)(a.norm_w + k0 + kk);
        v0 = xv.x * s_rs[row] * gv.x;
        v1 = xv.y * s_rs[row] * gv.y;
      }
      As[kk][row] = v0;
      As[kk + 1][row] = v1;
    }
    if (t < E) {  // B tile: expert t, 32 k
      const uint4* src = (const uint4*)(a.router + (int64_t)t * H + k0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float f[8];
        unpack8(src[q], f);
#pragma unroll
        for (int u = 0; u < 8; ++u) Bs[(q * 8 + u) * E + t] = f[u];
      }
    }
    __syncthreads();
    if (eg < E) {
#pragma unroll 8
      for (int kk = 0; kk < kKT; ++kk) {
        const float4 av = *(const float4*)&As[kk][rg];
        const float4 bv = *(const float4*)&Bs[kk * E + eg];
        const float ar[4] = {av.x, av.y, av.z, av.w};
        const float br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
      }
    }
    __syncthreads();
  }
  // 3. logits to LDS and workspace, then route each row with one wave
  if (eg < E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rg + i;
#pragma unroll
      for (int j = 0; j < 4; ++j) Bs[row * E + eg + j] = acc[i][j];
      if (row < nrows) {
        float4 o = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        *(float4*)(a.logits + (r0 + row) * E + eg) = o;
      }
    }
  }
  __syncthreads();
  for (int j = wv; j < nrows; j += kThreads / kWave) {
    const int64_t r = r0 + j;
    const int32_t tok = (a.layer_kind == MOE_LAYER_HASH) ? a.token_ids[r] : 0;
    RowRoute rr = route_row(Bs + j * E, E, K, a.layer_kind, a.bias, a.table, a.table_rows, tok);
    if (lane < K) {
      int iv = 0;
      float wv_ = 0.f;
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k)
        if (k == lane) { iv = rr.idx[k]; wv_ = rr.w[k]; }
      a.idx[r * K + lane] = iv;
      a.wts[r * K + lane] = wv_;
    }
    if (lane == 0) a.rowflags[r] = rr.flags;
  }
}

// ===========================================================================
// Counting sort: block e < E collects the rows that chose expert e (each row
// once, even if a malformed table lists e twice), in ascending row order,
// and the rank of each such slot.  Block E records the shared group's row
// count and folds the per-row status bits into the status word.
constexpr int kSortPer = 16;  // slots per thread per pass

__global__ __launch_bounds__(kThreads) void k_pre_sort(const FwdArgs a) {
  __shared__ int s_wsum[kThreads / kWave];
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  const int e = blockIdx.x, E = a.E, K = a.K;
  const int64_t R = a.R, S = R * K;
  if (e == E) {
    uint32_t f = 0;
    for (int64_t r = t; r < R; r += kThreads) f |= a.rowflags[r];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o, kWave);
    if (lane == 0) s_wsum[wv] = (int)f;
    __syncthreads();
    if (t == 0) {
      uint32_t tot = 0;
      for (int w = 0; w < kThreads / kWave; ++w) tot |= (uint32_t)s_wsum[w];
      a.status[0] = tot;
      a.sync->last_epoch = 0;  // no decode-path wait in this call
      a.cnt[E] = (int)R;
    }
    return;
  }
  int running = 0;
  for (int64_t c0 = 0; c0 < S; c0 += (int64_t)kThreads * kSortPer) {
    const int64_t s0 = c0 + (int64_t)t * kSortPer;
    unsigned flags = 0;
#pragma unroll
    for (int q = 0; q < kSortPer; ++q) {
      const int64_t s = s0 + q;
      if (s < S && a.idx[s] == e) {
        // count a row once: skip if an earlier slot of the row has e too
        const int64_t rb = s - s % K;
        bool dup = false;
        for (int64_t p = rb; p < s; ++p) dup |= (a.idx[p] == e);
        if (!dup) flags |= 1u << q;
      }
    }
    const int mine = __popc(flags);
    // block-wide exclusive scan of `mine`
    int incl = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) s_wsum[wv] = incl;
    __syncthreads();
    int before = running, total = running;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
      const int v = s_wsum[w];
      if (w < wv) before += v;
      total += v;
    }
    before += incl - mine;
    int rank = before;
#pragma unroll
    for (int q = 0; q < kSortPer; ++q) {
      if (flags & (1u << q)) {
        const int64_t s = s0 + q;
        a.perm[(int64_t)e * R + rank] = (int)(s / K);
        a.slot_rank[s] = rank;
        ++rank;
      }
    }
    running = total;
    __syncthreads();
  }
  if (t == 0) a.cnt[e] = running;
}

// ===========================================================================
// Grouped GEMM on fp16 MFMA.  Tile 128 (rows) x 128 (output columns) x 64
// (k), 4 waves in a 2 x 2 arrangement, each wave 64 x 64 from 32x32x16
// MFMAs.  MODE 0 (gate/up): the B tile holds 128 gate rows and the matching
// 128 up rows, and the epilogue writes silu(gate) * up as fp16.  MODE 1
// (down): the B tile holds 128 down rows, epilogue writes f32.
constexpr int BM = 128, BN = 128, BK = 64, LDSK = BK + 8;

template <int MODE>
struct GemmShape;
template <>
struct GemmShape<0> {
  static constexpr int BROWS = 2 * BN;
};
template <>
struct GemmShape<1> {
  static constexpr int BROWS = BN;
};

__device__ __forceinline__ uint2 bf16x4_to_f16x4(uint32_t lo, uint32_t hi) {
  // bf16 -> f32 -> f16 (round toward zero; exact whenever the value is an
  // fp16 normal, since bf16 carries fewer mantissa bits)
  auto p0 = __builtin_amdgcn_cvt_pkrtz(bf16lo(lo), bf16hi(lo));
  auto p1 = __builtin_amdgcn_cvt_pkrtz(bf16lo(hi), bf16hi(hi));
  uint2 r;
  r.x = *(uint32_t*)&p0;
  r.y = *(uint32_t*)&p1;
  return r;
}

template <int MODE, int KD, int ND>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(const FwdArgs a) {
  constexpr int BROWS = GemmShape<MODE>::BROWS;
  constexpr int NT = ND / BN;       // column tiles per group
  constexpr int NK = KD / BK;       // k tiles
  constexpr int AV = BM * BK / 8 / kThreads;     // 16B A vectors per thread (4)
  constexpr int BV = BROWS * BK / 8 / kThreads;  // 16B B vectors per thread (8 or 4)
  __shared__ _Float16 As[2][BM][LDSK];
  __shared__ _Float16 Bs[2][BROWS][LDSK];
  __shared__ int s_tbase[kMaxExperts + 2];
  __shared__ int s_rbase[kMaxExperts + 2];
  __shared__ int s_cnt[kMaxExperts + 1];

  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  const int E = a.E, G = E + 1;
  const int64_t R = a.R;

  // group prefix sums (rows and tiles), computed by wave 0
  if (wv == 0) {
    int rrun = 0, trun = 0;
    for (int g0 = 0; g0 < G; g0 += kWave) {
      const int g = g0 + lane;
      const int c = g < G ? a.cnt[g] : 0;
      const int tm = (c + BM - 1) / BM * NT;
      int ci = c, ti = tm;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        int v1 = __shfl_up(ci, o, kWave), v2 = __shfl_up(ti, o, kWave);
        if (lane >= o) { ci += v1; ti += v2; }
      }
      if (g < G) {
        s_cnt[g] = c;
        s_rbase[g] = rrun + ci - c;
        s_tbase[g] = trun + ti - tm;
      }
      rrun += __shfl(ci, kWave - 1, kWave);
      trun += __shfl(ti, kWave - 1, kWave);
    }
    if (lane == 0) {
      s_rbase[G] = rrun;
      s_tbase[G] = trun;
    }
  }
  __syncthreads();
  if (MODE == 0 && blockIdx.x == 0) {
    for (int g = t; g <= G; g += kThreads) a.base[g] = s_rbase[g];
  }
  const int total = s_tbase[G];
  const int wm = wv >> 1, wn = wv & 1;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    // locate the group: largest g with s_tbase[g] <= tile
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tbase[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int cntg = s_cnt[g];
    const int tm = (cntg + BM - 1) / BM;
    const int local = tile - s_tbase[g];
    const int mt = local % tm, nt = local / tm;
    const int m0 = mt * BM, n0 = nt * BN;
    const bool shared = g == E;

    // A row sources for this thread's vectors
    const _Float16* arow[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int v = t + kThreads * i;
      const int m = m0 + (v >> 3);
      if (m < cntg) {
        if (MODE == 0) {
          const int64_t r = shared ? (int64_t)m : (int64_t)a.perm[(int64_t)g * R + m];
          arow[i] = a.xn16 + r * KD + (v & 7) * 8;
        } else {
          arow[i] = a.h16 + (int64_t)(s_rbase[g] + m) * KD + (v & 7) * 8;
        }
      } else {
        arow[i] = nullptr;
      }
    }
    const uint16_t* brow[BV];
#pragma unroll
    for (int i = 0; i < BV; ++i) {
      const int v = t + kThreads * i;
      const int br = v >> 3;
      const uint16_t* basep;
      int64_t row;
      if (MODE == 0) {
        const bool is_up = br >= BN;
        basep = shared ? (is_up ? a.up_sh : a.gate_sh) : (is_up ? a.up : a.gate) + (int64_t)g * ND * KD;
        row = n0 + (is_up ? br - BN : br);
      } else {
        basep = shared ? a.down_sh : a.down + (int64_t)g * ND * KD;
        row = n0 + br;
      }
      brow[i] = basep + row * KD + (v & 7) * 8;
    }

    uint4 ra[AV], rb[BV];
    auto gload = [&](int kt) {
#pragma unroll
      for (int i = 0; i < AV; ++i)
        ra[i] = arow[i] ? *(const uint4*)(arow[i] + kt * BK) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < BV; ++i) rb[i] = *(const uint4*)(brow[i] + kt * BK);
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < AV; ++i) {
        const int v = t + kThreads * i;
        *(uint4*)&As[buf][v >> 3][(v & 7) * 8] = ra[i];
      }
#pragma unroll
      for (int i = 0; i < BV; ++i) {
        const int v = t + kThreads * i;
        const uint2 lo = bf16x4_to_f16x4(rb[i].x, rb[i].y);
        const uint2 hi = bf16x4_to_f16x4(rb[i].z, rb[i].w);
        *(uint4*)&Bs[buf][v >> 3][(v & 7) * 8] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    };

    constexpr int NB = (MODE == 0) ? 4 : 2;  // B fragments per wave (gate 2 + up 2, or 2)
    floatx16 acc[2][NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = floatx16{};

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < NK; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < NK) gload(kt + 1);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int kof = kk * 16 + (lane >> 5) * 8;
        half8 af[2], bfr[NB];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = *(const half8*)&As[buf][wm * 64 + i * 32 + (lane & 31)][kof];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          int brow_l;
          if (MODE == 0) brow_l = (j < 2 ? 0 : BN) + wn * 64 + (j & 1) * 32 + (lane & 31);
          else brow_l = wn * 64 + j * 32 + (lane & 31);
          bfr[j] = *(const half8*)&Bs[buf][brow_l][kof];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < NK) sstore(buf ^ 1);
      __syncthreads();
    }

    // epilogue: D[i][j] of a 32x32 tile sits in lane j + 32*((i/4)%2),
    // register 4*(i/8) + i%4
    const int rb0 = s_rbase[g];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int mrow = m0 + wm * 64 + i * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v & 3);
        if (mrow >= cntg) continue;
        const int64_t orow = (int64_t)(rb0 + mrow);
        if (MODE == 0) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + (lane & 31);
            const float gv = acc[i][j][v], uv = acc[i][j + 2][v];
            a.h16[orow * ND + col] = (_Float16)swiglu_f32(gv, uv);
          }
        } else {
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int col = n0 + wn * 64 + j * 32 + (lane & 31);
            a.dbuf[orow * ND + col] = acc[i][j][v];
          }
        }
      }
    }
  }
}

// ===========================================================================
// Weighted reduce: out[r] = sum_k w[r,k] * down(expert idx[r,k]) + shared,
// slots in k order; masked slots skipped.  One block per row.
template <int H>
__global__ __launch_bounds__(kThreads) void k_pre_reduce(const FwdArgs a) {
  const int64_t r = blockIdx.x;
  const int K = a.K, E = a.E, t = threadIdx.x;
  int pos[kMaxTopK];
  float wk[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    pos[k] = -1;
    wk[k] = 0.f;
    if (k < K) {
      const int e = a.idx[r * K + k];
      if (e >= 0 && e < E) {
        int kf = k;  // first slot of this row with the same expert
        for (int p = k - 1; p >= 0; --p)
          if (a.idx[r * K + p] == e) kf = p;
        pos[k] = a.base[e] + a.slot_rank[r * K + kf];
        wk[k] = a.wts[r * K + k];
      }
    }
  }
  const int64_t shpos = (int64_t)a.base[E] + r;
#pragma unroll
  for (int c = t; c < H / 4; c += kThreads) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
      if (pos[k] >= 0) {
        const float4 d = ((const float4*)(a.dbuf + (int64_t)pos[k] * H))[c];
        acc.x = fmaf(wk[k], d.x, acc.x); acc.y = fmaf(wk[k], d.y, acc.y);
        acc.z = fmaf(wk[k], d.z, acc.z); acc.w = fmaf(wk[k], d.w, acc.w);
      }
    }
    const float4 s = ((const float4*)(a.dbuf + shpos * H))[c];
    acc.x += s.x; acc.y += s.y; acc.z += s.z; acc.w += s.w;
    ((float4*)(a.out + r * H))[c] = acc;
  }
}

// ===========================================================================
// Stand-alone routing from given logits: one wave per row.
__global__ __launch_bounds__(kThreads) void k_route(const RouteArgs a) {
  const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int64_t r = (int64_t)blockIdx.x * (kThreads / kWave) + wv;
  if (r >= a.R) return;
  const int32_t tok = (a.layer_kind == MOE_LAYER_HASH) ? a.token_ids[r] : 0;
  RowRoute rr = route_row(a.logits + r * a.E, a.E, a.K, a.layer_kind, a.bias, a.table, a.table_rows, tok);
  if (lane < a.K) {
    int iv = 0;
    float wv_ = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
      if (k == lane) { iv = rr.idx[k]; wv_ = rr.w[k]; }
    a.idx[r * a.K + lane] = iv;
    a.w[r * a.K + lane] = wv_;
  }
}

int gemm_grid() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

template <int H, int I>
hipError_t run_prefill_t(const FwdArgs& a, hipStream_t s) {
  FwdArgs args = a;
  hipError_t err = launch("pre_router", (const void*)k_pre_router<H>, dim3((a.R + kRB - 1) / kRB), dim3(kThreads), 0,
                          s, &args);
  if (err != hipSuccess) return err;
  err = launch("pre_sort", (const void*)k_pre_sort, dim3(a.E + 1), dim3(kThreads), 0, s, &args);
  if (err != hipSuccess) return err;
  const int grid = gemm_grid();
  err = launch("gemm_gateup_swiglu", (const void*)k_gemm<0, H, I>, dim3(grid), dim3(kThreads), 0, s, &args);
  if (err != hipSuccess) return err;
  err = launch("gemm_down", (const void*)k_gemm<1, I, H>, dim3(grid), dim3(kThreads), 0, s, &args);
  if (err != hipSuccess) return err;
  return launch("pre_reduce", (const void*)k_pre_reduce<H>, dim3(a.R), dim3(kThreads), 0, s, &args);
}

}  // namespace

hipError_t run_prefill(const FwdArgs& a, hipStream_t s) {
  if (a.H == 4096 && a.I == 2048) return run_prefill_t<4096, 2048>(a, s);
  if (a.H == 512 && a.I == 256) return run_prefill_t<512, 256>(a, s);
  return hipErrorInvalidValue;
}

hipError_t run_route(const RouteArgs& a, hipStream_t s) {
  RouteArgs args = a;
  const int per = kThreads / kWave;
  return launch("route", (const void*)k_route, dim3((a.R + per - 1) / per), dim3(kThreads), 0, s, &args);
}

}  // namespace moe
