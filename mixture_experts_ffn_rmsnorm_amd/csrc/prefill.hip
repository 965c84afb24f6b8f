// Prefill path (more than 4 rows): routed rows are grouped by expert and
// every projection is a grouped GEMM on the fp16 matrix cores.
//
//   k_pre_norm     RMSNorm -> xn16 (fp16 GEMM operand) and its rounding
//                  remainder xlo16, one wave per row
//   k_pre_router   router logits on the matrix cores (hi/lo split
//                  activations), experts sliced over blocks for small
//                  batches; routing of each row; per expert a mask of the
//                  group's rows that chose it
//   k_pre_sort     per expert the ascending list of rows that chose it, plus
//                  each slot's rank in that list (one block per expert)
//   k_gemm<0>      gate/up GEMM of every (expert, row-tile, column-tile),
//                  the shared expert being one more group, with SwiGLU in
//                  the epilogue -> h16
//   k_gemm<1>      routed down GEMM -> per-(expert,row) outputs in fp16
//   k_gemm<2>      shared down GEMM whose epilogue adds the weighted routed
//                  outputs, slots in k order -> out
//
// Steps and their order follow forward_ffn_rows on the hf2q ffn_forward.rs
// page; its "slotted" indexed matmul over [rows, top_k] becomes the sort +
// grouped GEMM here.
//
// Matrix-core precision: weights are bf16, or block-scaled 8-bit or 4-bit
// codes (E4M3, or E2M1 two per byte, with an E8M0 scale per 32 inputs: OCP
// MXFP8 / MXFP4); activations (xn, and the
// SwiGLU output h) are rounded to fp16 and multiplied by the weights
// converted to fp16 (bf16: exact for 2^-14 <= |w| <= 65504, within 2^-25
// below; MX: the decoded value code * 2^(scale-127) rounded to nearest even
// fp16, so exact in the same range), accumulating in f32 on
// v_mfma_f32_32x32x16_f16.  fp16 keeps 3 more mantissa bits than
// bf16 at the same matrix-core rate, at the price of its range: an operand
// beyond 65504 in magnitude becomes infinite, and the router (non-finite
// logit) or a GEMM epilogue (non-finite h, routed down output or layer
// output) then sets MOE_FLAG_F16_RANGE in the status word.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f32x2_to_f16x2(float a, float b) {
  // one v_cvt_pk_f16_f32: round to nearest even, so a magnitude beyond
  // fp16's range becomes infinite (and is reported) instead of clamped
  const half2v h = __builtin_convertvector((float2v){a, b}, half2v);
  return *(const uint32_t*)&h;
}

__device__ __forceinline__ uint2 bf16x4_to_f16x4(uint32_t lo, uint32_t hi) {
  // bf16 -> f32 -> f16: exact for every bf16 value in fp16's normal range
  // (bf16 carries fewer mantissa bits), within 2^-25 below it (subnormal),
  // infinite above 65504
  uint2 r;
  r.x = f32x2_to_f16x2(bf16lo(lo), bf16hi(lo));
  r.y = f32x2_to_f16x2(bf16lo(hi), bf16hi(hi));
  return r;
}

__device__ __forceinline__ uint4 bf16x8_to_f16x8(const uint4& q) {
  const uint2 lo = bf16x4_to_f16x4(q.x, q.y);
  const uint2 hi = bf16x4_to_f16x4(q.z, q.w);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// SwiGLU for an fp16 result: silu(g) * u with the hardware exp2 and
// reciprocal (relative error ~1e-6, far below the fp16 rounding that follows)
__device__ __forceinline__ float swiglu_fast(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// chunk swizzle of a 128-byte LDS row
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// chunk swizzle of a row of weight codes in LDS: 8 chunks (one 128-byte
// row per line) as above; 4 chunks (two 64-byte rows per line) by
// (row / 4) & 3; 2 chunks (four 32-byte rows per line) by (row / 8) & 1 --
// so that 16 consecutive rows read at one chunk hit 16 distinct 16-byte bank
// groups
__device__ __forceinline__ int mxsw(int row, int cpr) {
  return cpr == 8 ? swz(row) : cpr == 4 ? (row >> 2) & 3 : (row >> 3) & 1;
}
// dword swizzle of a scale row of `dpr` dwords: the rows that share a
// 256-byte span rotate their dwords, so 32 consecutive rows reading one
// dword hit 32 distinct banks
__device__ __forceinline__ int ssw(int row, int dpr) { return (row / (64 / dpr)) & (dpr - 1); }

// 16 bytes per lane from global memory into LDS, lanes filling consecutive
// 16-byte slots from the wave-uniform LDS byte address `lds`.  Completion is
// counted by vmcnt like any vector load.
// m0 is a reserved register the compiler may assume unchanged; none of the
// code generated for these kernels reads or writes it other than here (the
// kernels' assembly holds no other m0 access), so clobbering it is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
// 4 bytes per lane, lanes filling consecutive 4-byte slots from `lds`
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// An E8M0 block scale 2^(c-127) as an f32 operand of the scaled conversions
// (c = 0 is the subnormal 2^-127, c = 255 is NaN).
__device__ __forceinline__ float e8m0_scale(uint32_t c) {
  return c == 0 ? __uint_as_float(0x00400000u) : (c == 255 ? __uint_as_float(0x7fc00000u) : __uint_as_float(c << 23));
}

// Eight E4M3 codes (little-endian bytes of lo, hi) times `scale`, rounded to
// nearest even fp16, in k order: v_cvt_scalef32_pk_f16_fp8 converts the two
// codes of one 16-bit half of its source.  Each result is taken as a whole
// 32-bit word: extracting the halves of the builtin's vector result
// duplicates its low half (measured: every odd code read back as its even
// neighbour), while the word itself holds both conversions exactly.
__device__ __forceinline__ uint4 fp8x8_to_f16x8(uint32_t lo, uint32_t hi, float scale) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, scale, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, scale, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, scale, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, scale, true));
  return r;
}

// Eight E2M1 codes (the nibbles of w, lowest first) times `scale`, rounded
// to nearest even fp16, in k order: v_cvt_scalef32_pk_f16_fp4 converts the
// two codes of one byte; results taken as whole 32-bit words as above.
__device__ __forceinline__ uint4 fp4x8_to_f16x8(uint32_t w, float scale) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 3));
  return r;
}

// s_waitcnt vmcnt(N) with the other counters left alone
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ===========================================================================
// Routing of one row by 8 consecutive lanes (lane `sub` of the group); the
// returned slot is slot `sub` (meaningful for sub < K).  Same results as the
// one-wave routines: score route by key sigmoid(logit) + bias (float64)
// descending, equal keys to the lower expert, weights the unbiased sigmoids
// of the chosen logits over their sum in slot order; hash route by the token
// id's table row with invalid ids / entries masked.
struct RowPick {
  int idx;
  float w;
  bool valid;
  uint32_t flags;
};

// weights of the K picks: s_k = sigmoid(l_k) (0 if masked), w_k = s_k / sum
// with the sum taken in slot order; lane `sub` holds slot sub's s
__device__ __forceinline__ float weight_8(double s_mine, int K, int sub) {
  const int base = (threadIdx.x & (kWave - 1)) & ~7;
  double tot = 0.0;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    const double sk = __shfl(s_mine, base + k, kWave);
    if (k < K) tot += sk;
  }
  return (sub < K && tot > 0.0) ? (float)(s_mine / tot) : 0.0f;
}

// (key, expert) of the lane DPP control CTRL selects, kept if it ranks first
template <int CTRL>
__device__ __forceinline__ void pick_best_dpp(uint64_t& bu, int& be) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)bu, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(bu >> 32), CTRL, 0xF, 0xF, false);
  const int oe = __builtin_amdgcn_update_dpp(0, be, CTRL, 0xF, 0xF, false);
  const uint64_t ou = ((uint64_t)hi << 32) | lo;
  if (ou > bu || (ou == bu && oe < be)) { bu = ou; be = oe; }
}

template <int EMAX>
__device__ __forceinline__ RowPick pick_score_8_t(const double* key, const float* lg, int E, int K, int sub) {
  constexpr int PER = EMAX / 8;  // experts per lane: e = sub + 8 i
  uint64_t u[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = sub + 8 * i;
    u[i] = e < E ? ordered_key(key[e]) : 0ull;
  }
  int mine = 0;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k >= K) break;
    // the lane's best: four independent chains (keys i = c, c + 4, ...;
    // the first of equal keys kept), then the chains by (key, lower expert)
    uint64_t cu[4] = {0ull, 0ull, 0ull, 0ull};
    int ce[4] = {0x7fffffff, 0x7fffffff, 0x7fffffff, 0x7fffffff};
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (u[i] > cu[i % 4]) { cu[i % 4] = u[i]; ce[i % 4] = sub + 8 * i; }
    uint64_t bu = cu[0];
    int be = ce[0];
#pragma unroll
    for (int c = 1; c < 4; ++c)
      if (cu[c] > bu || (cu[c] == bu && ce[c] < be)) { bu = cu[c]; be = ce[c]; }
    // the 8 lanes' best, by DPP moves (lane pairs 1 apart, 2 apart, then
    // the mirror of the 8); the order (key, then lower expert) is total, so
    // every lane ends with the group's best
    pick_best_dpp<0xB1>(bu, be);
    pick_best_dpp<0x4E>(bu, be);
    pick_best_dpp<0x141>(bu, be);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (sub + 8 * i == be) u[i] = 0ull;
    if (k == sub) mine = be;
  }
  RowPick rp;
  rp.idx = mine;
  rp.valid = sub < K;
  rp.flags = 0;
  rp.w = weight_8(sub < K ? sigmoid_f64(lg[mine]) : 0.0, K, sub);
  return rp;
}

__device__ __forceinline__ RowPick pick_score_8(const double* key, const float* lg, int E, int K, int sub) {
  return E <= 32 ? pick_score_8_t<32>(key, lg, E, K, sub) : pick_score_8_t<kMaxExperts>(key, lg, E, K, sub);
}

__device__ __forceinline__ RowPick pick_hash_8(const float* lg, int E, int K, const int32_t* __restrict__ table,
                                              int64_t table_rows, int32_t token, int sub) {
  RowPick rp;
  const bool tok_ok = token >= 0 && (int64_t)token < table_rows;
  const int e = (tok_ok && sub < K) ? table[(int64_t)token * K + sub] : -1;
  rp.idx = e;
  rp.valid = tok_ok && sub < K && e >= 0 && e < E;
  rp.flags = !tok_ok ? (uint32_t)MOE_FLAG_BAD_TOKEN : 0u;
  // a bad entry anywhere in the row flags the row (each slot reports its own)
  const bool bad_entry = tok_ok && sub < K && !rp.valid;
  uint32_t any_bad = bad_entry ? 1u : 0u;
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) any_bad |= (uint32_t)__shfl_xor((int)any_bad, m, kWave);
  if (any_bad) rp.flags |= MOE_FLAG_BAD_TABLE_ENTRY;
  rp.w = weight_8(rp.valid ? sigmoid_f64(lg[e]) : 0.0, K, sub);
  return rp;
}

// ===========================================================================
// RMSNorm of the batch, one wave per row: rs = rsqrt(mean(x^2) + eps) and
// xn = x * rs * g (f32), split into hi = fp16(xn) and lo = fp16(xn - hi),
// which together carry about 22 significant bits.  hi is the fp16 operand
// the expert GEMMs take (xn16); lo (xlo16) joins it in the router GEMM.
// Block 0 also clears the router's per-group arrival counters and the
// GEMM launches' tail-tile counters.
constexpr int kRR = kPrefillBlockRows;  // rows per router group (one MFMA row fragment)

template <int H>
__global__ __launch_bounds__(kThreads) void k_pre_norm(const FwdArgs a) {
  constexpr int V4 = H / 4 / kWave;  // float4 of a row per lane
  static_assert(H % (4 * kWave) == 0, "row split over the lanes");
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  if (blockIdx.x == 0) {
    const int64_t nb = (a.R + kRR - 1) / kRR;
    for (int64_t i = t; i < nb; i += kThreads) a.rcnt[i] = 0;
    if (t < 4) a.gctr[t] = 0;
  }
  const int64_t r = (int64_t)blockIdx.x * (kThreads / kWave) + wv;
  if (r >= a.R) return;
  float4 v[V4], g[V4];
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    v[i] = ((const float4*)(a.x + r * H))[i * kWave + lane];
    g[i] = ((const float4*)a.norm_w)[i * kWave + lane];
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    ss = fmaf(v[i].x, v[i].x, ss); ss = fmaf(v[i].y, v[i].y, ss);
    ss = fmaf(v[i].z, v[i].z, ss); ss = fmaf(v[i].w, v[i].w, ss);
  }
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / (float)H + a.eps);
  half4* hp = (half4*)(a.xn16 + r * H);
  half4* lp = (half4*)(a.xlo16 + r * H);
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    float xn[4] = {v[i].x * rs * g[i].x, v[i].y * rs * g[i].y, v[i].z * rs * g[i].z, v[i].w * rs * g[i].w};
    half4 h, l;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // xn is pinned as an f32 value first: hi must be the rounding of the
      // same f32 xn that lo is taken from (a multiply fused with the fp16
      // rounding can round a tie the other way)
      asm volatile("" : "+v"(xn[u]));
      h[u] = (_Float16)xn[u];
      l[u] = (_Float16)(xn[u] - (float)h[u]);
    }
    hp[i * kWave + lane] = h;
    lp[i * kWave + lane] = l;
  }
}

// ===========================================================================
// Router on the matrix cores.  Block (s, b) takes the 32 rows of group b and
// experts s*E/S .. (s+1)*E/S - 1 (S expert slices; more slices when the
// batch has few groups, so that small batches still spread over the chip).
//  1. logits = hi.W + lo.W on the 32x32x16 fp16 MFMA with f32 accumulation;
//     the bf16 router weights convert to fp16 exactly (for magnitudes in the
//     fp16 normal range).  Operand tiles reach LDS by direct global->LDS
//     loads through a ring as deep as LDS allows (a narrower expert slice
//     leaves room for more k-tiles in flight).  With fewer 32-expert
//     fragments than waves, the waves of a fragment split its k-steps and
//     add their partial sums in a fixed order.
//  2. With S > 1 a block writes its logit columns through to the workspace
//     and counts itself in the group's arrival counter; the group's last
//     block reads all E logits of its rows back and routes them.
//  3. Selection keys sigmoid(l) + bias (float64; the bias staged in LDS) of
//     all 32 x E logits, by all threads at once; then 8 lanes per row pick
//     its top-k (each lane's best of its experts, the 8 lanes' best by DPP
//     moves; or look up its hash row), and the block publishes, per expert,
//     the 32-bit mask of its rows that chose the expert, which is all the
//     sort needs.
constexpr int kRK = 64;                 // k-tile (one 128-byte row per operand row)
constexpr int kRBudget = 144 * 1024;    // LDS bytes of the router ring

template <int E, int S>
struct RouterShape {
  static constexpr int EL = E / S;                             // experts per block
  static constexpr int ST = 2 * kRR * kRK * 2 + EL * kRK * 2;  // hi + lo + router tile
  static constexpr int NSTG = kRBudget / ST < 12 ? kRBudget / ST : 12;
};

template <int H, int E, int S>
__global__ __launch_bounds__(kThreads, 1) void k_pre_router(const FwdArgs a) {
  constexpr int EL = RouterShape<E, S>::EL;
  constexpr int NF = EL / 32;                 // 32-expert fragments
  constexpr int FPW = (NF + 3) / 4;           // fragments per wave
  constexpr int NK = H / kRK;
  constexpr int A_ST = kRR * kRK * 2;         // one of the hi / lo tiles
  constexpr int B_ST = EL * kRK * 2;
  constexpr int ST = RouterShape<E, S>::ST;
  constexpr int NSTG = RouterShape<E, S>::NSTG;
  constexpr int BI = B_ST / 16 / kThreads;    // B DMA instructions per thread per k-tile
  constexpr int LPS = 2 + BI;                 // vector-memory ops per thread per k-tile
  static_assert(EL % 32 == 0 && BI >= 1 && BI * kThreads * 16 == B_ST && A_ST == kThreads * 16, "router tiling");
  static_assert(NSTG >= 3 && (NSTG - 2) * LPS < 64, "router ring");
  static_assert(kRR * E * 4 + kRR * E * 8 <= NSTG * ST, "logits and keys reuse the ring");
  static_assert(kRR * E * 12 + 4 * 16 * kWave * 4 <= NSTG * ST, "partial sums after the logits and keys");
  static_assert(NK >= 2, "router k loop");
  __shared__ __align__(16) unsigned char s_ring[NSTG * ST];
  __shared__ uint32_t s_mask[E];
  __shared__ float s_bias[E];  // the selection bias, staged once (score layers)
  __shared__ uint32_t s_flags;
  __shared__ int s_last;
  float* s_logit = reinterpret_cast<float*>(s_ring);                 // [kRR][E] after the k loop
  double* s_key = reinterpret_cast<double*>(s_ring + kRR * E * 4);   // [kRR][E]

  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  const int K = a.K;
  const int64_t nb = (a.R + kRR - 1) / kRR;
  const int64_t rb = blockIdx.x % nb;  // row group; its S slices are nb blocks apart
  const int e0 = (int)(blockIdx.x / nb) * EL;
  const int64_t r0 = rb * kRR;
  const int nrows = (int)((a.R - r0) < kRR ? (a.R - r0) : kRR);
  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)s_ring;
  for (int e = t; e < E; e += kThreads) {
    s_mask[e] = 0;
    s_bias[e] = a.layer_kind != MOE_LAYER_HASH && e < a.E ? a.bias[e] : 0.f;
  }
  if (t == 0) s_flags = 0;

  // 1. logits[32][e0 .. e0+EL).  DMA: the hi and lo tiles take one
  //    instruction each (wave w: rows 8w..8w+7), the router tile BI (rows
  //    (w*BI + i)*8 + lane/8); chunk (lane & 7) ^ swz(row) of each 128-byte row.
  const int chunk_even = ((lane & 7) ^ (lane >> 3)) * 16, chunk_odd = chunk_even ^ 16;
  const int arow_l = wv * 8 + (lane >> 3);
  const int64_t arow_g = r0 + (arow_l < nrows ? arow_l : nrows - 1);
  const unsigned char* ahi = (const unsigned char*)(a.xn16 + arow_g * H) + ((wv & 1) ? chunk_odd : chunk_even);
  const unsigned char* alo = (const unsigned char*)(a.xlo16 + arow_g * H) + ((wv & 1) ? chunk_odd : chunk_even);
  const unsigned char* bsrc = (const unsigned char*)(a.router + (int64_t)(e0 + wv * BI * 8 + (lane >> 3)) * H);
  const uint32_t a_wave = __builtin_amdgcn_readfirstlane(wv * 1024);
  const uint32_t b_wave = __builtin_amdgcn_readfirstlane(2 * A_ST + wv * BI * 1024);
  auto issue = [&](int kt) {
    const uint32_t base = ring + (uint32_t)(kt % NSTG) * ST;
    dma16(ahi + kt * (kRK * 2), base + a_wave);
    dma16(alo + kt * (kRK * 2), base + A_ST + a_wave);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      dma16(bsrc + (int64_t)i * 8 * H * 2 + kt * (kRK * 2) + (((wv * BI + i) & 1) ? chunk_odd : chunk_even),
            base + b_wave + i * 1024);
  };
  // fragment rows: A row lane & 31; B rows of fragment f: f*32 + lane & 31
  // (fragments past NF, on the small shapes, repeat fragment f % NF and are
  // not stored)
  int bro[FPW];
#pragma unroll
  for (int q = 0; q < FPW; ++q) bro[q] = ((wv + 4 * q) % NF) * 32 + (lane & 31);
  const int aro = lane & 31;
  floatx16 acc_hi[FPW], acc_lo[FPW];
#pragma unroll
  for (int q = 0; q < FPW; ++q) { acc_hi[q] = floatx16{}; acc_lo[q] = floatx16{}; }
  // With fewer fragments than waves, the WPF waves of one fragment split each
  // k-tile's k-steps (wave split s takes steps s, s + WPF, ...) and their
  // partial sums are added at the end in split order.
  constexpr int WPF = NF < 4 ? 4 / NF : 1;
  constexpr int NSW = (kRK / 16) / WPF;  // k-steps per k-tile of one wave
  static_assert(NF >= 4 || 4 % NF == 0, "fragments share the waves evenly");
  const int split = NF < 4 ? wv / NF : 0;
  auto read = [&](int kt, int st, half8& ah, half8& al, uint4 (&bq)[FPW]) {
    const unsigned char* Sb = s_ring + (kt % NSTG) * ST;
    const int c = 2 * st + (lane >> 5);
    const int ao = aro * 128 + ((c ^ swz(aro)) << 4);
    ah = *(const half8*)(Sb + ao);
    al = *(const half8*)(Sb + A_ST + ao);
#pragma unroll
    for (int q = 0; q < FPW; ++q) bq[q] = *(const uint4*)(Sb + 2 * A_ST + bro[q] * 128 + ((c ^ swz(bro[q])) << 4));
  };
  auto mma = [&](const half8& ah, const half8& al, const uint4 (&bq)[FPW]) {
#pragma unroll
    for (int q = 0; q < FPW; ++q) {
      const uint4 cv = bf16x8_to_f16x8(bq[q]);
      const half8 bf = *(const half8*)&cv;
      acc_hi[q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bf, acc_hi[q], 0, 0, 0);
      acc_lo[q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bf, acc_lo[q], 0, 0, 0);
    }
  };
  // NSTG-1 k-tiles in flight; past the end the refill re-loads the last
  // k-tile into the buffer just freed, so every wait counts the same loads.
  // A wave's next k-step is read before the current one's MFMAs, across
  // k-tile boundaries too (the barrier comes before the next tile's read).
#pragma unroll
  for (int st = 0; st + 1 < NSTG; ++st) issue(st < NK ? st : NK - 1);
  wait_vmcnt<(NSTG - 2) * LPS>();
  __syncthreads();  // k-tile 0 landed for every wave
  issue(NSTG - 1 < NK ? NSTG - 1 : NK - 1);
  half8 ah, al;
  uint4 bq[FPW];
  read(0, split, ah, al, bq);
#pragma unroll 1
  for (int kt = 0; kt < NK; ++kt) {
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
      half8 ahn, aln;
      uint4 bqn[FPW];
      if (i + 1 < NSW) {
        read(kt, split + WPF * (i + 1), ahn, aln, bqn);
      } else if (kt + 1 < NK) {
        wait_vmcnt<(NSTG - 2) * LPS>();
        __syncthreads();  // k-tile kt+1 landed for every wave; every wave is done reading kt's buffer
        issue(kt + NSTG < NK ? kt + NSTG : NK - 1);
        read(kt + 1, split, ahn, aln, bqn);
      } else {  // the last step: nothing follows
        ahn = ah;
        aln = al;
#pragma unroll
        for (int q = 0; q < FPW; ++q) bqn[q] = bq[q];
      }
      mma(ah, al, bq);
      ah = ahn;
      al = aln;
#pragma unroll
      for (int q = 0; q < FPW; ++q) bq[q] = bqn[q];
    }
  }
  wait_vmcnt<0>();   // the trailing refills land before the ring is reused
  __syncthreads();  // the ring becomes the logit and key tiles
  if constexpr (WPF > 1) {
    // the partial sums of each fragment, added in split order by the wave
    // with split 0 (which then holds the fragment's logits in acc_hi)
    float* s_part = reinterpret_cast<float*>(s_ring + kRR * E * 12);  // [4 waves][16][64]
#pragma unroll
    for (int v = 0; v < 16; ++v) s_part[(wv * 16 + v) * kWave + lane] = acc_hi[0][v] + acc_lo[0][v];
    __syncthreads();
    if (split == 0) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float sum = s_part[(wv * 16 + v) * kWave + lane];
        for (int sp = 1; sp < WPF; ++sp) sum += s_part[((wv + sp * NF) * 16 + v) * kWave + lane];
        acc_hi[0][v] = sum;
        acc_lo[0][v] = 0.f;
      }
    }
    __syncthreads();
  }

  // logits (D[i][j] of a 32x32 tile sits in lane j + 32*((i/4)%2), register
  // 4*(i/8) + i%4)
  if constexpr (S == 1) {
#pragma unroll
    for (int q = 0; q < FPW; ++q) {
      const int f = wv + 4 * q;
      if (f < NF) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          s_logit[i * E + f * 32 + (lane & 31)] = acc_hi[q][v] + acc_lo[q][v];
        }
      }
    }
    __syncthreads();
    for (int v = t; v < nrows * E / 4; v += kThreads)
      ((float4*)(a.logits + r0 * E))[v] = ((const float4*)s_logit)[v];
  } else {
    // 2. this block's columns, written through; the group's last block
    //    routes
#pragma unroll
    for (int q = 0; q < FPW; ++q) {
      const int f = wv + 4 * q;
      if (f < NF) {  // (with split k-steps, f < NF is the split-0 wave)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (i < nrows)
            __hip_atomic_store(&a.logits[(r0 + i) * E + e0 + f * 32 + (lane & 31)], acc_hi[q][v] + acc_lo[q][v],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __threadfence();  // release: the columns are visible device-wide before the count
    __syncthreads();
    if (t == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&a.rcnt[rb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev + 1 == (uint32_t)S;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();  // acquire: every slice's columns are visible to the loads below
    for (int v = t; v < nrows * E / 4; v += kThreads)
      ((float4*)s_logit)[v] = ((const float4*)(a.logits + r0 * E))[v];
    __syncthreads();
  }

  // 3. keys; routing.  A non-finite logit (an fp16 operand beyond range,
  //    or a non-finite input) is reported in the status word.
  const bool score = a.layer_kind != MOE_LAYER_HASH;
  {
    bool bad = false;
#pragma unroll 4
    for (int q = t; q < nrows * E; q += kThreads) {
      const float l = s_logit[q];
      bad |= !__builtin_isfinite(l);
      if (score) s_key[q] = score_key(l, s_bias[q % E]);
    }
    if (bad) atomicOr(&s_flags, (uint32_t)MOE_FLAG_F16_RANGE);
    __syncthreads();
  }
  // one row per 8 consecutive lanes: all 32 rows at once
  {
    const int j = t >> 3, sub = t & 7;
    if (j < nrows) {
      const int64_t r = r0 + j;
      RowPick rp = score ? pick_score_8(s_key + j * E, s_logit + j * E, E, K, sub)
                         : pick_hash_8(s_logit + j * E, E, K, a.table, a.table_rows, a.token_ids[r], sub);
      if (sub < K) {
        a.idx[r * K + sub] = rp.idx;
        a.wts[r * K + sub] = rp.w;
        if (rp.valid) atomicOr(&s_mask[rp.idx], 1u << j);
        else a.slot_rank[r * K + sub] = -1;
      }
      if (sub == 0 && rp.flags) atomicOr(&s_flags, rp.flags);
    }
  }
  __syncthreads();
  for (int e = t; e < E; e += kThreads) a.mask[(int64_t)e * nb + rb] = s_mask[e];
  if (t == 0) a.rowflags[rb] = s_flags;
}

// ===========================================================================
// Sort: block e < E turns the router blocks' row masks for expert e into the
// ascending list of rows that chose e (perm) and each such slot's rank in
// it (slot_rank; a row listed twice by a malformed table gets one rank for
// both slots).  Thread t owns a contiguous run of masks, so one block-wide
// scan of the per-thread popcounts places every row.  Block E records the
// shared group's row count and folds the router blocks' status bits into
// the status word.
__global__ __launch_bounds__(kThreads) void k_pre_sort(const FwdArgs a) {
  __shared__ int s_wsum[kThreads / kWave];
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  const int e = blockIdx.x, E = a.E, K = a.K;
  const int64_t R = a.R, nb = (R + kRR - 1) / kRR;
  if (e == E) {
    uint32_t f = 0;
    for (int64_t b = t; b < nb; b += kThreads) f |= a.rowflags[b];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o, kWave);
    if (lane == 0) s_wsum[wv] = (int)f;
    __syncthreads();
    if (t == 0) {
      uint32_t tot = 0;
      for (int w = 0; w < kThreads / kWave; ++w) tot |= (uint32_t)s_wsum[w];
      a.status[0] = tot;
      a.cnt[E] = (int)R;
    }
    return;
  }
  const uint32_t* m = a.mask + (int64_t)e * nb;
  const int64_t per = (nb + kThreads - 1) / kThreads;
  const int64_t b0 = (int64_t)t * per, b1 = (b0 + per < nb) ? b0 + per : nb;
  int mine = 0;
  for (int64_t b = b0; b < b1; ++b) mine += __popc(m[b]);
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) s_wsum[wv] = incl;
  __syncthreads();
  int rank = incl - mine, total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) {
    const int v = s_wsum[w];
    if (w < wv) rank += v;
    total += v;
  }
  // rows of each mask word in ascending order, 8 at a time: their slots'
  // expert indices are all requested before any is compared (one memory
  // round trip per 8 rows, not one per slot)
  int32_t* perm = a.perm + (int64_t)e * R;
  constexpr int kB = 8;
  for (int64_t b = b0; b < b1; ++b) {
    uint32_t bits = m[b];
    while (bits) {
      int64_t rows[kB];
      int n = 0;
#pragma unroll
      for (int q = 0; q < kB; ++q) {
        rows[q] = -1;
        if (bits) {
          rows[q] = b * kRR + (__ffs(bits) - 1);
          bits &= bits - 1;
          n = q + 1;
        }
      }
      int ids[kB][kMaxTopK];
#pragma unroll
      for (int q = 0; q < kB; ++q)
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) ids[q][k] = (rows[q] >= 0 && k < K) ? a.idx[rows[q] * K + k] : -1;
#pragma unroll
      for (int q = 0; q < kB; ++q) {
        if (q < n) {
          perm[rank + q] = (int32_t)rows[q];
#pragma unroll
          for (int k = 0; k < kMaxTopK; ++k)
            if (k < K && ids[q][k] == e) a.slot_rank[rows[q] * K + k] = rank + q;
        }
      }
      rank += n;
    }
  }
  if (t == 0) a.cnt[e] = total;
}

// ===========================================================================
// Grouped GEMM on fp16 MFMA.  Block tile 256 (rows) x 256 (B rows), 4 waves
// in a 2 x 2 arrangement, each wave 128 x 128 from 32x32x16 MFMAs (4 A
// fragments x 4 B fragments, 256 accumulators per lane).  Groups are the
// routed experts (rows listed by the sort) and the shared expert (every
// row).  Three modes:
//   0  gate/up, every group: the B tile holds 128 gate rows and the matching
//      128 up rows; the epilogue writes silu(gate) * up as fp16 (h16)
//   1  down, routed groups: fp16 output per (expert, row) pair (d16)
//   2  down, shared group: the epilogue forms the layer output
//      out[r] = sum_k w[r,k] * d16[pair (idx[r,k], r)] + shared down(r),
//      slots in k order
// Operands travel global -> LDS directly (global_load_lds_dwordx4, no
// register round trip) in k-tiles of 64 through a 2-stage ring: the next
// k-tile loads while the current one is multiplied.  A tile row is 64 k =
// 128 bytes, one cache line; its eight 16-byte chunks are stored
// XOR-swizzled by the row index so the fragment reads of consecutive rows
// hit distinct LDS banks.  B stays bf16 in LDS and is converted to fp16
// after the fragment read, interleaved with the MFMAs of the previous
// k-step.
// Block-scaled weights (MX) travel the same way as codes: 8-bit (MXFP8), a
// k-tile row of BK bytes (BK 128: one 128-byte row; BK 64: two rows per
// 128-byte line, 16-byte chunks swizzled by (row / 4) & 3), or 4-bit
// (MXFP4), BK / 2 bytes (two 64-byte rows per line; BK 64: four 32-byte
// rows, chunks swizzled by (row / 8) & 1); each tile's block scales (one
// byte per 32 inputs) land in LDS once per tile.  The k order inside a
// group of k-steps is permuted so that a lane's codes of the group are one
// 16-byte read under one scale: MXFP8, pairs -- k-step 2p + o takes k =
// 32p + 16 * (lane / 32) + 8o + 0..7; MXFP4, quads -- k-step 4p + o takes
// k = 64p + 32 * (lane / 32) + 8o + 0..7 (the A fragments follow the same
// map).  v_cvt_scalef32_pk_f16_fp8 / _fp4 turn the codes into fp16 with
// the scale.
// The grid is persistent (one block per compute unit); tiles are ordered by
// group, then in blocks of 4 row tiles x 8 column tiles, and handed out so
// that each XCD takes a contiguous run of them: the tiles that share
// activation tiles and weight slices run at the same time behind one L2.
constexpr int kSlab = 64; // epilogue rows staged per pass

// Tile configurations: BM tile rows (WM A fragments per wave), BROWS tile B
// rows (WN B fragments per wave), k-tiles of BK held in LDS as BK/64 halves
// of 64 k (one 128-byte row each), a ring of STAGES k-tiles, THREADS / 64
// waves in a grid of (THREADS / 64 / GWN) x GWN.
//   Big: 256 x 256, BK 64, 2 stages -- groups of many rows.
//   Small: 64 x 128, BK 128, 3 stages -- groups of a few rows, where the
//   kernel mostly streams weights: a lane fetches the two adjacent 128-byte
//   lines of a weight row back to back, so each row is read 256 bytes at a
//   time (DRAM page locality), and two k-tiles are in flight per compute
//   unit.
template <int BM_, int WM_, int BROWS_, int WN_, int BK_, int STAGES_, int GWN_, int THREADS_>
struct GemmCfg {
  static constexpr int BM = BM_, WM = WM_, BROWS = BROWS_, WN = WN_, BK = BK_, kStages = STAGES_;
  static constexpr int GWN = GWN_, kGT = THREADS_, GWM = THREADS_ / 64 / GWN_;  // wave grid GWM x GWN
  static_assert(BM == GWM * WM * 32 && BROWS == GWN * WN * 32, "wave grid of 32-row fragments");
  static_assert(BK % 64 == 0, "k-tiles of whole 64-k halves");
};
using GemmBig = GemmCfg<256, 4, 256, 2, 64, 2, 4, 512>;
using GemmSmall = GemmCfg<64, 1, 128, 1, 128, 3, 4, 512>;

// output columns per block tile
template <int MODE, class Cfg>
struct GemmShape {
  static constexpr int BN = MODE == 0 ? Cfg::BROWS / 2 : Cfg::BROWS;
};

template <int MODE, int KD, int ND, class Cfg, int MX>
__global__ __launch_bounds__(Cfg::kGT, 1) void k_gemm(const FwdArgs a) {
  constexpr int BM = Cfg::BM, WM = Cfg::WM, BROWS = Cfg::BROWS, WN = Cfg::WN, BK = Cfg::BK;
  constexpr int kGT = Cfg::kGT, GWN = Cfg::GWN;
  constexpr int kStages = Cfg::kStages;
  constexpr int BN = GemmShape<MODE, Cfg>::BN;
  constexpr int NT = ND / BN;                // column tiles per group
  constexpr int NK = KD / BK;                // k slices
  constexpr int NH = BK / 64;              // 64-k halves per k-tile
  constexpr int HA = BM * 128, HB = BROWS * 128;  // bytes of one half of the A / B tile (bf16 B)
  // epilogue staging per 64-row slab, reusing the ring: f32 [64][BROWS + 4]
  // (gate/up: gate columns, then up columns)
  constexpr int CPITCH = BROWS + 4;
  constexpr int SLAB = kSlab * CPITCH * 4;
  // MX: the B tile holds BK bytes per row; with three stages they are
  // padded to a slab so that the epilogue can stage through one of them
  constexpr int RB = MX == 2 ? BK / 2 : BK;  // MX: bytes of a k-tile row of codes
  constexpr int KB = MX == 2 ? KD / 2 : KD;  // MX: bytes of a whole row of codes
  constexpr int A_ST = NH * HA, B_ST = MX ? BROWS * RB : NH * HB;
  constexpr bool kPad = MX && kStages == 3 && MODE != 2 && A_ST + B_ST < SLAB;
  constexpr int ST = kPad ? (SLAB + 1023) / 1024 * 1024 : A_ST + B_ST;
  constexpr int AI = A_ST / 16 / kGT;  // A DMA instructions per thread per k-tile
  constexpr int BI = B_ST / 16 / kGT;  // B DMA instructions per thread per k-tile
  constexpr int AG = AI / NH, BG = MX ? BI : BI / NH;  // 8-line groups per wave (A, B)
  static_assert(AG >= 1 && BG >= 1 && AI * kGT * 16 == A_ST && BI * kGT * 16 == B_ST, "DMA tiling");
  static_assert(kStages == 2 || AG == 1, "the ring's wait counts at most one A row group per wave");
  static_assert(SLAB <= kStages * ST, "staging fits");
  static_assert(NK >= 2 && ND % BN == 0, "tiling");
  // MX B rows: RPL rows per 128-byte line, CPR 16-byte chunks per row
  constexpr int RPL = MX ? 128 / RB : 1, CPR = MX ? RB / 16 : 8;
  static_assert(!MX || ((RB == 32 || RB == 64 || RB == 128) && BROWS % (8 * RPL) == 0), "MX B layout");
  // MX block scales of the tile's B rows: SR bytes per row (DPR dwords),
  // dword w of row r stored at slot w ^ ssw(r); one buffer padded to whole
  // rounds of 4-byte DMA, SCI per thread
  constexpr int SR = KD / 32, DPR = SR / 4;
  static_assert(!MX || (KD % 128 == 0 && DPR <= 64 && (DPR & (DPR - 1)) == 0), "MX scale rows");
  constexpr int SCL = MX ? (BROWS * SR + kGT * 4 - 1) / (kGT * 4) * (kGT * 4) : 0;
  constexpr int SCI = SCL / (kGT * 4);
  // With three stages and a slab that fits in one stage, the k-tiles of
  // consecutive statically dealt tiles form one stream: the last two
  // refills of a tile's k loop request the next tile's first two k-tiles
  // (instead of re-loading a dead one), so the next tile starts with them
  // landed; the epilogue stages through the buffer of the tile's last
  // k-tile, the one buffer left free.  k-tile kt of a tile sits in buffer
  // (off + kt) % kStages.  Not for the shared expert's down + reduce, whose
  // per-tile slot table lives in LDS.  MX: the next tile's scales land in
  // the second scale buffer along with them.
  constexpr bool kPre = MODE != 2 && kStages == 3 && SLAB <= ST;
  __shared__ __align__(16) unsigned char s_ring[kStages * ST];
  __shared__ __align__(16) unsigned char s_scl[MX ? (kPre ? 2 : 1) * SCL : 16];
  __shared__ int s_tbase[kMaxExperts + 2];
  __shared__ int s_rbase[kMaxExperts + 2];
  __shared__ int s_cnt[kMaxExperts + 1];
  __shared__ int s_pos[MODE == 2 ? BM * kMaxTopK : 1];
  __shared__ float s_w[MODE == 2 ? BM * kMaxTopK : 1];

  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  const int E = a.E, G = E + 1, K = a.K;
  const int64_t R = a.R;
  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)s_ring;
  const uint32_t scl = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)s_scl;
  const uint32_t a_wave = __builtin_amdgcn_readfirstlane(wv * AG * 1024);
  const uint32_t b_wave = __builtin_amdgcn_readfirstlane(A_ST + wv * BG * 1024);

  // row bases of every group, and tile bases of the groups this mode covers
  if (wv == 0) {
    int rrun = 0, trun = 0;
    for (int g0 = 0; g0 < G; g0 += kWave) {
      const int g = g0 + lane;
      const int c = g < G ? a.cnt[g] : 0;
      const bool mine = MODE == 0 ? g < G : MODE == 1 ? g < E : g == E;
      const int tm = mine ? (c + BM - 1) / BM * NT : 0;
      int ci = c, ti = tm;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v1 = __shfl_up(ci, o, kWave), v2 = __shfl_up(ti, o, kWave);
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
  const int total = s_tbase[G];
  const int wm = wv / GWN, wn = wv % GWN;
  int first = blockIdx.x;
  if (gridDim.x % 8 == 0) first = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;

  // fragment rows of this lane (tile-relative) and their swizzles
  int arow[WM], brow[WN];
#pragma unroll
  for (int i = 0; i < WM; ++i) arow[i] = wm * (WM * 32) + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < WN; ++j)
    brow[j] = (MODE == 0 && WN >= 2 ? (j < WN / 2 ? 0 : BROWS / 2) + wn * (WN / 2) * 32 + (j % (WN / 2 > 0 ? WN / 2 : 1)) * 32
                                    : wn * (WN * 32) + j * 32) + (lane & 31);
  // DMA: row group q of a wave (8 tile rows, (wave * groups + q) * 8 +
  // lane / 8) is filled half by half, the halves of a row back to back; the
  // lane moves chunk (lane & 7) ^ swz(row) = (lane & 7) ^ (lane / 8) ^
  // ((wave * groups + q) & 1) of its row
  const int chunk0 = ((lane & 7) ^ (lane >> 3)) * 16;  // bytes, even row group
  const int chunk1 = chunk0 ^ 16;                       // odd row group

  // Tiles: all but the last two rounds are dealt statically (first, first
  // + grid, ...; an XCD's blocks get neighbouring tiles); the rest go to
  // whichever block asks next, through a counter per launch, so that blocks
  // that ran fast take the tail.
  __shared__ int s_next;
  const int grid = (int)gridDim.x, rounds = total / grid;
  const int nstatic = total <= grid ? total : (rounds > 3 ? rounds - 2 : 1) * grid;
  auto grab = [&]() { return nstatic + (int)__hip_atomic_fetch_add(&a.gctr[MODE], 1u, __ATOMIC_RELAXED,
                                                                      __HIP_MEMORY_SCOPE_AGENT); };
  // group and position of a tile: largest g with s_tbase[g] <= tl (empty
  // groups share their successor's base and lose the search); within the
  // group, tiles go in bands of SN column tiles, each band in blocks of SM
  // row tiles x SN column tiles (row tile fastest): an XCD's 32 concurrent
  // tiles then share 4 activation tiles and 8 weight slices
  auto locate = [&](int tl, int& g, int& cntg, int& m0, int& n0) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tbase[mid] <= tl) lo = mid; else hi = mid - 1;
    }
    g = lo;
    cntg = s_cnt[g];
    const int tm = (cntg + BM - 1) / BM;
    const int local = tl - s_tbase[g];
    constexpr int SN = NT < 8 ? NT : 8, SM = 4;
    static_assert(NT % SN == 0, "column bands");
    const int band = local / (tm * SN), inband = local - band * tm * SN;
    const int mb = inband / (SM * SN), ms = (tm - mb * SM) < SM ? (tm - mb * SM) : SM;
    const int ib = inband - mb * SM * SN;
    m0 = (mb * SM + ib % ms) * BM;
    n0 = (band * SN + ib / ms) * BN;
  };
  // DMA source of A row group i / B row group i of this wave for a tile.
  // Rows past the group's end read its last row; their results are never
  // stored.  B: each wave's rows are all gate or all up rows.
  auto a_src = [&](int g, int cntg, int m0, int i) {
    const int row = (wv * AG + i) * 8 + (lane >> 3);
    const int m = (m0 + row < cntg) ? m0 + row : cntg - 1;
    int64_t r;
    if (MODE == 0) {
      r = g == E ? (int64_t)m : (int64_t)a.perm[(int64_t)g * R + m];
      check_index(a.status, r >= 0 && r < R);
      r = r < 0 ? 0 : (r >= R ? R - 1 : r);
    } else {
      r = (int64_t)s_rbase[g] + m;
    }
    return (MODE == 0 ? (const unsigned char*)a.xn16 : (const unsigned char*)a.h16) + r * (KD * 2) +
           (((wv * AG + i) & 1) ? chunk1 : chunk0);
  };
  auto b_src = [&](int g, int n0, int i) {
    const int bw_row = wv * BG * 8;  // first tile B row of this wave
    const bool sh = g == E;
    const uint16_t* bmat;
    int brow0;
    if (MODE == 0) {
      const bool is_up = bw_row >= BN;
      bmat = sh ? (is_up ? a.up_sh : a.gate_sh) : (is_up ? a.up : a.gate) + (int64_t)g * ND * KD;
      brow0 = n0 + (is_up ? bw_row - BN : bw_row) + (lane >> 3);
    } else {
      bmat = sh ? a.down_sh : a.down + (int64_t)g * ND * KD;
      brow0 = n0 + bw_row + (lane >> 3);
    }
    return (const unsigned char*)bmat + (int64_t)(brow0 + i * 8) * (KD * 2) + (((wv * BG + i) & 1) ? chunk1 : chunk0);
  };
  // MX: codes (or scales) of tile B row `r` (0 <= r < BROWS)
  auto mx_row = [&](int g, int n0, int r, bool scales) {
    const bool sh = g == E;
    const uint8_t* m;
    int row;
    if (MODE == 0) {
      const bool is_up = r >= BN;
      m = scales ? (sh ? (is_up ? a.up_sh_s : a.gate_sh_s) : (is_up ? a.up_s : a.gate_s))
                 : (sh ? (is_up ? a.up_sh_q : a.gate_sh_q) : (is_up ? a.up_q : a.gate_q));
      row = n0 + (is_up ? r - BN : r);
    } else {
      m = scales ? (sh ? a.down_sh_s : a.down_s) : (sh ? a.down_sh_q : a.down_q);
      row = n0 + r;
    }
    const int64_t rows_before = sh ? 0 : (int64_t)g * ND;
    return m + (rows_before + row) * (scales ? SR : KB);
  };
  // MX B DMA: instruction i of the wave fills 1024 bytes of the B tile,
  // lane l the 16-byte slot l & 7 of line (wave * BI + i) * 8 + l / 8: row
  // line * RPL + slot / CPR, chunk (slot % CPR) ^ mxsw(row)
  auto b_src_mx = [&](int g, int n0, int i) {
    const int line = (wv * BI + i) * 8 + (lane >> 3), slot = lane & 7;
    const int r = line * RPL + slot / CPR;
    return mx_row(g, n0, r, false) + ((slot % CPR) ^ mxsw(r, CPR)) * 16;
  };
  // MX scales of a tile into scale buffer `sb`: dword d of the buffer (row
  // d / DPR, slot d % DPR) holds source dword slot ^ ssw(row); rows past the
  // tile (padding) re-read its last row.  Not unrolled: unrolled, the
  // tile-invariant offsets of every round were kept live across the k loop
  // and spilled.
  auto issue_scales = [&](int g, int n0, int sb) {
#pragma unroll 1
    for (int u = 0; u < SCI; ++u) {
      const int d = u * kGT + t, r = d / DPR < BROWS ? d / DPR : BROWS - 1;
      dma4(mx_row(g, n0, r, true) + (((d % DPR) ^ ssw(r, DPR)) << 2), scl + (uint32_t)(sb * SCL + (u * kGT + wv * kWave) * 4));
    }
  };
  int off = 0;   // ring offset of the current tile
  int npre = 0;  // its first k-tiles the previous tile requested (0 or 2)
  int sb = 0;    // MX: the scale buffer of the current tile
  bool range_bad = false;  // a non-finite value written by this thread's epilogues
  int tile = first;
  if (tile >= nstatic) {
    if (t == 0) s_next = nstatic < total ? grab() : total;
    __syncthreads();
    tile = s_next;
  }
  while (tile < total) {
    const bool dyn_next = tile + grid >= nstatic;  // the next tile comes from the counter
    int next_dyn = total;
    int g, cntg, m0, n0;
    locate(tile, g, cntg, m0, n0);

    if (MODE == 2) {
      // slots of this tile's rows: position of each (expert, row) pair in
      // d16, and its weight
      for (int q = t; q < BM * K; q += kGT) {
        const int rl = q / K, k = q - rl * K;
        const int64_t r = (int64_t)m0 + rl;
        int pos = -1;
        float w = 0.f;
        if (r < R) {
          const int e = a.idx[r * K + k];
          const int rank = a.slot_rank[r * K + k];
          if (e >= 0 && e < E && rank >= 0) {
            pos = s_rbase[e] + rank;
            check_index(a.status, rank < s_cnt[e] && pos < s_rbase[E]);
            pos = pos < s_rbase[E] ? pos : s_rbase[E] - 1;
            w = a.wts[r * K + k];
          }
        }
        s_pos[rl * kMaxTopK + k] = pos;
        s_w[rl * kMaxTopK + k] = w;
      }
    }

    // DMA sources
    const unsigned char* asrc[AG];
#pragma unroll
    for (int i = 0; i < AG; ++i) asrc[i] = a_src(g, cntg, m0, i);
    const unsigned char* bsrc[BG];
#pragma unroll
    for (int i = 0; i < BG; ++i) bsrc[i] = MX ? b_src_mx(g, n0, i) : b_src(g, n0, i);
    // whether this wave loads A rows at all (the small configuration's one
    // A row group per wave; the big one waits with vmcnt(0))
    const bool a_loads = m0 + wv * AG * 8 < cntg;
    // the next statically dealt tile, whose first k-tiles this tile's k loop
    // requests: its DMA sources now (their row-list loads land under the k
    // loop's first full wait)
    const bool pref = kPre && !dyn_next && tile + grid < total;
    const unsigned char* nasrc[AG];
    const unsigned char* nbsrc[BG];
    bool na_loads = false;
    int nm0 = 0, ncnt = 0, ng = 0, nn0 = 0;
    if (kPre && pref) {
      locate(tile + grid, ng, ncnt, nm0, nn0);
#pragma unroll
      for (int i = 0; i < AG; ++i) nasrc[i] = a_src(ng, ncnt, nm0, i);
#pragma unroll
      for (int i = 0; i < BG; ++i) nbsrc[i] = MX ? b_src_mx(ng, nn0, i) : b_src(ng, nn0, i);
      na_loads = nm0 + wv * AG * 8 < ncnt;
    }
    // k-tile `src` into ring buffer `buf`
    // (A row groups wholly past the group's end are not loaded: the ring
    // waits with vmcnt(0), so the number of loads may differ per wave)
    auto issue = [&](int src, int buf) {
      const uint32_t base = ring + (uint32_t)buf * ST;
#pragma unroll
      for (int i = 0; i < AG; ++i)
        if (m0 + (wv * AG + i) * 8 < cntg)
#pragma unroll
          for (int h = 0; h < NH; ++h) dma16(asrc[i] + src * (BK * 2) + h * 128, base + a_wave + h * HA + i * 1024);
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < BG; ++i) dma16(bsrc[i] + src * RB, base + b_wave + i * 1024);
      } else {
#pragma unroll
        for (int i = 0; i < BG; ++i)
#pragma unroll
          for (int h = 0; h < NH; ++h) dma16(bsrc[i] + src * (BK * 2) + h * 128, base + b_wave + h * HB + i * 1024);
      }
    };
    // the same for k-tile `src` of the next tile
    auto issue_next = [&](int src, int buf) {
      const uint32_t base = ring + (uint32_t)buf * ST;
#pragma unroll
      for (int i = 0; i < AG; ++i)
        if (nm0 + (wv * AG + i) * 8 < ncnt)
#pragma unroll
          for (int h = 0; h < NH; ++h) dma16(nasrc[i] + src * (BK * 2) + h * 128, base + a_wave + h * HA + i * 1024);
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < BG; ++i) dma16(nbsrc[i] + src * RB, base + b_wave + i * 1024);
      } else {
#pragma unroll
        for (int i = 0; i < BG; ++i)
#pragma unroll
          for (int h = 0; h < NH; ++h) dma16(nbsrc[i] + src * (BK * 2) + h * 128, base + b_wave + h * HB + i * 1024);
      }
    };
    auto ring_buf = [&](int kt) { return kPre ? (off + kt) % kStages : kt % kStages; };
    // fragment reads of k-step `st` (16 k) of k-tile `kt` from ring buffer
    // `buf`.  MX: the B codes of a step pair (MXFP8) or quad (MXFP4) and
    // their scale are read at its first step and kept for the others.
    auto read_step = [&](int buf, int st, half8 (&af)[WM], uint4 (&rb)[WN], float (&sc)[WN], int nv, int kt) {
      const unsigned char* As = s_ring + buf * ST + (st >> 2) * HA;
      const int c = MX == 2 ? 4 * (lane >> 5) + (st & 3)
                    : MX    ? 4 * ((st >> 1) & 1) + 2 * (lane >> 5) + (st & 1)
                            : 2 * (st & 3) + (lane >> 5);
#pragma unroll
      for (int i = 0; i < WM; ++i)
        if (i < nv) af[i] = *(const half8*)(As + arow[i] * 128 + ((c ^ swz(arow[i])) << 4));
      if constexpr (!MX) {
        const unsigned char* Bs = s_ring + buf * ST + A_ST + (st >> 2) * HB;
#pragma unroll
        for (int j = 0; j < WN; ++j) rb[j] = *(const uint4*)(Bs + brow[j] * 128 + ((c ^ swz(brow[j])) << 4));
      } else if ((st & (MX == 2 ? 3 : 1)) == 0) {
        const unsigned char* Bs = s_ring + buf * ST + A_ST;
        const int q = MX == 2 ? 2 * (st >> 2) + (lane >> 5) : 2 * (st >> 1) + (lane >> 5);
        // 32-k block of the lane's codes
        const int b = kt * (BK / 32) + (MX == 2 ? 2 * (st >> 2) + (lane >> 5) : st >> 1);
        const unsigned char* Ss = s_scl + sb * SCL + (b & 3);
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          rb[j] = *(const uint4*)(Bs + (brow[j] / RPL) * 128 + (brow[j] % RPL) * RB + ((q ^ mxsw(brow[j], CPR)) << 4));
          sc[j] = e8m0_scale(Ss[brow[j] * SR + (((b >> 2) ^ ssw(brow[j], DPR)) << 2)]);
        }
      }
    };
    // B fragment j of k-step `st` in fp16
    auto conv1 = [&](int j, int st, const uint4 (&rb)[WN], const float (&sc)[WN], half8& out) {
      uint4 cv;
      if constexpr (MX == 2) {
        const int o = st & 3;
        cv = fp4x8_to_f16x8(o == 0 ? rb[j].x : o == 1 ? rb[j].y : o == 2 ? rb[j].z : rb[j].w, sc[j]);
      } else if constexpr (MX) {
        cv = (st & 1) ? fp8x8_to_f16x8(rb[j].z, rb[j].w, sc[j]) : fp8x8_to_f16x8(rb[j].x, rb[j].y, sc[j]);
      } else {
        cv = bf16x8_to_f16x8(rb[j]);
      }
      out = __builtin_bit_cast(half8, cv);
    };

    floatx16 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[i][j] = floatx16{};

    // Ring of kStages buffers: later k-tiles load while kt is multiplied.
    // The next k-step's fragments are read and converted while the MFMAs of
    // the current step run, across k-tile boundaries too: before the last
    // step of k-tile kt (its fragments already in registers) every wave
    // waits for k-tile kt+1, passes the barrier, reads kt+1's first step and
    // refills kt's buffer with kt+kStages.  Past the end the refill re-loads
    // the last k-tile into the dead buffer and the read repeats it -- or,
    // with the cross-tile stream, requests the next tile's first k-tiles
    // (and the read past the end reads the next tile's first, unused).
    constexpr int NS = BK / 16;  // k-steps per k-tile
    // The k loop is instantiated per count NV of this wave's A fragments
    // that hold rows of the group (a partly filled row tile runs only the
    // MFMAs of its filled fragments); every variant passes the same barriers.
    auto kloop = [&](auto nv_c) {
    constexpr int NV = decltype(nv_c)::value;
    half8 af[WM], bf[WN];
    if constexpr (kPre) {
      if (npre == 0) {
        if constexpr (MX) issue_scales(g, n0, sb);
        issue(0, ring_buf(0));
      }
      wait_vmcnt<0>();
      __syncthreads();
#pragma unroll
      for (int st = 1; st < kStages; ++st)
        if (st >= npre) issue(st < NK ? st : NK - 1, ring_buf(st));
    } else {
      if constexpr (MX) issue_scales(g, n0, 0);
      issue(0, 0);
      wait_vmcnt<0>();
      __syncthreads();
#pragma unroll
      for (int st = 1; st < kStages; ++st) issue(st < NK ? st : NK - 1, st);
    }
    // raw B fragments (MX: of the current step pair or quad) and their scales
    uint4 rb[WN];
    float sc[WN];
    read_step(ring_buf(0), 0, af, rb, sc, NV, 0);
#pragma unroll
    for (int j = 0; j < WN; ++j) conv1(j, 0, rb, sc, bf[j]);
    // one B fragment's four MFMAs
    auto mfma_j = [&](int j) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    };
    // The schedule inside a k-step is pinned with scheduling fences: the
    // next step's fragment reads go first, then each B fragment's MFMAs run
    // while the next step's fragment of the previous column converts.
#pragma unroll 1
    for (int kt = 0; kt < NK; ++kt) {
      const int buf = ring_buf(kt), nbuf = ring_buf(kt + 1);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        half8 afn[WM], bfn[WN];
        if (st + 1 < NS) {
          read_step(buf, st + 1, afn, rb, sc, NV, kt);
          __builtin_amdgcn_sched_barrier(0);
          mfma_j(0);
          __builtin_amdgcn_sched_barrier(0);
        } else {
          // k-tile kt+1 landed for this wave: only the loads of the
          // kStages-2 later tiles may still be in flight (with three
          // stages, k-tile kt+2: the next tile's first when kt+2 >= NK)
          const bool later_a = (kPre && pref && kt + 2 >= NK) ? na_loads : a_loads;
          if (kStages == 2 || !later_a) wait_vmcnt<(kStages - 2) * BI>();
          else wait_vmcnt<(kStages - 2) * (BI + NH)>();
          __syncthreads();  // k-tile kt+1 landed for every wave; every wave is done reading buffer `buf`
          read_step(nbuf, 0, afn, rb, sc, NV, kt + 1 < NK ? kt + 1 : NK - 1);
          __builtin_amdgcn_sched_barrier(0);
          mfma_j(0);
          if constexpr (!kPre) {
            issue(kt + kStages < NK ? kt + kStages : NK - 1, buf);
          } else {
            if (kt + kStages < NK) issue(kt + kStages, buf);
            else if (!pref) issue(NK - 1, buf);  // dead refill: the loop body stays the same
            else if (kt + kStages - NK < kStages - 1) {
              // MX: the next tile's scales go ahead of its first k-tile
              if (MX && kt + kStages == NK) issue_scales(ng, nn0, sb ^ 1);
              issue_next(kt + kStages - NK, buf);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 1; j < WN; ++j) {
          conv1(j - 1, (st + 1) % NS, rb, sc, bfn[j - 1]);
          mfma_j(j);
          __builtin_amdgcn_sched_barrier(0);
        }
        conv1(WN - 1, (st + 1) % NS, rb, sc, bfn[WN - 1]);
#pragma unroll
        for (int i = 0; i < NV; ++i) af[i] = afn[i];
#pragma unroll
        for (int j = 0; j < WN; ++j) bf[j] = bfn[j];
      }
    }
    };
    {
      const int rows_left = cntg - m0 - wm * (WM * 32);
      const int nv = rows_left <= 0 ? 0 : (rows_left >= WM * 32 ? WM : (rows_left + 31) / 32);
      switch (nv) {
        case 4: kloop(std::integral_constant<int, 4>{}); break;
        case 3: kloop(std::integral_constant<int, 3>{}); break;
        case 2: kloop(std::integral_constant<int, 2>{}); break;
        case 1: kloop(std::integral_constant<int, 1>{}); break;
        default: kloop(std::integral_constant<int, 0>{}); break;
      }
    }
    // the trailing refills land before the ring turns into staging (with the
    // cross-tile stream there are none: the staging buffer gets no refill,
    // and the next tile's k-tiles may stay in flight)
    if (!kPre || !pref) wait_vmcnt<0>();
    // the next tile's number is requested now; the epilogue covers the wait
    if (t == 0 && dyn_next && nstatic < total) next_dyn = grab();
    __syncthreads();
    unsigned char* const s_stage = s_ring + (kPre ? ring_buf(NK - 1) * ST : 0);

    // epilogue, through LDS in 64-row slabs: D[i][j] of a 32x32 tile sits in
    // lane j + 32*((i/4)%2), register 4*(i/8) + i%4
    constexpr int CH = BN / 8;  // 8-column chunks per row
    // unrolled: the accumulator indices must stay compile-time constants
#pragma unroll
    for (int sl = 0; sl < BM / kSlab; ++sl) {
      __syncthreads();  // the ring (or the previous slab) is free
      __builtin_amdgcn_sched_barrier(0);  // keep each slab's accumulator reads in place
      if constexpr (WM * 32 >= kSlab) {
        // a wave row spans whole slabs: slab sl holds fragments
        // (sl % S) * F .. + F-1 of wave row sl / S (F per slab, S slabs per row)
        constexpr int F = kSlab / 32, S = WM / F;
        if (wm == sl / S) {
#pragma unroll
          for (int ii = 0; ii < F; ++ii) {
            const int i = (sl % S) * F + ii;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rl = ii * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
#pragma unroll
              for (int j = 0; j < WN; ++j) ((float*)s_stage)[rl * CPITCH + brow[j]] = acc[i][j][v];
            }
          }
        }
      } else {
        // a slab spans several wave rows: every fragment lands in slab 0
        static_assert(BM == kSlab, "one slab");
#pragma unroll
        for (int i = 0; i < WM; ++i) {
          const int base = wm * (WM * 32) + i * 32;  // tile row of fragment i
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rl = base + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
#pragma unroll
            for (int j = 0; j < WN; ++j) ((float*)s_stage)[rl * CPITCH + brow[j]] = acc[i][j][v];
          }
        }
      }
      __syncthreads();
#pragma unroll 1
      for (int q = t; q < kSlab * CH; q += kGT) {
        const int rl = q / CH, cc = (q % CH) * 8;
        const int m = m0 + sl * kSlab + rl;
        if (m >= cntg) continue;
        if (MODE != 2) {
          const float* sv = &((const float*)s_stage)[rl * CPITCH + cc];
          half8 h;
          if (MODE == 0) {
#pragma unroll
            for (int u = 0; u < 8; ++u) h[u] = (_Float16)swiglu_fast(sv[u], sv[BN + u]);
          } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) h[u] = (_Float16)sv[u];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) range_bad |= !__builtin_isfinite((float)h[u]);
          _Float16* dst = MODE == 0 ? a.h16 : a.d16;
          *(half8*)(dst + (int64_t)(s_rbase[g] + m) * ND + n0 + cc) = h;
        } else {
          const int tr = sl * kSlab + rl;  // tile row
          // all K gathers in flight before the sum (masked slots load row 0
          // and are dropped by a select, never multiplied)
          half8 d[kMaxTopK];
#pragma unroll
          for (int k = 0; k < kMaxTopK; ++k) {
            if (k < K) {
              const int pos = s_pos[tr * kMaxTopK + k];
              d[k] = *(const half8*)(a.d16 + (int64_t)(pos >= 0 ? pos : 0) * ND + n0 + cc);
            }
          }
          float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < kMaxTopK; ++k) {
            if (k < K && s_pos[tr * kMaxTopK + k] >= 0) {
              const float w = s_w[tr * kMaxTopK + k];
#pragma unroll
              for (int u = 0; u < 8; ++u) o[u] = fmaf(w, (float)d[k][u], o[u]);
            }
          }
          const float* sh = &((const float*)s_stage)[rl * CPITCH + cc];
          float4 o0, o1;
          o0.x = o[0] + sh[0]; o0.y = o[1] + sh[1]; o0.z = o[2] + sh[2]; o0.w = o[3] + sh[3];
          o1.x = o[4] + sh[4]; o1.y = o[5] + sh[5]; o1.z = o[6] + sh[6]; o1.w = o[7] + sh[7];
          range_bad |= !(__builtin_isfinite(o0.x) && __builtin_isfinite(o0.y) && __builtin_isfinite(o0.z) &&
                         __builtin_isfinite(o0.w) && __builtin_isfinite(o1.x) && __builtin_isfinite(o1.y) &&
                         __builtin_isfinite(o1.z) && __builtin_isfinite(o1.w));
          float* dst = a.out + (int64_t)m * ND + n0 + cc;
          *(float4*)dst = o0;
          *(float4*)(dst + 4) = o1;
        }
      }
    }
    if (t == 0) s_next = dyn_next ? next_dyn : tile + grid;
    if constexpr (kPre) {
      off = pref ? ring_buf(NK) : 0;
      npre = pref ? kStages - 1 : 0;
      if (MX && pref) sb ^= 1;
    }
    __syncthreads();  // staging and s_pos are rewritten by the next tile
    tile = s_next;
  }
  // the sort has written the status word; this launch only adds to it
  if (range_bad) atomicOr(a.status, (uint32_t)MOE_FLAG_F16_RANGE);
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

template <int H, int E, int S>
const void* router_fn() {
  if constexpr (E / S >= 32) return (const void*)k_pre_router<H, E, S>;
  else return (const void*)k_pre_router<H, E, 1>;
}

template <int H, int I, int E, int MX>
hipError_t run_prefill_t(const FwdArgs& a, hipStream_t s) {
  FwdArgs args = a;
  const int nb = (a.R + kRR - 1) / kRR;
  hipError_t err = launch("pre_norm", (const void*)k_pre_norm<H>, dim3((a.R + 3) / 4), dim3(kThreads), 0, s, &args);
  if (err != hipSuccess) return err;
  // expert slices: as many as keep the router blocks within one per compute
  // unit, up to 8 (32 experts, one fragment, per block)
  const int grid = gemm_grid();
  int S = 1;
  while (S < 8 && E / (2 * S) >= 32 && (int64_t)nb * 2 * S <= grid) S *= 2;
  const void* router = S == 8   ? router_fn<H, E, 8>()
                       : S == 4 ? router_fn<H, E, 4>()
                       : S == 2 ? router_fn<H, E, 2>()
                                : router_fn<H, E, 1>();
  err = launch("pre_router", router, dim3(nb * S), dim3(kThreads), 0, s, &args);
  if (err != hipSuccess) return err;
  err = launch("pre_sort", (const void*)k_pre_sort, dim3(a.E + 1), dim3(kThreads), 0, s, &args);
  if (err != hipSuccess) return err;
  // groups of a few rows on average: the small row tile and the deeper ring
  const bool small = (int64_t)a.R * a.K <= 32LL * a.E;
  err = launch(MX == 2 ? "gemm_gateup_swiglu_mx4" : MX ? "gemm_gateup_swiglu_mx" : "gemm_gateup_swiglu",
               small ? (const void*)k_gemm<0, H, I, GemmSmall, MX> : (const void*)k_gemm<0, H, I, GemmBig, MX>,
               dim3(grid), dim3(small ? GemmSmall::kGT : GemmBig::kGT), 0, s, &args);
  if (err != hipSuccess) return err;
  err = launch(MX == 2 ? "gemm_down_mx4" : MX ? "gemm_down_mx" : "gemm_down",
               small ? (const void*)k_gemm<1, I, H, GemmSmall, MX> : (const void*)k_gemm<1, I, H, GemmBig, MX>,
               dim3(grid), dim3(small ? GemmSmall::kGT : GemmBig::kGT), 0, s, &args);
  if (err != hipSuccess) return err;
  // the shared down covers R rows only: small tiles when big ones would
  // leave compute units idle
  const int64_t big_tiles = (a.R + GemmBig::BM - 1) / GemmBig::BM * (H / GemmShape<2, GemmBig>::BN);
  const bool sh_small = big_tiles < grid;
  const int64_t sh_tiles =
      sh_small ? (a.R + GemmSmall::BM - 1) / GemmSmall::BM * (H / GemmShape<2, GemmSmall>::BN) : big_tiles;
  const int sh_grid = sh_tiles < grid ? (int)sh_tiles : grid;
  return launch(MX == 2 ? "gemm_down_shared_reduce_mx4" : MX ? "gemm_down_shared_reduce_mx" : "gemm_down_shared_reduce",
                sh_small ? (const void*)k_gemm<2, I, H, GemmSmall, MX> : (const void*)k_gemm<2, I, H, GemmBig, MX>,
                dim3(sh_grid), dim3(sh_small ? GemmSmall::kGT : GemmBig::kGT), 0, s, &args);
}

}  // namespace

hipError_t run_prefill(const FwdArgs& a, hipStream_t s) {
  if (a.H == 4096 && a.I == 2048 && a.E == 256)
    return a.mx == 2   ? run_prefill_t<4096, 2048, 256, 2>(a, s)
           : a.mx == 1 ? run_prefill_t<4096, 2048, 256, 1>(a, s)
                       : run_prefill_t<4096, 2048, 256, 0>(a, s);
  if (a.H == 512 && a.I == 256 && a.E == 32)
    return a.mx == 2   ? run_prefill_t<512, 256, 32, 2>(a, s)
           : a.mx == 1 ? run_prefill_t<512, 256, 32, 1>(a, s)
                       : run_prefill_t<512, 256, 32, 0>(a, s);
  return hipErrorInvalidValue;
}

hipError_t run_route(const RouteArgs& a, hipStream_t s) {
  RouteArgs args = a;
  const int per = kThreads / kWave;
  return launch("route", (const void*)k_route, dim3((a.R + per - 1) / per), dim3(kThreads), 0, s, &args);
}

}  // namespace moe
