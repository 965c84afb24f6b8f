// Host-side interface between the C ABI (abi.hip) and the kernel files.
// Every kernel takes one argument struct by value; launch() sends it with
// hipExtLaunchKernel so the optional stage timer can bracket the kernel's
// own execution with start/stop events.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace moe {

// Launch `fn(args)` on `stream`; returns the launch status.
hipError_t launch(const char* name, const void* fn, dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                  void* args);

// Everything one forward call needs, resolved to device pointers.
struct FwdArgs {
  // problem
  int R, H, E, K, I;
  float eps;
  int layer_kind;
  int64_t table_rows;
  // inputs / outputs
  const float* x;
  const int32_t* token_ids;
  const float* norm_w;
  const uint16_t* router;
  const float* bias;
  const int32_t* table;
  const uint16_t* gate;
  const uint16_t* up;
  const uint16_t* down;
  const uint16_t* gate_sh;
  const uint16_t* up_sh;
  const uint16_t* down_sh;
  // block-scaled 8-bit expert weights (moe_ffn_forward_mxfp8; mx != 0): E4M3
  // codes [out][in] and E8M0 scales [out][in/32] of the same six matrices
  int mx;
  const uint8_t *gate_q, *up_q, *down_q, *gate_sh_q, *up_sh_q, *down_sh_q;
  const uint8_t *gate_s, *up_s, *down_s, *gate_sh_s, *up_sh_s, *down_sh_s;
  float* out;
  // hyper-connection wrapper folded into a decode call (hc > 0, 1-4 rows):
  // every head block adds the mix launch's slice partials and splits (block
  // 0 stores the mixes and maps), the input row is x[r] = sum_i pre[r][i] *
  // state[r][i] (block 0 stores it to hc_x), and the reduce writes
  // new[r][j] = post[r][j] * out[r] + sum_i comb[r][j][i] * state[r][i]
  int hc, hc_iters;
  int64_t hc_slices;
  const float* hc_state;    // [R][hc][H]
  const float* hc_partial;  // [slices][4][(2+hc)*hc + 1] mix sums, then the sum of squares
  const float* hc_scale;    // [3]
  const float* hc_base;     // [(2+hc)*hc]
  float* hc_mixes;          // [R][(2+hc)*hc]
  float* hc_maps;           // [R][(2+hc)*hc]: pre | post | comb
  float* hc_x;              // [R][H]
  float* hc_out;            // [R][hc][H]
  // workspace pieces
  uint32_t* status;
  DecodeSync* sync;
  float* logits;
  int32_t* idx;
  float* wts;
  uint32_t* rowflags;
  float* xn32;
  DecodePlan* plan;
  float* h32;
  float* d32;
  _Float16* xn16;
  _Float16* xlo16;
  uint32_t* mask;
  uint32_t* rcnt;
  uint32_t* gctr;
  int32_t* cnt;
  int32_t* slot_rank;
  int32_t* perm;
  _Float16* h16;
  _Float16* d16;
};

hipError_t run_decode(const FwdArgs& a, hipStream_t s);
hipError_t run_prefill(const FwdArgs& a, hipStream_t s);

// The hyper-connection wrapper's launches (hc.hip).
struct HcArgs {
  int R, H, hc, iters;
  float eps;
  int64_t slices;
  int slice_k;           // flattened inputs per slice
  int tile_rows;         // rows per mix tile: 4 (1-4 rows) or 32 (more, on the matrix cores)
  const float* state;    // [R][hc][H]
  const uint16_t* fn;    // bf16 [(2+hc)*hc][hc*H]
  const float* scale;    // [3]
  const float* base;     // [(2+hc)*hc]
  float* mixes;          // [R][(2+hc)*hc]
  float* maps;           // [R][(2+hc)*hc]
  float* partial;
  float* ffn_in;         // [R][H]
  const float* ffn_out;  // [R][H]
  float* out;            // [R][hc][H]
};
// before the FFN: the mixes' slice partials -- and, with more than 4 rows,
// the split and the FFN input in a second launch (1-4 rows: the decode head
// splits and forms the input)
hipError_t run_hc_pre(const HcArgs& a, hipStream_t s);
// the new state (after the FFN)
hipError_t run_hc_post(const HcArgs& a, hipStream_t s);

struct RouteArgs {
  int R, E, K, layer_kind;
  int64_t table_rows;
  const float* logits;
  const int32_t* token_ids;
  const float* bias;
  const int32_t* table;
  int32_t* idx;
  float* w;
};
hipError_t run_route(const RouteArgs& a, hipStream_t s);

}  // namespace moe
