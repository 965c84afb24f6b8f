// Workspace layout of moe_ffn_forward: one caller-provided device block is
// carved into the per-call intermediates.  ffn_forward.rs (forward_ffn_rows)
// allocates the same set per call -- logits, I32 indices, U32 safe
// indices, weights, routed/shared gate, up, activation and down buffers;
// here they live at fixed offsets so a call allocates nothing.
//
// Pure host/device arithmetic, no HIP calls: the CPU-side validation and the
// kernels use the same offsets.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moe {

// Rows up to this count take the decode path (weight-streaming GEMV with
// f32 activations); larger batches take the grouped-GEMM prefill path.
constexpr int kDecodeMaxRows = 4;
constexpr int kMaxTopK = 8;
constexpr int kDecodeMaxSlots = kDecodeMaxRows * kMaxTopK;  // 32
constexpr int kMaxExperts = 256;
// Rows per prefill router block: the routing of a block's rows is handed to
// the sort as one 32-bit row mask per expert.
constexpr int kPrefillBlockRows = 32;

// Routing plan of a decode call: the distinct experts of the batch, each
// with the distinct rows that chose it and the summed weight of those
// slots.  Written by the routing prologue of the gate/up kernel, read by the
// down kernel.
struct DecodePlan {
  int32_t ngroups;                            // distinct routed experts
  int32_t nentries;                           // distinct (expert, row) pairs
  int32_t group_expert[kDecodeMaxSlots];
  int32_t group_begin[kDecodeMaxSlots + 1];   // entry range of each group
  int32_t entry_row[kDecodeMaxSlots];
  float entry_w[kDecodeMaxSlots];
};

// Cross-workgroup words of the decode path, after the status word.  The
// arrival count starts every call at 0: the router block that completes it
// resets it (the workspace is zero-filled before its first use).
struct DecodeSync {
  uint32_t arrive;                       // router blocks of the current call that have written their logits
  uint32_t pad[15];
  // one-row path: each expert's ordered selection key and float64 sigmoid,
  // written by the router launch for the gate/up blocks that route
  uint64_t route_key[kMaxExperts];
  double route_sig[kMaxExperts];
};

struct Layout {
  size_t status;     // u32 status word, then the decode path's sync words (DecodeSync)
  size_t logits;     // f32 [R][E]
  size_t idx;        // i32 [R][K]
  size_t wts;        // f32 [R][K]
  size_t rowflags;   // u32 [R]
  size_t xn32;       // f32 [R][H]   (decode)
  size_t plan;       // DecodePlan    (decode)
  size_t h32;        // f32 [kDecodeMaxSlots + R][I]   (decode)
  size_t d32;        // f32 [kDecodeMaxSlots + R][H]   (decode) down output per entry
  size_t xn16;       // f16 [R][H]   normalised activations, rounded (prefill)
  size_t xlo16;      // f16 [R][H]   their rounding remainders (prefill router)
  size_t mask;       // u32 [E][ceil(R/32)]  bit j of word b: row 32b+j chose the expert (prefill)
  size_t rcnt;       // u32 [ceil(R/32)]  router blocks finished per 32-row group (prefill)
  size_t gctr;       // u32 [4]      tail-tile counters of the three GEMM launches (prefill)
  size_t cnt;        // i32 [E + 1]  rows per group (routed experts, then shared)
  size_t slot_rank;  // i32 [R][K]   rank of the slot's row inside its expert, -1 if masked
  size_t perm;       // i32 [E][R]   rows of each expert in ascending order
  size_t h16;        // f16 [S + R][I]   SwiGLU output, grouped order
  size_t d16;        // f16 [S][H]   routed down output, grouped order
  size_t total;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Returns false on size overflow.
inline bool make_layout(int64_t R, int H, int E, int K, int I, Layout* L) {
  const unsigned __int128 lim = (unsigned __int128)1 << 62;
  unsigned __int128 r = (unsigned __int128)R;
  unsigned __int128 S = r * K;
  if (R <= 0 || S >= lim) return false;
  const bool decode = R <= kDecodeMaxRows;
  unsigned __int128 off = 0;
  auto take = [&](unsigned __int128 bytes) -> size_t {
    off = (off + 255) / 256 * 256;
    size_t at = (size_t)off;
    off += bytes;
    return at;
  };
  L->status = take(64 + sizeof(DecodeSync));
  L->logits = take(r * E * 4);
  L->idx = take(S * 4);
  L->wts = take(S * 4);
  L->rowflags = take(r * 4);
  if (decode) {
    L->xn32 = take(r * H * 4);
    L->plan = take(sizeof(DecodePlan));
    L->h32 = take((unsigned __int128)(kDecodeMaxSlots + R) * I * 4);
    L->d32 = take((unsigned __int128)(kDecodeMaxSlots + R) * H * 4);
    L->xn16 = L->xlo16 = L->mask = L->rcnt = L->gctr = L->cnt = L->slot_rank = L->perm = L->h16 = L->d16 = 0;
  } else {
    L->xn32 = L->plan = L->h32 = L->d32 = 0;
    L->xn16 = take(r * H * 2);
    L->xlo16 = take(r * H * 2);
    L->mask = take((unsigned __int128)E * ((r + kPrefillBlockRows - 1) / kPrefillBlockRows) * 4);
    L->rcnt = take((r + kPrefillBlockRows - 1) / kPrefillBlockRows * 4);
    L->gctr = take(16);
    L->cnt = take((unsigned __int128)(E + 1) * 4);
    L->slot_rank = take(S * 4);
    L->perm = take((unsigned __int128)E * r * 4);
    L->h16 = take((S + r) * I * 2);
    L->d16 = take(S * H * 2);
  }
  off = (off + 255) / 256 * 256;
  if (off >= lim) return false;
  L->total = (size_t)off;
  return true;
}

// Hyper-connection wrapper (moe_ffn_forward_hc): the FFN's layout at offset
// 0, then the wrapper's intermediates.  The mix launch works on tiles of
// tile_rows rows x slice_k flattened inputs and leaves one partial sum per
// tile, slice and row; the next launch adds them.  1-4 rows (one tile of
// kHcRows, a latency-bound call on the vector ALUs) take slices of
// kHcSlice inputs, one block each; more rows go to the matrix cores in
// tiles of kHcMfmaRows rows, with slices of a multiple of kHcMfmaK inputs,
// as few as keep about kHcMixBlocks blocks in the launch.
constexpr int kHcMax = 4;       // streams
constexpr int kHcRows = 4;      // rows per mix tile
static_assert(kHcRows == kDecodeMaxRows, "a decode call is one mix tile");
constexpr int kHcSlice = 1024;   // flattened state values per mix block (1-4 rows: 256 threads x 4)
constexpr int kHcMfmaRows = 32;  // rows per mix tile with more than 4 rows (one 32x32 MFMA tile)
constexpr int kHcMfmaK = 64;     // slice granule with more than 4 rows (4 waves x 16 k)
constexpr int kHcMixBlocks = 512;
struct HcLayout {
  Layout ffn;
  int64_t tile_rows, tiles, slices, slice_k;  // slice_k: flattened inputs per slice
  size_t mixes;    // f32 [R][(2+hc)*hc]
  size_t maps;     // f32 [R][(2+hc)*hc]  pre | post | comb (output stream, input stream)
  size_t ffn_in;   // f32 [R][H]
  size_t ffn_out;  // f32 [R][H]
  size_t partial;  // f32 [tiles][slices][tile_rows][(2+hc)*hc + 1]  partial dots, then the sum of squares
  size_t total;
};

inline bool make_hc_layout(int64_t R, int H, int E, int K, int I, int hc, HcLayout* L) {
  if (hc < 1 || hc > kHcMax || !make_layout(R, H, E, K, I, &L->ffn)) return false;
  const unsigned __int128 lim = (unsigned __int128)1 << 62;
  const unsigned __int128 r = (unsigned __int128)R;
  const int mw = (2 + hc) * hc;
  L->tile_rows = R <= kHcRows ? kHcRows : kHcMfmaRows;
  L->tiles = (R + L->tile_rows - 1) / L->tile_rows;
  const int64_t gran = R <= kHcRows ? kHcSlice : kHcMfmaK;
  const int64_t passes = ((int64_t)hc * H + gran - 1) / gran;  // granule-wide pieces of a row
  int64_t want = R <= kHcRows ? passes : (kHcMixBlocks + L->tiles - 1) / L->tiles;
  want = want < 1 ? 1 : (want > passes ? passes : want);
  L->slice_k = (passes + want - 1) / want * gran;
  L->slices = ((int64_t)hc * H + L->slice_k - 1) / L->slice_k;
  unsigned __int128 off = L->ffn.total;
  auto take = [&](unsigned __int128 bytes) -> size_t {
    off = (off + 255) / 256 * 256;
    size_t at = (size_t)off;
    off += bytes;
    return at;
  };
  L->mixes = take(r * mw * 4);
  L->maps = take(r * mw * 4);
  L->ffn_in = take(r * H * 4);
  L->ffn_out = take(r * H * 4);
  L->partial = take((unsigned __int128)L->tiles * L->slices * L->tile_rows * (mw + 1) * 4);
  off = (off + 255) / 256 * 256;
  if (off >= lim) return false;
  L->total = (size_t)off;
  return true;
}

}  // namespace moe
