// C ABI of libmoeffn.so (declared in include/moe_ffn.h).
//
// Argument checks mirror the bails of forward_ffn_rows on the hf2q
// ffn_forward.rs page (layer/rows range, routed-row overflow, fixed MoE
// shape, state dtype/shape, "no routing source") and run on the host before
// any HIP call, so a rejected call leaves nothing on the stream and can be
// exercised without a GPU.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <string.h>
#include <vector>

#include "kernels.h"
#include "layout.h"
#include "moe_ffn.h"

namespace moe {
namespace {

bool dims_supported(const moe_dims_t* d) {
  if (d->reserved0 != 0 || d->reserved1 != 0 || d->n_shared != 1) return false;
  if (!(d->eps >= 0.0f) || !isfinite(d->eps)) return false;
  const bool full = d->hidden == 4096 && d->experts == 256 && d->top_k == 6 && d->inter == 2048;
  const bool tiny = d->hidden == 512 && d->experts == 32 && d->top_k == 6 && d->inter == 256;
  return full || tiny;
}

constexpr int64_t kMaxRows = (int64_t)1 << 24;  // keeps rows*top_k and every index within int32

int check_dims_rows(const moe_dims_t* d, int64_t rows) {
  if (!d) return MOE_EINVAL;
  if (rows <= 0) return MOE_EINVAL;
  if (!dims_supported(d)) return MOE_EUNSUPPORTED;
  if (rows > kMaxRows) return MOE_EOVERFLOW;
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_weights(const moe_dims_t* d, int layer_kind, const moe_weights_t* w, const int32_t* token_ids,
                  bool need_experts) {
  if (!w) return MOE_EINVAL;
  if (layer_kind != MOE_LAYER_SCORE && layer_kind != MOE_LAYER_HASH) return MOE_EINVAL;
  if (layer_kind == MOE_LAYER_SCORE && !w->sel_bias) return MOE_EINVAL;
  if (layer_kind == MOE_LAYER_HASH && (!w->tid2eid || !token_ids || d->table_rows <= 0)) return MOE_EINVAL;
  if (need_experts) {
    const void* req[] = {w->norm_w, w->router, w->gate_exps, w->up_exps, w->down_exps,
                         w->gate_sh, w->up_sh, w->down_sh};
    for (const void* p : req)
      if (!p || !aligned(p, 16)) return MOE_EINVAL;
  }
  return MOE_OK;
}

// The block-scaled weight struct checked like the bf16 one: the small
// parameters are shared, every code and scale array must be present and
// 16-byte aligned.  *common receives the small parameters (and the code
// arrays in the expert slots, only for the presence checks).
int check_mx_weights(const moe_mx_weights_t* w, moe_weights_t* common) {
  if (!w) return MOE_EINVAL;
  const moe_mx_matrix_t* m[] = {&w->gate_exps, &w->up_exps, &w->down_exps, &w->gate_sh, &w->up_sh, &w->down_sh};
  for (const moe_mx_matrix_t* p : m)
    if (!p->codes || !p->scales || !aligned(p->codes, 16) || !aligned(p->scales, 16)) return MOE_EINVAL;
  *common = moe_weights_t{w->norm_w, w->router, w->sel_bias, w->tid2eid,
                          (const uint16_t*)w->gate_exps.codes, (const uint16_t*)w->up_exps.codes,
                          (const uint16_t*)w->down_exps.codes, (const uint16_t*)w->gate_sh.codes,
                          (const uint16_t*)w->up_sh.codes, (const uint16_t*)w->down_sh.codes};
  return MOE_OK;
}

struct TimerRec {
  const char* name;
  hipEvent_t start, stop;
};

struct StageTimer {
  std::mutex mu;
  bool enabled = false;
  std::vector<TimerRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

StageTimer& timer() {
  static StageTimer t;
  return t;
}

}  // namespace

hipError_t launch(const char* name, const void* fn, dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                  void* args) {
  void* argv[1] = {args};
  hipEvent_t e0 = nullptr, e1 = nullptr;
  StageTimer& T = timer();
  std::unique_lock<std::mutex> lk(T.mu);
  if (T.enabled) {
    e0 = T.get();
    e1 = T.get();
  } else {
    lk.unlock();
  }
  hipError_t err = hipExtLaunchKernel(fn, grid, block, argv, shmem, stream, e0, e1, 0);
  if (e0 && e1) T.recs.push_back({name, e0, e1});
  return err;
}

// The wrapper's parameters: hc streams supported, a positive round count,
// every array present (hc_fn 16-byte aligned for its 8-byte loads).
int check_hc_weights(const moe_hc_weights_t* hw) {
  if (!hw) return MOE_EINVAL;
  if (hw->hc < 1 || hw->hc > kHcMax) return MOE_EUNSUPPORTED;
  if (hw->sinkhorn_iters < 1 || hw->sinkhorn_iters > MOE_HC_MAX_ITERS) return MOE_EINVAL;
  if (!hw->hc_fn || !hw->hc_scale || !hw->hc_base || !aligned(hw->hc_fn, 16) || !aligned(hw->hc_scale, 4) ||
      !aligned(hw->hc_base, 4))
    return MOE_EINVAL;
  return MOE_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_ffn_workspace_bytes(const moe_dims_t* d, int64_t rows, size_t* bytes) {
  int rc = check_dims_rows(d, rows);
  if (rc) return rc;
  if (!bytes) return MOE_EINVAL;
  Layout L;
  if (!make_layout(rows, d->hidden, d->experts, d->top_k, d->inter, &L)) return MOE_EOVERFLOW;
  *bytes = L.total;
  return MOE_OK;
}

}  // extern "C"

namespace moe {
namespace {

// Host checks of a forward call that need no workspace: dims, rows,
// pointers, layer kind, overlap of x and out.  Fills *L with the workspace
// layout for `rows`.
int check_forward_args(const moe_dims_t* d, const float* x, const int32_t* token_ids, int64_t rows, int layer_kind,
                       const moe_weights_t* w, const float* out, Layout* L) {
  int rc = check_dims_rows(d, rows);
  if (rc) return rc;
  if (!x || !out || !aligned(x, 16) || !aligned(out, 16)) return MOE_EINVAL;
  rc = check_weights(d, layer_kind, w, token_ids, true);
  if (rc) return rc;
  if (!make_layout(rows, d->hidden, d->experts, d->top_k, d->inter, L)) return MOE_EOVERFLOW;
  const size_t nbytes = (size_t)rows * d->hidden * sizeof(float);
  const uintptr_t xb = (uintptr_t)x, ob = (uintptr_t)out;
  if (xb < ob + nbytes && ob < xb + nbytes) return MOE_EOVERLAP;
  return MOE_OK;
}

// The forward with its intermediates carved from `workspace` (already
// checked: at least L.total bytes, 256-byte aligned).  With `mx` the expert
// matrices are the block-scaled ones there, in format `mx_format` (1 MXFP8,
// 2 MXFP4; w then supplies only the small parameters).
// The hyper-connection wrapper folded into a decode call: the split in the
// head (from the mix launch's partials), the pre-mix in its staging, the
// post-mix in the reduce.
struct HcPost {
  int hc, iters;
  int64_t slices;
  const float* state;
  const float* partial;
  const float* scale;
  const float* base;
  float* mixes;
  float* maps;
  float* x;  // the FFN input, stored for the view
  float* out;
};

int forward_in(const moe_dims_t* d, const float* x, const int32_t* token_ids, int64_t rows, int layer_kind,
               const moe_weights_t* w, const moe_mx_weights_t* mx, int mx_format, float* out, void* workspace,
               const Layout& L, void* stream, const HcPost* post = nullptr) {
  char* ws = (char*)workspace;
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.R = (int)rows;
  a.H = d->hidden;
  a.E = d->experts;
  a.K = d->top_k;
  a.I = d->inter;
  a.eps = d->eps;
  a.layer_kind = layer_kind;
  a.table_rows = d->table_rows;
  a.x = x;
  a.token_ids = token_ids;
  a.norm_w = w->norm_w;
  a.router = w->router;
  a.bias = w->sel_bias;
  a.table = w->tid2eid;
  a.gate = w->gate_exps;
  a.up = w->up_exps;
  a.down = w->down_exps;
  a.gate_sh = w->gate_sh;
  a.up_sh = w->up_sh;
  a.down_sh = w->down_sh;
  if (mx) {
    a.gate = a.up = a.down = a.gate_sh = a.up_sh = a.down_sh = nullptr;
    a.mx = mx_format;
    a.gate_q = mx->gate_exps.codes;
    a.up_q = mx->up_exps.codes;
    a.down_q = mx->down_exps.codes;
    a.gate_sh_q = mx->gate_sh.codes;
    a.up_sh_q = mx->up_sh.codes;
    a.down_sh_q = mx->down_sh.codes;
    a.gate_s = mx->gate_exps.scales;
    a.up_s = mx->up_exps.scales;
    a.down_s = mx->down_exps.scales;
    a.gate_sh_s = mx->gate_sh.scales;
    a.up_sh_s = mx->up_sh.scales;
    a.down_sh_s = mx->down_sh.scales;
  }
  a.out = out;
  if (post) {
    a.hc = post->hc;
    a.hc_iters = post->iters;
    a.hc_slices = post->slices;
    a.hc_state = post->state;
    a.hc_partial = post->partial;
    a.hc_scale = post->scale;
    a.hc_base = post->base;
    a.hc_mixes = post->mixes;
    a.hc_maps = post->maps;
    a.hc_x = post->x;
    a.hc_out = post->out;
  }
  a.status = (uint32_t*)(ws + L.status);
  a.sync = (DecodeSync*)(ws + L.status + 64);  // both paths: the status block
  a.logits = (float*)(ws + L.logits);
  a.idx = (int32_t*)(ws + L.idx);
  a.wts = (float*)(ws + L.wts);
  a.rowflags = (uint32_t*)(ws + L.rowflags);
  const bool decode = rows <= kDecodeMaxRows;
  if (decode) {
    a.xn32 = (float*)(ws + L.xn32);
    a.plan = (DecodePlan*)(ws + L.plan);
    a.h32 = (float*)(ws + L.h32);
    a.d32 = (float*)(ws + L.d32);
  } else {
    a.xn16 = (_Float16*)(ws + L.xn16);
    a.xlo16 = (_Float16*)(ws + L.xlo16);
    a.cnt = (int32_t*)(ws + L.cnt);
    a.mask = (uint32_t*)(ws + L.mask);
    a.rcnt = (uint32_t*)(ws + L.rcnt);
    a.gctr = (uint32_t*)(ws + L.gctr);
    a.slot_rank = (int32_t*)(ws + L.slot_rank);
    a.perm = (int32_t*)(ws + L.perm);
    a.h16 = (_Float16*)(ws + L.h16);
    a.d16 = (_Float16*)(ws + L.d16);
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = decode ? run_decode(a, s) : run_prefill(a, s);
  return err == hipSuccess ? MOE_OK : MOE_EHIP;
}

// ---- the allocation-free entry point's scratch ---------------------------
// The intermediates of moe_ffn_forward_noalloc live in this array, one copy
// per GPU (each device that loads the library's code holds its own, until
// the process ends).  In host code `scratch` names a host-side stand-in, not
// the device array: its device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// ever passed to a kernel.
constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  void* ptr = nullptr;   // device address of this device's `scratch`
  bool zeroed = false;   // its handoff words were zeroed by a call that ran (not only captured)
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxDevices];

__global__ void k_zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// Device address of the scratch on the device `stream` belongs to.  Until
// a call on that device has run outside stream capture, the call first
// enqueues a fill kernel that zeroes the status block (the decode path's
// handoff words must start at 0); inside a capture the fill becomes part of
// the graph and runs before the forward on every replay, which is harmless.
int scratch_for(hipStream_t stream, size_t zero_bytes, void** out) {
  int dev = 0, cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return MOE_EHIP;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return MOE_EHIP;
  } else {
    dev = cur;
  }
  if (dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchSlot& sl = g_scratch[dev];
  if (!sl.ptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return MOE_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p || !aligned(p, 256)) return MOE_EHIP;
    sl.ptr = p;
  }
  if (!sl.zeroed) {
    const int n = (int)(zero_bytes / 4);
    void* argv[2];
    uint32_t* wp = (uint32_t*)sl.ptr;
    int nn = n;
    argv[0] = &wp;
    argv[1] = &nn;
    if (hipLaunchKernel((const void*)k_zero_words, dim3((n + 255) / 256), dim3(256), argv, 0, stream) != hipSuccess)
      return MOE_EHIP;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return MOE_EHIP;
    if (cs == hipStreamCaptureStatusNone) sl.zeroed = true;
  }
  *out = sl.ptr;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_ffn_forward(const moe_dims_t* d, const float* x, const int32_t* token_ids, int64_t rows, int layer_kind,
                    const moe_weights_t* w, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  Layout L;
  const int rc = check_forward_args(d, x, token_ids, rows, layer_kind, w, out, &L);
  if (rc) return rc;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total) return MOE_EWORKSPACE;
  return forward_in(d, x, token_ids, rows, layer_kind, w, nullptr, 0, out, workspace, L, stream);
}

int moe_ffn_forward_noalloc(const moe_dims_t* d, const float* x, const int32_t* token_ids, int64_t rows,
                            int layer_kind, const moe_weights_t* w, float* out, void* stream) {
  Layout L;
  int rc = check_forward_args(d, x, token_ids, rows, layer_kind, w, out, &L);
  if (rc) return rc;
  if (L.total > kScratchBytes) return MOE_ESCRATCH;
  void* ws = nullptr;
  rc = scratch_for((hipStream_t)stream, L.logits, &ws);  // the status block precedes the logits
  if (rc) return rc;
  return forward_in(d, x, token_ids, rows, layer_kind, w, nullptr, 0, out, ws, L, stream);
}

int moe_ffn_forward_mxfp8(const moe_dims_t* d, const float* x, const int32_t* token_ids, int64_t rows, int layer_kind,
                          const moe_mx_weights_t* w, float* out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  moe_weights_t common;
  int rc = check_dims_rows(d, rows);
  if (rc) return rc;
  rc = check_mx_weights(w, &common);
  if (rc) return rc;
  Layout L;
  rc = check_forward_args(d, x, token_ids, rows, layer_kind, &common, out, &L);
  if (rc) return rc;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total) return MOE_EWORKSPACE;
  return forward_in(d, x, token_ids, rows, layer_kind, &common, w, 1, out, workspace, L, stream);
}

int moe_ffn_forward_mxfp4(const moe_dims_t* d, const float* x, const int32_t* token_ids, int64_t rows, int layer_kind,
                          const moe_mx_weights_t* w, float* out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  moe_weights_t common;
  int rc = check_dims_rows(d, rows);
  if (rc) return rc;
  rc = check_mx_weights(w, &common);
  if (rc) return rc;
  Layout L;
  rc = check_forward_args(d, x, token_ids, rows, layer_kind, &common, out, &L);
  if (rc) return rc;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total) return MOE_EWORKSPACE;
  return forward_in(d, x, token_ids, rows, layer_kind, &common, w, 2, out, workspace, L, stream);
}

int moe_route(const moe_dims_t* d, const float* logits, const int32_t* token_ids, int64_t rows, int layer_kind,
              const moe_weights_t* w, int32_t* idx, float* wout, void* stream) {
  int rc = check_dims_rows(d, rows);
  if (rc) return rc;
  if (!logits || !idx || !wout) return MOE_EINVAL;
  rc = check_weights(d, layer_kind, w, token_ids, false);
  if (rc) return rc;
  RouteArgs a;
  a.R = (int)rows;
  a.E = d->experts;
  a.K = d->top_k;
  a.layer_kind = layer_kind;
  a.table_rows = d->table_rows;
  a.logits = logits;
  a.token_ids = token_ids;
  a.bias = w->sel_bias;
  a.table = w->tid2eid;
  a.idx = idx;
  a.w = wout;
  return run_route(a, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_ffn_hc_workspace_bytes(const moe_dims_t* d, int32_t hc, int64_t rows, size_t* bytes) {
  int rc = check_dims_rows(d, rows);
  if (rc) return rc;
  if (!bytes) return MOE_EINVAL;
  if (hc < 1 || hc > kHcMax) return MOE_EUNSUPPORTED;
  HcLayout L;
  if (!make_hc_layout(rows, d->hidden, d->experts, d->top_k, d->inter, hc, &L)) return MOE_EOVERFLOW;
  *bytes = L.total;
  return MOE_OK;
}

int moe_ffn_forward_hc(const moe_dims_t* d, const float* state_in, const int32_t* token_ids, int64_t rows,
                       int layer_kind, const moe_weights_t* w, const moe_hc_weights_t* hw, float* state_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims_rows(d, rows);
  if (rc) return rc;
  rc = check_hc_weights(hw);
  if (rc) return rc;
  if (!state_in || !state_out || !aligned(state_in, 16) || !aligned(state_out, 16)) return MOE_EINVAL;
  rc = check_weights(d, layer_kind, w, token_ids, true);
  if (rc) return rc;
  HcLayout L;
  if (!make_hc_layout(rows, d->hidden, d->experts, d->top_k, d->inter, hw->hc, &L)) return MOE_EOVERFLOW;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total) return MOE_EWORKSPACE;
  const size_t sbytes = (size_t)rows * hw->hc * d->hidden * sizeof(float);
  if (overlaps(state_in, sbytes, state_out, sbytes) || overlaps(state_out, sbytes, workspace, L.total) ||
      overlaps(state_in, sbytes, workspace, L.total))
    return MOE_EOVERLAP;
  char* ws = (char*)workspace;
  HcArgs a;
  memset(&a, 0, sizeof(a));
  a.R = (int)rows;
  a.H = d->hidden;
  a.hc = hw->hc;
  a.iters = hw->sinkhorn_iters;
  a.eps = d->eps;
  a.slices = L.slices;
  a.slice_k = (int)L.slice_k;
  a.tile_rows = (int)L.tile_rows;
  a.state = state_in;
  a.fn = hw->hc_fn;
  a.scale = hw->hc_scale;
  a.base = hw->hc_base;
  a.mixes = (float*)(ws + L.mixes);
  a.maps = (float*)(ws + L.maps);
  a.partial = (float*)(ws + L.partial);
  a.ffn_in = (float*)(ws + L.ffn_in);
  a.ffn_out = (float*)(ws + L.ffn_out);
  a.out = state_out;
  // 1-4 rows: the mix launch leaves its slice partials, the decode head
  // splits and forms the FFN input from the streams, and the decode reduce
  // does the post-mix
  const bool small = rows <= kDecodeMaxRows;
  hipStream_t s = (hipStream_t)stream;
  if (run_hc_pre(a, s) != hipSuccess) return MOE_EHIP;
  const HcPost post{hw->hc, a.iters, a.slices, state_in, a.partial, a.scale, a.base, a.mixes, a.maps, a.ffn_in,
                    state_out};
  rc = forward_in(d, a.ffn_in, token_ids, rows, layer_kind, w, nullptr, 0, (float*)(ws + L.ffn_out), workspace,
                  L.ffn, stream, small ? &post : nullptr);
  if (rc) return rc;
  if (small) return MOE_OK;
  return run_hc_post(a, s) == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_ffn_hc_view(const moe_dims_t* d, int32_t hc, int64_t rows, void* workspace, size_t workspace_bytes,
                    const float** mixes, const float** maps, const float** ffn_in, const float** ffn_out) {
  int rc = check_dims_rows(d, rows);
  if (rc) return rc;
  if (hc < 1 || hc > kHcMax) return MOE_EUNSUPPORTED;
  HcLayout L;
  if (!make_hc_layout(rows, d->hidden, d->experts, d->top_k, d->inter, hc, &L)) return MOE_EOVERFLOW;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total) return MOE_EWORKSPACE;
  char* ws = (char*)workspace;
  if (mixes) *mixes = (const float*)(ws + L.mixes);
  if (maps) *maps = (const float*)(ws + L.maps);
  if (ffn_in) *ffn_in = (const float*)(ws + L.ffn_in);
  if (ffn_out) *ffn_out = (const float*)(ws + L.ffn_out);
  return MOE_OK;
}

int moe_ffn_routing_view(const moe_dims_t* d, int64_t rows, void* workspace, size_t workspace_bytes,
                         const float** logits, const int32_t** idx, const float** wout) {
  int rc = check_dims_rows(d, rows);
  if (rc) return rc;
  Layout L;
  if (!make_layout(rows, d->hidden, d->experts, d->top_k, d->inter, &L)) return MOE_EOVERFLOW;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total) return MOE_EWORKSPACE;
  char* ws = (char*)workspace;
  if (logits) *logits = (const float*)(ws + L.logits);
  if (idx) *idx = (const int32_t*)(ws + L.idx);
  if (wout) *wout = (const float*)(ws + L.wts);
  return MOE_OK;
}

int moe_ffn_status(const void* workspace, void* stream, uint32_t* flags) {
  if (!workspace || !flags) return MOE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_EHIP;
  uint32_t v = 0;
  if (hipMemcpy(&v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return MOE_EHIP;
  *flags = v;
  return MOE_OK;
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported layer dimensions";
    case MOE_EOVERFLOW: return "size overflow";
    case MOE_EWORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_EHIP: return "HIP launch or runtime error";
    case MOE_EOVERLAP: return "x and out overlap";
    case MOE_ESCRATCH: return "rows need more intermediate memory than the allocation-free entry point's scratch holds";
    default: return "unknown status";
  }
}

int moe_ffn_stage_timing_begin(void) {
  StageTimer& T = timer();
  std::lock_guard<std::mutex> lk(T.mu);
  T.enabled = true;
  return MOE_OK;
}

int moe_ffn_stage_timing_end(int max, const char** names, double* total_ms, int64_t* launches, int* n) {
  if (max < 0 || !n || (max > 0 && (!names || !total_ms || !launches))) return MOE_EINVAL;
  StageTimer& T = timer();
  std::lock_guard<std::mutex> lk(T.mu);
  T.enabled = false;
  std::vector<const char*> nm;
  std::vector<double> ms;
  std::vector<int64_t> cnt;
  int rc = MOE_OK;
  for (auto& r : T.recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) rc = MOE_EHIP;
    float el = 0.f;
    if (rc == MOE_OK && hipEventElapsedTime(&el, r.start, r.stop) != hipSuccess) rc = MOE_EHIP;
    size_t i = 0;
    while (i < nm.size() && strcmp(nm[i], r.name) != 0) ++i;
    if (i == nm.size()) {
      nm.push_back(r.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[i] += el;
    cnt[i] += 1;
    T.pool.push_back(r.start);
    T.pool.push_back(r.stop);
  }
  T.recs.clear();
  *n = (int)nm.size();
  for (int i = 0; i < max && i < (int)nm.size(); ++i) {
    names[i] = nm[i];
    total_ms[i] = ms[i];
    launches[i] = cnt[i];
  }
  return rc;
}

}  // extern "C"
