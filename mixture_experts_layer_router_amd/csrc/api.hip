// C-ABI entry points of lc_moe: argument checks, workspace carving, launch sequence.
// The layer definition and every argument's meaning are documented in include/lc_moe.h.
#include <mutex>

#include "common.h"

using namespace lcm;

// Workspace of lc_moe_forward_noalloc: one copy per GPU, allocated by the runtime with the
// library's code object.  In host code `scratch` is a stand-in symbol, not a device
// address: host code only ever uses the address hipGetSymbolAddress returns for the
// current device.
static __device__ __align__(256) unsigned char scratch[LC_MOE_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's `scratch`, looked up once per device with the device
// current (each GPU holds its own copy at its own address).
lc_moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LC_MOE_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LC_MOE_E_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LC_MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

lc_moe_status check_shape(const lc_moe_shape* s) {
  if (!s) return LC_MOE_E_NULLPTR;
  if (s->dtype != LC_MOE_F32 && s->dtype != LC_MOE_BF16) return LC_MOE_E_DTYPE;
  if (s->T < 1 || s->d < 1 || s->N < 1 || s->K < 1 || s->I < 1 || s->Z < 0) return LC_MOE_E_SHAPE;
  const long long E = static_cast<long long>(s->N) + s->Z;
  if (s->K > E || E > kMaxE || s->N > kMaxN) return LC_MOE_E_SHAPE;
  if (static_cast<long long>(s->T) * s->K >= (1LL << 31)) return LC_MOE_E_SHAPE;
  const int vec = s->dtype == LC_MOE_BF16 ? 8 : 4;
  if (s->d % vec != 0 || s->I % vec != 0) return LC_MOE_E_SHAPE;
  if (!grids_fit(*s)) return LC_MOE_E_SHAPE;
  return LC_MOE_OK;
}

// Non-null and 16-byte aligned (optional pointers may be null).
lc_moe_status check_ptr(const void* p, bool optional = false) {
  if (!p) return optional ? LC_MOE_OK : LC_MOE_E_NULLPTR;
  return aligned16(p) ? LC_MOE_OK : LC_MOE_E_ALIGN;
}

lc_moe_status check_ws(const lc_moe_shape* s, const void* ws, size_t bytes, WsPlan& plan) {
  plan = plan_workspace(*s);
  if (!ws) return LC_MOE_E_NULLPTR;
  if (!aligned16(ws)) return LC_MOE_E_ALIGN;
  if (bytes < plan.total) return LC_MOE_E_WORKSPACE;
  return LC_MOE_OK;
}

#define LCM_CHECK(expr)                        \
  do {                                         \
    lc_moe_status _st = (expr);                \
    if (_st != LC_MOE_OK) return _st;          \
  } while (0)
#define LCM_LAUNCH(expr)                       \
  do {                                         \
    if ((expr) != hipSuccess) return LC_MOE_E_DEVICE; \
  } while (0)

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

// route -> histogram -> scan -> scatter, shared by permute and forward.
lc_moe_status permute_core(const lc_moe_shape& s, const int32_t* idx, const WsPlan& p, void* ws,
                           int32_t* load, int32_t* offsets, int32_t* slot_row,
                           int32_t* perm_token, int32_t* ffn_cnt, hipStream_t st) {
  if (p.nblocks == 1) {  // one token block: the three steps in one workgroup
    LCM_LAUNCH(launch_permute_small(s, idx, load, ffn_cnt, offsets, at<MTile>(ws, p.mtiles),
                                    at<int32_t>(ws, p.n_mtiles), p.bm, slot_row, perm_token, st));
    return LC_MOE_OK;
  }
  int32_t* bc = at<int32_t>(ws, p.block_counts);
  int32_t* bb = at<int32_t>(ws, p.block_base);
  LCM_LAUNCH(launch_histogram(s, idx, bc, ffn_cnt, p.nblocks, st));
  LCM_LAUNCH(launch_scan(s, bc, p.nblocks, load, offsets, bb, at<MTile>(ws, p.mtiles),
                         at<int32_t>(ws, p.n_mtiles), p.bm, st));
  LCM_LAUNCH(launch_scatter(s, idx, bb, p.nblocks, slot_row, perm_token, st));
  return LC_MOE_OK;
}

}  // namespace

extern "C" {

size_t lc_moe_workspace_size(const lc_moe_shape* shape) {
  if (check_shape(shape) != LC_MOE_OK) return 0;
  return plan_workspace(*shape).total;
}

const char* lc_moe_status_str(lc_moe_status status) {
  switch (status) {
    case LC_MOE_OK: return "ok";
    case LC_MOE_E_NULLPTR: return "a required pointer is NULL";
    case LC_MOE_E_SHAPE: return "shape out of range";
    case LC_MOE_E_DTYPE: return "unknown dtype";
    case LC_MOE_E_ALIGN: return "pointer not 16-byte aligned";
    case LC_MOE_E_WORKSPACE: return "workspace too small";
    case LC_MOE_E_DEVICE: return "HIP launch error";
  }
  return "unknown status";
}

const char* lc_moe_stage_name(int stage) {
  static const char* names[LC_MOE_NUM_STAGES] = {"route", "permute", "gate_up", "down", "combine"};
  return (stage >= 0 && stage < LC_MOE_NUM_STAGES) ? names[stage] : "unknown";
}

lc_moe_status lc_moe_route(const lc_moe_shape* shape, const void* x, const float* w_router,
                           const float* bias, int32_t* topk_idx, float* topk_gate,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  LCM_CHECK(check_shape(shape));
  LCM_CHECK(check_ptr(x));
  LCM_CHECK(check_ptr(w_router));
  LCM_CHECK(check_ptr(bias));
  LCM_CHECK(check_ptr(topk_idx));
  LCM_CHECK(check_ptr(topk_gate));
  WsPlan p;
  LCM_CHECK(check_ws(shape, workspace, workspace_bytes, p));
  float* logits = at<float>(workspace, p.logits);
  LCM_LAUNCH(launch_router_logits(*shape, x, w_router, at<bf16_t>(workspace, p.wsplit), logits,
                                  at<float>(workspace, p.rpart), stream));
  LCM_LAUNCH(launch_router_topk(*shape, logits, bias, topk_idx, topk_gate, stream));
  return LC_MOE_OK;
}

lc_moe_status lc_moe_expert_load(const lc_moe_shape* shape, const int32_t* topk_idx,
                                 int32_t* load, int32_t* ffn_per_token, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  LCM_CHECK(check_shape(shape));
  LCM_CHECK(check_ptr(topk_idx));
  LCM_CHECK(check_ptr(load));
  LCM_CHECK(check_ptr(ffn_per_token, true));
  WsPlan p;
  LCM_CHECK(check_ws(shape, workspace, workspace_bytes, p));
  int32_t* bc = at<int32_t>(workspace, p.block_counts);
  LCM_LAUNCH(launch_histogram(*shape, topk_idx, bc, ffn_per_token, p.nblocks, stream));
  LCM_LAUNCH(launch_scan(*shape, bc, p.nblocks, load, at<int32_t>(workspace, p.offsets),
                         at<int32_t>(workspace, p.block_base), at<MTile>(workspace, p.mtiles),
                         at<int32_t>(workspace, p.n_mtiles), p.bm, stream));
  return LC_MOE_OK;
}

lc_moe_status lc_moe_permute(const lc_moe_shape* shape, const void* x, const int32_t* topk_idx,
                             int32_t* ffn_offsets, int32_t* perm_token, int32_t* slot_row,
                             void* x_perm, int32_t* load, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  LCM_CHECK(check_shape(shape));
  LCM_CHECK(check_ptr(x, x_perm == nullptr));
  LCM_CHECK(check_ptr(topk_idx));
  LCM_CHECK(check_ptr(ffn_offsets));
  LCM_CHECK(check_ptr(perm_token));
  LCM_CHECK(check_ptr(slot_row));
  LCM_CHECK(check_ptr(x_perm, true));
  LCM_CHECK(check_ptr(load, true));
  WsPlan p;
  LCM_CHECK(check_ws(shape, workspace, workspace_bytes, p));
  int32_t* ld = load ? load : at<int32_t>(workspace, p.load);
  LCM_CHECK(permute_core(*shape, topk_idx, p, workspace, ld, ffn_offsets, slot_row, perm_token,
                         nullptr, stream));
  if (x_perm) LCM_LAUNCH(launch_gather_rows(*shape, x, perm_token, ffn_offsets, x_perm, stream));
  return LC_MOE_OK;
}

lc_moe_status lc_moe_forward_staged(const lc_moe_shape* shape, const void* x,
                                    const lc_moe_weights* weights, void* y, int32_t* topk_idx,
                                    float* topk_gate, int32_t* load, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t* stage_events) {
  LCM_CHECK(check_shape(shape));
  if (!weights) return LC_MOE_E_NULLPTR;
  LCM_CHECK(check_ptr(x));
  LCM_CHECK(check_ptr(weights->w_router));
  LCM_CHECK(check_ptr(weights->bias));
  if (weights->fp8 && weights->packed) return LC_MOE_E_DTYPE;  // one weight format
  if (weights->fp8_act && !weights->fp8) return LC_MOE_E_DTYPE;
  if (weights->fp8) {
    LCM_CHECK(check_ptr(weights->fp8));
    if (shape->dtype != LC_MOE_BF16) return LC_MOE_E_DTYPE;
    if (plan_fp8(*shape).total == 0) return LC_MOE_E_SHAPE;
    if (weights->fp8_act && !fp8_mfma_ok(*shape)) return LC_MOE_E_SHAPE;
  } else if (weights->packed) {
    LCM_CHECK(check_ptr(weights->packed));
    if (shape->dtype != LC_MOE_BF16) return LC_MOE_E_DTYPE;
    if (plan_packed(*shape).total == 0) return LC_MOE_E_SHAPE;
  } else {
    LCM_CHECK(check_ptr(weights->w_gate));
    LCM_CHECK(check_ptr(weights->w_up));
    LCM_CHECK(check_ptr(weights->w_down));
  }
  LCM_CHECK(check_ptr(y));
  LCM_CHECK(check_ptr(topk_idx, true));
  LCM_CHECK(check_ptr(topk_gate, true));
  LCM_CHECK(check_ptr(load, true));
  WsPlan p;
  LCM_CHECK(check_ws(shape, workspace, workspace_bytes, p));
  if (stage_events) {
    for (int i = 0; i <= LC_MOE_NUM_STAGES; ++i)
      if (!stage_events[i]) return LC_MOE_E_NULLPTR;
  }
  const lc_moe_shape& s = *shape;
  auto mark = [&](int i) -> bool {
    return !stage_events || hipEventRecord(stage_events[i], stream) == hipSuccess;
  };
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(workspace, p.idx);
  float* gate = topk_gate ? topk_gate : at<float>(workspace, p.gate);
  int32_t* ld = load ? load : at<int32_t>(workspace, p.load);
  int32_t* offsets = at<int32_t>(workspace, p.offsets);
  int32_t* perm_token = at<int32_t>(workspace, p.perm_token);
  int32_t* slot_row = at<int32_t>(workspace, p.slot_row);
  const MTile* mtiles = at<MTile>(workspace, p.mtiles);
  const int32_t* n_mtiles = at<int32_t>(workspace, p.n_mtiles);
  void* hbuf = at<char>(workspace, p.hbuf);
  void* ybuf = at<char>(workspace, p.ybuf);

  // A layer of one token block runs top-K and permutation as one kernel (counted in the
  // route stage; the permute stage's span is then empty).
  const bool fused = p.nblocks == 1;
  int32_t* done = at<int32_t>(workspace, p.done);
  if (!mark(0)) return LC_MOE_E_DEVICE;
  LCM_LAUNCH(launch_router_logits(s, x, weights->w_router, at<bf16_t>(workspace, p.wsplit),
                                  at<float>(workspace, p.logits), at<float>(workspace, p.rpart),
                                  stream, fused ? done : nullptr));
  if (fused)
    LCM_LAUNCH(launch_topk_permute(s, at<float>(workspace, p.logits), weights->bias, idx, gate, done, ld,
                                   offsets, at<MTile>(workspace, p.mtiles), at<int32_t>(workspace, p.n_mtiles),
                                   p.bm, slot_row, perm_token, stream));
  else
    LCM_LAUNCH(launch_router_topk(s, at<float>(workspace, p.logits), weights->bias, idx, gate, stream));
  if (!mark(1)) return LC_MOE_E_DEVICE;
  if (!fused) LCM_CHECK(permute_core(s, idx, p, workspace, ld, offsets, slot_row, perm_token, nullptr, stream));
  if (!mark(2)) return LC_MOE_E_DEVICE;
  if (weights->fp8_act) {  // x quantized, then the FP8 MFMA gate/up (H quantized in it)
    LCM_LAUNCH(launch_quantize_act(x, s.T, s.d, at<unsigned char>(workspace, p.xq),
                                   at<unsigned char>(workspace, p.xs), stream));
    LCM_LAUNCH(launch_ffn_fp8_mfma(s, p, workspace, weights->fp8, 0, stream));
  } else {
    LCM_LAUNCH(launch_ffn_gate_up(s, x, perm_token, weights->w_gate, weights->w_up, weights->fp8,
                                  weights->packed, hbuf, mtiles, offsets, n_mtiles, p.mt_max, stream));
  }
  if (!mark(3)) return LC_MOE_E_DEVICE;
  if (weights->fp8_act)
    LCM_LAUNCH(launch_ffn_fp8_mfma(s, p, workspace, weights->fp8, 1, stream));
  else
    LCM_LAUNCH(launch_ffn_down(s, hbuf, weights->w_down, weights->fp8, weights->packed, ybuf, mtiles, offsets,
                               n_mtiles, p.mt_max, stream));
  if (!mark(4)) return LC_MOE_E_DEVICE;
  LCM_LAUNCH(launch_combine(s, x, ybuf, slot_row, gate, y, stream));
  if (!mark(5)) return LC_MOE_E_DEVICE;
  return LC_MOE_OK;
}

size_t lc_moe_fp8_weights_size(const lc_moe_shape* shape) {
  if (check_shape(shape) != LC_MOE_OK || shape->dtype != LC_MOE_BF16) return 0;
  return plan_fp8(*shape).total;
}

lc_moe_status lc_moe_quantize_weights(const lc_moe_shape* shape, const void* w_gate,
                                      const void* w_up, const void* w_down, void* fp8_weights,
                                      size_t fp8_weights_bytes, hipStream_t stream) {
  LCM_CHECK(check_shape(shape));
  if (shape->dtype != LC_MOE_BF16) return LC_MOE_E_DTYPE;
  if (plan_fp8(*shape).total == 0) return LC_MOE_E_SHAPE;
  LCM_CHECK(check_ptr(w_gate));
  LCM_CHECK(check_ptr(w_up));
  LCM_CHECK(check_ptr(w_down));
  LCM_CHECK(check_ptr(fp8_weights));
  if (fp8_weights_bytes < plan_fp8(*shape).total) return LC_MOE_E_WORKSPACE;
  LCM_LAUNCH(launch_quantize_weights(*shape, w_gate, w_up, w_down, fp8_weights, stream));
  return LC_MOE_OK;
}

lc_moe_status lc_moe_quantize_activations(const void* x, int32_t rows, int32_t cols, void* codes,
                                          void* scales, hipStream_t stream) {
  if (cols < 64 || cols > 16384 || cols % 64 != 0 || rows < 0 || rows >= (1 << 24)) return LC_MOE_E_SHAPE;
  if (rows == 0) return LC_MOE_OK;
  LCM_CHECK(check_ptr(x));
  LCM_CHECK(check_ptr(codes));
  LCM_CHECK(check_ptr(scales));
  LCM_LAUNCH(launch_quantize_act(x, rows, cols, static_cast<unsigned char*>(codes),
                                 static_cast<unsigned char*>(scales), stream));
  return LC_MOE_OK;
}

size_t lc_moe_packed_weights_size(const lc_moe_shape* shape) {
  if (check_shape(shape) != LC_MOE_OK || shape->dtype != LC_MOE_BF16) return 0;
  return plan_packed(*shape).total;
}

lc_moe_status lc_moe_pack_weights(const lc_moe_shape* shape, const void* w_gate,
                                  const void* w_up, const void* w_down, void* packed_weights,
                                  size_t packed_weights_bytes, hipStream_t stream) {
  LCM_CHECK(check_shape(shape));
  if (shape->dtype != LC_MOE_BF16) return LC_MOE_E_DTYPE;
  if (plan_packed(*shape).total == 0) return LC_MOE_E_SHAPE;
  LCM_CHECK(check_ptr(w_gate));
  LCM_CHECK(check_ptr(w_up));
  LCM_CHECK(check_ptr(w_down));
  LCM_CHECK(check_ptr(packed_weights));
  if (packed_weights_bytes < plan_packed(*shape).total) return LC_MOE_E_WORKSPACE;
  LCM_LAUNCH(launch_pack_weights(*shape, w_gate, w_up, w_down, packed_weights, stream));
  return LC_MOE_OK;
}

lc_moe_status lc_moe_bias_update(const lc_moe_shape* shape, const lc_moe_pid* gains,
                                 const int32_t* load, const float* target, float* bias,
                                 float* integral, float* prev_err, hipStream_t stream) {
  LCM_CHECK(check_shape(shape));
  if (!gains) return LC_MOE_E_NULLPTR;
  LCM_CHECK(check_ptr(load));
  LCM_CHECK(check_ptr(target));
  LCM_CHECK(check_ptr(bias));
  LCM_CHECK(check_ptr(integral));
  LCM_CHECK(check_ptr(prev_err));
  const int E = shape->N + shape->Z;
  LCM_LAUNCH(launch_bias_update(E, static_cast<long long>(shape->T) * shape->K, gains->kp,
                                gains->ki, gains->kd, load, target, bias, integral, prev_err,
                                stream));
  return LC_MOE_OK;
}

lc_moe_status lc_moe_forward_noalloc(const lc_moe_shape* shape, const void* x,
                                     const lc_moe_weights* weights, void* y, int32_t* topk_idx,
                                     float* topk_gate, int32_t* load, hipStream_t stream) {
  LCM_CHECK(check_shape(shape));
  if (plan_workspace(*shape).total > LC_MOE_STATIC_WORKSPACE_BYTES) return LC_MOE_E_WORKSPACE;
  void* ws = nullptr;
  LCM_CHECK(scratch_of_current_device(&ws));
  return lc_moe_forward_staged(shape, x, weights, y, topk_idx, topk_gate, load, ws,
                               LC_MOE_STATIC_WORKSPACE_BYTES, stream, nullptr);
}

size_t lc_moe_backward_workspace_size(const lc_moe_shape* shape) {
  if (check_shape(shape) != LC_MOE_OK || shape->dtype != LC_MOE_BF16 || shape->d % 32 || shape->I % 32) return 0;
  return plan_backward(*shape).total;
}

lc_moe_status lc_moe_ffn_backward(const lc_moe_shape* shape, const void* x,
                                  const lc_moe_weights* weights, const int32_t* topk_idx,
                                  const float* topk_gate, const void* dy, void* dx, void* dw_gate,
                                  void* dw_up, void* dw_down, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  LCM_CHECK(check_shape(shape));
  if (shape->dtype != LC_MOE_BF16) return LC_MOE_E_DTYPE;
  if (shape->d % 32 || shape->I % 32) return LC_MOE_E_SHAPE;
  if (!weights) return LC_MOE_E_NULLPTR;
  LCM_CHECK(check_ptr(x));
  LCM_CHECK(check_ptr(weights->w_gate));
  LCM_CHECK(check_ptr(weights->w_up));
  LCM_CHECK(check_ptr(weights->w_down));
  LCM_CHECK(check_ptr(topk_idx));
  LCM_CHECK(check_ptr(topk_gate));
  LCM_CHECK(check_ptr(dy));
  LCM_CHECK(check_ptr(dx));
  LCM_CHECK(check_ptr(dw_gate));
  LCM_CHECK(check_ptr(dw_up));
  LCM_CHECK(check_ptr(dw_down));
  if (!workspace) return LC_MOE_E_NULLPTR;
  if (!aligned16(workspace)) return LC_MOE_E_ALIGN;
  const BwPlan p = plan_backward(*shape);
  if (workspace_bytes < p.total) return LC_MOE_E_WORKSPACE;
  const lc_moe_shape& s = *shape;
  int32_t* load = at<int32_t>(workspace, p.load);
  int32_t* offsets = at<int32_t>(workspace, p.offsets);
  int32_t* slot_row = at<int32_t>(workspace, p.slot_row);
  int32_t* perm_token = at<int32_t>(workspace, p.perm_token);
  MTile* mtiles = at<MTile>(workspace, p.mtiles);
  int32_t* n_mtiles = at<int32_t>(workspace, p.n_mtiles);
  if (p.nblocks == 1) {
    LCM_LAUNCH(launch_permute_small(s, topk_idx, load, nullptr, offsets, mtiles, n_mtiles, kBmBwd, slot_row,
                                    perm_token, stream));
  } else {
    int32_t* bc = at<int32_t>(workspace, p.block_counts);
    int32_t* bb = at<int32_t>(workspace, p.block_base);
    LCM_LAUNCH(launch_histogram(s, topk_idx, bc, nullptr, p.nblocks, stream));
    LCM_LAUNCH(launch_scan(s, bc, p.nblocks, load, offsets, bb, mtiles, n_mtiles, kBmBwd, stream));
    LCM_LAUNCH(launch_scatter(s, topk_idx, bb, p.nblocks, slot_row, perm_token, stream));
  }
  LCM_LAUNCH(launch_ffn_backward(s, p, workspace, x, weights->w_gate, weights->w_up, weights->w_down, topk_idx,
                                 topk_gate, dy, dx, dw_gate, dw_up, dw_down, stream));
  return LC_MOE_OK;
}

lc_moe_status lc_moe_forward(const lc_moe_shape* shape, const void* x,
                             const lc_moe_weights* weights, void* y, int32_t* topk_idx,
                             float* topk_gate, int32_t* load, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return lc_moe_forward_staged(shape, x, weights, y, topk_idx, topk_gate, load, workspace,
                               workspace_bytes, stream, nullptr);
}

}  // extern "C"
