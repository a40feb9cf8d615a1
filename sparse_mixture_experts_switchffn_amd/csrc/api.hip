// C-ABI entry points of the SwitchFFN library: argument checks, capacity,
// workspace carve-up and the launch sequence (all on the caller's stream).
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "sffn_internal.h"
#include "../../include/switch_ffn.h"

namespace {

thread_local char g_hip_error[256] = "no HIP error recorded";

const char* const kStageNames[] = {"router_logits", "softmax_route", "dispatch_scan",
                                   "dispatch_scatter", "ffn1", "ffn2"};
constexpr int kNumStages = (int)(sizeof(kStageNames) / sizeof(kStageNames[0]));

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15) == 0; }

}  // namespace

int sffn::record_hip_error(hipError_t e, const char* what) {
  snprintf(g_hip_error, sizeof(g_hip_error), "%s: %s", what, hipGetErrorString(e));
  return SFFN_EHIP;
}

using sffn::record_hip_error;

namespace sffn {

size_t workspace_layout(const Shape& s, Workspace* ws, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  const size_t T = (size_t)s.T, N = (size_t)s.N, nb = (size_t)s.n_route_blocks;
  const size_t esize = s.dtype == SFFN_BF16 ? 2 : 4;
  Workspace w;
  w.tag = (uint32_t*)take(kTagBytes);
  w.logits = (float*)take(T * N * sizeof(float));
  w.ppart = (float*)take(nb * N * sizeof(float));
  const size_t K = (size_t)s.k;
  w.cnt = (int*)take(nb * N * sizeof(int));
  w.cnt1 = (int*)take(K == 2 ? nb * N * sizeof(int) : 0);
  w.base = (int*)take(nb * N * sizeof(int));
  const size_t R = s.reroute ? 1 : 0;
  w.lrank = (int*)take(T * (R ? 2 : K) * sizeof(int));
  w.hist = (int*)take(N * sizeof(int));
  w.hist1 = (int*)take(K == 2 ? N * sizeof(int) : 0);
  w.acc = (int*)take(N * sizeof(int));
  w.acc2 = (int*)take(R * N * sizeof(int));
  w.choice = (int32_t*)take(R * 2 * T * sizeof(int32_t));
  w.gate2 = (float*)take(R * 2 * T * sizeof(float));
  w.slot1 = (int32_t*)take(R * T * sizeof(int32_t));
  w.offset = (int*)take((N + 1) * sizeof(int));
  w.psum = (double*)take(N * sizeof(double));
  w.row2tok = (int*)take((size_t)s.max_rows * sizeof(int) + 4);
  w.rowgate = (float*)take((size_t)s.max_rows * sizeof(float) + 4);
  w.H = (void*)take((size_t)s.max_rows * (size_t)s.F * esize + 16);
  w.Y2 = (void*)take(K == 2 ? (size_t)s.max_rows * (size_t)s.d * esize + 16 : 0);
  w.planes = (uint16_t*)take(sffn::router_planes_bytes(s));
  if (ws) *ws = w;
  return off;
}

WsTag make_tag(const Shape& s, uint32_t flags) {
  WsTag t{};
  t.w[kTagWMagic] = kTagMagic;
  t.w[kTagWVersion] = kTagVersion;
  t.w[kTagWK] = (uint32_t)s.k;
  t.w[kTagWFlags] = flags;
  t.w[kTagWT] = (uint32_t)s.T;
  t.w[kTagWD] = (uint32_t)s.d;
  t.w[kTagWF] = (uint32_t)s.F;
  t.w[kTagWN] = (uint32_t)s.N;
  t.w[kTagWC] = (uint32_t)s.C;
  t.w[kTagWDtype] = (uint32_t)s.dtype;
  return t;
}

}  // namespace sffn

// Shape checks shared by workspace sizing and the forward pass.
static int make_shape(int64_t T, int64_t d, int64_t F, int64_t N, double CF, int dtype, int k,
                      bool reroute, sffn::Shape* s, bool glu = false) {
  if (T <= 0 || d <= 0 || F <= 0 || N <= 0 || !isfinite(CF) || CF < 0) return SFFN_EINVAL;
  if ((k != 1 && k != 2) || N < k) return SFFN_EINVAL;
  if (reroute && (k != 1 || N < 2)) return SFFN_EINVAL;
  if (dtype != SFFN_FP32 && dtype != SFFN_BF16) return SFFN_EDTYPE;
  if (N > SFFN_MAX_EXPERTS) return SFFN_EUNSUPPORTED;
  const int64_t widest = N > d ? (N > F ? N : F) : (d > F ? d : F);
  // Element offsets of every tensor (the fp32 router logits [T, N] included) and of one
  // expert's weights stay below 2^29, so byte offsets of fp32 and bf16 tensors stay below
  // 2^31: the offset the buffer accesses use for masked lanes (2^31) lies past them all.
  if (T > ((int64_t)1 << 29) / widest - 1) return SFFN_EUNSUPPORTED;
  if (d * F >= ((int64_t)1 << 29)) return SFFN_EUNSUPPORTED;
  if (dtype == SFFN_BF16 && ((d % 8) != 0 || (F % 8) != 0)) return SFFN_EUNSUPPORTED;
  const int64_t C = switch_ffn_capacity(k * T, N, CF);
  const int64_t Ce = C < T ? C : T;  // a rank never reaches T (one position per token and expert)
  s->T = (int)T;
  s->d = (int)d;
  s->F = (int)F;
  s->N = (int)N;
  s->C = (int)Ce;
  s->dtype = dtype;
  s->k = k;
  s->reroute = reroute ? 1 : 0;
  s->glu = glu ? 1 : 0;
  s->n_route_blocks = (int)((T + sffn::kRouteTokens - 1) / sffn::kRouteTokens);
  const int64_t cap_rows = N * Ce;
  s->max_rows = (int)(cap_rows < k * T ? cap_rows : k * T);
  // k = 2: the expert buffers hold up to 2T rows; their byte offsets stay below 2^31.
  if (k == 2 && (int64_t)s->max_rows * (d > F ? d : F) * 4 >= ((int64_t)1 << 31))
    return SFFN_EUNSUPPORTED;
  return SFFN_OK;
}

extern "C" {

int64_t switch_ffn_capacity(int64_t T, int64_t N, double CF) {
  if (T < 0 || N <= 0 || !isfinite(CF) || CF < 0) return -1;
  const double c = floor((CF * (double)T) / (double)N);
  if (c >= 9.2e18) return INT64_MAX;
  return (int64_t)c;
}

size_t switch_ffn_workspace_bytes_topk(int64_t T, int64_t d, int64_t F, int64_t N, double CF,
                                       int k, int dtype) {
  sffn::Shape s;
  if (make_shape(T, d, F, N, CF, dtype, k, false, &s) != SFFN_OK) return 0;
  size_t bytes = sffn::workspace_layout(s, nullptr, nullptr);
  // k = 1: room for rerouting too, so one workspace serves both forms of the call.
  sffn::Shape r;
  if (k == 1 && make_shape(T, d, F, N, CF, dtype, k, true, &r) == SFFN_OK) {
    const size_t rb = sffn::workspace_layout(r, nullptr, nullptr);
    if (rb > bytes) bytes = rb;
  }
  return bytes;
}

size_t switch_ffn_workspace_bytes(int64_t T, int64_t d, int64_t F, int64_t N, double CF,
                                  int dtype) {
  return switch_ffn_workspace_bytes_topk(T, d, F, N, CF, 1, dtype);
}

int switch_ffn_num_stages(void) { return kNumStages; }

const char* switch_ffn_stage_name(int stage) {
  return (stage >= 0 && stage < kNumStages) ? kStageNames[stage] : nullptr;
}

const char* switch_ffn_status_string(int status) {
  switch (status) {
    case SFFN_OK: return "ok";
    case SFFN_EINVAL: return "invalid argument (null pointer, non-positive size, or bad CF)";
    case SFFN_EDTYPE: return "unknown dtype (expected SFFN_FP32 or SFFN_BF16)";
    case SFFN_EWORKSPACE: return "workspace missing or smaller than switch_ffn_workspace_bytes()";
    case SFFN_EUNSUPPORTED:
      return "unsupported shape or alignment (N <= 4096, T*max(N,d,F) < 2^30, d*F < 2^30; bf16 "
             "needs d, F "
             "multiples of 8 and 16-byte aligned x, Wr, W1, W2, y; workspace 256-byte aligned)";
    case SFFN_EHIP: return g_hip_error;
    case SFFN_ESCRATCH:
      return "the shape needs more workspace than switch_ffn_forward_noalloc's built-in scratch "
             "(switch_ffn_noalloc_scratch_bytes())";
    default: return "unknown status";
  }
}

int switch_ffn_forward_topk(const void* x, const float* Wr, const void* W1, const void* b1,
                            const void* W2, const void* b2, int64_t T, int64_t d, int64_t F,
                            int64_t N, double CF, int k, int dtype, void* y, int32_t* expert_idx,
                            int32_t* slot, float* gate, float* aux_loss, void* workspace,
                            size_t workspace_bytes, void* stream, uint32_t flags,
                            const sffn_stats* stats, void* const* stage_events) {
  if (!x || !Wr || !W1 || !W2 || !y || !expert_idx || !slot || !gate || !aux_loss)
    return SFFN_EINVAL;
  if (flags & ~(uint32_t)(SFFN_NO_RESIDUAL | SFFN_REROUTE_OVERFLOW | SFFN_GEGLU))
    return SFFN_EINVAL;
  sffn::Shape s;
  const int rc = make_shape(T, d, F, N, CF, dtype, k, (flags & SFFN_REROUTE_OVERFLOW) != 0, &s,
                            (flags & SFFN_GEGLU) != 0);
  if (rc != SFFN_OK) return rc;
  if (dtype == SFFN_BF16 &&
      !(aligned16(x) && aligned16(Wr) && aligned16(W1) && aligned16(W2) && aligned16(y)))
    return SFFN_EUNSUPPORTED;
  const size_t need = sffn::workspace_layout(s, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return SFFN_EWORKSPACE;
  if (((uintptr_t)workspace & 255) != 0) return SFFN_EUNSUPPORTED;

  sffn::Workspace ws;
  sffn::workspace_layout(s, &ws, (char*)workspace);
  const sffn::Inputs in{x, Wr, W1, b1, W2, b2};
  const sffn::Outputs out{y,
                          expert_idx,
                          slot,
                          gate,
                          aux_loss,
                          stats ? stats->expert_count : nullptr,
                          stats ? stats->accepted_count : nullptr,
                          stats ? stats->n_dropped : nullptr};
  const bool no_res = (flags & SFFN_NO_RESIDUAL) != 0;
  hipStream_t st = (hipStream_t)stream;

  auto mark = [&](int i) -> hipError_t {
    if (!stage_events) return hipSuccess;
    return hipEventRecord((hipEvent_t)stage_events[i], st);
  };
  hipError_t e;
  if ((e = mark(0)) != hipSuccess) return record_hip_error(e, "event record");
  if ((e = sffn::launch_router_logits(s, in, ws, st)) != hipSuccess)
    return record_hip_error(e, kStageNames[0]);
  if ((e = mark(1)) != hipSuccess) return record_hip_error(e, "event record");
  if ((e = sffn::launch_softmax_route(s, in, ws, out, st)) != hipSuccess)
    return record_hip_error(e, kStageNames[1]);
  if ((e = mark(2)) != hipSuccess) return record_hip_error(e, "event record");
  if ((e = sffn::launch_dispatch_scan(s, ws, st)) != hipSuccess)
    return record_hip_error(e, kStageNames[2]);
  if ((e = mark(3)) != hipSuccess) return record_hip_error(e, "event record");
  if ((e = sffn::launch_dispatch_scatter(s, in, ws, out, no_res, sffn::make_tag(s, flags), st)) !=
      hipSuccess)
    return record_hip_error(e, kStageNames[3]);
  if ((e = mark(4)) != hipSuccess) return record_hip_error(e, "event record");
  if ((e = sffn::launch_ffn1(s, in, ws, st)) != hipSuccess)
    return record_hip_error(e, kStageNames[4]);
  if ((e = mark(5)) != hipSuccess) return record_hip_error(e, "event record");
  if ((e = sffn::launch_ffn2(s, in, ws, out, no_res, st)) != hipSuccess)
    return record_hip_error(e, kStageNames[5]);
  if (s.k == 2 && (e = sffn::launch_combine(s, in, ws, out, no_res, st)) != hipSuccess)
    return record_hip_error(e, "combine");
  if ((e = mark(6)) != hipSuccess) return record_hip_error(e, "event record");
  return SFFN_OK;
}

namespace {
const char* const kBwdStageNames[] = {"expert_dgrad_hidden", "router_grad",
                                      "expert_dgrad_input", "dx", "router_wgrad",
                                      "expert_wgrad", "bias_grad"};
constexpr int kNumBwdStages = (int)(sizeof(kBwdStageNames) / sizeof(kBwdStageNames[0]));

// Backward scratch: checked offsets [N+1], counts [N] and the guard flag |
// dz [T, N] fp32 | dA [max_rows, F] | partial dg | dXe [T, d] fp32 | partial dWr.
size_t bwd_layout(const sffn::Shape& s, char* base, sffn::BwdState* b) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  const size_t T = (size_t)s.T, N = (size_t)s.N, esize = s.dtype == SFFN_BF16 ? 2 : 4;
  const int n_dgp = sffn::bwd_dgp_tiles(s), parts = sffn::bwd_wr_parts(s);
  int* guard = (int*)take((2 * N + 2) * sizeof(int));
  float* dz = (float*)take(T * N * 4);
  void* dA = take((size_t)s.max_rows * s.F * esize + 16);
  float* dgp = (float*)take((size_t)n_dgp * s.max_rows * 4 + 4);
  float* dxe = (float*)take(T * s.d * 4);
  float* wrp = (float*)take((size_t)parts * N * s.d * 4);
  if (b) {
    b->offset = guard;
    b->hist = guard ? guard + N + 1 : nullptr;
    b->bad = guard ? guard + 2 * N + 1 : nullptr;
    b->dz = dz;
    b->dA = dA;
    b->dgp = dgp;
    b->n_dgp = n_dgp;
    b->dxe = dxe;
    b->wrp = wrp;
    b->n_wr_parts = parts;
  }
  return off;
}
}  // namespace

size_t switch_ffn_backward_workspace_bytes(int64_t T, int64_t d, int64_t F, int64_t N, double CF,
                                           int dtype) {
  sffn::Shape s;
  if (make_shape(T, d, F, N, CF, dtype, 1, false, &s) != SFFN_OK) return 0;
  return bwd_layout(s, nullptr, nullptr);
}

int switch_ffn_backward_num_stages(void) { return kNumBwdStages; }

const char* switch_ffn_backward_stage_name(int stage) {
  return (stage >= 0 && stage < kNumBwdStages) ? kBwdStageNames[stage] : nullptr;
}

int switch_ffn_backward(const void* x, const float* Wr, const void* W1, const void* b1,
                        const void* W2, const void* b2, int64_t T, int64_t d, int64_t F,
                        int64_t N, double CF, int dtype, const int32_t* expert_idx,
                        const int32_t* slot, const void* fwd_workspace,
                        size_t fwd_workspace_bytes, const void* dy, float d_aux, void* dx,
                        float* dWr, void* dW1, void* db1, void* dW2, void* db2, void* workspace,
                        size_t workspace_bytes, void* stream, void* const* stage_events) {
  if (!x || !Wr || !W1 || !W2 || !expert_idx || !slot || !fwd_workspace || !dy || !dx || !dWr ||
      !dW1 || !dW2 || !isfinite(d_aux))
    return SFFN_EINVAL;
  sffn::Shape s;
  const int rc = make_shape(T, d, F, N, CF, dtype, 1, false, &s);
  if (rc != SFFN_OK) return rc;
  if (dtype == SFFN_BF16 && !(aligned16(x) && aligned16(Wr) && aligned16(W1) && aligned16(W2) &&
                              aligned16(dy) && aligned16(dx) && aligned16(dW1) && aligned16(dW2)))
    return SFFN_EUNSUPPORTED;
  if (fwd_workspace_bytes < sffn::workspace_layout(s, nullptr, nullptr)) return SFFN_EWORKSPACE;
  if (!workspace || workspace_bytes < bwd_layout(s, nullptr, nullptr)) return SFFN_EWORKSPACE;
  if ((((uintptr_t)workspace | (uintptr_t)fwd_workspace) & 255) != 0) return SFFN_EUNSUPPORTED;

  hipStream_t st = (hipStream_t)stream;
  // The forward's layout tag (16 words at the start of its workspace) must name
  // a top-1 forward without rerouting or GEGLU experts of this shape: the only
  // form whose workspace this pass can read.  Read on the host while the
  // stream is not being captured (it waits for the stream's earlier work);
  // under capture the forward has not run yet, and the guard kernel checks the
  // same tag on the device (see the header).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t he = hipStreamIsCapturing(st, &cap);
  if (he != hipSuccess) return record_hip_error(he, "stream capture query");
  if (cap == hipStreamCaptureStatusNone) {
    uint32_t got[16];
    he = hipMemcpyAsync(got, fwd_workspace, sizeof(got), hipMemcpyDeviceToHost, st);
    if (he == hipSuccess) he = hipStreamSynchronize(st);
    if (he != hipSuccess) return record_hip_error(he, "layout tag read");
    const sffn::WsTag want = sffn::make_tag(s, 0u);
    for (int i = 0; i < 16; ++i) {
      const bool ok = i == sffn::kTagWFlags ? (got[i] & ~(uint32_t)SFFN_NO_RESIDUAL) == 0
                                            : got[i] == want.w[i];
      if (!ok) return SFFN_EINVAL;
    }
  }

  sffn::Workspace fw;
  sffn::workspace_layout(s, &fw, (char*)const_cast<void*>(fwd_workspace));
  sffn::BwdState b{};
  bwd_layout(s, (char*)workspace, &b);
  b.fwd_tag = fw.tag;
  b.fwd_offset = fw.offset;
  b.fwd_hist = fw.hist;
  b.expert_idx = expert_idx;
  b.slot = slot;
  b.row2tok = fw.row2tok;
  b.rowgate = fw.rowgate;
  b.H = fw.H;
  b.logits = fw.logits;
  b.dy = dy;
  b.d_aux = d_aux;
  b.dx = dx;
  b.dWr = dWr;
  b.dW1 = dW1;
  b.db1 = db1;
  b.dW2 = dW2;
  b.db2 = db2;
  const sffn::Inputs in{x, Wr, W1, b1, W2, b2};
  const hipError_t e = sffn::launch_backward(s, in, b, st, stage_events);
  if (e != hipSuccess) return record_hip_error(e, "backward");
  return SFFN_OK;
}

int switch_ffn_forward_ex(const void* x, const float* Wr, const void* W1, const void* b1,
                          const void* W2, const void* b2, int64_t T, int64_t d, int64_t F,
                          int64_t N, double CF, int dtype, void* y, int32_t* expert_idx,
                          int32_t* slot, float* gate, float* aux_loss, void* workspace,
                          size_t workspace_bytes, void* stream, uint32_t flags,
                          const sffn_stats* stats) {
  return switch_ffn_forward_topk(x, Wr, W1, b1, W2, b2, T, d, F, N, CF, 1, dtype, y, expert_idx,
                                 slot, gate, aux_loss, workspace, workspace_bytes, stream, flags,
                                 stats, nullptr);
}

int switch_ffn_forward(const void* x, const float* Wr, const void* W1, const void* b1,
                       const void* W2, const void* b2, int64_t T, int64_t d, int64_t F,
                       int64_t N, double CF, int dtype, void* y, int32_t* expert_idx,
                       int32_t* slot, float* gate, float* aux_loss, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return switch_ffn_forward_ex(x, Wr, W1, b1, W2, b2, T, d, F, N, CF, dtype, y, expert_idx, slot,
                               gate, aux_loss, workspace, workspace_bytes, stream, 0u, nullptr);
}

}  // extern "C"
