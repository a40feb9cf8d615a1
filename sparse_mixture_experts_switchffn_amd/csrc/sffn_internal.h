// Internal interfaces of the SwitchFFN library: workspace carve-up and the
// kernel launchers each stage file provides.  Not part of the C-ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sffn {

// Tokens per routing block: one softmax/route block handles this many tokens
// and produces one row of per-expert probability sums and counts.
constexpr int kRouteTokens = 32;

struct Shape {
  int T, d, F, N, C;
  int k;                // experts per token (1: Switch routing, 2: top-2)
  int reroute;          // k = 1 with overflow tokens rerouted to their second choice
  int glu;              // GEGLU experts: W1 [N, 2F, d], b1 [N, 2F]
  int dtype;            // SFFN_FP32 / SFFN_BF16
  int n_route_blocks;   // ceil(T / kRouteTokens)
  int max_rows;         // min(k*T, N*C): rows the expert buffers can hold
};

// The router ranks two experts per token (top-2 routing, or rerouting).
inline bool two_choices(const Shape& s) { return s.k == 2 || s.reroute != 0; }
// The logits go through the workspace (no fused router).

// Layout tag: 16 words a forward call leaves at the start of its workspace, so
// that a later call reading the workspace (the backward pass) can tell which
// form of the layer carved it up and for which shape.
constexpr uint32_t kTagMagic = 0x4E464653u;  // "SFFN" in little-endian bytes
constexpr uint32_t kTagVersion = 1u;
constexpr size_t kTagBytes = 256;  // the tag's region (16 words used)
struct WsTag {
  uint32_t w[16];  // magic, version, k, flags, T, d, F, N, C, dtype, rest 0
};
enum TagWord { kTagWMagic = 0, kTagWVersion, kTagWK, kTagWFlags, kTagWT, kTagWD, kTagWF,
               kTagWN, kTagWC, kTagWDtype };
WsTag make_tag(const Shape& s, uint32_t flags);

struct Workspace {
  uint32_t* tag;   // [16] layout tag (kTagBytes region)
  float* logits;   // [T, N] fp32 router logits
  float* ppart;    // [n_route_blocks, N] sum of p[t,i] over a block's tokens
  int* cnt;        // [n_route_blocks, N] top-1 counts per block (rerouting: then the
                   //   per-block counts of overflowed tokens by second choice)
  int* base;       // [n_route_blocks, N] tokens of expert i in earlier blocks (rerouting:
                   //   then acc[i] + overflowed tokens of second choice i in earlier blocks)
  int* cnt1;       // [n_route_blocks, N] top-1 counts per block (k = 2; the aux loss)
  int* lrank;      // [T, k] rank of a choice among its block's tokens holding the same expert
                   //   (rerouting, [T, 2]: rank among the block's first choices, then among
                   //   the block's overflowed tokens with the same second choice)
  int* hist;       // [N] tokens holding each expert among their k choices (before capacity)
  int* hist1;      // [N] top-1 counts (k = 2; for k = 1 the aux loss uses hist)
  int* acc;        // [N] accepted counts min(hist, C) (rerouting: after the first stage)
  int* acc2;       // [N] rerouting: rows of each expert after both stages
  int32_t* choice; // [T, 2] rerouting: first and second choice of each token
  float* gate2;    // [T, 2] rerouting: p[t, choice] of both choices
  int32_t* slot1;  // [T] rerouting: first-stage slot of each token, -1 if it overflowed
  int* offset;     // [N+1] exclusive scan of acc: start row of each expert
  double* psum;    // [N] sum over all tokens of p[t,i]
  int* row2tok;    // [max_rows] token of each expert-buffer row
  float* rowgate;  // [max_rows] gate of each expert-buffer row's token
  void* H;         // [max_rows, F] expert hidden activations (dtype)
  void* Y2;        // [max_rows, d] gate-scaled expert outputs per buffer row (k = 2, dtype)
  uint16_t* planes;  // router weights split into three bf16 planes, fragment order (tiled router; fused router for > 64 experts)
};

// Records the HIP error text for switch_ffn_status_string and returns SFFN_EHIP.
int record_hip_error(hipError_t e, const char* what);

// Bytes of each region, in order, 256-byte aligned; returns the total.
size_t workspace_layout(const Shape& s, Workspace* ws, char* base);

struct Inputs {
  const void* x;
  const float* Wr;
  const void* W1;
  const void* b1;
  const void* W2;
  const void* b2;
};

struct Outputs {
  void* y;
  int32_t* expert_idx;
  int32_t* slot;
  float* gate;
  float* aux_loss;
  int32_t* stat_count;
  int32_t* stat_accepted;
  int32_t* stat_dropped;
};

// Stage launchers (each enqueues on `st` and returns hipGetLastError()).
hipError_t launch_router_logits(const Shape& s, const Inputs& in, const Workspace& ws,
                                hipStream_t st);
// Softmax, top-1 and per-block statistics; for bf16 with N <= 128 this also
// computes the logits (fused) and launch_router_logits does nothing.
hipError_t launch_softmax_route(const Shape& s, const Inputs& in, const Workspace& ws,
                                const Outputs& out, hipStream_t st);
bool router_is_fused(const Shape& s);
size_t router_planes_bytes(const Shape& s);
bool dispatch_scan_in_scatter(const Shape& s);
// Rerouting: also the overflow count of the second stage and its scan.
hipError_t launch_dispatch_scan(const Shape& s, const Workspace& ws, hipStream_t st);
// Also writes the layout tag `tag` into ws.tag (block 0).
hipError_t launch_dispatch_scatter(const Shape& s, const Inputs& in, const Workspace& ws,
                                   const Outputs& out, bool no_residual, const WsTag& tag,
                                   hipStream_t st);
hipError_t launch_ffn1(const Shape& s, const Inputs& in, const Workspace& ws, hipStream_t st);
hipError_t launch_ffn2(const Shape& s, const Inputs& in, const Workspace& ws, const Outputs& out,
                       bool no_residual, hipStream_t st);
// k = 2: y_t = x_t (or 0) + the gate-scaled expert rows of t's accepted choices.
hipError_t launch_combine(const Shape& s, const Inputs& in, const Workspace& ws,
                          const Outputs& out, bool no_residual, hipStream_t st);

// Backward pass (top-1, ReLU experts): the forward's dispatch state, the
// backward's own scratch, and the gradients.
struct BwdState {
  // from the forward
  const uint32_t* fwd_tag;    // [16] the forward workspace's layout tag
  const int* fwd_offset;      // [N+1] as the forward left them (read by the guard only)
  const int* fwd_hist;        // [N]
  const int32_t* expert_idx;  // [T]
  const int32_t* slot;        // [T]
  int* offset;                // [N+1] the guard's checked copy (backward workspace)
  const int* row2tok;         // [max_rows]
  const float* rowgate;       // [max_rows]
  int* hist;                  // [N] top-1 counts, the guard's checked copy
  int* bad;                   // [1] set by the guard when the forward workspace fails it
  const void* H;              // [max_rows, F] hidden activations (dtype)
  const float* logits;        // [T, N] fp32 router logits
  // upstream gradients
  const void* dy;             // [T, d] (dtype)
  float d_aux;
  // scratch
  float* dz;                  // [T, N] dL/dz
  void* dA;                   // [max_rows, F] (dtype)
  float* dgp;                 // [n_dgp, max_rows] partial dg per column tile of F
  int n_dgp;
  float* dxe;                 // [T, d] expert part of dx (accepted tokens)
  float* wrp;                 // [n_wr_parts, N, d] partial dWr
  int n_wr_parts;
  // gradients
  void* dx;                   // [T, d] (dtype)
  float* dWr;                 // [N, d]
  void* dW1;                  // [N, F, d] (dtype)
  void* db1;                  // [N, F] (dtype), nullable
  void* dW2;                  // [N, d, F] (dtype)
  void* db2;                  // [N, d] (dtype), nullable
};
// Column tiles of F in the backward's first expert GEMM (partial dg rows).
int bwd_dgp_tiles(const Shape& s);
// Token parts of the split router-weight gradient.
int bwd_wr_parts(const Shape& s);
hipError_t launch_backward(const Shape& s, const Inputs& in, const BwdState& b, hipStream_t st,
                           void* const* stage_events);

}  // namespace sffn
