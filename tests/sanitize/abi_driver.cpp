// Host-side driver of the C-ABI for the sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of the entry points).  It calls
// every host-only path -- capacity, workspace sizing for every form of the
// layer, stage names, status strings -- and every argument check that rejects
// a call before anything is enqueued, with fake device addresses that are
// never dereferenced.  Exit status 0 when every call returns what the header
// promises; any sanitizer report aborts the run.
//
// `asan_probe` / `ubsan_probe` as the only argument plant a heap overflow or a
// signed overflow in this driver (host memory, on the CPU) to show that the
// build really is instrumented.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/switch_ffn.h"

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,    \
              __LINE__, #cond);                                        \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

namespace {

void* const kFake = (void*)0x100000;

struct Fwd {
  const void* x = kFake;
  const float* Wr = (const float*)kFake;
  const void* W1 = kFake;
  const void* b1 = nullptr;
  const void* W2 = kFake;
  const void* b2 = nullptr;
  int64_t T = 64, d = 32, F = 64, N = 4;
  double CF = 1.0;
  int dtype = SFFN_BF16;
  void* y = kFake;
  int32_t* ei = (int32_t*)kFake;
  int32_t* slot = (int32_t*)kFake;
  float* gate = (float*)kFake;
  float* aux = (float*)kFake;
  void* ws = kFake;
  size_t ws_bytes = (size_t)1 << 40;
  uint32_t flags = 0;
  int k = 1;
  int ex() const {
    return switch_ffn_forward_ex(x, Wr, W1, b1, W2, b2, T, d, F, N, CF, dtype, y, ei, slot, gate,
                                 aux, ws, ws_bytes, nullptr, flags, nullptr);
  }
  int topk() const {
    return switch_ffn_forward_topk(x, Wr, W1, b1, W2, b2, T, d, F, N, CF, k, dtype, y, ei, slot,
                                   gate, aux, ws, ws_bytes, nullptr, flags, nullptr, nullptr);
  }
};

struct Bwd {
  Fwd f;
  const int32_t* ei = (const int32_t*)kFake;
  const int32_t* slot = (const int32_t*)kFake;
  const void* fws = kFake;
  size_t fws_bytes = 0;
  const void* dy = kFake;
  float d_aux = 0.01f;
  void* dx = kFake;
  float* dWr = (float*)kFake;
  void* dW1 = kFake;
  void* dW2 = kFake;
  void* ws = kFake;
  size_t ws_bytes = 0;
  Bwd() {
    fws_bytes = switch_ffn_workspace_bytes(f.T, f.d, f.F, f.N, f.CF, f.dtype);
    ws_bytes = switch_ffn_backward_workspace_bytes(f.T, f.d, f.F, f.N, f.CF, f.dtype);
  }
  int call() const {
    return switch_ffn_backward(f.x, f.Wr, f.W1, f.b1, f.W2, f.b2, f.T, f.d, f.F, f.N, f.CF,
                               f.dtype, ei, slot, fws, fws_bytes, dy, d_aux, dx, dWr, dW1,
                               nullptr, dW2, nullptr, ws, ws_bytes, nullptr, nullptr);
  }
};

void capacity_cases() {
  EXPECT(switch_ffn_capacity(64, 4, 1.0) == 16);
  EXPECT(switch_ffn_capacity(8192, 64, 1.25) == 160);
  EXPECT(switch_ffn_capacity(65536, 2048, 1.0) == 32);
  EXPECT(switch_ffn_capacity(0, 3, 1.0) == 0);
  EXPECT(switch_ffn_capacity(INT64_MAX, 1, 1e300) == INT64_MAX);  // saturates, no UB cast
  EXPECT(switch_ffn_capacity(5, 0, 1.0) == -1);
  EXPECT(switch_ffn_capacity(-1, 2, 1.0) == -1);
  EXPECT(switch_ffn_capacity(5, 2, -0.5) == -1);
  EXPECT(switch_ffn_capacity(5, 2, NAN) == -1);
  EXPECT(switch_ffn_capacity(5, 2, INFINITY) == -1);
}

void sizing_cases() {
  const int64_t shapes[][5] = {{64, 32, 64, 4, 0},       {8192, 768, 3072, 64, 0},
                               {16384, 768, 3072, 128, 0}, {32768, 1024, 4096, 128, 0},
                               {65536, 2080, 6144, 2048, 0}, {1, 8, 8, 1, 0},
                               {33000, 64, 32, 128, 0},   {300, 72, 16, 4096, 0}};
  const double cfs[] = {0.0, 0.5, 1.0, 1.25, 4.0, 1e9};
  for (const auto& s : shapes)
    for (double cf : cfs)
      for (int dt = 0; dt < 2; ++dt) {
        const size_t a = switch_ffn_workspace_bytes(s[0], s[1], s[2], s[3], cf, dt);
        const size_t b1 = switch_ffn_workspace_bytes_topk(s[0], s[1], s[2], s[3], cf, 1, dt);
        const size_t b2 = switch_ffn_workspace_bytes_topk(s[0], s[1], s[2], s[3], cf, 2, dt);
        const size_t c = switch_ffn_backward_workspace_bytes(s[0], s[1], s[2], s[3], cf, dt);
        EXPECT(a == b1);
        EXPECT(a > 0 && c > 0);
        if (s[3] < 2) EXPECT(b2 == 0);  // top-2 needs two experts
      }
  // bad shapes: zero, never a crash or an overflowed size
  EXPECT(switch_ffn_workspace_bytes(0, 8, 8, 2, 1.0, 1) == 0);
  EXPECT(switch_ffn_workspace_bytes(8, 8, 8, 2, -1.0, 1) == 0);
  EXPECT(switch_ffn_workspace_bytes(8, 8, 8, 5000, 1.0, 1) == 0);
  EXPECT(switch_ffn_workspace_bytes(INT64_MAX, INT64_MAX, INT64_MAX, 2, 1.0, 1) == 0);
  EXPECT(switch_ffn_workspace_bytes((int64_t)1 << 40, 8, 8, 2, 1.0, 1) == 0);
  EXPECT(switch_ffn_workspace_bytes(8, 32768, 32768, 2, 1.0, 1) == 0);
  EXPECT(switch_ffn_workspace_bytes_topk(8, 8, 8, 2, 1.0, 3, 1) == 0);
  EXPECT(switch_ffn_backward_workspace_bytes(8, 8, 8, 2, 1.0, 7) == 0);
}

void names_and_strings() {
  const int n = switch_ffn_num_stages();
  EXPECT(n == 6);
  for (int i = 0; i < n; ++i) EXPECT(switch_ffn_stage_name(i) != nullptr);
  EXPECT(switch_ffn_stage_name(n) == nullptr && switch_ffn_stage_name(-1) == nullptr);
  const int nb = switch_ffn_backward_num_stages();
  for (int i = 0; i < nb; ++i) EXPECT(switch_ffn_backward_stage_name(i) != nullptr);
  EXPECT(switch_ffn_backward_stage_name(nb) == nullptr);
  const int codes[] = {SFFN_OK, SFFN_EINVAL, SFFN_EDTYPE, SFFN_EWORKSPACE, SFFN_EUNSUPPORTED,
                       SFFN_EHIP, -99, INT32_MIN};
  for (int c : codes) EXPECT(strlen(switch_ffn_status_string(c)) > 0);
}

void forward_rejects() {
  struct Case {
    void (*set)(Fwd&);
    int code;
  };
  const Case cases[] = {
      {[](Fwd& f) { f.x = nullptr; }, SFFN_EINVAL},
      {[](Fwd& f) { f.Wr = nullptr; }, SFFN_EINVAL},
      {[](Fwd& f) { f.W1 = nullptr; }, SFFN_EINVAL},
      {[](Fwd& f) { f.W2 = nullptr; }, SFFN_EINVAL},
      {[](Fwd& f) { f.y = nullptr; }, SFFN_EINVAL},
      {[](Fwd& f) { f.ei = nullptr; }, SFFN_EINVAL},
      {[](Fwd& f) { f.slot = nullptr; }, SFFN_EINVAL},
      {[](Fwd& f) { f.gate = nullptr; }, SFFN_EINVAL},
      {[](Fwd& f) { f.aux = nullptr; }, SFFN_EINVAL},
      {[](Fwd& f) { f.T = 0; }, SFFN_EINVAL},
      {[](Fwd& f) { f.T = INT64_MIN; }, SFFN_EINVAL},
      {[](Fwd& f) { f.d = -1; }, SFFN_EINVAL},
      {[](Fwd& f) { f.F = 0; }, SFFN_EINVAL},
      {[](Fwd& f) { f.N = 0; }, SFFN_EINVAL},
      {[](Fwd& f) { f.CF = -1.0; }, SFFN_EINVAL},
      {[](Fwd& f) { f.CF = NAN; }, SFFN_EINVAL},
      {[](Fwd& f) { f.CF = -INFINITY; }, SFFN_EINVAL},
      {[](Fwd& f) { f.flags = 8; }, SFFN_EINVAL},
      {[](Fwd& f) { f.flags = 0x80000000u; }, SFFN_EINVAL},
      {[](Fwd& f) { f.dtype = 3; }, SFFN_EDTYPE},
      {[](Fwd& f) { f.dtype = -1; }, SFFN_EDTYPE},
      {[](Fwd& f) { f.N = 5000; }, SFFN_EUNSUPPORTED},
      {[](Fwd& f) { f.N = INT64_MAX; }, SFFN_EUNSUPPORTED},
      {[](Fwd& f) { f.d = 36; }, SFFN_EUNSUPPORTED},
      {[](Fwd& f) { f.F = 70; }, SFFN_EUNSUPPORTED},
      {[](Fwd& f) { f.T = (int64_t)1 << 25; f.d = 64; }, SFFN_EUNSUPPORTED},
      {[](Fwd& f) { f.T = INT64_MAX; }, SFFN_EUNSUPPORTED},
      {[](Fwd& f) { f.d = INT64_MAX - 7; }, SFFN_EUNSUPPORTED},
      {[](Fwd& f) { f.d = 32768; f.F = 32768; }, SFFN_EUNSUPPORTED},
      {[](Fwd& f) { f.x = (const void*)0x100004; }, SFFN_EUNSUPPORTED},
      {[](Fwd& f) { f.ws = nullptr; }, SFFN_EWORKSPACE},
      {[](Fwd& f) { f.ws_bytes = 1000; }, SFFN_EWORKSPACE},
      {[](Fwd& f) { f.ws = (void*)0x100010; }, SFFN_EUNSUPPORTED},
      {[](Fwd& f) { f.flags = SFFN_REROUTE_OVERFLOW; f.N = 1; }, SFFN_EINVAL},
  };
  for (const Case& c : cases) {
    Fwd f;
    c.set(f);
    EXPECT(f.ex() == c.code);
    EXPECT(f.topk() == c.code);
  }
  const Case topk_cases[] = {
      {[](Fwd& f) { f.k = 0; }, SFFN_EINVAL},
      {[](Fwd& f) { f.k = 3; }, SFFN_EINVAL},
      {[](Fwd& f) { f.k = 2; f.N = 1; }, SFFN_EINVAL},
      {[](Fwd& f) { f.k = 2; f.flags = SFFN_REROUTE_OVERFLOW; }, SFFN_EINVAL},
      {[](Fwd& f) { f.k = 2; f.ws_bytes = 1000; }, SFFN_EWORKSPACE},
      {[](Fwd& f) { f.k = 2; f.T = (int64_t)1 << 20; f.d = 512; f.F = 512; f.N = 2; },
       SFFN_EUNSUPPORTED},
  };
  for (const Case& c : topk_cases) {
    Fwd f;
    c.set(f);
    EXPECT(f.topk() == c.code);
  }
}

void backward_rejects() {
  struct Case {
    void (*set)(Bwd&);
    int code;
  };
  const Case cases[] = {
      {[](Bwd& b) { b.f.x = nullptr; }, SFFN_EINVAL},
      {[](Bwd& b) { b.f.Wr = nullptr; }, SFFN_EINVAL},
      {[](Bwd& b) { b.ei = nullptr; }, SFFN_EINVAL},
      {[](Bwd& b) { b.slot = nullptr; }, SFFN_EINVAL},
      {[](Bwd& b) { b.fws = nullptr; }, SFFN_EINVAL},
      {[](Bwd& b) { b.dy = nullptr; }, SFFN_EINVAL},
      {[](Bwd& b) { b.dx = nullptr; }, SFFN_EINVAL},
      {[](Bwd& b) { b.dWr = nullptr; }, SFFN_EINVAL},
      {[](Bwd& b) { b.dW1 = nullptr; }, SFFN_EINVAL},
      {[](Bwd& b) { b.dW2 = nullptr; }, SFFN_EINVAL},
      {[](Bwd& b) { b.d_aux = NAN; }, SFFN_EINVAL},
      {[](Bwd& b) { b.d_aux = -INFINITY; }, SFFN_EINVAL},
      {[](Bwd& b) { b.f.T = 0; }, SFFN_EINVAL},
      {[](Bwd& b) { b.f.CF = NAN; }, SFFN_EINVAL},
      {[](Bwd& b) { b.f.dtype = 2; }, SFFN_EDTYPE},
      {[](Bwd& b) { b.f.N = 5000; }, SFFN_EUNSUPPORTED},
      {[](Bwd& b) { b.f.T = INT64_MAX; }, SFFN_EUNSUPPORTED},
      {[](Bwd& b) { b.dy = (const void*)0x100004; }, SFFN_EUNSUPPORTED},
      {[](Bwd& b) { b.dW2 = (void*)0x100002; }, SFFN_EUNSUPPORTED},
      {[](Bwd& b) { b.fws_bytes = 1000; }, SFFN_EWORKSPACE},
      {[](Bwd& b) { b.ws = nullptr; }, SFFN_EWORKSPACE},
      {[](Bwd& b) { b.ws_bytes = 1000; }, SFFN_EWORKSPACE},
      {[](Bwd& b) { b.ws = (void*)0x100010; }, SFFN_EUNSUPPORTED},
      {[](Bwd& b) { b.fws = (const void*)0x100010; }, SFFN_EUNSUPPORTED},
  };
  for (const Case& c : cases) {
    Bwd b;
    c.set(b);
    EXPECT(b.call() == c.code);
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc > 1 && strcmp(argv[1], "asan_probe") == 0) {
    volatile char* p = (volatile char*)malloc(16);
    const int i = argc + 14;  // 16: one past the end
    p[0] = p[i];
    free((void*)p);
    return 0;
  }
  if (argc > 1 && strcmp(argv[1], "ubsan_probe") == 0) {
    volatile int big = INT32_MAX;
    const int r = big + argc;  // signed overflow
    return r == 0;
  }
  capacity_cases();
  sizing_cases();
  names_and_strings();
  forward_rejects();
  backward_rejects();
  if (g_fail) {
    fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  printf("abi_driver: all host-side cases passed\n");
  return 0;
}
