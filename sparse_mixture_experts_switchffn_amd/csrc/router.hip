// Router of the Switch layer: fp32 logits z = Wr x, softmax, top-1 with the
// lowest index on ties, gate p[t, e_t], and per-block sums of p for the aux
// loss ("Switch Transformers: Scaling to Trillion Parameter Models with Simple
// and Efficient Sparsity", section 3.4, "Switch Routing: The k=1
// Simplification" and "Selective Precision Training": the router runs in
// float32 inside a bfloat16 model).
#include "sffn_device.h"
#include "sffn_internal.h"
#include "../../include/switch_ffn.h"

namespace sffn {

// ---------------------------------------------------------------------------
// Logits for bf16 token states on the matrix cores.
//
// Each fp32 router weight w is split exactly into three bf16 terms
// w = hi + mid + lo (each the round-to-nearest of what is left).  Every product
// of a bf16 token value with a bf16 term is exact in fp32, and the matrix core
// accumulates in fp32, so z comes out as an fp32-accumulated dot product of the
// exact fp32 operands -- the router's float32 arithmetic -- at bf16 MFMA rate.
//
// Tile: rows = experts (staged in LDS as the three bf16 planes), columns =
// tokens (each lane streams 16 consecutive k of one token row per step straight
// into registers).  A wave owns 32 tokens; the block owns RW_WAVES*32 tokens and
// RM*32 experts.  K advances 32 per step, double-buffered.
// ---------------------------------------------------------------------------
constexpr int RW_WAVES = 4;
constexpr int RBK = 32;
constexpr int RLDS = RBK + 8;  // bf16 per LDS row (80 B) to spread banks

template <int RM>
__global__ void __launch_bounds__(RW_WAVES * 64)
router_logits_bf16_kernel(const uint16_t* __restrict__ x, const float* __restrict__ Wr,
                          float* __restrict__ logits, int T, int d, int N) {
  constexpr int EM = RM * 32;                  // experts per block
  constexpr int NTHR = RW_WAVES * 64;
  constexpr int CHUNKS = RBK / 4;              // 16-byte fp32 chunks per row per step (8)
  constexpr int ROWS_PER_PASS = NTHR / CHUNKS; // 32
  constexpr int A_LOADS = EM / ROWS_PER_PASS;  // RM
  __shared__ __attribute__((aligned(16))) uint16_t As[2][3][EM * RLDS];

  const int n_etiles = (N + EM - 1) / EM;
  const int tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
  const int et = tile % n_etiles;   // expert chunk fastest: blocks sharing tokens sit together
  const int tt = tile / n_etiles;
  const int e0 = et * EM;
  const int t0 = tt * (RW_WAVES * 32);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // Router-weight rows this thread stages (fp32, 4 per chunk).
  const int chunk = tid % CHUNKS;
  const float* a_src[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int r = tid / CHUNKS + i * ROWS_PER_PASS;
    a_src[i] = (e0 + r < N) ? Wr + (size_t)(e0 + r) * d : nullptr;
  }
  // Token row this lane streams.
  const int tok = t0 + wave * 32 + (lane & 31);
  const int khalf = lane >> 5;
  const uint16_t* b_src = (tok < T) ? x + (size_t)tok * d + khalf * 16 : nullptr;

  f32x16 acc[RM];
#pragma unroll
  for (int m = 0; m < RM; ++m) acc[m] = f32x16{};

  const int n_active = min(RM, (N - e0 + 31) / 32);
  const int nk = (d + RBK - 1) / RBK;

  u32x4 ra[A_LOADS];
  u32x4 rb0[2], rb1[2];

  auto load_a = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int k = k0 + chunk * 4;
      ra[i] = (a_src[i] && k < d) ? load16(a_src[i] + k) : u32x4{0, 0, 0, 0};
    }
  };
  auto load_b = [&](u32x4 (&rb)[2], int k0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int k = k0 + khalf * 16 + q * 8;
      rb[q] = (b_src && k < d) ? load16(b_src + k0 + q * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int r = tid / CHUNKS + i * ROWS_PER_PASS;
      uint32_t hi[4], mid[4], lo[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float w = __uint_as_float(ra[i][c]);
        hi[c] = f32_to_bf16_bits(w);
        const float r1 = w - bf16_bits_to_f32(hi[c]);
        mid[c] = f32_to_bf16_bits(r1);
        const float r2 = r1 - bf16_bits_to_f32(mid[c]);
        lo[c] = f32_to_bf16_bits(r2);
      }
      const int off = r * RLDS + chunk * 4;
      *reinterpret_cast<u32x2*>(&As[buf][0][off]) = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
      *reinterpret_cast<u32x2*>(&As[buf][1][off]) = u32x2{mid[0] | (mid[1] << 16), mid[2] | (mid[3] << 16)};
      *reinterpret_cast<u32x2*>(&As[buf][2][off]) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
    }
  };
  // Lane l holds k = k0 + 16*(l/32) + 8*q + 0..7 of its token in rb[q]; MFMA q
  // pairs it with the same k of the expert rows.
  auto compute = [&](int buf, const u32x4 (&rb)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const bf16x8 b = as_bf16x8(rb[q]);
#pragma unroll
      for (int m = 0; m < RM; ++m) {
        if (m < n_active) {
          const int off = (m * 32 + (lane & 31)) * RLDS + khalf * 16 + q * 8;
#pragma unroll
          for (int p = 0; p < 3; ++p) {
            const bf16x8 a = as_bf16x8(load16(&As[buf][p][off]));
            acc[m] = mfma_32x32x16(a, b, acc[m]);
          }
        }
      }
    }
  };

  load_b(rb0, 0);
  load_a(0);
  store_a(0);
  if (nk > 1) {
    load_b(rb1, RBK);
    load_a(RBK);
  }
  __syncthreads();
  for (int ks = 0; ks < nk; ks += 2) {
    compute(0, rb0);
    if (ks + 1 < nk) store_a(1);
    if (ks + 2 < nk) {
      load_b(rb0, (ks + 2) * RBK);
      load_a((ks + 2) * RBK);
    }
    __syncthreads();
    if (ks + 1 >= nk) break;
    compute(1, rb1);
    if (ks + 2 < nk) store_a(0);
    if (ks + 3 < nk) {
      load_b(rb1, (ks + 3) * RBK);
      load_a((ks + 3) * RBK);
    }
    __syncthreads();
  }

  if (tok >= T) return;
  float* zrow = logits + (size_t)tok * N;
#pragma unroll
  for (int m = 0; m < RM; ++m) {
    if (m < n_active) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = e0 + m * 32 + g * 8 + khalf * 4;
        if (e + 3 < N && (N & 3) == 0) {
          *reinterpret_cast<f32x4*>(zrow + e) =
              f32x4{acc[m][4 * g], acc[m][4 * g + 1], acc[m][4 * g + 2], acc[m][4 * g + 3]};
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (e + c < N) zrow[e + c] = acc[m][4 * g + c];
        }
      }
    }
  }
}

// Logits for fp32 token states: one thread per (token, expert), fp32 FMA in k order.
__global__ void __launch_bounds__(256)
router_logits_f32_kernel(const float* __restrict__ x, const float* __restrict__ Wr,
                         float* __restrict__ logits, int T, int d, int N) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)T * N) return;
  const int t = (int)(idx / N);
  const int i = (int)(idx % N);
  const float* xr = x + (size_t)t * d;
  const float* wr = Wr + (size_t)i * d;
  float s = 0.f;
  for (int k = 0; k < d; ++k) s = fmaf(xr[k], wr[k], s);
  logits[idx] = s;
}

hipError_t launch_router_logits(const Shape& s, const Inputs& in, const Workspace& ws,
                                hipStream_t st) {
  if (s.dtype == SFFN_FP32) {
    const long n = (long)s.T * s.N;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(router_logits_f32_kernel, dim3(blocks), dim3(256), 0, st,
                       (const float*)in.x, in.Wr, ws.logits, s.T, s.d, s.N);
    return hipGetLastError();
  }
  const int ttiles = (s.T + RW_WAVES * 32 - 1) / (RW_WAVES * 32);
  const int rm = s.N >= 128 ? 4 : (s.N + 31) / 32;
  const int etiles = (s.N + rm * 32 - 1) / (rm * 32);
  const dim3 grid((unsigned)(ttiles * etiles));
  const uint16_t* x = (const uint16_t*)in.x;
  switch (rm) {
    case 1: hipLaunchKernelGGL(router_logits_bf16_kernel<1>, grid, dim3(RW_WAVES * 64), 0, st, x, in.Wr, ws.logits, s.T, s.d, s.N); break;
    case 2: hipLaunchKernelGGL(router_logits_bf16_kernel<2>, grid, dim3(RW_WAVES * 64), 0, st, x, in.Wr, ws.logits, s.T, s.d, s.N); break;
    case 3: hipLaunchKernelGGL(router_logits_bf16_kernel<3>, grid, dim3(RW_WAVES * 64), 0, st, x, in.Wr, ws.logits, s.T, s.d, s.N); break;
    default: hipLaunchKernelGGL(router_logits_bf16_kernel<4>, grid, dim3(RW_WAVES * 64), 0, st, x, in.Wr, ws.logits, s.T, s.d, s.N); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Softmax, top-1, gate and per-block statistics.  One block handles
// kRouteTokens consecutive tokens; each wave takes every 4th token of the
// block.  Lane l holds experts l, l+64, ... (NPL of them).
//   m_t = max_i z, e_t = lowest i with z = m_t, S_t = sum_i exp(z - m_t),
//   gate = 1/S_t = p[t, e_t],  ppart[b, i] = sum over the block's tokens of p,
//   cnt[b, i] = tokens of the block whose top-1 is i,
//   lrank[t] = tokens of the block before t with the same top-1.
// All sums run in a fixed order, so results are bitwise reproducible.
// ---------------------------------------------------------------------------
template <int NPL>
__global__ void __launch_bounds__(256)
softmax_route_kernel(const float* __restrict__ logits, int T, int N,
                     int32_t* __restrict__ expert_idx, float* __restrict__ gate,
                     float* __restrict__ ppart, int* __restrict__ cnt, int* __restrict__ lrank) {
  constexpr int WAVES = 4;
  __shared__ float pacc[WAVES][NPL * 64];
  __shared__ int eid_s[kRouteTokens];
  __shared__ int cnt_s[NPL * 64];

  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tb = b * kRouteTokens;

  for (int i = threadIdx.x; i < NPL * 64; i += 256) cnt_s[i] = 0;

  float acc[NPL];
#pragma unroll
  for (int q = 0; q < NPL; ++q) acc[q] = 0.f;

  for (int j = wave; j < kRouteTokens; j += WAVES) {
    const int t = tb + j;
    if (t >= T) {
      if (lane == 0) eid_s[j] = -1;
      continue;
    }
    const float* z = logits + (size_t)t * N;
    float v[NPL];
    float m = -INFINITY;
    int arg = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int i = lane + 64 * q;
      v[q] = (i < N) ? z[i] : -INFINITY;
      if (i < N && (v[q] > m || (v[q] == m && i < arg))) {
        m = v[q];
        arg = i;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float om = __shfl_xor(m, off);
      const int oa = __shfl_xor(arg, off);
      if (om > m || (om == m && oa < arg)) {
        m = om;
        arg = oa;
      }
    }
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      v[q] = (lane + 64 * q < N) ? expf(v[q] - m) : 0.f;
      s += v[q];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    const float inv = 1.0f / s;
#pragma unroll
    for (int q = 0; q < NPL; ++q) acc[q] += v[q] * inv;
    if (lane == 0) {
      expert_idx[t] = arg;
      gate[t] = inv;
      eid_s[j] = arg;
    }
  }
#pragma unroll
  for (int q = 0; q < NPL; ++q) pacc[wave][lane + 64 * q] = acc[q];
  __syncthreads();

  for (int i = threadIdx.x; i < N; i += 256) {
    float p = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) p += pacc[w][i];
    ppart[(size_t)b * N + i] = p;
  }
  if (threadIdx.x < kRouteTokens) {
    const int j = threadIdx.x;
    const int e = eid_s[j];
    if (e >= 0) {
      int r = 0;
      for (int s2 = 0; s2 < j; ++s2) r += (eid_s[s2] == e);
      lrank[tb + j] = r;
      atomicAdd(&cnt_s[e], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += 256) cnt[(size_t)b * N + i] = cnt_s[i];
}

hipError_t launch_softmax_route(const Shape& s, const Workspace& ws, const Outputs& out,
                                hipStream_t st) {
  const dim3 grid((unsigned)s.n_route_blocks), block(256);
  const int npl = (s.N + 63) / 64;
#define SFFN_SOFTMAX(K)                                                                          \
  hipLaunchKernelGGL(softmax_route_kernel<K>, grid, block, 0, st, ws.logits, s.T, s.N,           \
                     out.expert_idx, out.gate, ws.ppart, ws.cnt, ws.lrank)
  if (npl <= 1) SFFN_SOFTMAX(1);
  else if (npl <= 2) SFFN_SOFTMAX(2);
  else if (npl <= 4) SFFN_SOFTMAX(4);
  else if (npl <= 8) SFFN_SOFTMAX(8);
  else if (npl <= 16) SFFN_SOFTMAX(16);
  else if (npl <= 32) SFFN_SOFTMAX(32);
  else SFFN_SOFTMAX(64);
#undef SFFN_SOFTMAX
  return hipGetLastError();
}

}  // namespace sffn
