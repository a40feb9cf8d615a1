// Expert FFNs of the Switch layer as grouped GEMMs over the expert-contiguous
// buffers, with the combine folded into the second GEMM's epilogue.
//
// E_e(v) = W2[e] ReLU(W1[e] v + b1[e]) + b2[e] ("Switch Transformer" paper
// note, section "Expert FFN Layer"); the output is scaled by the gate and added
// to the token's residual stream ("Switch Transformers: Scaling to Trillion
// Parameter Models with Simple and Efficient Sparsity", section 3.2,
// information flow through a Switch layer).  Only accepted rows are computed:
// expert e owns rows offset[e] .. offset[e+1]-1 of the buffers, in slot order.
//
//   FFN1: H[r, :] = ReLU(x[row2tok[r], :] W1[e]^T + b1[e])   (bf16 H)
//   FFN2: y[t, :] = x[t, :] + gate[t] (H[r, :] W2[e]^T + b2[e]),  t = row2tok[r]
#include "sffn_device.h"
#include "sffn_internal.h"
#include "../../include/switch_ffn.h"

namespace sffn {

// ---------------------------------------------------------------------------
// bf16 grouped GEMM on the matrix cores (v_mfma_f32_32x32x16_bf16).
//
// A block owns up to MT*32 rows of one expert and FW*32 output columns.  The
// weights are the streamed operand: each lane loads 32 consecutive k of one
// weight row (64 bytes) straight from HBM into registers, two k-steps ahead,
// and every weight byte is fetched once per row chunk.  The activations are
// the reused operand: the block gathers its rows (token rows of x for FFN1,
// rows of H for FFN2) into LDS, 64 k per step, double-buffered, and all four
// waves read them from there.  Within a k-step, the 64 k are permuted
// identically on both operands (lane half h, MFMA q covers k = 32h + 8q + i),
// which leaves the dot products unchanged.
// ---------------------------------------------------------------------------
constexpr int FW = 4;           // waves per block
constexpr int FBK = 64;         // k per step
constexpr int FLDS = FBK + 8;   // bf16 per LDS row (144 B)

template <int MT, bool SECOND>
__global__ void __launch_bounds__(FW * 64)
ffn_bf16_kernel(const uint16_t* __restrict__ act, const uint16_t* __restrict__ W,
                const uint16_t* __restrict__ bias, const int* __restrict__ offset,
                const int* __restrict__ row2tok, const float* __restrict__ gate,
                const uint16_t* __restrict__ xres, uint16_t* __restrict__ out, int K, int Nout,
                int n_mchunks, int d_model, int no_residual) {
  constexpr int ROWS = MT * 32;
  constexpr int NTHR = FW * 64;
  constexpr int RPP = NTHR / 8;        // rows per pass of the A loader (8 chunks of 16 B a row)
  constexpr int A_LOADS = ROWS / RPP;  // == MT
  __shared__ __attribute__((aligned(16))) uint16_t As[2][ROWS * FLDS];
  __shared__ int tok_s[ROWS];
  __shared__ float gate_s[ROWS];

  const int n_ntiles = (Nout + FW * 32 - 1) / (FW * 32);
  const int tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
  const int nt = tile % n_ntiles;
  const int rest = tile / n_ntiles;
  const int mc = rest % n_mchunks;
  const int e = rest / n_mchunks;
  const int rbeg = offset[e] + mc * ROWS;
  const int nrows = min(offset[e + 1] - rbeg, ROWS);
  if (nrows <= 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int khalf = lane >> 5;

  for (int r = tid; r < ROWS; r += NTHR) {
    const int t = r < nrows ? row2tok[rbeg + r] : -1;
    tok_s[r] = t;
    if (SECOND) gate_s[r] = t >= 0 ? gate[t] : 0.f;
  }
  __syncthreads();

  const int chunk = tid & 7;
  const uint16_t* a_src[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int r = (tid >> 3) + i * RPP;
    a_src[i] = nullptr;
    if (r < nrows)
      a_src[i] = SECOND ? act + (size_t)(rbeg + r) * K : act + (size_t)tok_s[r] * K;
  }
  const int n = nt * (FW * 32) + wave * 32 + (lane & 31);
  const uint16_t* b_src = n < Nout ? W + ((size_t)e * Nout + n) * K + khalf * 32 : nullptr;

  f32x16 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x16{};
  const int n_active = (nrows + 31) / 32;
  const int nk = (K + FBK - 1) / FBK;

  u32x4 ra[A_LOADS];
  u32x4 rb0[4], rb1[4];

  auto load_a = [&](int k0) {
    const int k = k0 + chunk * 8;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      ra[i] = (a_src[i] && k < K) ? load16(a_src[i] + k) : u32x4{0, 0, 0, 0};
  };
  auto load_b = [&](u32x4 (&rb)[4], int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = k0 + khalf * 32 + q * 8;
      rb[q] = (b_src && k < K) ? load16(b_src + k0 + q * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int r = (tid >> 3) + i * RPP;
      store16(&As[buf][r * FLDS + chunk * 8], ra[i]);
    }
  };
  auto compute = [&](int buf, const u32x4 (&rb)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8 b = as_bf16x8(rb[q]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < n_active) {
          const bf16x8 a =
              as_bf16x8(load16(&As[buf][(m * 32 + (lane & 31)) * FLDS + khalf * 32 + q * 8]));
          acc[m] = mfma_32x32x16(a, b, acc[m]);
        }
      }
    }
  };

  load_b(rb0, 0);
  load_a(0);
  store_a(0);
  if (nk > 1) {
    load_b(rb1, FBK);
    load_a(FBK);
  }
  __syncthreads();
  for (int ks = 0; ks < nk; ks += 2) {
    compute(0, rb0);
    if (ks + 1 < nk) store_a(1);
    if (ks + 2 < nk) {
      load_b(rb0, (ks + 2) * FBK);
      load_a((ks + 2) * FBK);
    }
    __syncthreads();
    if (ks + 1 >= nk) break;
    compute(1, rb1);
    if (ks + 2 < nk) store_a(0);
    if (ks + 3 < nk) {
      load_b(rb1, (ks + 3) * FBK);
      load_a((ks + 3) * FBK);
    }
    __syncthreads();
  }

  if (n >= Nout) return;
  const float bv = bias ? bf16_bits_to_f32(bias[(size_t)e * Nout + n]) : 0.f;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= n_active) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = m * 32 + (v >> 2) * 8 + khalf * 4 + (v & 3);
      if (r >= nrows) continue;
      const float val = acc[m][v] + bv;
      if (!SECOND) {
        out[(size_t)(rbeg + r) * Nout + n] = (uint16_t)f32_to_bf16_bits(fmaxf(val, 0.f));
      } else {
        const size_t o = (size_t)tok_s[r] * d_model + n;
        float yv = gate_s[r] * val;
        if (!no_residual) yv += bf16_bits_to_f32(xres[o]);
        out[o] = (uint16_t)f32_to_bf16_bits(yv);
      }
    }
  }
}

template <bool SECOND>
static void launch_ffn_bf16(int mt, dim3 grid, hipStream_t st, const uint16_t* act,
                            const uint16_t* W, const uint16_t* bias, const int* offset,
                            const int* row2tok, const float* gate, const uint16_t* xres,
                            uint16_t* out, int K, int Nout, int n_mchunks, int d_model,
                            int no_residual) {
#define SFFN_FFN(M)                                                                              \
  hipLaunchKernelGGL((ffn_bf16_kernel<M, SECOND>), grid, dim3(FW * 64), 0, st, act, W, bias,     \
                     offset, row2tok, gate, xres, out, K, Nout, n_mchunks, d_model, no_residual)
  switch (mt) {
    case 1: SFFN_FFN(1); break;
    case 2: SFFN_FFN(2); break;
    case 3: SFFN_FFN(3); break;
    case 4: SFFN_FFN(4); break;
    case 5: SFFN_FFN(5); break;
    case 6: SFFN_FFN(6); break;
    case 7: SFFN_FFN(7); break;
    default: SFFN_FFN(8); break;
  }
#undef SFFN_FFN
}

static int rows_tiles(int C) { return C <= 0 ? 1 : min(8, (C + 31) / 32); }

// ---------------------------------------------------------------------------
// fp32 experts: one thread per output element, fp32 FMA in k order.  Used for
// the fp32 variant of the layer (small parity shapes).
// ---------------------------------------------------------------------------
template <bool SECOND>
__global__ void __launch_bounds__(256)
ffn_f32_kernel(const float* __restrict__ act, const float* __restrict__ W,
               const float* __restrict__ bias, const int* __restrict__ offset,
               const int* __restrict__ row2tok, const float* __restrict__ gate,
               const float* __restrict__ xres, float* __restrict__ out, int K, int Nout,
               int d_model, int no_residual) {
  const int e = blockIdx.z;
  const int r = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int n = blockIdx.x * 16 + (threadIdx.x & 15);
  const int rbeg = offset[e];
  if (r >= offset[e + 1] - rbeg || n >= Nout) return;
  const int row = rbeg + r;
  const int tok = row2tok[row];
  const float* a = SECOND ? act + (size_t)row * K : act + (size_t)tok * K;
  const float* w = W + ((size_t)e * Nout + n) * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(a[k], w[k], s);
  if (bias) s += bias[(size_t)e * Nout + n];
  if (!SECOND) {
    out[(size_t)row * Nout + n] = fmaxf(s, 0.f);
  } else {
    const size_t o = (size_t)tok * d_model + n;
    float yv = gate[tok] * s;
    if (!no_residual) yv += xres[o];
    out[o] = yv;
  }
}

hipError_t launch_ffn1(const Shape& s, const Inputs& in, const Workspace& ws, hipStream_t st) {
  if (s.C <= 0) return hipSuccess;
  if (s.dtype == SFFN_FP32) {
    const dim3 grid((unsigned)((s.F + 15) / 16), (unsigned)((s.C + 15) / 16), (unsigned)s.N);
    hipLaunchKernelGGL(ffn_f32_kernel<false>, grid, dim3(256), 0, st, (const float*)in.x,
                       (const float*)in.W1, (const float*)in.b1, ws.offset, ws.row2tok,
                       (const float*)nullptr, (const float*)nullptr, (float*)ws.H, s.d, s.F, s.d,
                       0);
    return hipGetLastError();
  }
  const int mt = rows_tiles(s.C);
  const int n_mchunks = (s.C + mt * 32 - 1) / (mt * 32);
  const int n_ntiles = (s.F + FW * 32 - 1) / (FW * 32);
  const dim3 grid((unsigned)((long)n_ntiles * n_mchunks * s.N));
  launch_ffn_bf16<false>(mt, grid, st, (const uint16_t*)in.x, (const uint16_t*)in.W1,
                         (const uint16_t*)in.b1, ws.offset, ws.row2tok, nullptr, nullptr,
                         (uint16_t*)ws.H, s.d, s.F, n_mchunks, s.d, 0);
  return hipGetLastError();
}

hipError_t launch_ffn2(const Shape& s, const Inputs& in, const Workspace& ws, const Outputs& out,
                       bool no_residual, hipStream_t st) {
  if (s.C <= 0) return hipSuccess;
  if (s.dtype == SFFN_FP32) {
    const dim3 grid((unsigned)((s.d + 15) / 16), (unsigned)((s.C + 15) / 16), (unsigned)s.N);
    hipLaunchKernelGGL(ffn_f32_kernel<true>, grid, dim3(256), 0, st, (const float*)ws.H,
                       (const float*)in.W2, (const float*)in.b2, ws.offset, ws.row2tok, out.gate,
                       (const float*)in.x, (float*)out.y, s.F, s.d, s.d, no_residual ? 1 : 0);
    return hipGetLastError();
  }
  const int mt = rows_tiles(s.C);
  const int n_mchunks = (s.C + mt * 32 - 1) / (mt * 32);
  const int n_ntiles = (s.d + FW * 32 - 1) / (FW * 32);
  const dim3 grid((unsigned)((long)n_ntiles * n_mchunks * s.N));
  launch_ffn_bf16<true>(mt, grid, st, (const uint16_t*)ws.H, (const uint16_t*)in.W2,
                        (const uint16_t*)in.b2, ws.offset, ws.row2tok, out.gate,
                        (const uint16_t*)in.x, (uint16_t*)out.y, s.F, s.d, n_mchunks, s.d,
                        no_residual ? 1 : 0);
  return hipGetLastError();
}

}  // namespace sffn
