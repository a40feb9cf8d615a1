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
// A block owns up to MT*32 rows of one expert and FW*32 output columns (32 per
// wave).  The weights are the streamed operand: every weight byte is fetched
// once per row chunk, straight from HBM into registers, eight lanes per
// 128-byte line (one k-step of one weight row), so each load instruction covers
// eight whole lines.  Each wave then passes its 32 x 64 weight tile through a
// small private LDS slot to put it in the matrix-core operand layout.  The
// activations are the reused operand: the block gathers its rows (token rows of
// x for FFN1, rows of H for FFN2) into LDS, 64 k per step, and all waves read
// them from there; the activation bytes a block moves per weight byte are
// MT*32 / (FW*32), so wider blocks (FW up to 8) move fewer.  Both operands are
// fetched FP steps ahead into registers (buffer loads: out-of-range rows and k
// return zero, so the loop has no branches), and the activations pass through a
// double-buffered LDS tile one step ahead of use.  Within a k-step the 64 k are
// permuted identically on both operands (lane half h, MFMA q covers
// k = 32h + 8q + i), which leaves the dot products unchanged.
// ---------------------------------------------------------------------------
#ifndef SFFN_FFN_STAGES
#define SFFN_FFN_STAGES 3
#endif
constexpr int FBK = 64;              // k per step
constexpr int FLDS = FBK + 8;        // bf16 per LDS row (144 B): rows start 4 banks apart
constexpr int FP = SFFN_FFN_STAGES;  // k-steps in flight per operand

template <int MT, int FW, bool SECOND>
__global__ void __launch_bounds__(FW * 64)
ffn_bf16_kernel(const uint16_t* __restrict__ act, uint32_t act_bytes,
                const uint16_t* __restrict__ W, const uint16_t* __restrict__ bias,
                const int* __restrict__ offset, const int* __restrict__ row2tok,
                const float* __restrict__ gate, const uint16_t* __restrict__ xres,
                uint16_t* __restrict__ out, int K, int Nout, int n_mchunks, int d_model,
                int no_residual) {
  constexpr int ROWS = MT * 32;
  constexpr int NTHR = FW * 64;
  static_assert(ROWS <= NTHR, "one thread per row for the row lookups");
  constexpr int RPP = NTHR / 8;                    // rows per pass of the A loader (8 chunks a row)
  constexpr int A_LOADS = (ROWS + RPP - 1) / RPP;
  // One LDS buffer: [A tiles x2 | wave weight slots] in the k-loop, the result
  // staging tile in the epilogue.
  constexpr int AS_ELEMS = ROWS * FLDS;
  constexpr int LOOP_BYTES = (2 * AS_ELEMS + FW * 32 * FLDS) * 2;
  constexpr int STAGE_BYTES = SECOND ? ROWS * (FW * 16 + 4) * 4 : ROWS * (FW * 32 + 8) * 2;
  constexpr int SMEM_BYTES = LOOP_BYTES > STAGE_BYTES ? LOOP_BYTES : STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  uint16_t* const As0 = reinterpret_cast<uint16_t*>(smem);
  uint16_t* const Bs0 = As0 + 2 * AS_ELEMS;
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

  // The wave's 32 weight rows (expert e's block of Nout rows of K): load i of a
  // step brings rows 8i + lane/8, 16-byte chunk lane%8, of the k-step.
  const int n0 = nt * (FW * 32) + wave * 32;
  const __amdgpu_buffer_rsrc_t rb_src =
      make_rsrc(W + (size_t)e * Nout * K, (uint32_t)((size_t)Nout * K * 2));
  uint32_t b_off[4];
  bool b_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nr = n0 + i * 8 + (lane >> 3);
    b_ok[i] = nr < Nout;
    b_off[i] = ((uint32_t)(b_ok[i] ? nr : 0) * (uint32_t)K + (uint32_t)(lane & 7) * 8u) * 2u;
  }
  const int n = n0 + (lane & 31);  // output column of this lane in the MFMA result layout
  auto load_b = [&](u32x4 (&rb)[4], int ks) {
    const bool kin = ks * FBK + (lane & 7) * 8 < K;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rb[i] = buffer_load16(rb_src, (b_ok[i] && kin) ? b_off[i] + (uint32_t)ks * (FBK * 2) : kOob);
  };
  // Weights do not depend on the routing: start streaming them first.
  u32x4 rb[FP][4];
#pragma unroll
  for (int s = 0; s < FP; ++s) {
    load_b(rb[s], s);
    __builtin_amdgcn_sched_barrier(0);  // keep the prologue in step order
  }

  // Token of each row (one thread per row).  FFN1 needs it to find its
  // activation rows; FFN2 only in the epilogue, so there the load stays in
  // flight through the k-loop.
  const int my_tok = tid < nrows ? row2tok[rbeg + tid] : -1;
  if (!SECOND) {
    if (tid < ROWS) tok_s[tid] = my_tok;
    lds_barrier();
  }

  // Activation rows this thread stages: byte offset of (row, chunk) at k = 0.
  const __amdgpu_buffer_rsrc_t ra_src = make_rsrc(act, act_bytes);
  const int chunk = tid & 7;
  uint32_t a_off[A_LOADS];
  bool a_ok[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int r = (tid >> 3) + i * RPP;
    a_ok[i] = r < nrows;
    const uint32_t row = a_ok[i] ? (SECOND ? (uint32_t)(rbeg + r) : (uint32_t)tok_s[r]) : 0u;
    a_off[i] = (row * (uint32_t)K + (uint32_t)chunk * 8u) * 2u;
  }

  f32x16 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x16{};
  // Steps rounded up to whole pipeline rounds: the loop body is then free of
  // branches (extra steps load zeros), which keeps the load-wait counts exact.
  const int nk = ((K + FBK - 1) / FBK + FP - 1) / FP * FP;

  auto load_a = [&](u32x4 (&ra)[A_LOADS], int ks) {
    const bool kin = ks * FBK + chunk * 8 < K;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      ra[i] = buffer_load16(ra_src, (a_ok[i] && kin) ? a_off[i] + (uint32_t)ks * (FBK * 2) : kOob);
  };
  auto store_a = [&](int buf, const u32x4 (&ra)[A_LOADS]) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int r = (tid >> 3) + i * RPP;
      if (ROWS % RPP == 0 || r < ROWS) store16(As0 + buf * AS_ELEMS + r * FLDS + chunk * 8, ra[i]);
    }
  };
  uint16_t* bslot = Bs0 + wave * 32 * FLDS;
  auto compute = [&](int buf, const u32x4 (&rb)[4]) {
    // Weight tile into the wave's LDS slot (row-major), back out in operand layout.
    // LDS accesses of one wave complete in order, so no barrier is needed.
#pragma unroll
    for (int i = 0; i < 4; ++i) store16(bslot + (i * 8 + (lane >> 3)) * FLDS + (lane & 7) * 8, rb[i]);
    const uint16_t* base = As0 + buf * AS_ELEMS + (lane & 31) * FLDS + khalf * 32;
    const uint16_t* bbase = bslot + (lane & 31) * FLDS + khalf * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8 b = as_bf16x8(load16(bbase + q * 8));
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bf16x8 a = as_bf16x8(load16(base + m * 32 * FLDS + q * 8));
        acc[m] = mfma_32x32x16(a, b, acc[m]);
      }
    }
  };

  u32x4 ra[FP][A_LOADS];
#pragma unroll
  for (int s = 0; s < FP; ++s) {
    load_a(ra[s], s);
    __builtin_amdgcn_sched_barrier(0);
  }
  store_a(0, ra[0]);
  lds_barrier();
  for (int ks = 0; ks < nk; ks += FP) {
#pragma unroll
    for (int j = 0; j < FP; ++j) {
      const int k = ks + j;
      compute(k & 1, rb[j]);
      store_a((k + 1) & 1, ra[(j + 1) % FP]);   // A(k+1), fetched FP-1 steps ago
      load_a(ra[j], k + FP);                      // zero past the end of K
      load_b(rb[j], k + FP);
      lds_barrier();
    }
  }

  // Epilogue: the block's result tile goes through LDS (the activation buffers
  // are free after the loop's last barrier) and leaves in 16-byte row chunks.
  const float bv = (bias && n < Nout) ? bf16_bits_to_f32(bias[(size_t)e * Nout + n]) : 0.f;
  const int ccol = wave * 32 + (lane & 31);  // this lane's column within the block tile
  if (!SECOND) {
    // H rows: bias, ReLU, one rounding to bf16.
    constexpr int CST = FW * 32 + 8;  // bf16 per staged row
    uint16_t* Cs = As0;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m * 32 + (v >> 2) * 8 + khalf * 4 + (v & 3);
        Cs[r * CST + ccol] = (uint16_t)f32_to_bf16_bits(fmaxf(acc[m][v] + bv, 0.f));
      }
    }
    lds_barrier();
    constexpr int CPR = FW * 32 / 8;  // 16-byte chunks per staged row
    for (int idx = tid; idx < nrows * CPR; idx += NTHR) {
      const int r = idx / CPR, c = idx % CPR;
      const int col = nt * (FW * 32) + c * 8;
      if (col < Nout) store16(out + (size_t)(rbeg + r) * Nout + col, load16(&Cs[r * CST + c * 8]));
    }
  } else {
    // y rows: (acc + b2) * gate + x, one rounding to bf16; fp32 staging, half the
    // block's columns at a time.  The gate and residual loads go out first.
    constexpr int HALF = FW * 16;                       // columns per half
    constexpr int CST = HALF + 4;                       // fp32 per staged row
    constexpr int CPR = HALF / 8;                       // 16-byte output chunks per row and half
    constexpr int XPT = (ROWS * CPR + NTHR - 1) / NTHR; // chunks per thread and half
    if (tid < ROWS) {
      tok_s[tid] = my_tok;
      gate_s[tid] = my_tok >= 0 ? gate[my_tok] : 0.f;
    }
    lds_barrier();
    u32x4 xr[2][XPT];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < XPT; ++i) {
        const int idx = tid + i * NTHR;
        const int r = idx / CPR, c = idx % CPR;
        const int col = nt * (FW * 32) + h * HALF + c * 8;
        xr[h][i] = u32x4{0, 0, 0, 0};
        if (!no_residual && r < nrows && col < Nout)
          xr[h][i] = load16(xres + (size_t)tok_s[r] * d_model + col);
      }
    }
    float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (ccol / HALF == h) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = m * 32 + (v >> 2) * 8 + khalf * 4 + (v & 3);
            Cs[r * CST + (ccol - h * HALF)] = acc[m][v] + bv;
          }
        }
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < XPT; ++i) {
        const int idx = tid + i * NTHR;
        const int r = idx / CPR, c = idx % CPR;
        const int col = nt * (FW * 32) + h * HALF + c * 8;
        if (r >= nrows || col >= Nout) continue;
        const float g = gate_s[r];
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(&Cs[r * CST + c * 8]);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(&Cs[r * CST + c * 8 + 4]);
        const float val[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        u32x4 yr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = g * val[2 * j] + bf16_bits_to_f32(xr[h][i][j] & 0xffffu);
          const float hi = g * val[2 * j + 1] + bf16_bits_to_f32(xr[h][i][j] >> 16);
          yr[j] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
        }
        store16(out + (size_t)tok_s[r] * d_model + col, yr);
      }
      lds_barrier();
    }
  }
}

template <int FW, bool SECOND>
static void launch_ffn_bf16_fw(int mt, dim3 grid, hipStream_t st, const uint16_t* act,
                               uint32_t act_bytes, const uint16_t* W, const uint16_t* bias,
                               const int* offset, const int* row2tok, const float* gate,
                               const uint16_t* xres, uint16_t* out, int K, int Nout,
                               int n_mchunks, int d_model, int no_residual) {
#define SFFN_FFN(M)                                                                              \
  hipLaunchKernelGGL((ffn_bf16_kernel<M, FW, SECOND>), grid, dim3(FW * 64), 0, st, act,          \
                     act_bytes, W, bias, offset, row2tok, gate, xres, out, K, Nout, n_mchunks,   \
                     d_model, no_residual)
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

// Row tiles per block: the capacity's 32-row tiles split into as few chunks of at
// most 8 tiles as possible, evenly.
static int rows_tiles(int C) {
  const int tiles = C <= 0 ? 1 : (C + 31) / 32;
  const int chunks = (tiles + 7) / 8;
  return (tiles + chunks - 1) / chunks;
}

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

// Waves per block: the widest of 8, 6, 4 that still gives every CU a block
// (row chunks of 7-8 tiles keep 4 waves: wider blocks would spill registers).
static int pick_waves(int Nout, int mt, int n_mchunks, int N) {
  if (mt >= 7) return 4;
  const int fws[3] = {8, 6, 4};
  for (int fw : fws) {
    const long blocks = (long)((Nout + fw * 32 - 1) / (fw * 32)) * n_mchunks * N;
    if (blocks >= 256) return fw;
  }
  return 4;
}

template <bool SECOND>
static void launch_ffn_bf16(int Nout, const Shape& s, hipStream_t st, const uint16_t* act,
                            uint32_t act_bytes, const uint16_t* W, const uint16_t* bias,
                            const int* offset, const int* row2tok, const float* gate,
                            const uint16_t* xres, uint16_t* out, int K, int no_residual) {
  const int mt = rows_tiles(s.C);
  const int n_mchunks = (s.C + mt * 32 - 1) / (mt * 32);
  const int fw = pick_waves(Nout, mt, n_mchunks, s.N);
  const int n_ntiles = (Nout + fw * 32 - 1) / (fw * 32);
  const dim3 grid((unsigned)((long)n_ntiles * n_mchunks * s.N));
  if (fw == 8)
    launch_ffn_bf16_fw<8, SECOND>(mt, grid, st, act, act_bytes, W, bias, offset, row2tok, gate,
                                  xres, out, K, Nout, n_mchunks, s.d, no_residual);
  else if (fw == 6)
    launch_ffn_bf16_fw<6, SECOND>(mt, grid, st, act, act_bytes, W, bias, offset, row2tok, gate,
                                  xres, out, K, Nout, n_mchunks, s.d, no_residual);
  else
    launch_ffn_bf16_fw<4, SECOND>(mt, grid, st, act, act_bytes, W, bias, offset, row2tok, gate,
                                  xres, out, K, Nout, n_mchunks, s.d, no_residual);
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
  launch_ffn_bf16<false>(s.F, s, st, (const uint16_t*)in.x, (uint32_t)((size_t)s.T * s.d * 2),
                         (const uint16_t*)in.W1, (const uint16_t*)in.b1, ws.offset, ws.row2tok,
                         nullptr, nullptr, (uint16_t*)ws.H, s.d, 0);
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
  launch_ffn_bf16<true>(s.d, s, st, (const uint16_t*)ws.H,
                        (uint32_t)((size_t)s.max_rows * s.F * 2), (const uint16_t*)in.W2,
                        (const uint16_t*)in.b2, ws.offset, ws.row2tok, out.gate,
                        (const uint16_t*)in.x, (uint16_t*)out.y, s.F, no_residual ? 1 : 0);
  return hipGetLastError();
}

}  // namespace sffn
