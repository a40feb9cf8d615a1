// Backward pass of the Switch layer: top-1 routing, ReLU experts.
//
// The routing (argmax and capacity) is a piecewise-constant choice without a
// gradient; the router learns through the gate p[t, e_t] that scales the
// expert output ("Switch Transformers: Scaling to Trillion Parameter Models
// with Simple and Efficient Sparsity", section 3.4, "Switch Routing: The k=1
// Simplification") and through P_i of the aux loss, f_i being a count
// ("Switch Transformer, explained.", the symbol list under "Why one expert is
// enough").  With a = W1 x + b1, h = ReLU(a), o = W2 h + b2 for an accepted
// token t of expert e:
//   Q_t   = W2^T dy_t                         (E1: [rows, F] = dY_g W2_e)
//   dA_t  = g_t Q_t * [h_t > 0],  dg_t = Q_t . h_t + dy_t . b2_e
//   dXe_t = W1^T dA_t                         (E2: [rows, d] = dA W1_e)
//   dW2_e = sum_t g_t dy_t h_t^T               (E3: [d, F], contraction over rows)
//   dW1_e = sum_t dA_t x_t^T                   (E4: [F, d], contraction over rows)
//   db2_e = sum_t g_t dy_t,  db1_e = sum_t dA_t
//   u_{t,i} = d_aux N f_i / T + [t accepted][i = e_t] dg_t,  dz_t = p_t * (u_t - p_t . u_t)
//   dWr = dz^T x,  dx = dy + dXe + dz Wr       (fp32 router)
// h is the forward's bf16 H (its mask h > 0 is a > 0 up to rounding to zero).
#include "sffn_device.h"
#include "sffn_internal.h"
#include "../../include/switch_ffn.h"

namespace sffn {

// ---------------------------------------------------------------------------
// bf16 grouped GEMMs E1..E4 on the matrix cores: k-steps of 32 on
// v_mfma_f32_32x32x16_bf16, whose operand fragment is 8 consecutive k of one
// row or column per lane.  An operand that is k-contiguous in memory (E1 and
// E2's row operand) sits in LDS as [outer][k] rows (80-byte pitch) and a
// fragment is one 16-byte read.  The others hold k as their row index in
// memory (the weights of E1/E2 are [k][n]; E3/E4 contract over the expert's
// rows): they are copied into LDS as they are, [k][inner] rows of 320 bytes,
// and a fragment is two transposing reads (ds_read_b64_tr_b16: within each
// 16-lane group, lane i receives element i % 4 of the 8-byte chunks that
// lanes i/4 + 4c address, c = 0..3, so lanes addressing rows k..k+3 at
// columns 4 (j % 4) give each lane four consecutive k of one column).  The
// loads of the next PD steps are in flight in registers; LDS is
// double-buffered.
//
//   E1: rows x F,  K = d     A = dy[row2tok[r]]     B = W2_e [d][F]   (bwd_rows_kernel)
//   E2: rows x d,  K = F     A = dA[r]              B = W1_e [F][d]   (bwd_rows_kernel)
//   E3: d x F,     K = rows  A = g_r dy[row2tok[r]] B = H[r]          -> dW2_e
//   E4: F x d,     K = rows  A = dA[r]              B = x[row2tok[r]] -> dW1_e
// E1/E2 (bwd_rows_kernel): a whole row chunk of one expert against 32 NW output
// columns; E3/E4 (bwd_gemm_kernel): block tiles of (64 WMW) x (64 WNW), waves
// of 64 x 64 (2 x 2 MFMA tiles of 32 x 32), both operands [k][inner].
// ---------------------------------------------------------------------------
constexpr int GK = 32;
constexpr int GP = GK + 8;  // [outer][k] LDS row pitch in bf16 (80 bytes: fragment reads spread over banks)
constexpr int RP = 160;     // [k][inner] LDS row pitch in bf16 (320 bytes) of 128-wide tiles

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Operand fragment (8 consecutive k of inner index mbase + lane % 32, from k0 +
// 8 (lane / 32)) of a [k][inner] LDS tile, by two transposing reads.
__device__ __forceinline__ bf16x8 tr_fragment(const uint16_t* S, int k0, int mbase, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const uint16_t* p = S + (k0 + 8 * (g >> 1) + (j >> 2)) * RP + mbase + 16 * (g & 1) + 4 * (j & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * RP));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// k-steps whose loads are in flight: E1/E2 (long k-loops over d or F) and
// E3/E4 (k-loops over one expert's rows).
#ifndef SFFN_BWD_PD_ROWS
#define SFFN_BWD_PD_ROWS 2
#endif
#ifndef SFFN_BWD_PD_WGRAD
#define SFFN_BWD_PD_WGRAD 1
#endif
// Waves of E3/E4's block tile along its rows and columns (64 x 64 outputs each).
#ifndef SFFN_BWD_WGRAD_WM
#define SFFN_BWD_WGRAD_WM 2
#endif
#ifndef SFFN_BWD_WGRAD_WN
#define SFFN_BWD_WGRAD_WN 4
#endif
constexpr int kWgradWm = SFFN_BWD_WGRAD_WM, kWgradWn = SFFN_BWD_WGRAD_WN;
// Waves of E1's and E2's blocks (32 output columns each).  E2 produces d columns, a quarter of
// E1's F: 192-column tiles give it four column tiles at d = 768, so one block per CU with 64
// experts, where 256-column tiles leave a quarter of the CUs idle.
#ifndef SFFN_BWD_ROWS_NW
#define SFFN_BWD_ROWS_NW 8
#endif
#ifndef SFFN_BWD_E2_NW
#define SFFN_BWD_E2_NW 6
#endif
constexpr int kRowsWaves = SFFN_BWD_ROWS_NW, kRowsCols = 32 * kRowsWaves;  // E1
constexpr int kE2Waves = SFFN_BWD_E2_NW, kE2Cols = 32 * kE2Waves;          // E2

struct BwdGemmArgs {
  const uint16_t* a;
  const uint16_t* b;
  const int* offset;
  const int* row2tok;
  const float* rowgate;
  void* out;
  const int* bad;  // set by the guard: the results are written as NaN
  int T, d, F;
};

// A [k][inner] LDS tile's operand fragment as tr_fragment, for a tile of
// `pitch` bf16 per k row.
__device__ __forceinline__ bf16x8 tr_fragment_p(const uint16_t* S, int pitch, int k0, int mbase,
                                                int lane) {
  const int g = lane >> 4, j = lane & 15;
  const uint16_t* p = S + (k0 + 8 * (g >> 1) + (j >> 2)) * pitch + mbase + 16 * (g & 1) + 4 * (j & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * pitch));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// E3/E4: a block tile of (64 WMW) x (64 WNW) outputs, WMW x WNW waves of 64 x 64
// (2 x 2 matrix-core tiles each).  The contraction runs over the expert's rows
// (about C of them), so a tile reads (64 WMW + 64 WNW) x rows operand values
// and writes 64 WMW x 64 WNW results: wider tiles re-read the operands less per
// result written.
template <int KIND, int PD, int WMW, int WNW>
__global__ void __launch_bounds__(64 * WMW * WNW)
bwd_gemm_kernel(BwdGemmArgs g) {
  static_assert(KIND == 3 || KIND == 4, "the weight gradients");
  constexpr int NTHR = 64 * WMW * WNW;
  constexpr int TM = 64 * WMW, TN = 64 * WNW;   // block tile
  constexpr int RPA = TM + 32, RPB = TN + 32;   // [k][inner] LDS pitches (bf16): rows 16 banks apart
  constexpr int A_EL = GK * RPA, B_EL = GK * RPB;
  constexpr int SP = TN + 8;                    // staged tile pitch (bf16)
  constexpr int RING = 2 * (A_EL + B_EL);
  constexpr int LDS_EL = RING > TM * SP ? RING : TM * SP;
  // [A ring | B ring] (two buffers each); after the k-loop the epilogue stages its tile over it.
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_EL];
  uint16_t* const stg = lds;
  // Operand loads: CRx 16-byte chunks per k row, RPPx k rows per pass, NPx passes.
  constexpr int CRA = TM / 8, RPPA = NTHR / CRA, NPA = GK / RPPA;
  constexpr int CRB = TN / 8, RPPB = NTHR / CRB, NPB = GK / RPPB;
  static_assert(NTHR % CRA == 0 && GK % RPPA == 0 && NTHR % CRB == 0 && GK % RPPB == 0,
                "load mapping");
  constexpr int NPG = KIND == 3 ? NPA : NPB;  // passes of the gathered operand

  const int Nn = KIND == 3 ? g.F : g.d;
  const int M = KIND == 3 ? g.d : g.F;
  const int n_nt = (Nn + TN - 1) / TN;
  const int n_mt = (M + TM - 1) / TM;
  const int tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
  const int e = tile / (n_nt * n_mt);
  const int rest = tile % (n_nt * n_mt);
  const int mt = rest / n_nt, nt = rest % n_nt;
  const int rbeg = g.offset[e];
  const int Ae = g.offset[e + 1] - rbeg;
  const int K = Ae;
  const int m0 = mt * TM, n0 = nt * TN;
  const bool poison = *g.bad != 0;  // uniform

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WMW, wn = wave / WMW;

  // A: k row ar + RPPA q, chunk ac of the tile's TM-wide inner range; B likewise.
  const int ar = tid / CRA, ac = tid % CRA;
  const int br = tid / CRB, bc = tid % CRB;
  __amdgpu_buffer_rsrc_t a_src, b_src;
  if constexpr (KIND == 3) {
    a_src = make_rsrc(g.a, (uint32_t)g.T * (uint32_t)g.d * 2u);
    b_src = make_rsrc(g.b + (size_t)rbeg * g.F, (uint32_t)Ae * (uint32_t)g.F * 2u);
  } else {
    a_src = make_rsrc(g.a + (size_t)rbeg * g.F, (uint32_t)Ae * (uint32_t)g.F * 2u);
    b_src = make_rsrc(g.b, (uint32_t)g.T * (uint32_t)g.d * 2u);
  }
  const int ldA = KIND == 4 ? g.F : g.d;  // elements per memory row of A
  const int ldB = KIND == 3 ? g.F : g.d;  // ... and of B
  const int ma_chunk = m0 + ac * 8;       // A's inner chunk (m)
  const int nb_chunk = n0 + bc * 8;       // B's inner chunk (n)
  // k row of pass q of the gathered operand (E3: A, E4: B).
  auto grow = [&](int q) { return KIND == 3 ? ar + RPPA * q : br + RPPB * q; };

  // Register ring of PD k-steps in flight: slot s holds the loads of the steps
  // k with k % PD == s.  The gathered rows' tokens (and gates) are looked up
  // one ring ahead, so that no data load waits for its index.
  u32x4 ra[PD][NPA], rb[PD][NPB];
  int tk[PD][NPG];
  float gk[PD][NPG];
  auto lookup = [&](int k0, int (&t)[NPG], float (&gt)[NPG]) {
#pragma unroll
    for (int q = 0; q < NPG; ++q) {
      const int kk = k0 + grow(q);
      t[q] = kk < Ae ? g.row2tok[rbeg + kk] : -1;
      gt[q] = (KIND == 3 && kk < Ae) ? g.rowgate[rbeg + kk] : 0.f;
    }
  };
  auto load = [&](int k0, u32x4 (&a)[NPA], u32x4 (&b)[NPB], const int (&t)[NPG]) {
#pragma unroll
    for (int q = 0; q < NPA; ++q) {
      const int kk = k0 + ar + RPPA * q;
      // A: E3 gathered dy rows (scaled by the gate when staged), E4 expert rows of dA
      const uint32_t arow = KIND == 3 ? (uint32_t)(t[q] < 0 ? 0 : t[q]) : (uint32_t)kk;
      a[q] = buffer_load16(a_src, (kk < Ae && ma_chunk < M)
                                      ? (arow * (uint32_t)ldA + (uint32_t)ma_chunk) * 2u : kOob);
    }
#pragma unroll
    for (int q = 0; q < NPB; ++q) {
      const int kk = k0 + br + RPPB * q;
      // B: E3 expert rows of H, E4 gathered x rows
      const uint32_t brow = KIND == 4 ? (uint32_t)(t[q] < 0 ? 0 : t[q]) : (uint32_t)kk;
      b[q] = buffer_load16(b_src, (kk < Ae && nb_chunk < Nn)
                                      ? (brow * (uint32_t)ldB + (uint32_t)nb_chunk) * 2u : kOob);
    }
  };
  auto a_tile = [&](int buf) { return lds + buf * A_EL; };
  auto b_tile = [&](int buf) { return lds + 2 * A_EL + buf * B_EL; };
  // [k][inner] tiles: each chunk goes to its row as it is (E3's A scaled by the
  // row's gate, rounded once more to bf16).
  auto store = [&](int buf, const u32x4 (&a)[NPA], const u32x4 (&b)[NPB], const float (&sv)[NPG]) {
#pragma unroll
    for (int q = 0; q < NPA; ++q) {
      u32x4 w = a[q];
      if constexpr (KIND == 3) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
          w[h] = pack_bf16x2(bf16_bits_to_f32(a[q][h] & 0xffffu) * sv[q],
                             bf16_bits_to_f32(a[q][h] >> 16) * sv[q]);
      }
      store16(a_tile(buf) + (ar + RPPA * q) * RPA + ac * 8, w);
    }
#pragma unroll
    for (int q = 0; q < NPB; ++q) store16(b_tile(buf) + (br + RPPB * q) * RPB + bc * 8, b[q]);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int khalf = lane >> 5;
  auto compute = [&](int buf) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = tr_fragment_p(a_tile(buf), RPA, kh * 16, wm * 64 + 32 * i, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = tr_fragment_p(b_tile(buf), RPB, kh * 16, wn * 64 + 32 * j, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16(fb[j], fa[i], acc[i][j]);
    }
  };

  // Step k: its loads were issued PD steps earlier into slot k % PD; LDS
  // buffer k % 2 receives it one step before its matrix ops.  The steps are
  // rounded up to whole rounds of PD and every load is issued (past the end
  // of K they read zeros): the loop body has no branches, so the compiler's
  // waits for a slot's registers leave the later slots' loads in flight.
  // The gates of a slot's rows travel with it (sc) for the staging.
  float sc[PD][NPG];
  const int nk = (K + GK - 1) / GK;
  const int nkr = (nk + PD - 1) / PD * PD;
  static_for<0, PD>([&](auto j) { lookup(j * GK, tk[j], gk[j]); });
  static_for<0, PD>([&](auto j) {
    load(j * GK, ra[j], rb[j], tk[j]);
#pragma unroll
    for (int q = 0; q < NPG; ++q) sc[j][q] = gk[j][q];
    lookup((j + PD) * GK, tk[j], gk[j]);
  });
  store(0, ra[0], rb[0], sc[0]);
  __syncthreads();
  for (int k0 = 0; k0 < nkr; k0 += PD) {
    static_for<0, PD>([&](auto j) {
      constexpr int J = decltype(j)::value;
      const int k = k0 + J;
      load((k + PD) * GK, ra[J], rb[J], tk[J]);
#pragma unroll
      for (int q = 0; q < NPG; ++q) sc[J][q] = gk[J][q];
      lookup((k + 2 * PD) * GK, tk[J], gk[J]);
      __builtin_amdgcn_sched_barrier(0);  // the loads go out before this step's work
      compute(k & 1);
      constexpr int N1 = (J + 1) % PD;
      store((k + 1) & 1, ra[N1], rb[N1], sc[N1]);
      lds_barrier();  // LDS only: the later steps' loads stay in flight
    });
  }

  // ---- epilogue: lane holds row (l % 32) of each 32-row tile i and, for
  // value 4 gq + q, column 8 gq + 4 (l / 32) + q of each 32-column tile j ----
  const int lr = lane & 31;
  // dW2_e [d][F] (E3) or dW1_e [F][d] (E4), bf16, staged and written in row chunks
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ml = wm * 64 + 32 * i + lr;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x16& a = acc[i][j];
        *reinterpret_cast<u32x2*>(&stg[ml * SP + wn * 64 + 32 * j + 8 * gq + 4 * khalf]) =
            u32x2{pack_bf16x2(a[4 * gq], a[4 * gq + 1]), pack_bf16x2(a[4 * gq + 2], a[4 * gq + 3])};
      }
    }
  }
  __syncthreads();
  uint16_t* out = reinterpret_cast<uint16_t*>(g.out) + (size_t)e * g.d * g.F;
  constexpr int CPR = TN / 8;  // 16-byte chunks per staged row
#pragma unroll
  for (int c = 0; c < TM * CPR / NTHR; ++c) {
    const int idx = tid + NTHR * c;
    const int row = idx / CPR, col = (idx % CPR) * 8;
    const int m = m0 + row, n = n0 + col;
    // stored non-temporal: nothing here reads the gradients again, and their
    // dirty lines would otherwise crowd the caches for the next kernels
    if (m < M && n < Nn)
      __builtin_nontemporal_store(
          poison ? u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u} : load16(&stg[row * SP + col]),
          reinterpret_cast<u32x4*>(out + (size_t)m * Nn + n));
  }
}

// ---------------------------------------------------------------------------
// E1 and E2 with a whole row chunk per tile: a block computes R = 32 MT rows
// of one expert (all of its rows when C <= 160) against 128 output columns,
// wave w taking columns 32 w .. 32 w + 31 of every row.  A weight tile then
// streams once per row chunk instead of once per 128 rows, and no tile is
// mostly empty.  Operands as in bwd_gemm_kernel: A [rows][k] in LDS (one
// 16-byte fragment read), the weights [k][n] read as fragments by transposing
// reads.
//   E1: Q = dY_g W2_e  (K = d),  epilogue dA = g Q [H > 0] and partial dg
//   E2: dXe = dA W1_e  (K = F),  fp32 rows at the tokens
// ---------------------------------------------------------------------------
struct BwdRowsArgs {
  const uint16_t* a;   // E1: dy [T][d] (rows through row2tok); E2: dA [max_rows][F]
  const uint16_t* w;   // E1: W2 [N][d][F]; E2: W1 [N][F][d]
  const int* offset;
  const int* row2tok;
  const float* rowgate;
  const uint16_t* H;
  void* out;           // E1: dA [max_rows][F]; E2: dXe [T][d] fp32
  float* dgp;
  int T, d, F, max_rows, n_mc;  // n_mc: row chunks per expert
};

template <int KIND, int MT, int PD, int NW>
__global__ void __launch_bounds__(64 * NW)
bwd_rows_kernel(BwdRowsArgs g) {
  constexpr int NTHR = 64 * NW;
  constexpr int R = 32 * MT;
  constexpr int CW = 32 * NW;               // output columns per tile
  constexpr int RPW = CW + 32;              // [k][n] weight tile pitch (bf16): rows 16 banks apart
  constexpr int AI = (R * 4 + NTHR - 1) / NTHR;  // A loads per thread and step (16 bytes each)
  constexpr int CRB = CW / 8;               // 16-byte chunks per weight row of the tile
  constexpr int SPW = 128;                  // E1's epilogue works in parts of 128 columns
  constexpr int SP = SPW + 8;               // staged part pitch (bf16)
  constexpr int NPART = CW / SPW;
  constexpr int RING = 2 * R * GP + 2 * GK * RPW;
  static_assert(NTHR / CRB == 16, "two weight passes of 16 k rows");
  static_assert(KIND != 1 || CW % SPW == 0, "E1's epilogue parts");
  static_assert(R * SP <= RING, "a staged part fits the rings");
  __shared__ __attribute__((aligned(16))) uint16_t lds[RING];
  __shared__ float red[NW][R];
  uint16_t (*As)[R][GP] = reinterpret_cast<uint16_t (*)[R][GP]>(lds);
  uint16_t* const Bs = lds + 2 * R * GP;   // two [GK][RPW] tiles
  uint16_t* const stg = lds;

  const int Nn = KIND == 1 ? g.F : g.d;
  const int Kfull = KIND == 1 ? g.d : g.F;
  const int n_nt = (Nn + CW - 1) / CW;
  const int tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
  const int nt = tile % n_nt;
  const int mc = (tile / n_nt) % g.n_mc;
  const int e = tile / (n_nt * g.n_mc);
  const int rbeg = g.offset[e];
  const int Ae = g.offset[e + 1] - rbeg;
  const int m0 = mc * R, n0 = nt * CW;
  if (m0 >= Ae) return;  // uniform over the block
  const int kend = Kfull;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int khalf = lane >> 5;

  // A: chunk c = tid + NTHR i is 16-byte chunk c % 4 (of the k-step) of tile row c / 4.
  __amdgpu_buffer_rsrc_t a_src;
  uint32_t a_off[AI];
  if constexpr (KIND == 1) a_src = make_rsrc(g.a, (uint32_t)g.T * (uint32_t)g.d * 2u);
  else a_src = make_rsrc(g.a + (size_t)rbeg * g.F, (uint32_t)Ae * (uint32_t)g.F * 2u);
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int c = tid + NTHR * i;
    const int r = m0 + (c >> 2);
    const bool ok = c < R * 4 && r < Ae;
    const uint32_t row = KIND == 1 ? (ok ? (uint32_t)g.row2tok[rbeg + r] : 0u) : (uint32_t)r;
    a_off[i] = ok ? row * (uint32_t)(KIND == 1 ? g.d : g.F) * 2u : kOob;  // the row's start
  }
  // B: k rows tid/CRB + {0, 16} of the step, chunk tid % CRB of the CW columns.
  const int kr = tid / CRB, pc = tid % CRB;
  const int nb = n0 + pc * 8;
  const __amdgpu_buffer_rsrc_t b_src =
      make_rsrc(g.w + (size_t)e * g.d * g.F, (uint32_t)((size_t)g.d * g.F * 2));

  u32x4 ra[PD][AI], rb[PD][2];
  auto load = [&](int k0, u32x4 (&a)[AI], u32x4 (&b)[2]) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int kc = k0 + ((tid + NTHR * i) & 3) * 8;
      a[i] = buffer_load16(a_src, kc < kend ? a_off[i] + (uint32_t)kc * 2u : kOob);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int kk = k0 + kr + 16 * q;
      b[q] = buffer_load16(b_src, (kk < kend && nb < Nn)
                                      ? ((uint32_t)kk * (uint32_t)Nn + (uint32_t)nb) * 2u : kOob);
    }
  };
  auto store = [&](int buf, const u32x4 (&a)[AI], const u32x4 (&b)[2]) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int c = tid + NTHR * i;
      if (c < R * 4) store16(&As[buf][c >> 2][(c & 3) * 8], a[i]);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) store16(Bs + buf * GK * RPW + (kr + 16 * q) * RPW + pc * 8, b[q]);
  };

  f32x16 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x16{};
  auto compute = [&](int buf) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const bf16x8 fb = tr_fragment_p(Bs + buf * GK * RPW, RPW, kh * 16, 32 * wave, lane);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bf16x8 fa = as_bf16x8(load16(&As[buf][32 * m + (lane & 31)][kh * 16 + khalf * 8]));
        acc[m] = mfma_32x32x16(fb, fa, acc[m]);
      }
    }
  };

  // The k-loop as in bwd_gemm_kernel: PD steps in flight in registers, whole
  // rounds, no branches (steps past the end of K read zeros).
  const int nk = (kend + GK - 1) / GK;
  const int nkr = (nk + PD - 1) / PD * PD;
  static_for<0, PD>([&](auto j) { load(j * GK, ra[j], rb[j]); });
  store(0, ra[0], rb[0]);
  __syncthreads();
  for (int k0 = 0; k0 < nkr; k0 += PD) {
    static_for<0, PD>([&](auto j) {
      constexpr int J = decltype(j)::value;
      const int k = k0 + J;
      load((k + PD) * GK, ra[J], rb[J]);
      __builtin_amdgcn_sched_barrier(0);  // the loads go out before this step's work
      compute(k & 1);
      constexpr int N1 = (J + 1) % PD;
      store((k + 1) & 1, ra[N1], rb[N1]);
      lds_barrier();  // LDS only: the later steps' loads stay in flight
    });
  }

  // Lane values: row 32 m + lane % 32 of the tile; for value 4 gq + q,
  // column 32 wave + 8 gq + 4 khalf + q.
  const int lr = lane & 31;
  if constexpr (KIND == 1) {
    // Per part of 128 columns (waves 4p .. 4p+3): the H part into LDS; dA =
    // g Q [H > 0] in place of it and each wave's partial dg (its 32 columns)
    // per row; then dA out in row chunks.  The waves' partials are summed in
    // wave order at the end.
    const __amdgpu_buffer_rsrc_t h_src =
        make_rsrc(g.H + (size_t)rbeg * g.F, (uint32_t)Ae * (uint32_t)g.F * 2u);
    uint16_t* dA = reinterpret_cast<uint16_t*>(g.out) + (size_t)rbeg * g.F;
    constexpr int PCH = R * (SPW / 8) / NTHR;  // 16-byte chunks per thread of a part
#pragma unroll
    for (int p = 0; p < NPART; ++p) {
      const int pn0 = n0 + p * SPW;
#pragma unroll
      for (int c = 0; c < PCH; ++c) {
        const int idx = tid + NTHR * c;
        const int row = idx >> 4, col = (idx & 15) * 8;
        const int r = m0 + row, n = pn0 + col;
        store16(&stg[row * SP + col],
                buffer_load16(h_src, (r < Ae && n < g.F) ? ((uint32_t)r * (uint32_t)g.F + (uint32_t)n) * 2u
                                                          : kOob));
      }
      __syncthreads();
      if (wave / 4 == p) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int ml = 32 * m + lr;
          const int r = m0 + ml;
          const float gate = r < Ae ? g.rowgate[rbeg + r] : 0.f;
          float part = 0.f;
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            u32x2* ptr = reinterpret_cast<u32x2*>(&stg[ml * SP + 32 * (wave % 4) + 8 * gq + 4 * khalf]);
            const u32x2 hv = *ptr;
            float da[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float h = bf16_bits_to_f32((hv[q >> 1] >> (16 * (q & 1))) & 0xffffu);
              const float qv = acc[m][4 * gq + q];
              part += qv * h;
              da[q] = h > 0.f ? gate * qv : 0.f;
            }
            *ptr = u32x2{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
          }
          part += __shfl_xor(part, 32);
          if (khalf == 0) red[wave][ml] = part;
        }
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < PCH; ++c) {
        const int idx = tid + NTHR * c;
        const int row = idx >> 4, col = (idx & 15) * 8;
        const int r = m0 + row, n = pn0 + col;
        // non-temporal, as measured faster for the kernels after E1
        if (r < Ae && n < g.F)
          __builtin_nontemporal_store(load16(&stg[row * SP + col]),
                                      reinterpret_cast<u32x4*>(dA + (size_t)r * g.F + n));
      }
      if (p + 1 < NPART) __syncthreads();  // the part is read out before the next one lands
    }
    if (tid < R && m0 + tid < Ae) {
      float sum = red[0][tid];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += red[w][tid];
      g.dgp[(size_t)nt * g.max_rows + rbeg + m0 + tid] = sum;
    }
  } else {
    float* dxe = reinterpret_cast<float*>(g.out);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int r = m0 + 32 * m + lr;
      if (r >= Ae) continue;
      float* row = dxe + (size_t)g.row2tok[rbeg + r] * g.d;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int n = n0 + 32 * wave + 8 * gq + 4 * khalf;
        if (n < g.d)
          *reinterpret_cast<f32x4*>(row + n) =
              f32x4{acc[m][4 * gq], acc[m][4 * gq + 1], acc[m][4 * gq + 2], acc[m][4 * gq + 3]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 experts: one thread per output (or per row for E1), fp32 FMA in k
// order.  The fp32 layer's backward (small parity shapes).
// ---------------------------------------------------------------------------
// E1: one thread per expert row: Q = W2^T dy, dA = g Q [H > 0], dg part = Q . H.
__global__ void __launch_bounds__(256)
bwd_e1_f32_kernel(const float* __restrict__ dy, const float* __restrict__ W2,
                  const int* __restrict__ offset, const int* __restrict__ row2tok,
                  const float* __restrict__ rowgate, const float* __restrict__ H, int n_rows,
                  int N, int d, int F, float* __restrict__ dA, float* __restrict__ dgp) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= n_rows || row >= offset[N]) return;
  int e = 0;
  while (e + 1 < N && offset[e + 1] <= row) ++e;
  const float* y = dy + (size_t)row2tok[row] * d;
  const float* w = W2 + (size_t)e * d * F;
  const float gate = rowgate[row];
  float part = 0.f;
  for (int n = 0; n < F; ++n) {
    float q = 0.f;
    for (int k = 0; k < d; ++k) q = fmaf(y[k], w[(size_t)k * F + n], q);
    const float h = H[(size_t)row * F + n];
    part = fmaf(q, h, part);
    dA[(size_t)row * F + n] = h > 0.f ? gate * q : 0.f;
  }
  dgp[row] = part;
}

// E2: dXe[tok(row)][n] = sum_j dA[row][j] W1_e[j][n].
__global__ void __launch_bounds__(256)
bwd_e2_f32_kernel(const float* __restrict__ dA, const float* __restrict__ W1,
                  const int* __restrict__ offset, const int* __restrict__ row2tok, int n_rows,
                  int N, int d, int F, float* __restrict__ dxe) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)n_rows * d) return;
  const int row = (int)(i / d), n = (int)(i % d);
  if (row >= offset[N]) return;
  int e = 0;
  while (e + 1 < N && offset[e + 1] <= row) ++e;
  const float* w = W1 + (size_t)e * F * d;
  float s = 0.f;
  for (int j = 0; j < F; ++j) s = fmaf(dA[(size_t)row * F + j], w[(size_t)j * d + n], s);
  dxe[(size_t)row2tok[row] * d + n] = s;
}

// E3 (SECOND = false): dW2_e[m][n] = sum_r g_r dy[tok_r][m] H[r][n] over M = d, N = F.
// E4 (SECOND = true):  dW1_e[m][n] = sum_r dA[r][m] x[tok_r][n]  over M = F, N = d.
template <bool E4>
__global__ void __launch_bounds__(256)
bwd_wgrad_f32_kernel(const float* __restrict__ rowsA, const float* __restrict__ rowsB,
                     const int* __restrict__ offset, const int* __restrict__ row2tok,
                     const float* __restrict__ rowgate, int d, int F, const int* __restrict__ bad,
                     float* __restrict__ out) {
  const int e = blockIdx.y;
  const int M = E4 ? F : d, Nn = E4 ? d : F;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)M * Nn) return;
  const int m = (int)(i / Nn), n = (int)(i % Nn);
  float s = 0.f;
  for (int r = offset[e]; r < offset[e + 1]; ++r) {
    const int tok = row2tok[r];
    const float a = E4 ? rowsA[(size_t)r * F + m] : rowgate[r] * rowsA[(size_t)tok * d + m];
    const float b = E4 ? rowsB[(size_t)tok * d + n] : rowsB[(size_t)r * F + n];
    s = fmaf(a, b, s);
  }
  out[(size_t)e * M * Nn + i] = *bad ? __uint_as_float(0x7fc00000u) : s;
}

// ---------------------------------------------------------------------------
// Router gradient, one wave per token: p from the forward's fp32 logits, dg from
// E1's partial sums plus dy . b2, then dz = p * (u - p . u) written over the
// logits.  u_i = d_aux N hist_i / T^2 (+ dg at the token's expert).
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ void __launch_bounds__(256)
bwd_router_grad_kernel(const float* __restrict__ z, float* __restrict__ dz, const int32_t* __restrict__ expert_idx,
                       const int32_t* __restrict__ slot, const int* __restrict__ offset,
                       const int* __restrict__ hist, const float* __restrict__ dgp, int n_dgp,
                       int max_rows, const void* __restrict__ dyv, const void* __restrict__ b2v,
                       int T, int d, int N, int C, float d_aux, const int* __restrict__ bad) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  if (*bad) {  // the forward's workspace failed the guard: every dz is NaN
    for (int i = lane; i < N; i += 64) dz[(size_t)t * N + i] = __builtin_nanf("");
    return;
  }
  const float* zr = z + (size_t)t * N;
  float* dzr = dz + (size_t)t * N;
  float m = -INFINITY;
  for (int i = lane; i < N; i += 64) m = fmaxf(m, zr[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float S = 0.f;
  for (int i = lane; i < N; i += 64) S += expf(zr[i] - m);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) S += __shfl_xor(S, off);
  const float inv = 1.0f / S;

  // A slot is accepted only below C for an expert in range (the caller's
  // expert_idx and slot from the forward; anything else reads as dropped).
  const int e = expert_idx[t];
  const int sl = ((unsigned)e < (unsigned)N && slot[t] < C) ? slot[t] : -1;
  float dg = 0.f;
  if (sl >= 0) {
    const int row = offset[e] + sl;
    for (int q = lane; q < n_dgp; q += 64) dg += dgp[(size_t)q * max_rows + row];
    if (b2v) {
      for (int k = lane; k < d; k += 64) {
        const float yk = BF16 ? bf16_bits_to_f32(((const uint16_t*)dyv)[(size_t)t * d + k])
                              : ((const float*)dyv)[(size_t)t * d + k];
        const float bk = BF16 ? bf16_bits_to_f32(((const uint16_t*)b2v)[(size_t)e * d + k])
                              : ((const float*)b2v)[(size_t)e * d + k];
        dg = fmaf(yk, bk, dg);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dg += __shfl_xor(dg, off);
  }
  const float caux = d_aux * (float)N / ((float)T * (float)T);
  float pu = 0.f;
  for (int i = lane; i < N; i += 64) {
    const float p = expf(zr[i] - m) * inv;
    const float u = caux * (float)hist[i] + (i == e && sl >= 0 ? dg : 0.f);
    pu = fmaf(p, u, pu);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) pu += __shfl_xor(pu, off);
  for (int i = lane; i < N; i += 64) {
    const float p = expf(zr[i] - m) * inv;
    const float u = caux * (float)hist[i] + (i == e && sl >= 0 ? dg : 0.f);
    dzr[i] = p * (u - pu);
  }
}

// ---------------------------------------------------------------------------
// fp32 router GEMMs on the matrix cores (v_mfma_f32_32x32x2_f32: one k per
// lane, so either operand layout loads directly).  Block tile 128 x 128, four
// waves of 64 x 64, k-steps of 32.
//   DX:  dx[t][n] = dy + [accepted] dXe + sum_j dz[t][j] Wr[j][n]   (K = N)
//   DWR: part[p][j][n] = sum over the tokens of part p of dz[t][j] x[t][n]
// ---------------------------------------------------------------------------
constexpr int FK = 32;
constexpr int FPA = FK + 1;   // [m][k] rows of dz (DX): odd pitch, conflict-free column reads
constexpr int FPB = 128 + 32; // [k][n] rows: the two k of a fragment 32 banks apart

__device__ __forceinline__ f32x16 mfma_f32_32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <bool DWR, bool BF16>
__global__ void __launch_bounds__(256)
bwd_router_gemm_kernel(const float* __restrict__ dz, const float* __restrict__ Wr,
                       const void* __restrict__ xv, const void* __restrict__ dyv,
                       const float* __restrict__ dxe, const int32_t* __restrict__ slot, int T,
                       int d, int N, int tokens_per_part, void* __restrict__ outv) {
  // DX: A = dz [T][N] kept as [m][k]; B = Wr [N][d] as [k][n].
  // DWR: A = dz^T, kept as [k][m] (dz rows); B = x [T][d] as [k][n].
  // [A | B] operand tiles; the dx epilogue stages its tile over them.
  __shared__ __attribute__((aligned(16))) float smem[(DWR ? FK * FPB : 128 * FPA) + FK * FPB];
  float* const As = smem;
  float* const Bs = smem + (DWR ? FK * FPB : 128 * FPA);
  const int Mdim = DWR ? N : T;
  const int n_nt = (d + 127) / 128;
  const int n_mt = (Mdim + 127) / 128;
  const int bid = blockIdx.x;
  const int part = bid / (n_mt * n_nt);
  const int mt = (bid / n_nt) % n_mt, nt = bid % n_nt;
  const int m0 = mt * 128, n0 = nt * 128;
  const int kbeg = DWR ? part * tokens_per_part : 0;
  const int kend = DWR ? min(T, kbeg + tokens_per_part) : N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // 32 x 128 elements per operand and k-step: 16 per thread (consecutive
  // threads on consecutive addresses), all loaded into registers at once; the
  // next step's are in flight during this step's matrix ops.
  // Both operands move in chunks of 4 consecutive elements along their
  // contiguous axis (16-byte loads when the whole chunk is in range and aligned,
  // else element by element), 4 chunks per thread and operand; the element at
  // chunk position e of chunk q is tile element 4 (tid + 256 q) + e in the
  // operand's row-major tile order.
  //   DWR: A [32 k][128 m] from dz rows (m contiguous), B [32 k][128 n] from x.
  //   DX:  A [128 m][32 k] from dz rows (k contiguous), B [32 k][128 n] from Wr.
  float pa[16], pb[16];
  const bool a_vec = (N & 3) == 0;
  const bool b_vec = (d & 3) == 0;
  auto load4 = [&](const float* row, int j, int lim, bool vec, float* out4) {
    if (vec && j + 3 < lim) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) out4[e] = v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) out4[e] = j + e < lim ? row[j + e] : 0.f;
    }
  };
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = tid + 256 * q;
      if (DWR) {
        const int k = k0 + (c >> 5), m = m0 + 4 * (c & 31);
        if (k < kend) load4(dz + (size_t)k * N, m, N, a_vec, &pa[4 * q]);
        else for (int e = 0; e < 4; ++e) pa[4 * q + e] = 0.f;
      } else {
        const int m = m0 + (c >> 3), k = k0 + 4 * (c & 7);
        if (m < T) load4(dz + (size_t)m * N, k, kend, a_vec, &pa[4 * q]);
        else for (int e = 0; e < 4; ++e) pa[4 * q + e] = 0.f;
      }
      const int k = k0 + (c >> 5), n = n0 + 4 * (c & 31);
      if (k >= kend) {
        for (int e = 0; e < 4; ++e) pb[4 * q + e] = 0.f;
      } else if (!DWR) {
        load4(Wr + (size_t)k * d, n, d, b_vec, &pb[4 * q]);
      } else if (!BF16) {
        load4((const float*)xv + (size_t)k * d, n, d, b_vec, &pb[4 * q]);
      } else {  // bf16 x: d % 8 == 0, so a 4-element chunk is in range as a whole
        const uint16_t* xr = (const uint16_t*)xv + (size_t)k * d;
        const u32x2 v = n < d ? *reinterpret_cast<const u32x2*>(xr + n) : u32x2{0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) pb[4 * q + e] = bf16_bits_to_f32((v[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = tid + 256 * q;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (DWR) As[(c >> 5) * FPB + 4 * (c & 31) + e] = pa[4 * q + e];
        else As[(c >> 3) * FPA + 4 * (c & 7) + e] = pa[4 * q + e];
        Bs[(c >> 5) * FPB + 4 * (c & 31) + e] = pb[4 * q + e];
      }
    }
  };
  if (kbeg < kend) gload(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += FK) {
    sstore();
    __syncthreads();
    if (k0 + FK < kend) gload(k0 + FK);
#pragma unroll 4
    for (int ks = 0; ks < FK; ks += 2) {
      const int kk = ks + (lane >> 5);
      float fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int mm = wm * 64 + 32 * i + (lane & 31);
        fa[i] = DWR ? As[kk * FPB + mm] : As[mm * FPA + kk];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = Bs[kk * FPB + wn * 64 + 32 * j + (lane & 31)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_f32_32x32x2(fb[j], fa[i], acc[i][j]);
    }
    __syncthreads();
  }

  // Lane values: row m0 + wm*64 + 32 i + lr, four consecutive columns per gq.
  const int lr = lane & 31, khalf = lane >> 5;
  if constexpr (BF16 && !DWR) {
    // dx of the bf16 layer: the tile leaves through LDS in two halves of 64
    // rows (over the operand tiles), then each thread takes 8-column row
    // chunks, coalesced: dx = acc + dXe (accepted tokens) + dy, rounded once
    // (d % 8 == 0: a chunk is in range as a whole).
    constexpr int STP = 128 + 4;  // staged row pitch (floats)
    static_assert(64 * STP <= 128 * FPA + FK * FPB, "staged half tile fits the operand tiles");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (wm == h) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
              *reinterpret_cast<f32x4*>(smem + (32 * i + lr) * STP + wn * 64 + 32 * j + 8 * gq +
                                        4 * khalf) =
                  f32x4{acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                        acc[i][j][4 * gq + 3]};
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int idx = tid + 256 * c;
        const int row = idx >> 4, col = (idx & 15) * 8;
        const int m = m0 + 64 * h + row, n = n0 + col;
        if (m >= T || n >= d) continue;
        const float* sp = smem + row * STP + col;
        f32x4 v0 = *reinterpret_cast<const f32x4*>(sp);
        f32x4 v1 = *reinterpret_cast<const f32x4*>(sp + 4);
        const size_t o = (size_t)m * d + n;
        if (slot[m] >= 0) {
          const f32x4 e0 = *reinterpret_cast<const f32x4*>(dxe + o);
          const f32x4 e1 = *reinterpret_cast<const f32x4*>(dxe + o + 4);
          v0 = f32x4{v0[0] + e0[0], v0[1] + e0[1], v0[2] + e0[2], v0[3] + e0[3]};
          v1 = f32x4{v1[0] + e1[0], v1[1] + e1[1], v1[2] + e1[2], v1[3] + e1[3]};
        }
        const u32x4 yb = *reinterpret_cast<const u32x4*>((const uint16_t*)dyv + o);
        const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        u32x4 r;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          r[q] = pack_bf16x2(v[2 * q] + bf16_bits_to_f32(yb[q] & 0xffffu),
                             v[2 * q + 1] + bf16_bits_to_f32(yb[q] >> 16));
        *reinterpret_cast<u32x4*>((uint16_t*)outv + o) = r;
      }
      __syncthreads();
    }
    return;
  }
  const bool vec = (d & 3) == 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * 64 + 32 * i + lr;
    if (m >= Mdim) continue;
    const bool accepted = !DWR && slot[m] >= 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int n = n0 + wn * 64 + 32 * j + 8 * gq + 4 * khalf;
        if (n >= d) continue;
        const size_t o = (size_t)m * d + n;
        float v[4] = {acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                      acc[i][j][4 * gq + 3]};
        if (vec) {
          if (DWR) {
            *reinterpret_cast<f32x4*>((float*)outv + (size_t)part * N * d + o) =
                f32x4{v[0], v[1], v[2], v[3]};
            continue;
          }
          if (accepted) {
            const f32x4 xe = *reinterpret_cast<const f32x4*>(dxe + o);
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] += xe[q];
          }
          if (BF16) {
            const u32x2 yb = *reinterpret_cast<const u32x2*>((const uint16_t*)dyv + o);
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] += bf16_bits_to_f32((yb[q >> 1] >> (16 * (q & 1))) & 0xffffu);
            *reinterpret_cast<u32x2*>((uint16_t*)outv + o) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          } else {
            const f32x4 yf = *reinterpret_cast<const f32x4*>((const float*)dyv + o);
            *reinterpret_cast<f32x4*>((float*)outv + o) =
                f32x4{v[0] + yf[0], v[1] + yf[1], v[2] + yf[2], v[3] + yf[3]};
          }
          continue;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (n + q >= d) break;
          if (DWR) {
            ((float*)outv)[(size_t)part * N * d + o + q] = v[q];
          } else {
            float val = v[q] + (accepted ? dxe[o + q] : 0.f);
            if (BF16) {
              val += bf16_bits_to_f32(((const uint16_t*)dyv)[o + q]);
              ((uint16_t*)outv)[o + q] = (uint16_t)f32_to_bf16_bits(val);
            } else {
              val += ((const float*)dyv)[o + q];
              ((float*)outv)[o + q] = val;
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Partial dWr of the bf16 layer on the bf16 matrix cores: part p holds
// sum over its tokens t of dz_t^T x_t.  dz is split exactly into three bf16
// planes (dz = hi + mid + lo, each the round-to-nearest of what is left, as
// the router splits Wr in the forward pass) and x is bf16, so every product
// is exact and the sums run in fp32: an fp32 GEMM up to summation order, at
// the bf16 rate (three bf16 products per fp32 one).  Block tile 128 experts
// x 128 columns, four waves of 64 x 64; per k-step of 32 tokens the three dz
// planes and x are [k][inner] LDS tiles read by transposing reads.
// ---------------------------------------------------------------------------
template <int PD>
__global__ void __launch_bounds__(256)
bwd_wr_bf16_kernel(const float* __restrict__ dz, const uint16_t* __restrict__ x, int T, int d,
                   int N, int tokens_per_part, float* __restrict__ part_out) {
  constexpr int TILE = GK * RP;                // one [GK][RP] bf16 tile
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 4 * TILE];  // per buffer: 3 planes, x
  const int n_nt = (d + 127) / 128, n_mt = (N + 127) / 128;
  const int bid = blockIdx.x;
  const int part = bid / (n_mt * n_nt);
  const int mt = (bid / n_nt) % n_mt, nt = bid % n_nt;
  const int m0 = mt * 128, n0 = nt * 128;
  const int kbeg = part * tokens_per_part;
  const int kend = min(T, kbeg + tokens_per_part);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1, khalf = lane >> 5;

  // dz: thread k row tid/8, experts m0 + 16 (tid % 8) .. +15 (four 4-float
  // chunks).  x: k rows tid/16 + {0, 16}, 16-byte chunk tid % 16.
  const int ak = tid >> 3, am = m0 + 16 * (tid & 7);
  const int kr = tid >> 4, pc = tid & 15, nb = n0 + pc * 8;
  const bool nvec = (N & 3) == 0;
  const __amdgpu_buffer_rsrc_t z_src = make_rsrc(dz, (uint32_t)((size_t)T * N * 4));
  const __amdgpu_buffer_rsrc_t x_src = make_rsrc(x, (uint32_t)((size_t)T * d * 2));

  u32x4 ra[PD][4], rb[PD][2];
  auto load = [&](int k0, u32x4 (&a)[4], u32x4 (&b)[2]) {
    const int t = kbeg + k0 + ak;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int m = am + 4 * c;
      const uint32_t off = ((uint32_t)t * (uint32_t)N + (uint32_t)m) * 4u;
      if (nvec) {
        a[c] = buffer_load16(z_src, (t < kend && m < N) ? off : kOob);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a[c][e] = buffer_load4(z_src, (t < kend && m + e < N) ? off + 4u * (uint32_t)e : kOob);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int tt = kbeg + k0 + kr + 16 * q;
      b[q] = buffer_load16(x_src, (tt < kend && nb < d) ? ((uint32_t)tt * (uint32_t)d + (uint32_t)nb) * 2u
                                                         : kOob);
    }
  };
  auto store = [&](int buf, const u32x4 (&a)[4], const u32x4 (&b)[2]) {
    uint16_t* base = lds + buf * 4 * TILE;
    uint32_t pl[3][8];  // packed bf16 pairs of each plane
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        uint32_t h[2], mi[2], lo[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float w = __uint_as_float(a[c][e + u]);
          h[u] = f32_to_bf16_bits(w);
          const float r1 = w - bf16_bits_to_f32(h[u]);
          mi[u] = f32_to_bf16_bits(r1);
          lo[u] = f32_to_bf16_bits(r1 - bf16_bits_to_f32(mi[u]));
        }
        pl[0][2 * c + e / 2] = h[0] | (h[1] << 16);
        pl[1][2 * c + e / 2] = mi[0] | (mi[1] << 16);
        pl[2][2 * c + e / 2] = lo[0] | (lo[1] << 16);
      }
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      uint16_t* row = base + p * TILE + ak * RP + 16 * (tid & 7);
      store16(row, u32x4{pl[p][0], pl[p][1], pl[p][2], pl[p][3]});
      store16(row + 8, u32x4{pl[p][4], pl[p][5], pl[p][6], pl[p][7]});
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) store16(base + 3 * TILE + (kr + 16 * q) * RP + pc * 8, b[q]);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  auto compute = [&](int buf) {
    const uint16_t* base = lds + buf * 4 * TILE;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      bf16x8 fb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = tr_fragment(base + 3 * TILE, kh * 16, wn * 64 + 32 * j, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (m0 + wm * 64 + 32 * i >= N) continue;  // uniform over the wave: experts past N
#pragma unroll
        for (int p = 2; p >= 0; --p) {  // smallest plane first
          const bf16x8 fa = tr_fragment(base + p * TILE, kh * 16, wm * 64 + 32 * i, lane);
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16(fb[j], fa, acc[i][j]);
        }
      }
    }
  };

  // k-loop as in bwd_gemm_kernel: PD steps in flight, whole rounds, no branches.
  const int nk = (kend - kbeg + GK - 1) / GK;
  const int nkr = nk <= 0 ? 0 : (nk + PD - 1) / PD * PD;
  static_for<0, PD>([&](auto j) { load(j * GK, ra[j], rb[j]); });
  store(0, ra[0], rb[0]);
  __syncthreads();
  for (int k0 = 0; k0 < nkr; k0 += PD) {
    static_for<0, PD>([&](auto j) {
      constexpr int J = decltype(j)::value;
      const int k = k0 + J;
      load((k + PD) * GK, ra[J], rb[J]);
      __builtin_amdgcn_sched_barrier(0);
      compute(k & 1);
      constexpr int N1 = (J + 1) % PD;
      store((k + 1) & 1, ra[N1], rb[N1]);
      lds_barrier();
    });
  }

  // lane: expert m0 + wm*64 + 32 i + lane % 32; columns n0 + wn*64 + 32 j +
  // 8 gq + 4 khalf + q (d % 8 == 0: a group of four is in range as a whole).
  const int lr = lane & 31;
  float* out = part_out + (size_t)part * N * d;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * 64 + 32 * i + lr;
    if (m >= N) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int n = n0 + wn * 64 + 32 * j + 8 * gq + 4 * khalf;
        if (n < d)
          *reinterpret_cast<f32x4*>(out + (size_t)m * d + n) =
              f32x4{acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                    acc[i][j][4 * gq + 3]};
      }
    }
  }
}

// dWr = sum over parts, in part order.
__global__ void __launch_bounds__(256)
bwd_wr_reduce_kernel(const float* __restrict__ part, int parts, long n, float* __restrict__ out) {
  // Four consecutive sums per thread when n % 4 == 0 (16-byte loads, the parts'
  // loads unrolled ahead of the in-order adds), else one.
  if ((n & 3) == 0) {
    const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int p = 0; p < parts; ++p) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(part + (size_t)p * n + i);
      s = f32x4{s[0] + v[0], s[1] + v[1], s[2] + v[2], s[3] + v[3]};
    }
    *reinterpret_cast<f32x4*>(out + i) = s;
    return;
  }
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
#pragma unroll 8
  for (int p = 0; p < parts; ++p) s += part[(size_t)p * n + i];
  out[i] = s;
}

// ---------------------------------------------------------------------------
// Bias gradients, one thread per (expert, column): db2_e = sum_r g_r dy[tok_r],
// db1_e = sum_r dA[r], rows in buffer order.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ void __launch_bounds__(256)
bwd_bias_kernel(const void* __restrict__ dyv, const void* __restrict__ dAv,
                const int* __restrict__ offset, const int* __restrict__ row2tok,
                const float* __restrict__ rowgate, int d, int F, const int* __restrict__ bad,
                void* __restrict__ db1v, void* __restrict__ db2v) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;  // columns of db2 then db1
  const bool first = c < d;
  const int col = first ? c : c - d;
  if (col >= (first ? d : F) || (first ? db2v == nullptr : db1v == nullptr)) return;
  float s = 0.f;
  for (int r = offset[e]; r < offset[e + 1]; ++r) {
    float v;
    if (first) {
      const size_t o = (size_t)row2tok[r] * d + col;
      v = rowgate[r] * (BF16 ? bf16_bits_to_f32(((const uint16_t*)dyv)[o]) : ((const float*)dyv)[o]);
    } else {
      const size_t o = (size_t)r * F + col;
      v = BF16 ? bf16_bits_to_f32(((const uint16_t*)dAv)[o]) : ((const float*)dAv)[o];
    }
    s += v;
  }
  const size_t o = first ? (size_t)e * d + col : (size_t)e * F + col;
  void* out = first ? db2v : db1v;
  const bool poison = *bad != 0;  // the guard failed: NaN
  if (BF16) ((uint16_t*)out)[o] = poison ? (uint16_t)0x7fc0u : (uint16_t)f32_to_bf16_bits(s);
  else ((float*)out)[o] = poison ? __uint_as_float(0x7fc00000u) : s;
}

// ---------------------------------------------------------------------------
// Guard of the forward's workspace.  The pass reads the forward's dispatch maps
// and H, which only a top-1 forward without rerouting or GEGLU experts, of this
// very shape, lays out as read here; that forward leaves a layout tag at the
// start of its workspace.  One block checks the tag and the expert offsets
// (from 0, non-decreasing, at most max_rows rows; counts not negative) and
// copies offsets and counts into the backward's own workspace, where every
// later kernel reads them.  On a mismatch it writes empty experts there
// instead, so that no later kernel indexes the forward's maps, and raises
// `bad`: dz, and through it dx and dWr, comes out NaN, and the kernels that
// write the weight and bias gradients (every element of them) write NaN.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
bwd_guard_kernel(const uint32_t* __restrict__ tag, const WsTag want, uint32_t flags_allowed,
                 const int* __restrict__ offset, const int* __restrict__ hist, int N,
                 int max_rows, int* __restrict__ offset_out, int* __restrict__ hist_out,
                 int* __restrict__ bad) {
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t v = tag[i];
    ok &= i == kTagWFlags ? (v & ~flags_allowed) == 0 : v == want.w[i];
  }
  if (ok) {
    ok = offset[0] == 0 && offset[N] <= max_rows;
    for (int i = threadIdx.x; i < N; i += 256) ok &= offset[i] <= offset[i + 1] && hist[i] >= 0;
  }
  ok = __syncthreads_and(ok);
  for (int i = threadIdx.x; i <= N; i += 256) {
    offset_out[i] = ok ? offset[i] : 0;
    if (i < N) hist_out[i] = ok ? hist[i] : 0;
  }
  if (threadIdx.x == 0) *bad = ok ? 0 : 1;
}

// ---------------------------------------------------------------------------
int bwd_dgp_tiles(const Shape& s) {
  return s.dtype == SFFN_BF16 ? (s.F + kRowsCols - 1) / kRowsCols : 1;
}

int bwd_wr_parts(const Shape& s) {
  // Enough token parts for about 1024 blocks, each part at least 128 tokens.
  const int tiles = ((s.N + 127) / 128) * ((s.d + 127) / 128);
  int parts = (1024 + tiles - 1) / tiles;
  const int max_parts = (s.T + 127) / 128;
  if (parts > max_parts) parts = max_parts;
  return parts < 1 ? 1 : parts;
}

// Row tiles (of 32 rows) per E1/E2 block: the capacity's tiles split into as
// few chunks of at most 5 as possible, evenly.
static int bwd_rows_mt(int C) {
  const int tiles = C <= 0 ? 1 : (C + 31) / 32;
  const int chunks = (tiles + 4) / 5;
  return (tiles + chunks - 1) / chunks;
}

template <int KIND>
static hipError_t launch_rows(const BwdRowsArgs& g, int mt, int blocks, hipStream_t st) {
  constexpr int PD = SFFN_BWD_PD_ROWS, NW = KIND == 1 ? kRowsWaves : kE2Waves;
  const dim3 grid((unsigned)blocks), block(64 * NW);
  switch (mt) {
    case 1: hipLaunchKernelGGL((bwd_rows_kernel<KIND, 1, PD, NW>), grid, block, 0, st, g); break;
    case 2: hipLaunchKernelGGL((bwd_rows_kernel<KIND, 2, PD, NW>), grid, block, 0, st, g); break;
    case 3: hipLaunchKernelGGL((bwd_rows_kernel<KIND, 3, PD, NW>), grid, block, 0, st, g); break;
    case 4: hipLaunchKernelGGL((bwd_rows_kernel<KIND, 4, PD, NW>), grid, block, 0, st, g); break;
    default: hipLaunchKernelGGL((bwd_rows_kernel<KIND, 5, PD, NW>), grid, block, 0, st, g); break;
  }
  return hipGetLastError();
}

hipError_t launch_backward(const Shape& s, const Inputs& in, const BwdState& b, hipStream_t st,
                           void* const* ev) {
  int stage = 0;
  auto mark = [&]() -> hipError_t {
    if (!ev) return hipSuccess;
    return hipEventRecord((hipEvent_t)ev[stage++], st);
  };
  hipError_t err;
#define SFFN_CHECK(x)                      \
  do {                                     \
    if ((err = (x)) != hipSuccess) return err; \
  } while (0)
  const bool bf16 = s.dtype == SFFN_BF16;
  const int n_rows = s.max_rows;  // rows beyond offset[N] are never read

  // 1. the guard: checked copies of the forward's offsets and counts (timed with E1)
  SFFN_CHECK(mark());
  hipLaunchKernelGGL(bwd_guard_kernel, dim3(1), dim3(256), 0, st, b.fwd_tag, make_tag(s, 0u),
                     (uint32_t)SFFN_NO_RESIDUAL, b.fwd_offset, b.fwd_hist, s.N, s.max_rows,
                     b.offset, b.hist, b.bad);
  SFFN_CHECK(hipGetLastError());

  // 2. E1: dA and partial dg
  const int mt = bwd_rows_mt(s.C), n_mc = (s.C + 32 * mt - 1) / (32 * mt);
  if (s.C > 0) {
    if (bf16) {
      BwdRowsArgs g{(const uint16_t*)b.dy, (const uint16_t*)in.W2, b.offset, b.row2tok, b.rowgate,
                    (const uint16_t*)b.H, b.dA, b.dgp, s.T, s.d, s.F, s.max_rows, n_mc};
      SFFN_CHECK(launch_rows<1>(g, mt, s.N * n_mc * ((s.F + kRowsCols - 1) / kRowsCols), st));
    } else {
      hipLaunchKernelGGL(bwd_e1_f32_kernel, dim3((unsigned)((n_rows + 255) / 256)), dim3(256), 0,
                         st, (const float*)b.dy, (const float*)in.W2, b.offset, b.row2tok,
                         b.rowgate, (const float*)b.H, n_rows, s.N, s.d, s.F, (float*)b.dA, b.dgp);
    }
    SFFN_CHECK(hipGetLastError());
  }

  // 3. router gradient dz
  SFFN_CHECK(mark());
  {
    const dim3 grid((unsigned)((s.T + 3) / 4));
    if (bf16)
      hipLaunchKernelGGL(bwd_router_grad_kernel<true>, grid, dim3(256), 0, st, b.logits, b.dz,
                         b.expert_idx,
                         b.slot, b.offset, b.hist, b.dgp, b.n_dgp, s.max_rows, b.dy, in.b2, s.T,
                         s.d, s.N, s.C, b.d_aux, b.bad);
    else
      hipLaunchKernelGGL(bwd_router_grad_kernel<false>, grid, dim3(256), 0, st, b.logits, b.dz,
                         b.expert_idx,
                         b.slot, b.offset, b.hist, b.dgp, b.n_dgp, s.max_rows, b.dy, in.b2, s.T,
                         s.d, s.N, s.C, b.d_aux, b.bad);
    SFFN_CHECK(hipGetLastError());
  }

  // 4. E2: expert part of dx
  SFFN_CHECK(mark());
  if (s.C > 0) {
    if (bf16) {
      BwdRowsArgs g{(const uint16_t*)b.dA, (const uint16_t*)in.W1, b.offset, b.row2tok, b.rowgate,
                    nullptr, b.dxe, nullptr, s.T, s.d, s.F, s.max_rows, n_mc};
      SFFN_CHECK(launch_rows<2>(g, mt, s.N * n_mc * ((s.d + kE2Cols - 1) / kE2Cols), st));
    } else {
      const long n = (long)n_rows * s.d;
      hipLaunchKernelGGL(bwd_e2_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                         (const float*)b.dA, (const float*)in.W1, b.offset, b.row2tok, n_rows,
                         s.N, s.d, s.F, b.dxe);
    }
    SFFN_CHECK(hipGetLastError());
  }

  // 5. dx = dy + dXe + dz Wr
  SFFN_CHECK(mark());
  {
    const int blocks = ((s.T + 127) / 128) * ((s.d + 127) / 128);
    if (bf16)
      hipLaunchKernelGGL((bwd_router_gemm_kernel<false, true>), dim3((unsigned)blocks), dim3(256),
                         0, st, b.dz, in.Wr, in.x, b.dy, b.dxe, b.slot, s.T, s.d, s.N, 0, b.dx);
    else
      hipLaunchKernelGGL((bwd_router_gemm_kernel<false, false>), dim3((unsigned)blocks), dim3(256),
                         0, st, b.dz, in.Wr, in.x, b.dy, b.dxe, b.slot, s.T, s.d, s.N, 0, b.dx);
    SFFN_CHECK(hipGetLastError());
  }

  // 6. dWr = dz^T x, split over token parts, then summed in part order
  SFFN_CHECK(mark());
  {
    const int parts = b.n_wr_parts;
    const int per = ((s.T + parts - 1) / parts + FK - 1) / FK * FK;
    const int blocks = parts * ((s.N + 127) / 128) * ((s.d + 127) / 128);
    // bf16 planes while dz's byte offsets stay below 2^31 (the out-of-range
    // placeholder offset must lie past the buffer)
    if (bf16 && (size_t)s.T * s.N * 4 < ((size_t)1 << 31))
      hipLaunchKernelGGL((bwd_wr_bf16_kernel<2>), dim3((unsigned)blocks), dim3(256), 0, st, b.dz,
                         (const uint16_t*)in.x, s.T, s.d, s.N, per, b.wrp);
    else if (bf16)
      hipLaunchKernelGGL((bwd_router_gemm_kernel<true, true>), dim3((unsigned)blocks), dim3(256),
                         0, st, b.dz, in.Wr, in.x, b.dy, b.dxe, b.slot, s.T, s.d, s.N, per, b.wrp);
    else
      hipLaunchKernelGGL((bwd_router_gemm_kernel<true, false>), dim3((unsigned)blocks), dim3(256),
                         0, st, b.dz, in.Wr, in.x, b.dy, b.dxe, b.slot, s.T, s.d, s.N, per, b.wrp);
    SFFN_CHECK(hipGetLastError());
    const long n = (long)s.N * s.d;
    const long threads = (n & 3) == 0 ? n / 4 : n;
    hipLaunchKernelGGL(bwd_wr_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       st, b.wrp, parts, n, b.dWr);
    SFFN_CHECK(hipGetLastError());
  }

  // 7. E3 and E4: dW2, dW1 (every expert; zero where no rows)
  SFFN_CHECK(mark());
  if (bf16) {
    BwdGemmArgs g3{(const uint16_t*)b.dy, (const uint16_t*)b.H, b.offset, b.row2tok, b.rowgate,
                   b.dW2, b.bad, s.T, s.d, s.F};
    constexpr int TM = 64 * kWgradWm, TN = 64 * kWgradWn;
    const int t3 = ((s.d + TM - 1) / TM) * ((s.F + TN - 1) / TN);
    hipLaunchKernelGGL((bwd_gemm_kernel<3, SFFN_BWD_PD_WGRAD, kWgradWm, kWgradWn>),
                       dim3((unsigned)(s.N * t3)), dim3(64 * kWgradWm * kWgradWn), 0, st, g3);
    SFFN_CHECK(hipGetLastError());
    BwdGemmArgs g4{(const uint16_t*)b.dA, (const uint16_t*)in.x, b.offset, b.row2tok, b.rowgate,
                   b.dW1, b.bad, s.T, s.d, s.F};
    const int t4 = ((s.F + TM - 1) / TM) * ((s.d + TN - 1) / TN);
    hipLaunchKernelGGL((bwd_gemm_kernel<4, SFFN_BWD_PD_WGRAD, kWgradWm, kWgradWn>),
                       dim3((unsigned)(s.N * t4)), dim3(64 * kWgradWm * kWgradWn), 0, st, g4);
  } else {
    const long n = (long)s.d * s.F;
    const dim3 grid((unsigned)((n + 255) / 256), (unsigned)s.N);
    hipLaunchKernelGGL(bwd_wgrad_f32_kernel<false>, grid, dim3(256), 0, st, (const float*)b.dy,
                       (const float*)b.H, b.offset, b.row2tok, b.rowgate, s.d, s.F, b.bad,
                       (float*)b.dW2);
    SFFN_CHECK(hipGetLastError());
    hipLaunchKernelGGL(bwd_wgrad_f32_kernel<true>, grid, dim3(256), 0, st, (const float*)b.dA,
                       (const float*)in.x, b.offset, b.row2tok, b.rowgate, s.d, s.F, b.bad,
                       (float*)b.dW1);
  }
  SFFN_CHECK(hipGetLastError());

  // 8. bias gradients
  SFFN_CHECK(mark());
  if (b.db1 || b.db2) {
    const dim3 grid((unsigned)((s.d + s.F + 255) / 256), (unsigned)s.N);
    if (bf16)
      hipLaunchKernelGGL(bwd_bias_kernel<true>, grid, dim3(256), 0, st, b.dy, b.dA, b.offset,
                         b.row2tok, b.rowgate, s.d, s.F, b.bad, b.db1, b.db2);
    else
      hipLaunchKernelGGL(bwd_bias_kernel<false>, grid, dim3(256), 0, st, b.dy, b.dA, b.offset,
                         b.row2tok, b.rowgate, s.d, s.F, b.bad, b.db1, b.db2);
    SFFN_CHECK(hipGetLastError());
  }
  SFFN_CHECK(mark());
#undef SFFN_CHECK
  return hipSuccess;
}

}  // namespace sffn
