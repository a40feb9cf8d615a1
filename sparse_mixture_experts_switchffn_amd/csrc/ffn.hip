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
//
// GEGLU experts (named beside ReLU in the same paper's section 3.2): W1[e]
// holds 2F rows, the gate projection W (rows 0..F-1) and the linear
// projection V (rows F..2F-1), b1[e] both biases, and
//   FFN1: H[r, f] = GELU(x W^T + b_W)[f] * (x V^T + b_V)[f],  GELU(a) = a Phi(a).
#include "sffn_device.h"
#include "sffn_internal.h"
#include "../../include/switch_ffn.h"

namespace sffn {

// ---------------------------------------------------------------------------
// bf16 grouped GEMM on the matrix cores (v_mfma_f32_32x32x16_bf16).
//
// A tile is up to MT*32 rows of one expert against FW*32 output columns (32
// per wave), computed over k-steps of 64.
//
// Weights (the streamed operand) go from HBM straight into registers, eight
// lanes per 128-byte line (one k-step of one weight row), so each load
// instruction covers eight whole lines; each wave then passes its 32 x 64
// weight tile through a small private LDS slot to put it in the matrix-core
// operand layout.
//
// Activations (the reused operand: token rows of x for FFN1, rows of H for
// FFN2) go from memory straight into LDS with buffer loads that write LDS
// (one instruction moves 8 rows x 128 bytes), into a ring of FP+1 tiles; all
// waves read them from there.  Within a row the eight 16-byte chunks are
// stored XOR-swizzled by the row's low bits, so the matrix-core operand reads
// (32 rows, same chunk) spread over all LDS banks.  The activation bytes a
// block moves per weight byte are MT*32 / (FW*32).
//
// Both operands run FP steps ahead.  Out-of-range rows and k read as zero
// (buffer range checks), so the k-loop has no branches.  The LDS-writing loads
// are not tracked by the compiler's wait insertion: each step waits for them
// explicitly with a vector-memory count derived from the fixed issue order
// below (loads of all kinds complete in issue order on this target), then a
// barrier makes every wave's part of the tile visible.  Within a k-step the 64
// k are permuted identically on both operands (lane half h, MFMA q covers
// k = 32h + 8q + i), which leaves the dot products unchanged.
//
// The grid is persistent: one block per resident slot, each walking the tiles
// t = b, b + G, b + 2G, ... (b its XCD-contiguous index, G the grid size; tiles
// ordered by expert, then row chunk, then column tile, so the blocks running at
// one time on one XCD share an expert's activations in its L2).  The step
// stream runs on across tiles: the last round of a tile already fetches the
// next tile's first FP steps, and the next tile's row tokens, gates and bias
// are fetched while the tile runs, so tile starts and epilogues hide under
// loads in flight.
// ---------------------------------------------------------------------------
#ifndef SFFN_FFN_STAGES
#define SFFN_FFN_STAGES 3
#endif
// Cache policy bits of gfx950 buffer accesses: non-temporal (streamed,
// not kept in the caches).  The results are stored non-temporal (FFN2 reads
// H back, but keeping the dirty lines in L2 costs more than re-reading them);
// the weights are loaded non-temporal when each weight byte is read once (one
// row chunk per expert) and every weight row starts on a 128-byte line, and
// cached otherwise: row chunks re-read them, and with rows off the line grid
// a k-step reads half of a line whose other half the next step reads.
constexpr int kCpolNonTemporal = 2;
// Weight policy for rows of an odd number of 64-byte halves (K % 64 == 32):
// every other row then starts mid-line.  The loads are grouped by row parity
// (load i of a step takes rows of parity i%2): rows on the line grid stream
// past the caches, the others stay cached for the next k-step, which reads
// the other half of their last line.
constexpr int kCpolSplitRows = -1;
// FFN1 weight policy for the same rows: every load takes whole lines.  A load
// of an odd row (which starts mid-line) takes the line holding the second half
// of its k-step and the first half of the next step; that first half waits in
// registers (one stash per load) until the next step, and each tile starts
// with one extra load per odd row of its first 32 k.  Each weight line is then
// requested once (the line two rows share, twice) and all of them stream past
// the caches.
constexpr int kCpolShiftOdd = -2;
constexpr int FBK = 64;              // k per step (one 128-byte chunk row)
constexpr int FLDS = FBK + 8;        // bf16 per row of a weight slot (144 B: rows 4 banks apart)
constexpr int kFfnStages = SFFN_FFN_STAGES;  // k-steps in flight (two for split-row tiles)
constexpr int kLdsBytes = 160 * 1024;

// Kinds of pipeline round (FP steps): the first of a tile, a middle one, and
// the last (whose loads fetch the next tile; it may also be the first).
enum : int { kRoundFirst = 0, kRoundMid = 1, kRoundLast = 2 };

// GELU(a) = a Phi(a) = a (1 + erf(a / sqrt 2)) / 2, fp32.
__device__ __forceinline__ float gelu_f32(float a) {
  return 0.5f * a * (1.0f + erff(a * 0.7071067811865476f));
}

template <int MT, int FW, int WN, bool SECOND, bool GLU = false, int HV = 1>
struct FfnGeom {
  // GEGLU (FFN1 only): a tile's COLS weight rows are its "virtual columns": in
  // each epilogue part of PCOLS of them, the first half are gate rows and the
  // second half the linear rows of the same PCOLS/2 features, so a part holds
  // both factors of its outputs.  The stage is fp32 then, as for FFN2.
  static_assert(!(SECOND && GLU), "GEGLU is an FFN1 form");
  // Split rows (HV = 2): the waves form HV row parts of FW/HV column groups;
  // the two waves of a column group (one per part) each load half of the
  // group's weight rows into a slot they share, and each computes its own
  // MT row tiles against the whole slot, so a tile of HV*MT*32 rows streams
  // each weight byte once.  The shared slots are double-buffered and the
  // step's barrier publishes them; two k-steps stay in flight (the 320-row
  // activation tiles of 40 KB fill the LDS).
  static_assert(HV == 1 || HV == 2, "one or two row parts");
  static constexpr bool F32STAGE = SECOND || GLU;
  static constexpr int FP = HV == 2 ? 2 : kFfnStages;  // k-steps in flight
  static constexpr int FNB = FP + 1;                   // activation tiles in the LDS ring
  static constexpr int CG = FW / HV;                   // column groups (waves per row part)
  static constexpr int WROWS = MT * 32;                // rows per wave
  static constexpr int ROWS = WROWS * HV;              // rows per tile
  static constexpr int NTHR = FW * 64;
  static constexpr int WCOLS = WN * 32;               // output columns per wave
  static constexpr int COLS = CG * WCOLS;             // output columns per tile
  static constexpr int GROUPS = ROWS / 8;             // 8-row groups: one LDS-writing load each
  static constexpr int AL = (GROUPS + FW - 1) / FW;   // such loads per wave and step
  static constexpr int BL = 4 * WN / HV;              // weight loads per wave and step
  static constexpr int A_BYTES = ROWS * 128;          // one activation tile
  static constexpr int B_BYTES = HV * COLS * FLDS * 2;  // the weight slots (HV buffers)
  static constexpr int FREE = A_BYTES + B_BYTES;      // LDS the epilogue may use
  static constexpr int part_bytes(int wpp) {
    return F32STAGE ? ROWS * (wpp * WCOLS + 4) * 4 : ROWS * (wpp * WCOLS + 8) * 2;
  }
  static constexpr int pick_wpp() {
    for (int w = CG; w > 1; --w)
      if (CG % w == 0 && part_bytes(w) <= FREE) return w;
    return 1;
  }
  // Epilogue: the result leaves through LDS in column parts of WPP column groups.
  static constexpr int WPP = pick_wpp();
  static constexpr int NPARTS = CG / WPP;
  static constexpr int PCOLS = WPP * WCOLS;
  static constexpr int OPC = GLU ? PCOLS / 2 : PCOLS;             // output columns per part
  static constexpr int OCOLS = GLU ? COLS / 2 : COLS;             // output columns per tile
  static constexpr int CPR = OPC / 8;                             // 16-byte chunks per part row
  static constexpr int CST = F32STAGE ? PCOLS + 4 : PCOLS + 8;    // staged elements per row
  static constexpr int XPT = (ROWS * CPR + NTHR - 1) / NTHR;      // chunks per thread and part
  // Vector-memory operations per thread, in issue order:
  static constexpr int G = AL + BL;                 // per step of a first/middle round
  static constexpr int S = NPARTS * XPT;            // epilogue stores
  static constexpr int T1 = SECOND ? 3 : 2;         // next tile's token, bias chunk (and gate)
  // FFN2 holds its residual rows in registers through the epilogue; it then
  // fetches the next tile's weights after the epilogue instead of during the
  // last round (its activations still go out before the epilogue).
  static constexpr bool LATE_B = SECOND;
  static constexpr int EXTRA = SECOND ? S : 0;      // FFN2 residual loads (last round, step 0)
  static constexpr int SMEM = FNB * A_BYTES + B_BYTES + 1024;
  static constexpr bool fits = SMEM + ROWS * 8 + COLS * 2 <= kLdsBytes && part_bytes(1) <= FREE;

  // Operations this wave issued after the activation loads of step j of a
  // round of kind KIND, when that step starts; the step waits until no more
  // than this many are outstanding.  Tile start: the tile's FP activation
  // steps were the last activation loads, followed by S stores (the previous
  // epilogue, or as many placeholder stores before the first tile), with
  // LATE_B the FP weight steps, and the T1 lookups.
  template <int KIND, int J>
  static constexpr int step_wait() {
    constexpr int start = (FP - 1 - J) * AL + S + (LATE_B ? BL * FP : 0) + T1;
    constexpr int extra = (LATE_B && J >= 1) ? EXTRA : 0;
    constexpr int last_b = LATE_B ? 0 : J * BL;
    if constexpr (KIND == kRoundFirst) return start + J * G;
    else if constexpr (KIND == kRoundMid) return (FP - 1) * G;
    else {
      // A tile's final round runs one code path whether or not it is also
      // its first (K <= FP*64): the smaller count serves both.
      constexpr int after_mid = (FP - 1 - J) * G + extra + last_b;
      constexpr int after_start = start + extra + last_b;
      return after_mid < after_start ? after_mid : after_start;
    }
  }
};

// Rows rbeg .. rbeg+nrows-1 of expert e's buffer against column tile nt.
struct FfnTile {
  int e, nt, rbeg, nrows;
};

// The first non-empty tile of t, t + stride, ...; n_tiles if there is none.
// Everything here is uniform across the block (scalar loads of the offsets).
template <int ROWS>
__device__ __forceinline__ int find_tile(int t, int stride, int n_tiles, int n_ntiles,
                                         int n_mchunks, const int* __restrict__ offset,
                                         FfnTile& d) {
  for (; t < n_tiles; t += stride) {
    const int nt = t % n_ntiles;
    const int rest = t / n_ntiles;
    const int mc = rest % n_mchunks;
    const int e = rest / n_mchunks;
    const int rbeg = offset[e] + mc * ROWS;
    const int nrows = min(offset[e + 1] - rbeg, ROWS);
    if (nrows > 0) {
      d = FfnTile{e, nt, rbeg, nrows};
      return t;
    }
  }
  return n_tiles;
}

#define SFFN_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

template <int MT, int FW, int WN, bool SECOND, int WPOL, bool GLU = false, int HV = 1>
__global__ void __launch_bounds__(FW * 64)
ffn_bf16_kernel(const uint16_t* __restrict__ act, uint32_t act_bytes,
                const uint16_t* __restrict__ W, const uint16_t* __restrict__ bias,
                const int* __restrict__ offset, const int* __restrict__ row2tok,
                const float* __restrict__ rowgate, const uint16_t* __restrict__ xres,
                uint16_t* __restrict__ out, uint32_t out_bytes, int K, int Nout,
                int n_mchunks, int n_experts, int max_rows, int T, int d_model,
                int no_residual) {
  using Geo = FfnGeom<MT, FW, WN, SECOND, GLU, HV>;
  constexpr int FP = Geo::FP, FNB = Geo::FNB, CG = Geo::CG, WROWS = Geo::WROWS;
  constexpr int ROWS = Geo::ROWS, NTHR = Geo::NTHR, AL = Geo::AL, A_BYTES = Geo::A_BYTES;
  constexpr int NPARTS = Geo::NPARTS, WPP = Geo::WPP, PCOLS = Geo::PCOLS, CPR = Geo::CPR;
  constexpr int CST = Geo::CST, XPT = Geo::XPT, BL = Geo::BL, WCOLS = Geo::WCOLS;
  constexpr int COLS = Geo::COLS, OPC = Geo::OPC, OCOLS = Geo::OCOLS;
  constexpr int WMUL = GLU ? 2 : 1;  // weight rows per output column
  constexpr bool SHIFT = WPOL == kCpolShiftOdd;
  constexpr bool PARITY = SHIFT || WPOL == kCpolSplitRows;  // loads grouped by row parity
  constexpr int HB = SHIFT ? BL / 2 : 1;                     // odd-row loads (stashes)
  static_assert(!SHIFT || !Geo::LATE_B, "the stash is refilled before a tile's activations");
  static_assert(HV == 1 || (!PARITY && !GLU), "split rows: weight rows on the line grid, ReLU");
  static_assert(ROWS <= NTHR, "one thread per row for the row lookups");
  static_assert(Geo::fits, "LDS budget");
  // [activation ring (FNB tiles) | weight slots | 1 KB sink for idle loads].
  // The epilogue stages its result over [ring tile FP | weight slots].
  __shared__ __attribute__((aligned(1024))) char smem[Geo::SMEM];
  __shared__ int tok_s[ROWS];
  __shared__ float gate_s[ROWS];
  __shared__ __attribute__((aligned(16))) uint16_t bias_s[COLS];
  char* const As = smem;
  uint16_t* const Bs = reinterpret_cast<uint16_t*>(smem + FNB * A_BYTES);
  char* const sink = smem + FNB * A_BYTES + Geo::B_BYTES;
  char* const stage = smem + FP * A_BYTES;

  const int n_ntiles = (Nout + OCOLS - 1) / OCOLS;
  const int n_tiles = n_ntiles * n_mchunks * n_experts;
  const int stride = gridDim.x;
  FfnTile cur;
  int t = find_tile<ROWS>(xcd_contiguous_tile(blockIdx.x, gridDim.x), stride, n_tiles, n_ntiles,
                          n_mchunks, offset, cur);
  if (t >= n_tiles) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cgrp = wave % CG;   // column group: output columns cgrp*WCOLS ..
  const int rpart = wave / CG;  // row part: rows rpart*WROWS ..
  const int khalf = lane >> 5;
  // Steps rounded up to whole pipeline rounds: the loop body is then free of
  // branches (extra steps load zeros).
  const int nk = ((K + FBK - 1) / FBK + FP - 1) / FP * FP;

  const __amdgpu_buffer_rsrc_t ra_src = make_rsrc(act, act_bytes);
  const __amdgpu_buffer_rsrc_t tok_src = make_rsrc(row2tok, (uint32_t)max_rows * 4u);
  const __amdgpu_buffer_rsrc_t gate_src = make_rsrc(rowgate, SECOND ? (uint32_t)max_rows * 4u : 0u);
  const __amdgpu_buffer_rsrc_t out_src = make_rsrc(out, out_bytes);
  const __amdgpu_buffer_rsrc_t x_src =
      make_rsrc(xres, (SECOND && !(no_residual & 1)) ? (uint32_t)T * (uint32_t)d_model * 2u : 0u);
  // FFN2 output rows: the tokens' rows of y, or (bit 1 of no_residual, top-2
  // routing) the expert buffer's own rows, gate-scaled without the residual.
  const bool rowout = SECOND && (no_residual & 2) != 0;

  // Per-tile lookups: row token and gate (thread r: row r) and the tile's
  // bias (thread i: 16-byte chunk i, staged in LDS for the epilogue).
  auto load_tok = [&](const FfnTile& dt) -> int {
    return (int)buffer_load4(tok_src, tid < dt.nrows ? (uint32_t)(dt.rbeg + tid) * 4u : kOob);
  };
  auto load_gate = [&](const FfnTile& dt) -> float {
    return __uint_as_float(
        buffer_load4(gate_src, tid < dt.nrows ? (uint32_t)(dt.rbeg + tid) * 4u : kOob));
  };
  // Weight row (and bias entry) of virtual column v of column tile nt; -1 past
  // the last output column.
  auto phys_row = [&](int nt, int v) -> int {
    if constexpr (!GLU) {
      const int n = nt * COLS + v;
      return n < Nout ? n : -1;
    } else {
      constexpr int H = PCOLS / 2;
      const int j = v % PCOLS;
      const int f = nt * OCOLS + (v / PCOLS) * H + j % H;
      return f < Nout ? (j >= H ? Nout + f : f) : -1;
    }
  };
  auto load_bias = [&](const FfnTile& dt) -> u32x4 {
    const __amdgpu_buffer_rsrc_t src =
        make_rsrc(bias ? bias + (size_t)dt.e * WMUL * Nout : bias,
                  bias ? (uint32_t)(WMUL * Nout) * 2u : 0u);
    // Nout % 8 == 0 and 8-column chunks never straddle a half: a chunk is all
    // in or all out, and contiguous in the bias.
    const int n = tid < COLS / 8 ? phys_row(dt.nt, tid * 8) : -1;
    return buffer_load16(src, (dt.nrows > 0 && n >= 0) ? (uint32_t)n * 2u : kOob);
  };
  // Weights: load i of a step brings rows wrow(i) of the wave's WCOLS (8i +
  // lane/8, or grouped by parity: load i takes rows of parity i%2), 16-byte
  // chunk lane%8 of the k-step (kCpolShiftOdd, odd rows: 32 k further on).
  auto wrow = [&](int i) {
    return PARITY ? 2 * (8 * (i / 2) + (lane >> 3)) + (i & 1) : i * 8 + (lane >> 3);
  };
  auto setup_b = [&](const FfnTile& dt, __amdgpu_buffer_rsrc_t& src, uint32_t (&off)[BL]) {
    src = make_rsrc(W + (size_t)dt.e * WMUL * Nout * K, (uint32_t)((size_t)WMUL * Nout * K * 2));
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int nr = phys_row(dt.nt, cgrp * WCOLS + wrow(rpart * BL + i));
      const uint32_t shift = (SHIFT && (i & 1)) ? 32u : 0u;
      off[i] = (dt.nrows > 0 && nr >= 0)
                   ? ((uint32_t)nr * (uint32_t)K + shift + (uint32_t)(lane & 7) * 8u) * 2u : kOob;
    }
  };
  auto load_b = [&](u32x4 (&rb)[BL], const __amdgpu_buffer_rsrc_t& src, const uint32_t (&off)[BL],
                    int ks) {
    const int kc = ks * FBK + (lane & 7) * 8;
    const bool kin = kc < K;
    const bool kin_odd = SHIFT ? kc + 32 < K : kin;
    constexpr int P0 = PARITY ? kCpolNonTemporal : WPOL;                      // even loads
    constexpr int P1 = SHIFT ? kCpolNonTemporal : (PARITY ? 0 : WPOL);        // odd loads
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      if (i & 1)
        rb[i] = __builtin_amdgcn_raw_buffer_load_b128(
            src, (int)(kin_odd ? off[i] + (uint32_t)ks * (FBK * 2) : kOob), 0, P1);
      else
        rb[i] = __builtin_amdgcn_raw_buffer_load_b128(
            src, (int)(kin ? off[i] + (uint32_t)ks * (FBK * 2) : kOob), 0, P0);
    }
  };
  // kCpolShiftOdd: the stash of a tile's first step, each odd row's first
  // 32 k (k-step -1 of its loads: lanes 4..7 hold them).
  auto load_head = [&](u32x4 (&h)[HB], const __amdgpu_buffer_rsrc_t& src,
                       const uint32_t (&off)[BL]) {
    const int kc = (lane & 7) * 8 - 32;
    const bool kin = kc >= 0 && kc < K;
#pragma unroll
    for (int j = 0; j < HB; ++j)
      h[j] = __builtin_amdgcn_raw_buffer_load_b128(
          src, (int)((kin && off[2 * j + 1] != kOob) ? off[2 * j + 1] - (uint32_t)(FBK * 2) : kOob),
          0, kCpolNonTemporal);
  };

  // Activations: load i of a step fills row group g = wave + i*FW (rows 8g ..
  // 8g+7); lane l writes LDS chunk l%8 of row 8g + l/8, which holds logical
  // chunk (l%8) ^ swizzle(row).  Groups past the tile go to the sink.
  uint32_t a_off[AL];
  int a_c8[AL];  // 8 x the logical chunk this lane loads (the swizzle parity follows the group)
#pragma unroll
  for (int i = 0; i < AL; ++i)
    a_c8[i] = (((lane & 7) ^ (lane >> 3) ^ ((wave + i * FW) & 1)) & 7) * 8;
  auto setup_a = [&](const FfnTile& dt) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int r = (wave + i * FW) * 8 + (lane >> 3);
      const bool ok = r < dt.nrows;
      const uint32_t row = SECOND ? (uint32_t)(dt.rbeg + r) : (uint32_t)tok_s[ok ? r : 0];
      a_off[i] = ok ? (row * (uint32_t)K + (uint32_t)a_c8[i]) * 2u : kOob;
    }
  };
  auto dma_a = [&](int buf, int ks) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int g = wave + i * FW;
      char* dst = g < Geo::GROUPS ? As + buf * A_BYTES + g * 1024 : sink;
      const bool kin = ks * FBK + a_c8[i] < K;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra_src, SFFN_LDS_PTR(dst), 16, (int)(kin ? a_off[i] + (uint32_t)ks * (FBK * 2) : kOob),
          0, 0, 0);
    }
  };
  // Matrix-core operand reads of the activation tile: lane l, MFMA q reads
  // row m*32 + l%32, logical chunk 4*khalf + q, stored at chunk
  // (4*khalf + q) ^ swizzle; the q term only flips address bits 4-5.
  const int rsw = (lane & 7) ^ ((lane >> 3) & 1);  // swizzle of rows with these low bits
  const uint32_t a_rd = (uint32_t)(lane & 31) * 128u + (uint32_t)(((khalf * 4) ^ rsw) * 16);
  f32x16 acc[MT * WN];
  u32x4 st[HB];  // kCpolShiftOdd: the next step's first half of each odd row
  // The weight slot of the wave's column group (HV = 2: buffer b of two).
  auto slot_of = [&](int b) { return Bs + ((HV == 2 ? b * CG : 0) + cgrp) * WCOLS * FLDS; };
  // This wave's weight rows of a step into a slot (row-major).
  auto write_slot = [&](uint16_t* bslot, const u32x4 (&rb)[BL]) {
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      if (SHIFT && (i & 1)) {
        // Lanes 0..3 hold chunks 4..7 of this step; lanes 4..7 take chunks
        // 0..3 from the stash and keep their own (the next step's) in it.
        const bool lo = (lane & 7) < 4;
        u32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = lo ? rb[i][q] : st[i / 2][q];
        store16(bslot + wrow(i) * FLDS + (((lane & 7) + 4) & 7) * 8, v);
        st[i / 2] = rb[i];
      } else {
        store16(bslot + wrow(rpart * BL + i) * FLDS + (lane & 7) * 8, rb[i]);
      }
    }
  };
  // The matrix-core work of a step: activation ring tile `buf` (this wave's
  // row part) against a weight slot, in operand layout.
  auto mma = [&](int buf, const uint16_t* bslot) {
    const char* abase = As + buf * A_BYTES + rpart * WROWS * 128;
    const uint16_t* bbase = bslot + (lane & 31) * FLDS + khalf * 32;
    // Operand fragments of sub-step q (16 k): read one sub-step ahead of the
    // matrix-core ops that use them; the scheduling fence per sub-step keeps
    // the compiler from hoisting all of a step's reads (registers).
    bf16x8 fa[2][MT], fb[2][WN];
    auto read_frags = [&](int q, bf16x8 (&a)[MT], bf16x8 (&b)[WN]) {
#pragma unroll
      for (int w = 0; w < WN; ++w) b[w] = as_bf16x8(load16(bbase + w * 32 * FLDS + q * 8));
#pragma unroll
      for (int m = 0; m < MT; ++m)
        a[m] = as_bf16x8(load16(abase + ((a_rd ^ (uint32_t)(q * 16)) + m * 32 * 128)));
    };
    read_frags(0, fa[0], fb[0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < 3) read_frags(q + 1, fa[(q + 1) & 1], fb[(q + 1) & 1]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int w = 0; w < WN; ++w)
          acc[m * WN + w] = mfma_32x32x16(fb[q & 1][w], fa[q & 1][m], acc[m * WN + w]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One wave per slot: the wave writes its slot and reads it back (LDS
  // accesses of one wave complete in order, so no barrier is needed).
  auto compute = [&](int buf, const u32x4 (&rb)[BL]) {
    write_slot(slot_of(0), rb);
    mma(buf, slot_of(0));
  };

  // First tile: its lookups, then the weights (independent of the routing)
  // and the activation rows (FFN1 needs the tokens for them), in the order a
  // tile start inside the loop sees them.
  __amdgpu_buffer_rsrc_t rb_src;
  uint32_t b_off[BL];
  u32x4 rb[FP][BL];
  int my_tok = load_tok(cur);
  u32x4 my_bias = load_bias(cur);
  float my_gate = SECOND ? load_gate(cur) : 0.f;
  setup_b(cur, rb_src, b_off);
  auto prologue_b = [&]() {
#pragma unroll
    for (int s = 0; s < FP; ++s) {
      load_b(rb[s], rb_src, b_off, s);
      __builtin_amdgcn_sched_barrier(0);  // keep the prologue in step order
    }
  };
  if (!Geo::LATE_B) prologue_b();
  if constexpr (SHIFT) load_head(st, rb_src, b_off);
  if (!SECOND) {
    if (tid < ROWS) tok_s[tid] = my_tok;
    dma_barrier();
  }
  setup_a(cur);
#pragma unroll
  for (int s = 0; s < FP; ++s) {
    dma_a(s, s);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Placeholders for the epilogue stores that precede a tile start inside the
  // loop: stores at distinct offsets past the output's range, which the
  // range check drops.  Every tile then starts with the same sequence of
  // outstanding operations.
#pragma unroll
  for (int i = 0; i < Geo::S; ++i) buffer_store16(out_src, kOob + 16u * (uint32_t)i, u32x4{0, 0, 0, 0});
  __builtin_amdgcn_sched_barrier(0);
  if (Geo::LATE_B) prologue_b();

  for (;;) {
    // Tile start: steps 0 .. FP-1 are in flight (weights in rb, activations
    // into ring tiles 0 .. FP-1).  The epilogue's index arithmetic derives from
    // an opaque copy of the thread index so that it is recomputed per tile
    // rather than hoisted out of the tile loop, where it would hold registers.
    int etid = tid;
    asm volatile("" : "+v"(etid));
#pragma unroll
    for (int m = 0; m < MT * WN; ++m) acc[m] = f32x16{};
    if (SECOND && tid < ROWS) {
      tok_s[tid] = my_tok;  // visible after the first step's barrier
      gate_s[tid] = my_gate;
    }
    if (tid < COLS / 8) store16(bias_s + tid * 8, my_bias);
    // The next tile and its lookups, in flight through this tile.
    FfnTile nxt{cur.e, cur.nt, 0, 0};
    const int tn = find_tile<ROWS>(t + stride, stride, n_tiles, n_ntiles, n_mchunks, offset, nxt);
    const int tok_n = load_tok(nxt);
    const u32x4 bias_n = load_bias(nxt);
    const float gate_n = SECOND ? load_gate(nxt) : 0.f;
    __amdgpu_buffer_rsrc_t rb_src_n;
    uint32_t b_off_n[BL];

    u32x4 xr[NPARTS][SECOND ? XPT : 1];
    auto load_residual = [&]() {
      if constexpr (SECOND) {
#pragma unroll
        for (int p = 0; p < NPARTS; ++p) {
#pragma unroll
          for (int i = 0; i < XPT; ++i) {
            const int idx = etid + i * NTHR;
            const int r = idx / CPR, c = idx % CPR;
            const int col = cur.nt * COLS + p * PCOLS + c * 8;
            const bool ok = r < cur.nrows && col < Nout;
            xr[p][i] = buffer_load16(
                x_src, ok ? ((uint32_t)tok_s[ok ? r : 0] * (uint32_t)d_model + (uint32_t)col) * 2u
                          : kOob);
          }
        }
      }
    };
    auto step = [&](auto kind_c, auto j_c, int ks) {
      constexpr int KIND = decltype(kind_c)::value;
      constexpr int J = decltype(j_c)::value;
      const int k = ks + J;
      wait_vmcnt<Geo::template step_wait<KIND, J>()>();  // this wave's A(k) is in LDS
      if constexpr (HV == 2) {
        // This wave's half of the group's weights of step k (its own loads:
        // the compiler waits for them) into slot buffer k % 2; the barrier
        // publishes both halves.  Buffer k % 2 was last read in step k - 2,
        // which every wave finished before the previous barrier.
        write_slot(slot_of(k & 1), rb[J]);
        dma_barrier();  // everyone's activations and slot halves; ring tile k-1 is free
        mma(k % FNB, slot_of(k & 1));
      } else {
        dma_barrier();  // everyone's activations; ring tile k-1 is free
        compute(k % FNB, rb[J]);
      }
      if constexpr (KIND == kRoundFirst || KIND == kRoundMid) {
        dma_a((k + FP) % FNB, k + FP);  // zero past the end of K
        load_b(rb[J], rb_src, b_off, k + FP);
      } else if constexpr (Geo::LATE_B) {
        if (J == 0) {  // FFN2's residual rows; tok_s is visible since the first step
          __builtin_amdgcn_sched_barrier(0);  // not into the compute above
          load_residual();
        }
      } else {
        // kCpolShiftOdd: the stash is free after the tile's final compute.
        if constexpr (SHIFT && J == FP - 1) load_head(st, rb_src_n, b_off_n);
        load_b(rb[J], rb_src_n, b_off_n, J);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto round = [&](auto kind_c, int ks) {
      static_for<0, FP>([&](auto j_c) { step(kind_c, j_c, ks); });
    };
    if (nk > FP) {
      round(std::integral_constant<int, kRoundFirst>{}, 0);
      for (int ks = FP; ks < nk - FP; ks += FP) round(std::integral_constant<int, kRoundMid>{}, ks);
    }
    if (!Geo::LATE_B) setup_b(nxt, rb_src_n, b_off_n);
    round(std::integral_constant<int, kRoundLast>{}, nk - FP);

    // The next tile's activation rows (ring tiles 0 .. FP-1), once every wave
    // is past its last read of the ring.
    if (!SECOND && tid < ROWS) tok_s[tid] = tok_n;
    dma_barrier();
    setup_a(nxt);
#pragma unroll
    for (int s = 0; s < FP; ++s) {
      dma_a(s, s);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Epilogue: the result goes through LDS in column parts and leaves in
    // 16-byte row chunks.
#pragma unroll
    for (int p = 0; p < NPARTS; ++p) {
      if (cgrp / WPP == p) {
        // The matrix-core result is C^T: lane l holds row l%32 of row tile m
        // and, for value 4g + j, column 8g + 4*(l/32) + j of column tile w --
        // four consecutive columns per g, staged as one 8- or 16-byte write.
        // Lane geometry from the opaque index keeps the staging addresses
        // immediates off one per-tile base.
        const int elane = etid & 63;
        const int ekh = elane >> 5;
        const int er = elane & 31;
#pragma unroll
        for (int w = 0; w < WN; ++w) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int cw = cgrp * WCOLS + w * 32 + 8 * g + 4 * ekh;  // column within the tile
            const u32x2 bb = *reinterpret_cast<const u32x2*>(bias_s + cw);
            const float b0 = bf16_bits_to_f32(bb[0] & 0xffffu), b1 = bf16_bits_to_f32(bb[0] >> 16);
            const float b2 = bf16_bits_to_f32(bb[1] & 0xffffu), b3 = bf16_bits_to_f32(bb[1] >> 16);
            const int pc = cw - p * PCOLS;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              const f32x16& a = acc[m * WN + w];
              const int r = rpart * WROWS + m * 32 + er;
              if (Geo::F32STAGE) {
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(stage) + r * CST + pc) =
                    f32x4{a[4 * g] + b0, a[4 * g + 1] + b1, a[4 * g + 2] + b2, a[4 * g + 3] + b3};
              } else {  // H: bias, ReLU, one rounding to bf16
                *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(stage) + r * CST + pc) =
                    u32x2{pack_bf16x2(fmaxf(a[4 * g] + b0, 0.f), fmaxf(a[4 * g + 1] + b1, 0.f)),
                          pack_bf16x2(fmaxf(a[4 * g + 2] + b2, 0.f), fmaxf(a[4 * g + 3] + b3, 0.f))};
              }
            }
          }
        }
      }
      dma_barrier();
#pragma unroll
      for (int i = 0; i < XPT; ++i) {
        const int idx = etid + i * NTHR;
        const int r = idx / CPR, c = idx % CPR;
        const int col = cur.nt * OCOLS + p * OPC + c * 8;
        const bool ok = r < cur.nrows && col < Nout;
        const int rr = ok ? r : 0;
        if (GLU) {
          // H = GELU(gate half) * linear half, one rounding to bf16.
          const float* srow = reinterpret_cast<const float*>(stage) + rr * CST + c * 8;
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(srow);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(srow + 4);
          const f32x4 l0 = *reinterpret_cast<const f32x4*>(srow + PCOLS / 2);
          const f32x4 l1 = *reinterpret_cast<const f32x4*>(srow + PCOLS / 2 + 4);
          const u32x4 v{pack_bf16x2(gelu_f32(g0[0]) * l0[0], gelu_f32(g0[1]) * l0[1]),
                        pack_bf16x2(gelu_f32(g0[2]) * l0[2], gelu_f32(g0[3]) * l0[3]),
                        pack_bf16x2(gelu_f32(g1[0]) * l1[0], gelu_f32(g1[1]) * l1[1]),
                        pack_bf16x2(gelu_f32(g1[2]) * l1[2], gelu_f32(g1[3]) * l1[3])};
          __builtin_amdgcn_raw_buffer_store_b128(
              v, out_src,
              (int)(ok ? ((uint32_t)(cur.rbeg + r) * (uint32_t)Nout + (uint32_t)col) * 2u : kOob), 0,
              kCpolNonTemporal);
        } else if (!SECOND) {
          const u32x4 v = load16(reinterpret_cast<const uint16_t*>(stage) + rr * CST + c * 8);
          __builtin_amdgcn_raw_buffer_store_b128(
              v, out_src,
              (int)(ok ? ((uint32_t)(cur.rbeg + r) * (uint32_t)Nout + (uint32_t)col) * 2u : kOob), 0,
              kCpolNonTemporal);
        } else {
          // y = (acc + b2) * gate + x, one rounding to bf16.
          const float* srow = reinterpret_cast<const float*>(stage) + rr * CST + c * 8;
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(srow);
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(srow + 4);
          const float val[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          const float g = gate_s[rr];
          u32x4 yr;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float lo = g * val[2 * j] + bf16_bits_to_f32(xr[p][i][j] & 0xffffu);
            const float hi = g * val[2 * j + 1] + bf16_bits_to_f32(xr[p][i][j] >> 16);
            yr[j] = pack_bf16x2(lo, hi);
          }
          __builtin_amdgcn_raw_buffer_store_b128(
              yr, out_src,
              (int)(ok ? ((uint32_t)(rowout ? cur.rbeg + rr : tok_s[rr]) * (uint32_t)d_model + (uint32_t)col) * 2u
                       : kOob),
              0,
              kCpolNonTemporal);
        }
      }
      dma_barrier();
    }

    if (tn >= n_tiles) break;
    if (Geo::LATE_B) {
      setup_b(nxt, rb_src_n, b_off_n);
#pragma unroll
      for (int s = 0; s < FP; ++s) {
        load_b(rb[s], rb_src_n, b_off_n, s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    cur = nxt;
    t = tn;
    my_tok = tok_n;
    my_bias = bias_n;
    my_gate = gate_n;
    rb_src = rb_src_n;
#pragma unroll
    for (int i = 0; i < BL; ++i) b_off[i] = b_off_n[i];
  }
  // The last activation loads (range-checked to nothing) still write LDS:
  // let them land before the block's LDS is released.
  wait_vmcnt<0>();
}

#undef SFFN_LDS_PTR

template <int MT, int FW, int WN, bool SECOND, bool GLU, int WPOL = 0, int HV = 1>
static int ffn_resident_blocks() {
  // Blocks of this kernel the device holds at once (a persistent grid's size).
  static const int n = [] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, ffn_bf16_kernel<MT, FW, WN, SECOND, WPOL, GLU, HV>, FW * 64, 0) != hipSuccess)
      return 256;
    return (cus > 0 ? cus : 256) * (per_cu > 0 ? per_cu : 1);
  }();
  return n;
}

struct FfnArgs {
  const uint16_t* act;
  uint32_t act_bytes;
  const uint16_t* W;
  const uint16_t* bias;
  const int* offset;
  const int* row2tok;
  const float* rowgate;
  const uint16_t* xres;
  uint16_t* out;
  uint32_t out_bytes;
  int K, Nout, n_mchunks, n_experts, max_rows, T, d_model, no_residual;
};

// Block shapes (waves, 32-column tiles per wave) the launcher chooses from.
// {8, 2}: 512-column tiles (one block per CU) for one or two row tiles, where
// the activation rows are re-read least and a launch has half as many tiles.
struct FfnShape {
  int fw, wn;
};
constexpr FfnShape kFfnShapes[] = {{8, 2}, {4, 2}, {3, 2}, {8, 1}, {6, 1}, {4, 1}};

template <int MT, int FW, int WN, bool SECOND, bool GLU>
static constexpr bool ffn_shape_ok() {
  // Two column tiles per wave only for up to 2 row tiles: beyond that the
  // registers allow one wave per SIMD, which leaves too little latency
  // hiding.  Blocks of more than 4 waves (2 per SIMD) only up to 6 row tiles
  // (registers).  One thread per row for the row lookups; the LDS budget holds.
  // 512-column tiles (eight waves of two column tiles) for one row tile only
  // (registers).
  return (WN == 1 || MT <= 2) && (FW <= 4 || MT <= 6) && MT * 32 <= FW * 64 &&
         (FW * WN <= 8 || MT == 1) && FfnGeom<MT, FW, WN, SECOND, GLU>::fits;
}

template <int MT, int FW, int WN, bool SECOND, bool GLU>
static long ffn_resident_if_ok() {
  if constexpr (ffn_shape_ok<MT, FW, WN, SECOND, GLU>())
    return ffn_resident_blocks<MT, FW, WN, SECOND, GLU>();
  else return 0;
}

// Column tiles of a launch: each covers FW*WN*32 weight rows, which are as many
// output columns (GEGLU: half as many).
static long ffn_col_tiles(const FfnArgs& a, long rows_per_tile, bool glu) {
  const long ocols = glu ? rows_per_tile / 2 : rows_per_tile;
  return (a.Nout + ocols - 1) / ocols;
}

// One launch with weight policy WPOL: a persistent grid of as many blocks as
// that kernel keeps resident, or fewer if there are fewer tiles.
template <int MT, int FW, int WN, bool SECOND, int WPOL, bool GLU, int HV = 1>
static void launch_ffn_pol(const FfnArgs& a, hipStream_t st) {
  const long n_tiles = ffn_col_tiles(a, FW / HV * WN * 32, GLU) * a.n_mchunks * a.n_experts;
  const long resident = ffn_resident_blocks<MT, FW, WN, SECOND, GLU, WPOL, HV>();
  const dim3 grid((unsigned)(n_tiles < resident ? n_tiles : resident)), block(FW * 64);
  hipLaunchKernelGGL((ffn_bf16_kernel<MT, FW, WN, SECOND, WPOL, GLU, HV>), grid, block, 0, st, a.act,
                     a.act_bytes, a.W, a.bias, a.offset, a.row2tok, a.rowgate, a.xres, a.out,
                     a.out_bytes, a.K, a.Nout, a.n_mchunks, a.n_experts, a.max_rows, a.T,
                     a.d_model, a.no_residual);
}

template <int MT, int FW, int WN, bool SECOND, bool GLU>
static void launch_ffn_bf16_t(const FfnArgs& a, hipStream_t st) {
  if constexpr (ffn_shape_ok<MT, FW, WN, SECOND, GLU>()) {
    // Weights are streamed past the caches when nothing re-reads their lines
    // (with rows off the line grid: FFN1 loads whole lines, FFN2 streams only
    // the rows on the grid).
    const bool odd_rows =
        a.n_mchunks == 1 && (a.K * 2) % 128 == 64 && ((size_t)a.W & 127) == 0 && a.Nout % 2 == 0;
    constexpr int kOddPol = SECOND ? kCpolSplitRows : kCpolShiftOdd;
    if (odd_rows) launch_ffn_pol<MT, FW, WN, SECOND, kOddPol, GLU>(a, st);
    else if (a.n_mchunks == 1 && (a.K * 2) % 128 == 0)
      launch_ffn_pol<MT, FW, WN, SECOND, kCpolNonTemporal, GLU>(a, st);
    else launch_ffn_pol<MT, FW, WN, SECOND, 0, GLU>(a, st);
  }
}

// Estimated time of one launch with a block shape, in units of one row of K
// streamed through a CU: each tile streams its weight rows (on average the
// output columns over the column tiles: a ragged last tile streams only its
// own rows) and re-reads its activation rows (mostly L2 hits, weighted 0.6);
// tiles run in rounds of the resident grid.  Returns a huge cost for shapes
// that cannot run.
template <int MT, bool SECOND, bool GLU>
static double ffn_shape_cost(const FfnArgs& a, FfnShape sh, int cus) {
  long resident = 0;
  if (sh.fw == 8 && sh.wn == 2) resident = ffn_resident_if_ok<MT, 8, 2, SECOND, GLU>();
  if (sh.fw == 4 && sh.wn == 2) resident = ffn_resident_if_ok<MT, 4, 2, SECOND, GLU>();
  if (sh.fw == 3 && sh.wn == 2) resident = ffn_resident_if_ok<MT, 3, 2, SECOND, GLU>();
  if (sh.fw == 8 && sh.wn == 1) resident = ffn_resident_if_ok<MT, 8, 1, SECOND, GLU>();
  if (sh.fw == 6 && sh.wn == 1) resident = ffn_resident_if_ok<MT, 6, 1, SECOND, GLU>();
  if (sh.fw == 4 && sh.wn == 1) resident = ffn_resident_if_ok<MT, 4, 1, SECOND, GLU>();
  if (resident <= 0) return 1e300;
  const long cols = sh.fw * sh.wn * 32;
  const long n_ct = ffn_col_tiles(a, cols, GLU);
  const long n_tiles = n_ct * a.n_mchunks * a.n_experts;
  const long rounds = (n_tiles + resident - 1) / resident;
  const double tile = (double)(GLU ? 2 * a.Nout : a.Nout) / (double)n_ct + 0.6 * MT * 32;
  return (double)rounds * (double)resident / (double)cus * tile;
}

template <int MT, bool SECOND, bool GLU>
static void launch_ffn_bf16_mt(const FfnArgs& a, hipStream_t st) {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return 256;
    return n;
  }();
  FfnShape best = kFfnShapes[0];
  double best_cost = 1e301;
  for (const FfnShape& sh : kFfnShapes) {  // first of equal cost wins (fewer LDS reads)
#ifdef SFFN_FFN_ONLY_WN  // tuning builds: restrict the choice to one wave width
    if (sh.wn != SFFN_FFN_ONLY_WN) continue;
#endif
#ifdef SFFN_FFN2_ONLY_FW  // tuning builds: restrict the second GEMM to one block shape
    if (SECOND && (sh.fw != SFFN_FFN2_ONLY_FW || sh.wn != 2)) continue;
#endif
    const double c = ffn_shape_cost<MT, SECOND, GLU>(a, sh, cus);
    if (c < best_cost) {
      best_cost = c;
      best = sh;
    }
  }
  if (best.fw == 8 && best.wn == 2) launch_ffn_bf16_t<MT, 8, 2, SECOND, GLU>(a, st);
  else if (best.fw == 4 && best.wn == 2) launch_ffn_bf16_t<MT, 4, 2, SECOND, GLU>(a, st);
  else if (best.fw == 3 && best.wn == 2) launch_ffn_bf16_t<MT, 3, 2, SECOND, GLU>(a, st);
  else if (best.fw == 8) launch_ffn_bf16_t<MT, 8, 1, SECOND, GLU>(a, st);
  else if (best.fw == 6) launch_ffn_bf16_t<MT, 6, 1, SECOND, GLU>(a, st);
  else launch_ffn_bf16_t<MT, 4, 1, SECOND, GLU>(a, st);
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
// FFN2 with bit 1 of no_residual (top-2 routing): out is the expert buffer's
// rows, gate the per-row gate, and no residual is added.
template <bool SECOND>
__global__ void __launch_bounds__(256)
ffn_f32_kernel(const float* __restrict__ act, const float* __restrict__ W,
               const float* __restrict__ bias, const int* __restrict__ offset,
               const int* __restrict__ row2tok, const float* __restrict__ gate,
               const float* __restrict__ xres, float* __restrict__ out, int K, int Nout,
               int d_model, int no_residual, int glu) {
  const int e = blockIdx.z;
  const int r = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int n = blockIdx.x * 16 + (threadIdx.x & 15);
  const int rbeg = offset[e];
  if (r >= offset[e + 1] - rbeg || n >= Nout) return;
  const int row = rbeg + r;
  const int tok = row2tok[row];
  const float* a = SECOND ? act + (size_t)row * K : act + (size_t)tok * K;
  const int wm = (!SECOND && glu) ? 2 : 1;  // GEGLU: gate row n, linear row Nout + n
  const float* w = W + ((size_t)e * wm * Nout + n) * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(a[k], w[k], s);
  if (bias) s += bias[(size_t)e * wm * Nout + n];
  if (!SECOND && glu) {
    const float* v = w + (size_t)Nout * K;
    float l = 0.f;
    for (int k = 0; k < K; ++k) l = fmaf(a[k], v[k], l);
    if (bias) l += bias[(size_t)e * wm * Nout + Nout + n];
    out[(size_t)row * Nout + n] = gelu_f32(s) * l;
  } else if (!SECOND) {
    out[(size_t)row * Nout + n] = fmaxf(s, 0.f);
  } else if (no_residual & 2) {
    out[(size_t)row * d_model + n] = gate[row] * s;
  } else {
    const size_t o = (size_t)tok * d_model + n;
    float yv = gate[tok] * s;
    if (!(no_residual & 1)) yv += xres[o];
    out[o] = yv;
  }
}

template <bool SECOND, bool GLU = false>
static void launch_ffn_bf16(FfnArgs a, const Shape& s, hipStream_t st) {
  a.n_experts = s.N;
  a.max_rows = s.max_rows;
  a.T = s.T;
  a.d_model = s.d;
  // Experts of 9 or 10 row tiles (capacity 257 .. 320 rows: Switch-Large-like,
  // top-2 Switch-Base-like) as one tile of two row parts: 8 waves, 5 row tiles
  // each, 128 columns, each weight byte streamed once (weight rows on the
  // 128-byte line grid, ReLU experts).
  // The grid is one block per CU (LDS), so the split tiles run only where
  // they make at least four rounds of the grid: with fewer, the last round
  // leaves CUs idle and two row chunks of wider tiles balance better.
  const int tiles = (s.C + 31) / 32;
#ifndef SFFN_FFN_NO_SPLIT  // tuning builds: the two-chunk path only
  if constexpr (!GLU) {
    if ((tiles == 9 || tiles == 10) && (a.K * 2) % 128 == 0) {
      a.n_mchunks = 1;
      const long n_split = ffn_col_tiles(a, 128, false) * a.n_experts;
      const long resident = ffn_resident_blocks<5, 8, 1, SECOND, false, kCpolNonTemporal, 2>();
      if (n_split >= 4 * resident) {
        launch_ffn_pol<5, 8, 1, SECOND, kCpolNonTemporal, false, 2>(a, st);
        return;
      }
    }
  }
#endif
  const int mt = rows_tiles(s.C);
  a.n_mchunks = (s.C + mt * 32 - 1) / (mt * 32);
  a.n_experts = s.N;
  a.max_rows = s.max_rows;
  a.T = s.T;
  a.d_model = s.d;
  switch (mt) {
    case 1: launch_ffn_bf16_mt<1, SECOND, GLU>(a, st); break;
    case 2: launch_ffn_bf16_mt<2, SECOND, GLU>(a, st); break;
    case 3: launch_ffn_bf16_mt<3, SECOND, GLU>(a, st); break;
    case 4: launch_ffn_bf16_mt<4, SECOND, GLU>(a, st); break;
    case 5: launch_ffn_bf16_mt<5, SECOND, GLU>(a, st); break;
    case 6: launch_ffn_bf16_mt<6, SECOND, GLU>(a, st); break;
    case 7: launch_ffn_bf16_mt<7, SECOND, GLU>(a, st); break;
    default: launch_ffn_bf16_mt<8, SECOND, GLU>(a, st); break;
  }
}

hipError_t launch_ffn1(const Shape& s, const Inputs& in, const Workspace& ws, hipStream_t st) {
  if (s.C <= 0) return hipSuccess;
  if (s.dtype == SFFN_FP32) {
    const dim3 grid((unsigned)((s.F + 15) / 16), (unsigned)((s.C + 15) / 16), (unsigned)s.N);
    hipLaunchKernelGGL(ffn_f32_kernel<false>, grid, dim3(256), 0, st, (const float*)in.x,
                       (const float*)in.W1, (const float*)in.b1, ws.offset, ws.row2tok,
                       (const float*)nullptr, (const float*)nullptr, (float*)ws.H, s.d, s.F, s.d,
                       0, s.glu);
    return hipGetLastError();
  }
  FfnArgs a{};
  a.act = (const uint16_t*)in.x;
  a.act_bytes = (uint32_t)((size_t)s.T * s.d * 2);
  a.W = (const uint16_t*)in.W1;
  a.bias = (const uint16_t*)in.b1;
  a.offset = ws.offset;
  a.row2tok = ws.row2tok;
  a.out = (uint16_t*)ws.H;
  a.out_bytes = (uint32_t)((size_t)s.max_rows * s.F * 2);
  a.K = s.d;
  a.Nout = s.F;
  if (s.glu) launch_ffn_bf16<false, true>(a, s, st);
  else launch_ffn_bf16<false>(a, s, st);
  return hipGetLastError();
}

hipError_t launch_ffn2(const Shape& s, const Inputs& in, const Workspace& ws, const Outputs& out,
                       bool no_residual, hipStream_t st) {
  if (s.C <= 0) return hipSuccess;
  if (s.dtype == SFFN_FP32) {
    const dim3 grid((unsigned)((s.d + 15) / 16), (unsigned)((s.C + 15) / 16), (unsigned)s.N);
    if (s.k == 2)
      hipLaunchKernelGGL(ffn_f32_kernel<true>, grid, dim3(256), 0, st, (const float*)ws.H,
                         (const float*)in.W2, (const float*)in.b2, ws.offset, ws.row2tok,
                         ws.rowgate, (const float*)nullptr, (float*)ws.Y2, s.F, s.d, s.d, 3, 0);
    else
      hipLaunchKernelGGL(ffn_f32_kernel<true>, grid, dim3(256), 0, st, (const float*)ws.H,
                         (const float*)in.W2, (const float*)in.b2, ws.offset, ws.row2tok,
                         out.gate, (const float*)in.x, (float*)out.y, s.F, s.d, s.d,
                         no_residual ? 1 : 0, 0);
    return hipGetLastError();
  }
  FfnArgs a{};
  a.act = (const uint16_t*)ws.H;
  a.act_bytes = (uint32_t)((size_t)s.max_rows * s.F * 2);
  a.W = (const uint16_t*)in.W2;
  a.bias = (const uint16_t*)in.b2;
  a.offset = ws.offset;
  a.row2tok = ws.row2tok;
  a.rowgate = ws.rowgate;
  a.xres = (const uint16_t*)in.x;
  a.out = (uint16_t*)out.y;
  a.out_bytes = (uint32_t)((size_t)s.T * s.d * 2);
  a.K = s.F;
  a.Nout = s.d;
  a.no_residual = no_residual ? 1 : 0;
  if (s.k == 2) {  // gate-scaled rows of the expert buffer; the combine adds them up
    a.out = (uint16_t*)ws.Y2;
    a.out_bytes = (uint32_t)((size_t)s.max_rows * s.d * 2);
    a.no_residual = 3;
  }
  launch_ffn_bf16<true>(a, s, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-2 combine: y_t = x_t + Y2[row of choice 0] + Y2[row of choice 1], over
// the accepted choices, summed in fp32 in that order and rounded once (Y2
// holds gate-scaled expert outputs).  One wave per token row; bf16: 8
// elements per lane and step (16-byte accesses), fp32: one.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ void __launch_bounds__(256)
combine_top2_kernel(const void* __restrict__ xv, const void* __restrict__ Y2v,
                    const int32_t* __restrict__ expert_idx, const int32_t* __restrict__ slot,
                    const int* __restrict__ offset, int T, int d, int no_residual,
                    void* __restrict__ yv) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  int row[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int sl = slot[2 * (size_t)t + c];
    row[c] = sl >= 0 ? offset[expert_idx[2 * (size_t)t + c]] + sl : -1;
  }
  if constexpr (BF16) {
    const uint16_t* x = (const uint16_t*)xv + (size_t)t * d;
    const uint16_t* Y2 = (const uint16_t*)Y2v;
    uint16_t* y = (uint16_t*)yv + (size_t)t * d;
    for (int i = lane * 8; i < d; i += 64 * 8) {  // d % 8 == 0
      float acc[8];
      const u32x4 xq = no_residual ? u32x4{0, 0, 0, 0} : load16(x + i);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = bf16_bits_to_f32(j & 1 ? xq[j / 2] >> 16 : xq[j / 2] & 0xffffu);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (row[c] < 0) continue;
        const u32x4 v = load16(Y2 + (size_t)row[c] * d + i);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += bf16_bits_to_f32(j & 1 ? v[j / 2] >> 16 : v[j / 2] & 0xffffu);
      }
      store16(y + i, u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                           pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])});
    }
  } else {
    const float* x = (const float*)xv + (size_t)t * d;
    const float* Y2 = (const float*)Y2v;
    float* y = (float*)yv + (size_t)t * d;
    for (int i = lane; i < d; i += 64) {
      float acc = no_residual ? 0.f : x[i];
#pragma unroll
      for (int c = 0; c < 2; ++c)
        if (row[c] >= 0) acc += Y2[(size_t)row[c] * d + i];
      y[i] = acc;
    }
  }
}

hipError_t launch_combine(const Shape& s, const Inputs& in, const Workspace& ws,
                          const Outputs& out, bool no_residual, hipStream_t st) {
  const dim3 grid((unsigned)((s.T + 3) / 4)), block(256);
  if (s.dtype == SFFN_BF16)
    hipLaunchKernelGGL(combine_top2_kernel<true>, grid, block, 0, st, in.x, ws.Y2, out.expert_idx,
                       out.slot, ws.offset, s.T, s.d, no_residual ? 1 : 0, out.y);
  else
    hipLaunchKernelGGL(combine_top2_kernel<false>, grid, block, 0, st, in.x, ws.Y2, out.expert_idx,
                       out.slot, ws.offset, s.T, s.d, no_residual ? 1 : 0, out.y);
  return hipGetLastError();
}

}  // namespace sffn
