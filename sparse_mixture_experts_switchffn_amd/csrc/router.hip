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

// ---------------------------------------------------------------------------
// Router planes: the exact three-way bf16 split of Wr (w = hi + mid + lo, each
// term the round-to-nearest of what remains), written in matrix-core fragment
// order so that a wave loads each 32x16 operand fragment as one contiguous
// 1 KB block:  planes[ks][p][m][q][lane][8] = plane p of
//   Wr[32 m + lane%32][32 ks + 16 (lane/32) + 8 q + 0..7],
// zero outside [0, N) x [0, d).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
router_planes_kernel(const float* __restrict__ Wr, int d, int N, int MT, int nks,
                     uint16_t* __restrict__ planes) {
  const int g = blockIdx.x * 256 + threadIdx.x;   // one (ks, m, q, lane) group of 8 weights
  const int total = nks * MT * 2 * 64;
  if (g >= total) return;
  const int lane = g & 63;
  const int q = (g >> 6) & 1;
  const int m = (g >> 7) % MT;
  const int ks = (g >> 7) / MT;
  const int row = 32 * m + (lane & 31);
  const int k0 = 32 * ks + 16 * (lane >> 5) + 8 * q;
  uint32_t hi[8], mid[8], lo[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float w = (row < N && k0 + c < d) ? Wr[(size_t)row * d + k0 + c] : 0.f;
    hi[c] = f32_to_bf16_bits(w);
    const float r1 = w - bf16_bits_to_f32(hi[c]);
    mid[c] = f32_to_bf16_bits(r1);
    lo[c] = f32_to_bf16_bits(r1 - bf16_bits_to_f32(mid[c]));
  }
  auto pack = [](const uint32_t* v) {
    return u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
  };
  const size_t frag = 64 * 8;  // bf16 per fragment
  uint16_t* base = planes + ((((size_t)ks * 3) * MT + m) * 2 + q) * frag + (size_t)lane * 8;
  store16(base, pack(hi));
  store16(base + (size_t)MT * 2 * frag, pack(mid));
  store16(base + (size_t)2 * MT * 2 * frag, pack(lo));
}

// ---------------------------------------------------------------------------
// Router with softmax, top-1 and the per-block statistics fused into the GEMM
// epilogue, for N <= 128 experts.  A block of four waves routes one routing
// block of kRouteTokens (32) tokens and computes all N logits, so the logits
// never leave the chip.  The reduction over k is split across the waves (wave w
// takes k-steps w, w+4, ...), which spreads the token stream over four times as
// many blocks; the four partial logit tiles are summed in LDS in wave order.
//
// GEMM: rows = experts, columns = tokens (four lanes per 64-byte row segment,
// re-laid out through a private LDS slot into the operand layout).  32 k per
// step, operands fetched 2-3 steps ahead.  The expert operand: for up to 64
// experts (MT <= 2) straight from fp32 Wr (16-byte aligned rows, d % 8 == 0):
// each lane loads the 16 consecutive weights of its row and k-half and splits
// them into the three bf16 planes in registers, one hardware conversion per
// pair and plane, so no planes pass runs first and Wr costs 4 bytes a weight
// against the planes' 6.  For more experts the split's VALU work outweighs
// that, and the block reads the router planes (one coalesced 1 KB fragment
// load per plane and tile).
// Epilogue (all four waves): the partial logit tiles meet in LDS and are
// summed in wave order (and the fp32 logits are written to the workspace, where
// the backward pass reads them); eight threads per token then take
//   m = max z, e = lowest index with z = m, S = sum exp(z - m), gate = 1/S,
// each over an eighth of the experts, combined by three cross-lane steps;
// finally one thread per expert sums p over the block's tokens in token order
// (ppart[b, i]) and counts the tokens whose top-1 is i (cnt[b, i]), and one
// thread per token counts the earlier tokens with its top-1 (lrank[t]).
// MODE 1 (top-2) also takes the second choice (the largest other logit, lowest
// index on ties) with gate exp(z2 - m)/S, writes both choices [T, 2], counts
// memberships in cnt and first choices in cnt1, and ranks each choice among
// the block's earlier choices of the same expert (lrank[2t + c]), as the
// staged top-2 route does.  MODE 2 (rerouting) writes both choices and gates
// [T, 2] to the workspace and counts and ranks the first choices only.
// ---------------------------------------------------------------------------
constexpr int FR_BK = 32;
constexpr int FR_LD = FR_BK + 8;  // bf16 per LDS row of the token slot (80 B)
constexpr int FR_KSPLIT = 4;      // waves per block, each a quarter of the k-steps
static_assert(kRouteTokens == 32, "one block routes 32 tokens");

template <int MT, int MODE>
__global__ void __launch_bounds__(64 * FR_KSPLIT)
router_fused_kernel(const uint16_t* __restrict__ x, const float* __restrict__ Wr,
                    const uint16_t* __restrict__ planes, uint32_t planes_bytes, int T, int d, int N,
                    int32_t* __restrict__ expert_idx,
                    float* __restrict__ gate, float* __restrict__ ppart, int* __restrict__ cnt,
                    int* __restrict__ lrank, int* __restrict__ cnt1,
                    float* __restrict__ logits) {
  constexpr int NE = MT * 32;       // expert rows of the tile
  constexpr int PST = 33;           // floats per staged expert row (32 tokens + 1: banks)
  constexpr int EPT = NE / 8;       // experts per thread in the softmax (8 threads a token)
  __shared__ __attribute__((aligned(16))) uint16_t Xs[FR_KSPLIT][32 * FR_LD];
  __shared__ float Ps[FR_KSPLIT][NE * PST];  // partial logits; then Ps[0] holds p
  __shared__ int ids_s[32];
  __shared__ int ids2_s[MODE != 0 ? 32 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const int t0 = b * kRouteTokens;
  const int khalf = lane >> 5;

  constexpr bool WF = MT <= 2;  // Wr split in registers, else the planes
  const __amdgpu_buffer_rsrc_t rw_src =
      WF ? make_rsrc(Wr, (uint32_t)((size_t)N * d * 4)) : make_rsrc(planes, planes_bytes);
  const __amdgpu_buffer_rsrc_t rx_src = make_rsrc(x, (uint32_t)((size_t)T * d * 2));
  // Byte offset of Wr[32 m + lane%32][16 khalf] (kOob past the experts).
  uint32_t w_row[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int row = 32 * m + (lane & 31);
    w_row[m] = row < N ? ((uint32_t)row * (uint32_t)d + 16u * (uint32_t)khalf) * 4u : kOob;
  }
  uint32_t x_off[2];
  bool x_ok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + i * 16 + (lane >> 2);
    x_ok[i] = t < T;
    x_off[i] = ((uint32_t)(x_ok[i] ? t : 0) * (uint32_t)d + (uint32_t)(lane & 3) * 8u) * 2u;
  }
  constexpr int RFP = MT <= 2 ? 3 : 2;  // k-steps in flight (register budget)
  const int nks = (d + FR_BK - 1) / FR_BK;
  const int nmine = (nks + FR_KSPLIT - 1) / FR_KSPLIT;      // this wave's steps, padded
  const int nk = (nmine + RFP - 1) / RFP * RFP;
  constexpr int NA = WF ? MT * 4 : 3 * MT * 2;  // 16-byte expert-operand loads a step
  const uint32_t step_bytes = 3u * MT * 2u * 1024u;  // planes of one k-step

  // Local step j of this wave is global k-step wave + 4 j.
  auto load_a = [&](u32x4 (&ra)[NA], int j) {
    const int ks = wave + FR_KSPLIT * j;
    if constexpr (WF) {
      // Chunk c holds k = 32 ks + 16 khalf + 4 c + 0..3; d % 4 == 0, so a chunk is
      // wholly inside or wholly past the row.
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool kin = ks * FR_BK + 16 * khalf + 4 * c < d;
          ra[m * 4 + c] = buffer_load16(
              rw_src, kin ? w_row[m] + (uint32_t)ks * (FR_BK * 4) + 16u * c : kOob);
        }
    } else {
      const bool kin = ks < nks;
#pragma unroll
      for (int f = 0; f < 3 * MT * 2; ++f)
        ra[f] = buffer_load16(rw_src, kin ? (uint32_t)ks * step_bytes + (uint32_t)f * 1024u +
                                                (uint32_t)lane * 16u : kOob);
    }
  };
  auto load_x = [&](u32x4 (&rx)[2], int j) {
    const int ks = wave + FR_KSPLIT * j;
    const bool kin = ks * FR_BK + (lane & 3) * 8 < d;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      rx[i] = buffer_load16(rx_src, (x_ok[i] && kin) ? x_off[i] + (uint32_t)ks * (FR_BK * 2) : kOob);
  };
  uint16_t* xslot = &Xs[wave][0];
  f32x16 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x16{};
  auto compute = [&](const u32x4 (&ra)[NA], const u32x4 (&rx)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) store16(xslot + (i * 16 + (lane >> 2)) * FR_LD + (lane & 3) * 8, rx[i]);
    const uint16_t* xbase = xslot + (lane & 31) * FR_LD + khalf * 16;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const bf16x8 bv = as_bf16x8(load16(xbase + q * 8));
      u32x4 pl[3][MT];  // the hi, mid and lo planes of this lane's 8 weights per tile
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if constexpr (WF) {
          // w = hi + mid + lo exactly: each plane is the round-to-nearest-even bf16 of
          // what the earlier planes leave, and each remainder is exact in fp32.
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x4& ch = ra[(m * 4 + 2 * q + (j >> 1)) % NA];
            float w0 = __uint_as_float(ch[(2 * j) & 3]), w1 = __uint_as_float(ch[(2 * j + 1) & 3]);
#pragma unroll
            for (int p = 0; p < 3; ++p) {
              const uint32_t h = pack_bf16x2(w0, w1);
              pl[p][m][j] = h;
              w0 -= __uint_as_float(h << 16);
              w1 -= __uint_as_float(h & 0xffff0000u);
            }
          }
        } else {
#pragma unroll
          for (int p = 0; p < 3; ++p) pl[p][m] = ra[(p * MT + m) * 2 + q];
        }
      }
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = mfma_32x32x16(as_bf16x8(pl[p][m]), bv, acc[m]);
    }
  };

  u32x4 ra[RFP][NA];
  u32x4 rx[RFP][2];
#pragma unroll
  for (int st = 0; st < RFP; ++st) {
    load_a(ra[st], st);
    load_x(rx[st], st);
    __builtin_amdgcn_sched_barrier(0);  // keep the prologue in step order
  }
  for (int js = 0; js < nk; js += RFP) {
#pragma unroll
    for (int j = 0; j < RFP; ++j) {
      compute(ra[j], rx[j]);
      load_a(ra[j], js + j + RFP);
      load_x(rx[j], js + j + RFP);
    }
  }

  // ---- partial logit tiles to LDS: Ps[w][e][t] ----
  const int tl = lane & 31;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      Ps[wave][(m * 32 + (v >> 2) * 8 + khalf * 4 + (v & 3)) * PST + tl] = acc[m][v];
  lds_barrier();

  // ---- softmax, top-1 and gate: token tt, experts g + 8 i ----
  const int tt = threadIdx.x >> 3;
  const int g = threadIdx.x & 7;
  const int t = t0 + tt;
  const bool live = t < T;
  float z[EPT];
  float mx = -INFINITY;
  int arg = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = g + 8 * i;
    const int o = e * PST + tt;
    z[i] = ((Ps[0][o] + Ps[1][o]) + Ps[2][o]) + Ps[3][o];  // waves in order
    if (live && e < N) logits[(size_t)t * N + e] = z[i];  // kept for the backward pass
    if (e < N && route_before(z[i], e, mx, arg)) {
      mx = z[i];
      arg = e;
    }
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    const float om = __shfl_xor(mx, off);
    const int oa = __shfl_xor(arg, off);
    if (route_before(om, oa, mx, arg)) {
      mx = om;
      arg = oa;
    }
  }
  float mx2 = -INFINITY;
  int arg2 = 0x7fffffff;
  if constexpr (MODE != 0) {  // second choice: the largest other logit, lowest index on ties
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = g + 8 * i;
      if (e < N && e != arg && route_before(z[i], e, mx2, arg2)) {
        mx2 = z[i];
        arg2 = e;
      }
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      const float om = __shfl_xor(mx2, off);
      const int oa = __shfl_xor(arg2, off);
      if (route_before(om, oa, mx2, arg2)) {
        mx2 = om;
        arg2 = oa;
      }
    }
  }
  float ssum = 0.f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    z[i] = (g + 8 * i) < N ? expf(z[i] - mx) : 0.f;
    ssum += z[i];
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) ssum += __shfl_xor(ssum, off);
  const float inv = 1.0f / ssum;
  if (g == 0) {
    ids_s[tt] = live ? arg : -1;
    if constexpr (MODE != 0) ids2_s[tt] = live ? arg2 : -1;
    if (live) {
      if constexpr (MODE == 0) {
        expert_idx[t] = arg;
        gate[t] = inv;
      } else {
        expert_idx[2 * (size_t)t] = arg;
        expert_idx[2 * (size_t)t + 1] = arg2;
        gate[2 * (size_t)t] = inv;
        gate[2 * (size_t)t + 1] = expf(mx2 - mx) * inv;
      }
    }
  }
  lds_barrier();  // every wave is past its reads of the partial tiles
#pragma unroll
  for (int i = 0; i < EPT; ++i) Ps[0][(g + 8 * i) * PST + tt] = live ? z[i] * inv : 0.f;
  lds_barrier();

  // ---- per expert: block sum of p (token order) and top-1 count ----
  for (int e = threadIdx.x; e < N; e += 64 * FR_KSPLIT) {
    float ps = 0.f;
    int c = 0, c2 = 0;
    for (int j = 0; j < 32; ++j) {
      ps += Ps[0][e * PST + j];
      c += ids_s[j] == e;
      if constexpr (MODE == 1) c2 += ids2_s[j] == e;
    }
    ppart[(size_t)b * N + e] = ps;
    cnt[(size_t)b * N + e] = c + c2;  // top-2: memberships
    if constexpr (MODE == 1) cnt1[(size_t)b * N + e] = c;
  }
  // ---- per token: earlier tokens of the block with the same top-1 ----
  if constexpr (MODE == 1) {  // each choice among the earlier choices of its expert
    const int j0 = threadIdx.x >> 1, c = threadIdx.x & 1;
    if (threadIdx.x < 64 && t0 + j0 < T) {
      const int me = c ? ids2_s[j0] : ids_s[j0];
      int r = 0;
      for (int j = 0; j < j0; ++j) r += (ids_s[j] == me) + (ids2_s[j] == me);
      lrank[2 * (size_t)(t0 + j0) + c] = r;
    }
  } else if (threadIdx.x < 32 && t0 + (int)threadIdx.x < T) {
    const int me = ids_s[threadIdx.x];
    int r = 0;
    for (int j = 0; j < (int)threadIdx.x; ++j) r += ids_s[j] == me;
    lrank[(MODE == 2 ? 2 : 1) * (size_t)(t0 + threadIdx.x)] = r;
  }
}

// ---------------------------------------------------------------------------
// Logits for many experts (N > 128, N % 4 == 0), bf16 token states: the same
// exact three-plane product, tiled for the matrix cores.
//
// A block of 8 waves computes 128 experts x 128 TN tokens; wave w takes
// expert half w%2 (two 32-expert tiles) and token quarter w/2 (TN 32-token
// tiles), so each 16-k sub-step is 6 TN matrix-core ops on 6 plane and TN
// token fragments (TN = 3 for many experts, 1 for 128 experts, where fewer
// tokens per block keep every CU busy).  Both operands go from memory straight into LDS rings with
// buffer loads that write LDS, 32 k per step:
//   * planes (fragment order, from router_planes_kernel): 24 KB a step, one
//     1 KB fragment per instruction; each lane reads back the 16 bytes it
//     loaded, so the reads need no swizzle.
//   * token rows: 128 TN x 64 B a step, 16 rows per instruction; the four 16-byte
//     chunks of row r are stored XOR-swizzled by (r/4)%4 so the operand reads
//     (32 rows, one chunk) spread over the banks.
// Three ring slots each: step k computes, then issues the loads of step k+2,
// so at its start everything but the loads of step k+1 must have landed: a
// fixed wait, then a barrier that completes LDS accesses only (the loads are
// issued after the step's LDS reads, which keeps the compiler from waiting
// for them there).
// Block order: tiles are grouped in runs of 8 token tiles x 4 expert groups
// (expert group fastest, XCD-contiguous ids), so the blocks running together
// on one XCD share both their token rows and their planes in its L2.
// ---------------------------------------------------------------------------
constexpr int RL_WAVES = 8;
constexpr int RL_EXP = 128;                   // experts per block
constexpr int RL_PSLOT = 24 * 1024;           // plane bytes per step: 3 planes x 4 tiles x 2 q
constexpr int RL_NB = 3;                      // ring slots (two steps in flight)
constexpr int RL_PLD = 24 / RL_WAVES;         // plane loads per wave per step

template <int TN>
__global__ void __launch_bounds__(RL_WAVES * 64)
router_logits_mfma_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ planes,
                          uint32_t planes_bytes, int T, int d, int N, int MTp, int nks,
                          float* __restrict__ logits) {
  constexpr int RL_TOK = 128 * TN;                // tokens per block
  constexpr int RL_TN = TN;                       // 32-token tiles per wave
  constexpr int RL_XSLOT = RL_TOK * 64;           // token bytes per step
  constexpr int RL_XLD = RL_TOK / 16 / RL_WAVES;  // token loads per wave per step
  // One LDS object for both rings (the compiler then leaves the waits for the
  // loads that write it to the explicit ones below).
  __shared__ __attribute__((aligned(1024))) char ring[RL_NB * (RL_PSLOT + RL_XSLOT)];
  char* const pring = ring;
  char* const xring = ring + RL_NB * RL_PSLOT;
  const int n_eg = MTp / 4;
  const int n_tt = (T + RL_TOK - 1) / RL_TOK;
  const int egc = (n_eg % 4 == 0) ? 4 : (n_eg % 2 == 0 ? 2 : 1);  // expert groups per run
  int tt, eg;
  {
    const int tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    const int row = tile / (8 * n_eg), rem = tile % (8 * n_eg);
    const int rows = min(8, n_tt - row * 8);
    const int chunk = rem / (rows * egc), inner = rem % (rows * egc);
    tt = row * 8 + inner / egc;
    eg = chunk * egc + inner % egc;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int khalf = lane >> 5;
  const int t0 = tt * RL_TOK;

  const __amdgpu_buffer_rsrc_t rp = make_rsrc(planes, planes_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)T * d * 2));
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(logits, (uint32_t)((size_t)T * N * 4));

  // Plane loads: fragment f = wave*PLD + i of a step is (plane f/8, tile
  // (f/2)%4, q f%2) and sits at f KB of the slot.
  const uint32_t pstep = (uint32_t)(3 * MTp * 2) * 1024u;
  uint32_t p_off[RL_PLD];
#pragma unroll
  for (int i = 0; i < RL_PLD; ++i) {
    const int f = wave * RL_PLD + i;
    p_off[i] = (uint32_t)(((f / 8) * MTp + 4 * eg + (f / 2) % 4) * 2 + f % 2) * 1024u + (uint32_t)lane * 16u;
  }
  // Token loads: instruction j = wave*XLD + i of a step covers rows 16 j ..
  // 16 j + 15; lane l fills row 16 j + l/4, stored chunk l%4, which holds
  // logical chunk (l%4) ^ ((row/4)%4) = k 8c .. 8c+7 of the step.  Rows past
  // T are pushed past the end of x (offsets stay below 2^32).
  uint32_t x_row[RL_XLD];
  int x_k[RL_XLD];
#pragma unroll
  for (int i = 0; i < RL_XLD; ++i) {
    const int r = 16 * (wave * RL_XLD + i) + (lane >> 2);
    const int t = t0 + r;
    x_row[i] = t < T ? (uint32_t)t * (uint32_t)d * 2u : kOob;
    x_k[i] = 8 * ((lane & 3) ^ ((r >> 2) & 3));
  }
  auto dma_p = [&](int k) {
    char* slot = pring + (k % RL_NB) * RL_PSLOT;
#pragma unroll
    for (int i = 0; i < RL_PLD; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rp, (__attribute__((address_space(3))) void*)(slot + (wave * RL_PLD + i) * 1024), 16,
          (int)((uint32_t)k * pstep + p_off[i]), 0, 0, 0);
  };
  auto dma_x = [&](int k) {
    char* slot = xring + (k % RL_NB) * RL_XSLOT;
#pragma unroll
    for (int i = 0; i < RL_XLD; ++i) {
      const int kk = 32 * k + x_k[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(slot + (wave * RL_XLD + i) * 1024), 16,
          (int)(kk < d ? x_row[i] + (uint32_t)kk * 2u : kOob), 0, 0, 0);
    }
  };

  // Operand reads: planes of tiles 2 (w%2) + m, tokens of tiles 3 (w/2) + n;
  // sub-step q (k = 16 khalf + 8 q + 0..7 of the step in lane half khalf).
  const int we = wave & 1, wt = wave >> 1;
  const uint32_t p_rd = (uint32_t)lane * 16u;
  const uint32_t x_rd = (uint32_t)(wt * RL_TN * 32 + (lane & 31)) * 64u;
  const int xsw = (lane >> 2) & 3;  // (row/4)%4 of every row this lane reads
  f32x16 acc[2][RL_TN];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < RL_TN; ++n) acc[m][n] = f32x16{};
  auto compute = [&](int k) {
    const char* ps = pring + (k % RL_NB) * RL_PSLOT + p_rd;
    const char* xs = xring + (k % RL_NB) * RL_XSLOT + x_rd;
    bf16x8 pf[3][2], xf[RL_TN];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          pf[p][m] = as_bf16x8(load16(ps + ((p * 4 + 2 * we + m) * 2 + q) * 1024));
      const int xc = ((2 * khalf + q) ^ xsw) * 16;
#pragma unroll
      for (int n = 0; n < RL_TN; ++n) xf[n] = as_bf16x8(load16(xs + n * 32 * 64 + xc));
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < RL_TN; ++n) acc[m][n] = mfma_32x32x16(pf[p][m], xf[n], acc[m][n]);
    }
  };

  dma_x(0);
  dma_p(0);
  dma_x(1);
  dma_p(1);
  for (int k = 0; k < nks; ++k) {
    wait_vmcnt<RL_XLD + RL_PLD>();  // all but the loads of step k+1 have landed
    dma_barrier();                  // everyone's; the slots of step k-1 are free
    compute(k);
    dma_x(k + 2);  // zero past the end of d
    dma_p(k + 2);
  }

  // Logits: lane holds, for tiles (m, n), token t0 + 32 TN (w/2) + 32 n + lane%32
  // and experts 128 eg + 64 (w%2) + 32 m + 8 g + 4 khalf + 0..3 in values 4g..4g+3.
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < RL_TN; ++n) {
      const int t = t0 + wt * RL_TN * 32 + 32 * n + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = eg * RL_EXP + we * 64 + 32 * m + 8 * g + 4 * khalf;
        const f32x4 v = f32x4{acc[m][n][4 * g], acc[m][n][4 * g + 1], acc[m][n][4 * g + 2],
                              acc[m][n][4 * g + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, v), rz,
            (int)(((t < T) & (e < N)) ? ((uint32_t)t * (uint32_t)N + (uint32_t)e) * 4u : kOob), 0, 0);
      }
    }
  // The last ring loads (zeros past the end of d) still write LDS.
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
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

// Many-expert logits on the matrix cores: planes for 32-k steps and 128-expert
// groups (zero-padded), offsets of the staged logits and of the planes below
// 2^31 so that the range-checked placeholder offset stays out of range.
static size_t tiled_planes_bytes(const Shape& s) {
  const size_t nks = (size_t)(s.d + 31) / 32;
  const size_t mtp = 4 * (size_t)((s.N + RL_EXP - 1) / RL_EXP);
  return nks * 3 * mtp * 2 * 1024;
}

static bool logits_fit_offsets(const Shape& s) {
  return (size_t)s.T * (size_t)s.N * 4 < ((size_t)1 << 31);
}

// The tiled router (logits staged in HBM, then the softmax pass) for many
// experts, and for 128-expert-scale layers with enough tokens to give every
// CU a 128-token block, where the fused router would fetch the planes once
// per 32 tokens.
static bool router_is_tiled(const Shape& s) {
  return s.dtype == SFFN_BF16 && s.N % 4 == 0 && logits_fit_offsets(s) &&
         tiled_planes_bytes(s) < ((size_t)1 << 31) - ((size_t)8 << 20) &&
         (s.N > 128 || (s.N > 64 && s.T >= 256 * 128));
}

// The forward forms (top-1, top-2, rerouting) all have a fused epilogue.
bool router_is_fused(const Shape& s) {
  return s.dtype == SFFN_BF16 && s.N <= 128 && !router_is_tiled(s);
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
  if (router_is_fused(s)) return hipSuccess;  // done by launch_softmax_route
  const uint16_t* x = (const uint16_t*)in.x;
  if (router_is_tiled(s)) {
    const int mtp = 4 * ((s.N + RL_EXP - 1) / RL_EXP);
    const int nks = (s.d + 31) / 32;
    const int groups = nks * mtp * 2 * 64;
    hipLaunchKernelGGL(router_planes_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                       st, in.Wr, s.d, s.N, mtp, nks, ws.planes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const uint32_t pbytes = (uint32_t)tiled_planes_bytes(s);
    if (s.N > 128) {
      const int n_tt = (s.T + 383) / 384;
      hipLaunchKernelGGL(router_logits_mfma_kernel<3>, dim3((unsigned)(n_tt * (mtp / 4))),
                         dim3(RL_WAVES * 64), 0, st, x, ws.planes, pbytes, s.T, s.d, s.N, mtp,
                         nks, ws.logits);
    } else {
      const int n_tt = (s.T + 127) / 128;
      hipLaunchKernelGGL(router_logits_mfma_kernel<1>, dim3((unsigned)(n_tt * (mtp / 4))),
                         dim3(RL_WAVES * 64), 0, st, x, ws.planes, pbytes, s.T, s.d, s.N, mtp,
                         nks, ws.logits);
    }
    return hipGetLastError();
  }
  const int ttiles = (s.T + RW_WAVES * 32 - 1) / (RW_WAVES * 32);
  const int rm = s.N >= 128 ? 4 : (s.N + 31) / 32;
  const int etiles = (s.N + rm * 32 - 1) / (rm * 32);
  const dim3 grid((unsigned)(ttiles * etiles));
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

  // Each wave takes every 4th token of the block; up to N = 2048 the next
  // token's logits are fetched while the current one is reduced.
  constexpr bool kPrefetch = NPL <= 32;
  float vn[NPL];
  auto fetch = [&](int j, float (&v)[NPL]) {
    const int t = tb + j;
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int i = lane + 64 * q;
      v[q] = (t < T && i < N) ? logits[(size_t)t * N + i] : -INFINITY;
    }
  };
  if (kPrefetch) fetch(wave, vn);
  for (int j = wave; j < kRouteTokens; j += WAVES) {
    const int t = tb + j;
    float v[NPL];
    if (kPrefetch) {
#pragma unroll
      for (int q = 0; q < NPL; ++q) v[q] = vn[q];
      if (j + WAVES < kRouteTokens) fetch(j + WAVES, vn);
    } else {
      fetch(j, v);
    }
    if (t >= T) {
      if (lane == 0) eid_s[j] = -1;
      continue;
    }
    float m = -INFINITY;
    int arg = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int i = lane + 64 * q;
      if (i < N && route_before(v[q], i, m, arg)) {
        m = v[q];
        arg = i;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float om = __shfl_xor(m, off);
      const int oa = __shfl_xor(arg, off);
      if (route_before(om, oa, m, arg)) {
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

// ---------------------------------------------------------------------------
// Top-2 routing over staged logits.  One block per routing block of
// kRouteTokens tokens, each wave every 4th token; lane l holds experts
// l, l+64, ... (NPL of them).
//   m = max z, e0 = lowest index with z = m, e1 = lowest index of the largest
//   logit other than e0 (fp32), S = sum exp(z - m): gate0 = 1/S = p[t, e0],
//   gate1 = exp(z[e1] - m)/S = p[t, e1] (raw gates);
//   ppart[b, i] = sum of p over the block, cnt[b, i] = tokens of the block
//   holding i among their two choices, cnt1[b, i] = tokens whose top-1 is i,
//   lrank[2t + c] = earlier tokens of the block holding e_c among their choices.
// With first_only (rerouting) cnt and lrank[2t] count the first choices alone,
// cnt1 is not written and lrank[2t + 1] is left to the overflow count, which
// needs the first stage's global ranks.
// Sums run in fixed orders, so results are bitwise reproducible.
// ---------------------------------------------------------------------------
template <int NPL>
__global__ void __launch_bounds__(256)
softmax_route_top2_kernel(const float* __restrict__ logits, int T, int N,
                          int32_t* __restrict__ expert_idx, float* __restrict__ gate,
                          float* __restrict__ ppart, int* __restrict__ cnt,
                          int* __restrict__ cnt1, int* __restrict__ lrank, int first_only) {
  constexpr int WAVES = 4;
  __shared__ float pacc[WAVES][NPL * 64];
  __shared__ int eid_s[kRouteTokens][2];
  __shared__ int cnt_s[NPL * 64], cnt1_s[NPL * 64];

  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tb = b * kRouteTokens;

  for (int i = threadIdx.x; i < NPL * 64; i += 256) {
    cnt_s[i] = 0;
    cnt1_s[i] = 0;
  }
  float acc[NPL];
#pragma unroll
  for (int q = 0; q < NPL; ++q) acc[q] = 0.f;

  // Lane-local then cross-lane maximum with the lowest index on ties, skipping `skip`.
  auto argmax = [&](const float (&v)[NPL], int skip, float& m, int& arg) {
    m = -INFINITY;
    arg = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int i = lane + 64 * q;
      if (i < N && i != skip && route_before(v[q], i, m, arg)) {
        m = v[q];
        arg = i;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float om = __shfl_xor(m, off);
      const int oa = __shfl_xor(arg, off);
      if (route_before(om, oa, m, arg)) {
        m = om;
        arg = oa;
      }
    }
  };
  for (int j = wave; j < kRouteTokens; j += WAVES) {
    const int t = tb + j;
    if (t >= T) {
      if (lane == 0) eid_s[j][0] = eid_s[j][1] = -1;
      continue;
    }
    float v[NPL];
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int i = lane + 64 * q;
      v[q] = i < N ? logits[(size_t)t * N + i] : -INFINITY;
    }
    float m, m1;
    int e0, e1;
    argmax(v, -1, m, e0);
    argmax(v, e0, m1, e1);
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
      expert_idx[2 * (size_t)t] = e0;
      expert_idx[2 * (size_t)t + 1] = e1;
      gate[2 * (size_t)t] = inv;
      gate[2 * (size_t)t + 1] = expf(m1 - m) * inv;
      eid_s[j][0] = e0;
      eid_s[j][1] = e1;
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
  if (threadIdx.x < 2 * kRouteTokens) {
    const int j = threadIdx.x >> 1, c = threadIdx.x & 1;
    const int e = eid_s[j][c];
    if (e >= 0 && !(first_only && c == 1)) {
      int r = 0;
      if (first_only) {
        for (int s2 = 0; s2 < j; ++s2) r += eid_s[s2][0] == e;
      } else {
        for (int s2 = 0; s2 < j; ++s2) r += (eid_s[s2][0] == e) + (eid_s[s2][1] == e);
      }
      lrank[2 * (size_t)(tb + j) + c] = r;
      atomicAdd(&cnt_s[e], 1);
      if (c == 0) atomicAdd(&cnt1_s[e], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += 256) {
    cnt[(size_t)b * N + i] = cnt_s[i];
    if (cnt1) cnt1[(size_t)b * N + i] = cnt1_s[i];
  }
}

// ---------------------------------------------------------------------------
// The same for N % 4 == 0 with 16-byte loads: lane l of a wave holds experts
// 4 (64 q + l) + c, c = 0..3, q = 0..NQ-1, so one load instruction of a wave
// covers 1 KB of a logit row.  A wave routes every 4th token of the block and
// has the next one's row in flight; the expert order within a lane rises with
// (q, c), so the first strict maximum is the lowest index of the lane's maxima.
// Sums: per lane in (q, c) order, then a fixed butterfly across the wave; p
// sums over the block: per lane in token order, then the four waves in order.
// ---------------------------------------------------------------------------
template <int NQ>
__global__ void __launch_bounds__(256)
softmax_route_vec_kernel(const float* __restrict__ logits, int T, int N,
                         int32_t* __restrict__ expert_idx, float* __restrict__ gate,
                         float* __restrict__ ppart, int* __restrict__ cnt, int* __restrict__ lrank) {
  constexpr int WAVES = 4;
  __shared__ __attribute__((aligned(16))) float pacc[WAVES][NQ * 256];
  __shared__ int eid_s[kRouteTokens];
  __shared__ int cnt_s[NQ * 256];

  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tb = b * kRouteTokens;
  const __amdgpu_buffer_rsrc_t src = make_rsrc(logits, (uint32_t)((size_t)T * N * 4));

  for (int i = threadIdx.x; i < NQ * 256; i += 256) cnt_s[i] = 0;

  f32x4 acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto fetch = [&](int j, u32x4 (&v)[NQ]) {
    const int t = tb + j;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int i = 4 * (64 * q + lane);
      v[q] = buffer_load16(src, (t < T && i < N) ? ((uint32_t)t * (uint32_t)N + (uint32_t)i) * 4u : kOob);
    }
  };
  u32x4 vn[NQ];
  fetch(wave, vn);
  for (int j = wave; j < kRouteTokens; j += WAVES) {
    const int t = tb + j;
    f32x4 v[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) v[q] = __builtin_bit_cast(f32x4, vn[q]);
    if (j + WAVES < kRouteTokens) fetch(j + WAVES, vn);
    if (t >= T) {
      if (lane == 0) eid_s[j] = -1;
      continue;
    }
    float m = -INFINITY;
    int arg = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 4 * (64 * q + lane) + c;
        if (i < N && route_before(v[q][c], i, m, arg)) {
          m = v[q][c];
          arg = i;
        }
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float om = __shfl_xor(m, off);
      const int oa = __shfl_xor(arg, off);
      if (route_before(om, oa, m, arg)) {
        m = om;
        arg = oa;
      }
    }
    // exp(z - m) as 2^((z - m) log2 e) on the hardware exp2: z - m <= 0, so the
    // terms are at most 1 and each carries a relative error of about
    // (|z - m| + 1) 2^-23, which bounds the gate's error near 3e-7 (the terms
    // far below the maximum carry the larger relative errors but weigh little).
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v[q][c] = (4 * (64 * q + lane) + c < N)
                      ? __builtin_amdgcn_exp2f((v[q][c] - m) * 1.4426950408889634f) : 0.f;
        s += v[q][c];
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    const float inv = 1.0f / s;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[q][c] += v[q][c] * inv;
    if (lane == 0) {
      expert_idx[t] = arg;
      gate[t] = inv;
      eid_s[j] = arg;
    }
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    *reinterpret_cast<f32x4*>(&pacc[wave][4 * (64 * q + lane)]) = acc[q];
  __syncthreads();

  for (int i4 = threadIdx.x; 4 * i4 < N; i4 += 256) {
    const int i = 4 * i4;
    f32x4 p = *reinterpret_cast<const f32x4*>(&pacc[0][i]);
#pragma unroll
    for (int w = 1; w < WAVES; ++w) p += *reinterpret_cast<const f32x4*>(&pacc[w][i]);
    *reinterpret_cast<f32x4*>(ppart + (size_t)b * N + i) = p;
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

int router_plane_tiles(int N) { return (N + 31) / 32; }

// The tiled router, and the fused one for more than 64 experts, read planes;
// the fused router for up to 64 experts splits Wr as it loads it.
size_t router_planes_bytes(const Shape& s) {
  if (router_is_tiled(s)) return tiled_planes_bytes(s);
  if (!router_is_fused(s) || router_plane_tiles(s.N) <= 2) return 0;
  const size_t nks = (size_t)(s.d + FR_BK - 1) / FR_BK;
  return nks * 3 * (size_t)router_plane_tiles(s.N) * 2 * 1024;
}

hipError_t launch_router_fused(const Shape& s, const Inputs& in, const Workspace& ws,
                               const Outputs& out, hipStream_t st) {
  const int mt = router_plane_tiles(s.N);
  if (mt > 2) {
    const int nks = (s.d + FR_BK - 1) / FR_BK;
    const int groups = nks * mt * 2 * 64;
    hipLaunchKernelGGL(router_planes_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                       st, in.Wr, s.d, s.N, mt, nks, ws.planes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)s.n_route_blocks), block(256);
  const uint16_t* x = (const uint16_t*)in.x;
  const uint32_t pbytes = (uint32_t)router_planes_bytes(s);
  // Rerouting keeps both choices in the workspace; the scatter writes the outputs.
  const int mode = s.k == 2 ? 1 : (s.reroute ? 2 : 0);
  int32_t* const eidx = mode == 2 ? ws.choice : out.expert_idx;
  float* const g = mode == 2 ? ws.gate2 : out.gate;
#define SFFN_FUSED(M, MO)                                                                      \
  hipLaunchKernelGGL((router_fused_kernel<M, MO>), grid, block, 0, st, x, in.Wr, ws.planes,     \
                     pbytes, s.T, s.d, s.N, eidx, g, ws.ppart, ws.cnt, ws.lrank, ws.cnt1,       \
                     ws.logits)
#define SFFN_FUSED_MODES(M)         \
  if (mode == 0) SFFN_FUSED(M, 0);  \
  else if (mode == 1) SFFN_FUSED(M, 1); \
  else SFFN_FUSED(M, 2)
  switch (mt) {
    case 1: SFFN_FUSED_MODES(1); break;
    case 2: SFFN_FUSED_MODES(2); break;
    case 3: SFFN_FUSED_MODES(3); break;
    default: SFFN_FUSED_MODES(4); break;
  }
#undef SFFN_FUSED_MODES
#undef SFFN_FUSED
  return hipGetLastError();
}

hipError_t launch_softmax_route(const Shape& s, const Inputs& in, const Workspace& ws,
                                const Outputs& out, hipStream_t st) {
  if (router_is_fused(s)) return launch_router_fused(s, in, ws, out, st);
  const dim3 grid((unsigned)s.n_route_blocks), block(256);
  if (two_choices(s)) {
    // Rerouting keeps both choices in the workspace; the scatter writes the outputs.
    const bool rr = s.reroute != 0;
    int32_t* const eidx = rr ? ws.choice : out.expert_idx;
    float* const g = rr ? ws.gate2 : out.gate;
    int* const cnt1 = rr ? nullptr : ws.cnt1;
    const int npl = (s.N + 63) / 64;
#define SFFN_TOP2(K)                                                                             \
  hipLaunchKernelGGL(softmax_route_top2_kernel<K>, grid, block, 0, st, ws.logits, s.T, s.N,      \
                     eidx, g, ws.ppart, ws.cnt, cnt1, ws.lrank, rr ? 1 : 0)
    if (npl <= 1) SFFN_TOP2(1);
    else if (npl <= 2) SFFN_TOP2(2);
    else if (npl <= 4) SFFN_TOP2(4);
    else if (npl <= 8) SFFN_TOP2(8);
    else if (npl <= 16) SFFN_TOP2(16);
    else if (npl <= 32) SFFN_TOP2(32);
    else SFFN_TOP2(64);
#undef SFFN_TOP2
    return hipGetLastError();
  }
  if (s.N % 4 == 0 && logits_fit_offsets(s)) {
    const int nq = (s.N + 255) / 256;
#define SFFN_SOFTMAX_VEC(K)                                                                      \
  hipLaunchKernelGGL(softmax_route_vec_kernel<K>, grid, block, 0, st, ws.logits, s.T, s.N,       \
                     out.expert_idx, out.gate, ws.ppart, ws.cnt, ws.lrank)
    if (nq <= 1) SFFN_SOFTMAX_VEC(1);
    else if (nq <= 2) SFFN_SOFTMAX_VEC(2);
    else if (nq <= 4) SFFN_SOFTMAX_VEC(4);
    else if (nq <= 8) SFFN_SOFTMAX_VEC(8);
    else SFFN_SOFTMAX_VEC(16);
#undef SFFN_SOFTMAX_VEC
    return hipGetLastError();
  }
  const int npl = (s.N + 63) / 64;
#define SFFN_SOFTMAX(K)                                                                         \
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
