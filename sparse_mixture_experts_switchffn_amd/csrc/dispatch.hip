// Capacity-limited dispatch of the Switch layer and its aux loss.
//
// "Switch Transformers: Scaling to Trillion Parameter Models with Simple and
// Efficient Sparsity", section 3.4, "Distributed Implementation and Expert
// Capacity": a running count down each expert's column gives every token its
// position in that expert's buffer; positions at or past the capacity C are
// masked out and the token overflows, bypassing the expert on the residual
// path.  Here the running count is an exact integer rank in flattened token
// order: rank_t = (tokens of e_t in earlier routing blocks) + (tokens of e_t
// earlier in t's own block).  No step depends on the order in which blocks
// run, so slots are bitwise reproducible.
//
// Same section, "The Load-Balancing Auxiliary Loss": aux = N sum_i f_i P_i with
// f_i the top-1 share before capacity and P_i the mean router probability.
#include "sffn_device.h"
#include "sffn_internal.h"
#include "../../include/switch_ffn.h"

namespace sffn {

// ---------------------------------------------------------------------------
// Column scan over routing blocks.  Block = EPB experts x 1024/EPB segments of
// routing blocks (1024 threads; EPB = 8 gives four times the blocks of EPB =
// 32, which the scan's short columns need to spread over the GPU).  Outputs
// base[b][e] (start[e] + tokens of e in blocks < b), hist[e], acc[e] =
// min(start[e] + hist[e], C) and psum[e] = sum_b ppart[b][e] (float64, segment
// partial sums combined in segment order).  start (rerouting's second stage),
// ppart/psum, hist and cnt1/hist1 may be null: start counts as 0 and the
// others are skipped.
// ---------------------------------------------------------------------------
constexpr int kScanEpb = 8;
constexpr int kScanSegs = 1024 / kScanEpb;

__global__ void __launch_bounds__(1024)
dispatch_scan_kernel(const int* __restrict__ cnt, const float* __restrict__ ppart, int nblk,
                     int N, int C, int* __restrict__ base, int* __restrict__ hist,
                     int* __restrict__ acc, double* __restrict__ psum,
                     const int* __restrict__ cnt1, int* __restrict__ hist1,
                     const int* __restrict__ start) {
  __shared__ int part[kScanSegs][kScanEpb + 1];
  __shared__ int part1[kScanSegs][kScanEpb + 1];
  __shared__ double ppart_s[kScanSegs][kScanEpb + 1];
  const int el = threadIdx.x % kScanEpb;
  const int seg = threadIdx.x / kScanEpb;
  const int e = blockIdx.x * kScanEpb + el;
  const int per = (nblk + kScanSegs - 1) / kScanSegs;
  const int c0 = min(nblk, seg * per);
  const int c1 = min(nblk, c0 + per);
  int s = 0, s1 = 0, s0 = 0;
  double ps = 0.0;
  if (e < N) {
    if (start) s0 = start[e];
#pragma unroll 4
    for (int c = c0; c < c1; ++c) s += cnt[(size_t)c * N + e];
    if (ppart)
      for (int c = c0; c < c1; ++c) ps += (double)ppart[(size_t)c * N + e];
    if (cnt1)
      for (int c = c0; c < c1; ++c) s1 += cnt1[(size_t)c * N + e];
  }
  part[seg][el] = s;
  part1[seg][el] = s1;
  ppart_s[seg][el] = ps;
  __syncthreads();
  if (e >= N) return;
  int run = s0;
  for (int q = 0; q < seg; ++q) run += part[q][el];
#pragma unroll 4
  for (int c = c0; c < c1; ++c) {
    const int v = cnt[(size_t)c * N + e];
    base[(size_t)c * N + e] = run;
    run += v;
  }
  if (seg == 0) {
    int total = 0, total1 = 0;
    double ptot = 0.0;
    for (int q = 0; q < kScanSegs; ++q) {
      total += part[q][el];
      total1 += part1[q][el];
      ptot += ppart_s[q][el];
    }
    if (hist) hist[e] = total;
    acc[e] = min(s0 + total, C);
    if (psum) psum[e] = ptot;
    if (hist1) hist1[e] = total1;
  }
}

// ---------------------------------------------------------------------------
// No-Token-Left-Behind rerouting ("Switch Transformers" summary, section 3.4,
// "Distributed Implementation and Expert Capacity", the No-Token-Left-Behind
// experiment of Appendix B and its two-stage Figure 11), second stage, count
// pass.  After the first stage's scan a token's position in its first choice is
// base[b][e1] + lrank[2t]; the slot it takes there (or -1) goes to slot1[t].
// Overflowed tokens are counted per block by second choice: cnt[b][e] (the
// first stage's counts are spent by then) and their rank among the block's
// overflowed tokens with the same second choice in lrank[2t + 1].
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
reroute_count_kernel(const int32_t* __restrict__ choice, const int* __restrict__ base, int T,
                     int N, int C, int* __restrict__ lrank, int32_t* __restrict__ slot1,
                     int* __restrict__ cnt) {
  __shared__ int cnt_s[SFFN_MAX_EXPERTS];
  __shared__ int e2_s[kRouteTokens];
  const int b = blockIdx.x;
  const int tb = b * kRouteTokens;
  for (int i = threadIdx.x; i < N; i += 256) cnt_s[i] = 0;
  if (threadIdx.x < kRouteTokens) {
    const int t = tb + threadIdx.x;
    int e2 = -1;
    if (t < T) {
      const int e1 = choice[2 * (size_t)t];
      const int r = (unsigned)e1 < (unsigned)N ? base[(size_t)b * N + e1] + lrank[2 * (size_t)t]
                                               : C;
      if (r < C) {
        slot1[t] = r;
      } else {
        slot1[t] = -1;
        e2 = choice[2 * (size_t)t + 1];
        if ((unsigned)e2 >= (unsigned)N) e2 = -1;  // refused by both stages
      }
    }
    e2_s[threadIdx.x] = e2;
  }
  __syncthreads();
  if (threadIdx.x < kRouteTokens) {
    const int e = e2_s[threadIdx.x];
    if (e >= 0) {
      int r = 0;
      for (int j = 0; j < (int)threadIdx.x; ++j) r += e2_s[j] == e;
      lrank[2 * (size_t)(tb + threadIdx.x) + 1] = r;
      atomicAdd(&cnt_s[e], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += 256) cnt[(size_t)b * N + i] = cnt_s[i];
}

hipError_t launch_dispatch_scan(const Shape& s, const Workspace& ws, hipStream_t st) {
  if (dispatch_scan_in_scatter(s)) return hipSuccess;  // done by dispatch_scatter_fold_kernel
  const dim3 grid((unsigned)((s.N + kScanEpb - 1) / kScanEpb)), block(1024);
  hipLaunchKernelGGL(dispatch_scan_kernel, grid, block, 0, st, ws.cnt, ws.ppart,
                     s.n_route_blocks, s.N, s.C, ws.base, ws.hist, ws.acc, ws.psum,
                     s.k == 2 ? ws.cnt1 : nullptr, s.k == 2 ? ws.hist1 : nullptr, nullptr);
  if (!s.reroute) return hipGetLastError();
  // Second stage: overflowed tokens by second choice, then their positions,
  // which start after each expert's first-stage rows: base = acc + earlier
  // blocks' overflowed tokens, acc2 = min(acc + overflowed tokens, C).
  hipLaunchKernelGGL(reroute_count_kernel, dim3((unsigned)s.n_route_blocks), dim3(256), 0, st,
                     ws.choice, ws.base, s.T, s.N, s.C, ws.lrank, ws.slot1, ws.cnt);
  hipLaunchKernelGGL(dispatch_scan_kernel, grid, block, 0, st, ws.cnt, nullptr,
                     s.n_route_blocks, s.N, s.C, ws.base, nullptr, ws.acc2, nullptr,
                     nullptr, nullptr, ws.acc);
  return hipGetLastError();
}

// Exclusive scan of acc[0..N) into off_s[0..N] by one 256-thread block.
__device__ void block_offsets(const int* __restrict__ acc, int N, int* off_s, int* tsum) {
  const int per = (N + 255) / 256;
  const int i0 = min(N, (int)threadIdx.x * per);
  const int i1 = min(N, i0 + per);
  int s = 0;
  for (int i = i0; i < i1; ++i) s += acc[i];
  tsum[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x < 64) {  // one wave scans the 256 thread sums, 4 per lane
    const int l = threadIdx.x;
    int v[4], run = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) { v[q] = tsum[4 * l + q]; run += v[q]; }
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (l >= off) incl += o;
    }
    int ex = incl - run;
#pragma unroll
    for (int q = 0; q < 4; ++q) { tsum[4 * l + q] = ex; ex += v[q]; }
  }
  __syncthreads();
  int run = tsum[threadIdx.x];
  for (int i = i0; i < i1; ++i) {
    off_s[i] = run;
    run += acc[i];
  }
  if (threadIdx.x == 255) off_s[N] = run;
  __syncthreads();
}

// Dropped tokens leave the layer unchanged (or as zero in the no-residual view):
// the four waves of the block copy the rows of the block's flagged tokens.
__device__ void pass_through_dropped(const int* dropped_s, int tb, int d, int esize,
                                     const void* __restrict__ x, void* __restrict__ y,
                                     int no_residual) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t row_bytes = (size_t)d * esize;
  for (int j = wave; j < kRouteTokens; j += 4) {
    if (!dropped_s[j]) continue;
    const size_t t = (size_t)(tb + j);
    char* dst = (char*)y + t * row_bytes;
    const char* src = (const char*)x + t * row_bytes;
    if (((row_bytes | (size_t)x | (size_t)y) & 15) == 0) {
      for (size_t c = (size_t)lane * 16; c < row_bytes; c += 64 * 16)
        store16(dst + c, no_residual ? u32x4{0, 0, 0, 0} : load16(src + c));
    } else {
      for (size_t c = (size_t)lane * 4; c < row_bytes; c += 64 * 4)
        *(uint32_t*)(dst + c) = no_residual ? 0u : *(const uint32_t*)(src + c);
    }
  }
}

// Block 0's share of a dispatch: the expert offsets, the aux loss
// N * sum_i (f_count_i / T) * (psum_i / T) summed in a fixed tree order, and the
// optional statistics (count[i], accepted = acc[i], dropped = slots - sum acc).
__device__ void finish_dispatch(const int* __restrict__ f_count, const int* __restrict__ count,
                                const int* __restrict__ acc, const double* __restrict__ psum,
                                int T, int N, int slots, const int* off_s, int* tsum, double* red,
                                int* __restrict__ offset, float* __restrict__ aux_loss,
                                int32_t* __restrict__ stat_count,
                                int32_t* __restrict__ stat_accepted,
                                int32_t* __restrict__ stat_dropped, uint32_t* __restrict__ tag,
                                const WsTag& tagv) {
  if (threadIdx.x == 0) {  // the layout tag (constant indices: the words stay in registers)
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      store16(tag + i, u32x4{tagv.w[i], tagv.w[i + 1], tagv.w[i + 2], tagv.w[i + 3]});
  }
  for (int i = threadIdx.x; i <= N; i += 256) offset[i] = off_s[i];
  double part = 0.0;
  int accepted = 0;
  for (int i = threadIdx.x; i < N; i += 256) {
    part += (double)f_count[i] * psum[i];
    accepted += acc[i];
    if (stat_count) stat_count[i] = count[i];
    if (stat_accepted) stat_accepted[i] = acc[i];
  }
  red[threadIdx.x] = part;
  tsum[threadIdx.x] = accepted;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) {
      red[threadIdx.x] += red[threadIdx.x + w];
      tsum[threadIdx.x] += tsum[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double Td = (double)T;
    aux_loss[0] = (float)((double)N * red[0] / (Td * Td));
    if (stat_dropped) stat_dropped[0] = slots - tsum[0];
  }
}

// ---------------------------------------------------------------------------
// Slots, the row-to-token map and the residual pass-through of dropped tokens.
// Block b handles routing block b (kRouteTokens tokens).  Block 0 also writes
// the expert offsets, the aux loss and the optional statistics.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
dispatch_scatter_kernel(const int32_t* __restrict__ expert_idx, const int* __restrict__ base,
                        const int* __restrict__ lrank, const int* __restrict__ hist,
                        const int* __restrict__ acc, const double* __restrict__ psum, int T, int N,
                        int C, int d, int esize, const void* __restrict__ x, void* __restrict__ y,
                        int no_residual, const float* __restrict__ gate,
                        int32_t* __restrict__ slot, int* __restrict__ row2tok,
                        float* __restrict__ rowgate, int* __restrict__ offset, float* __restrict__ aux_loss,
                        int32_t* __restrict__ stat_count, int32_t* __restrict__ stat_accepted,
                        int32_t* __restrict__ stat_dropped,
    uint32_t* __restrict__ tag, const WsTag tagv) {
  __shared__ int off_s[SFFN_MAX_EXPERTS + 1];
  __shared__ int tsum[256];
  __shared__ int dropped_s[kRouteTokens];
  __shared__ double red[256];

  block_offsets(acc, N, off_s, tsum);

  const int b = blockIdx.x;
  const int tb = b * kRouteTokens;
  if (threadIdx.x < kRouteTokens) {
    const int t = tb + threadIdx.x;
    int dropped = 0;
    if (t < T) {
      // The router gives every token an expert in [0, N); an index outside it
      // (a corrupted input) drops the token instead of indexing past the tables.
      const int e = expert_idx[t];
      const bool ok = (unsigned)e < (unsigned)N;
      const int r = ok ? base[(size_t)b * N + e] + lrank[t] : C;
      if (r < C) {
        slot[t] = r;
        row2tok[off_s[e] + r] = t;
        rowgate[off_s[e] + r] = gate[t];
      } else {
        slot[t] = -1;
        dropped = 1;
      }
    }
    dropped_s[threadIdx.x] = dropped;
  }
  __syncthreads();

  pass_through_dropped(dropped_s, tb, d, esize, x, y, no_residual);
  if (b != 0) return;
  finish_dispatch(hist, hist, acc, psum, T, N, T, off_s, tsum, red, offset, aux_loss, stat_count,
                  stat_accepted, stat_dropped, tag, tagv);
}

// ---------------------------------------------------------------------------
// Top-1 dispatch with the column scan folded in, for layers whose count table
// cnt[nblk][N] is small: every block sums the table itself, so no scan pass
// runs before it.  For each expert e, block b takes pre[e] = tokens of e in
// routing blocks < b and tot[e] = tokens of e in all blocks (integer sums, the
// same in any order), acc[e] = min(tot[e], C), and the offsets from acc.
// Threads read 16-byte chunks of four experts' counts: chunk j of a row by the
// threads of column j, routing blocks split into segments by thread row, the
// segment partials combined in LDS.  Block 0 also takes psum[e] = sum_b
// ppart[b][e] in float64 (each segment in block order, then the segments in
// order) and writes hist = tot, the offsets, the aux loss and the statistics.
// ---------------------------------------------------------------------------
constexpr int kFoldMaxExperts = 256;
constexpr int kFoldRowsPerThread = 16;  // all of a thread's table rows in flight at once

bool dispatch_scan_in_scatter(const Shape& s) {
  if (s.k != 1 || s.reroute || s.N % 4 != 0 || s.N > kFoldMaxExperts) return false;
  const int segs = 256 / (s.N / 4) < s.n_route_blocks ? 256 / (s.N / 4) : s.n_route_blocks;
  return (s.n_route_blocks + segs - 1) / segs <= kFoldRowsPerThread;
}

__global__ void __launch_bounds__(256)
dispatch_scatter_fold_kernel(const int32_t* __restrict__ expert_idx, const int* __restrict__ cnt,
                             const float* __restrict__ ppart, const int* __restrict__ lrank,
                             int nblk, int T, int N, int C, int d, int esize,
                             const void* __restrict__ x, void* __restrict__ y, int no_residual,
                             const float* __restrict__ gate, int32_t* __restrict__ slot,
                             int* __restrict__ row2tok, float* __restrict__ rowgate,
                             int* __restrict__ hist, int* __restrict__ offset,
                             float* __restrict__ aux_loss, int32_t* __restrict__ stat_count,
                             int32_t* __restrict__ stat_accepted,
                             int32_t* __restrict__ stat_dropped, uint32_t* __restrict__ tag,
                             const WsTag tagv) {
  __shared__ u32x4 part_pre[256], part_tot[256];
  __shared__ double part_ps[256][4];
  __shared__ int pre_s[kFoldMaxExperts], tot_s[kFoldMaxExperts], acc_s[kFoldMaxExperts];
  __shared__ double psum_s[kFoldMaxExperts];
  __shared__ int off_s[kFoldMaxExperts + 1];
  __shared__ int tsum[256];
  __shared__ int dropped_s[kRouteTokens];
  __shared__ double red[256];

  const int b = blockIdx.x;
  const int cpr = N >> 2;            // 16-byte chunks per row of the table
  const int segs = min(256 / cpr, nblk);  // segments of routing blocks
  const int j = threadIdx.x % cpr, sg = threadIdx.x / cpr;
  const int per = (nblk + segs - 1) / segs;  // at most kFoldRowsPerThread
  const int c0 = sg < segs ? min(nblk, sg * per) : nblk;
  const int c1 = min(nblk, c0 + per);
  u32x4 pre{0, 0, 0, 0}, tot{0, 0, 0, 0};
  double ps[4] = {0.0, 0.0, 0.0, 0.0};
  {
    u32x4 v[kFoldRowsPerThread];
#pragma unroll
    for (int r = 0; r < kFoldRowsPerThread; ++r)
      v[r] = c0 + r < c1 ? load16(cnt + (size_t)(c0 + r) * N + 4 * j) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < kFoldRowsPerThread; ++r) {
      tot += v[r];
      if (c0 + r < b) pre += v[r];
    }
  }
  if (b == 0) {
    u32x4 v[kFoldRowsPerThread];
#pragma unroll
    for (int r = 0; r < kFoldRowsPerThread; ++r)
      v[r] = c0 + r < c1 ? load16(ppart + (size_t)(c0 + r) * N + 4 * j) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < kFoldRowsPerThread; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) ps[q] += (double)__uint_as_float(v[r][q]);  // block order
  }
  part_pre[threadIdx.x] = pre;
  part_tot[threadIdx.x] = tot;
  if (b == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) part_ps[threadIdx.x][q] = ps[q];
  }
  __syncthreads();
  if ((int)threadIdx.x < N) {
    const int e = threadIdx.x, jj = e >> 2, q = e & 3;
    int p = 0, t = 0;
    double sp = 0.0;
    for (int g = 0; g < segs; ++g) {
      p += (int)part_pre[g * cpr + jj][q];
      t += (int)part_tot[g * cpr + jj][q];
      if (b == 0) sp += part_ps[g * cpr + jj][q];
    }
    pre_s[e] = p;
    tot_s[e] = t;
    acc_s[e] = min(t, C);
    psum_s[e] = sp;
  }
  __syncthreads();
  block_offsets(acc_s, N, off_s, tsum);

  const int tb = b * kRouteTokens;
  if (threadIdx.x < kRouteTokens) {
    const int t = tb + threadIdx.x;
    int dropped = 0;
    if (t < T) {
      const int e = expert_idx[t];
      const bool ok = (unsigned)e < (unsigned)N;  // as in dispatch_scatter_kernel
      const int r = ok ? pre_s[e] + lrank[t] : C;
      if (r < C) {
        slot[t] = r;
        row2tok[off_s[e] + r] = t;
        rowgate[off_s[e] + r] = gate[t];
      } else {
        slot[t] = -1;
        dropped = 1;
      }
    }
    dropped_s[threadIdx.x] = dropped;
  }
  __syncthreads();

  pass_through_dropped(dropped_s, tb, d, esize, x, y, no_residual);
  if (b != 0) return;
  for (int e = threadIdx.x; e < N; e += 256) hist[e] = tot_s[e];
  finish_dispatch(tot_s, tot_s, acc_s, psum_s, T, N, T, off_s, tsum, red, offset, aux_loss,
                  stat_count, stat_accepted, stat_dropped, tag, tagv);
}

// ---------------------------------------------------------------------------
// Top-2 dispatch: slots and the row maps of both choices of every token (each
// expert column in token order).  The residual path is left to the combine,
// which writes every y row.  Block 0 also writes the expert offsets, the aux
// loss (f from the top-1 counts) and the optional statistics.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
dispatch_scatter_top2_kernel(const int32_t* __restrict__ expert_idx, const int* __restrict__ base,
                             const int* __restrict__ lrank, const int* __restrict__ hist,
                             const int* __restrict__ hist1, const int* __restrict__ acc,
                             const double* __restrict__ psum, int T, int N, int C,
                             const float* __restrict__ gate, int32_t* __restrict__ slot,
                             int* __restrict__ row2tok, float* __restrict__ rowgate,
                             int* __restrict__ offset, float* __restrict__ aux_loss,
                             int32_t* __restrict__ stat_count, int32_t* __restrict__ stat_accepted,
                             int32_t* __restrict__ stat_dropped,
    uint32_t* __restrict__ tag, const WsTag tagv) {
  __shared__ int off_s[SFFN_MAX_EXPERTS + 1];
  __shared__ int tsum[256];
  __shared__ double red[256];

  block_offsets(acc, N, off_s, tsum);

  const int b = blockIdx.x;
  const int tb = b * kRouteTokens;
  if (threadIdx.x < 2 * kRouteTokens) {
    const int t = tb + (threadIdx.x >> 1);
    const size_t i = 2 * (size_t)t + (threadIdx.x & 1);
    if (t < T) {
      const int e = expert_idx[i];
      const bool ok = (unsigned)e < (unsigned)N;  // as in the top-1 dispatch
      const int r = ok ? base[(size_t)b * N + e] + lrank[i] : C;
      if (r < C) {
        slot[i] = r;
        row2tok[off_s[e] + r] = t;
        rowgate[off_s[e] + r] = gate[i];
      } else {
        slot[i] = -1;
      }
    }
  }

  if (b != 0) return;
  finish_dispatch(hist1, hist, acc, psum, T, N, 2 * T, off_s, tsum, red, offset, aux_loss,
                  stat_count, stat_accepted, stat_dropped, tag, tagv);
}

// ---------------------------------------------------------------------------
// Rerouting dispatch: each token's final expert, slot and gate, the row maps,
// and the pass-through of tokens refused by both choices.  A token keeps its
// first-stage slot if it has one; otherwise it takes position base[b][e2] +
// lrank[2t + 1] of its second choice e2 (base already starts after e2's
// first-stage rows) if that is below C, else it is dropped and reports its
// first choice.  Offsets come from acc2; the aux loss and expert_count use the
// first choices (hist), accepted_count is acc2.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
dispatch_scatter_reroute_kernel(const int32_t* __restrict__ choice,
                                const float* __restrict__ gate2, const int32_t* __restrict__ slot1,
                                const int* __restrict__ base, const int* __restrict__ lrank,
                                const int* __restrict__ hist, const int* __restrict__ acc2,
                                const double* __restrict__ psum, int T, int N, int C, int d,
                                int esize, const void* __restrict__ x, void* __restrict__ y,
                                int no_residual, int32_t* __restrict__ expert_idx,
                                float* __restrict__ gate, int32_t* __restrict__ slot,
                                int* __restrict__ row2tok, float* __restrict__ rowgate,
                                int* __restrict__ offset, float* __restrict__ aux_loss,
                                int32_t* __restrict__ stat_count,
                                int32_t* __restrict__ stat_accepted,
                                int32_t* __restrict__ stat_dropped,
    uint32_t* __restrict__ tag, const WsTag tagv) {
  __shared__ int off_s[SFFN_MAX_EXPERTS + 1];
  __shared__ int tsum[256];
  __shared__ int dropped_s[kRouteTokens];
  __shared__ double red[256];

  block_offsets(acc2, N, off_s, tsum);

  const int b = blockIdx.x;
  const int tb = b * kRouteTokens;
  if (threadIdx.x < kRouteTokens) {
    const int t = tb + threadIdx.x;
    int dropped = 0;
    if (t < T) {
      const size_t i0 = 2 * (size_t)t;
      int e = choice[i0], r = slot1[t];
      float g = gate2[i0];
      if (r < 0) {
        const int e2 = choice[i0 + 1];
        const bool ok = (unsigned)e2 < (unsigned)N;  // as in the top-1 dispatch
        const int r2 = ok ? base[(size_t)b * N + e2] + lrank[i0 + 1] : C;
        if (r2 < C) {
          e = e2;
          r = r2;
          g = gate2[i0 + 1];
        }
      }
      expert_idx[t] = e;
      gate[t] = g;
      if (r >= 0) {
        slot[t] = r;
        row2tok[off_s[e] + r] = t;
        rowgate[off_s[e] + r] = g;
      } else {
        slot[t] = -1;
        dropped = 1;
      }
    }
    dropped_s[threadIdx.x] = dropped;
  }
  __syncthreads();

  pass_through_dropped(dropped_s, tb, d, esize, x, y, no_residual);
  if (b != 0) return;
  finish_dispatch(hist, hist, acc2, psum, T, N, T, off_s, tsum, red, offset, aux_loss,
                  stat_count, stat_accepted, stat_dropped, tag, tagv);
}

hipError_t launch_dispatch_scatter(const Shape& s, const Inputs& in, const Workspace& ws,
                                   const Outputs& out, bool no_residual, const WsTag& tag,
                                   hipStream_t st) {
  const dim3 grid((unsigned)s.n_route_blocks), block(256);
  if (s.k == 2) {
    hipLaunchKernelGGL(dispatch_scatter_top2_kernel, grid, block, 0, st, out.expert_idx, ws.base,
                       ws.lrank, ws.hist, ws.hist1, ws.acc, ws.psum, s.T, s.N, s.C, out.gate,
                       out.slot, ws.row2tok, ws.rowgate, ws.offset, out.aux_loss,
                       out.stat_count, out.stat_accepted, out.stat_dropped, ws.tag, tag);
    return hipGetLastError();
  }
  const int esize = s.dtype == SFFN_BF16 ? 2 : 4;
  if (s.reroute) {
    hipLaunchKernelGGL(dispatch_scatter_reroute_kernel, grid, block, 0, st, ws.choice, ws.gate2,
                       ws.slot1, ws.base, ws.lrank, ws.hist, ws.acc2, ws.psum, s.T, s.N, s.C,
                       s.d, esize, in.x, out.y, no_residual ? 1 : 0, out.expert_idx, out.gate,
                       out.slot, ws.row2tok, ws.rowgate, ws.offset, out.aux_loss,
                       out.stat_count, out.stat_accepted, out.stat_dropped, ws.tag, tag);
    return hipGetLastError();
  }
  if (dispatch_scan_in_scatter(s)) {
    hipLaunchKernelGGL(dispatch_scatter_fold_kernel, grid, block, 0, st, out.expert_idx, ws.cnt,
                       ws.ppart, ws.lrank, s.n_route_blocks, s.T, s.N, s.C, s.d, esize, in.x,
                       out.y, no_residual ? 1 : 0, out.gate, out.slot, ws.row2tok, ws.rowgate,
                       ws.hist, ws.offset, out.aux_loss, out.stat_count, out.stat_accepted,
                       out.stat_dropped, ws.tag, tag);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_scatter_kernel, grid, block, 0, st, out.expert_idx, ws.base,
                     ws.lrank, ws.hist, ws.acc, ws.psum, s.T, s.N, s.C, s.d, esize, in.x, out.y,
                     no_residual ? 1 : 0, out.gate, out.slot, ws.row2tok, ws.rowgate,
                     ws.offset, out.aux_loss,
                     out.stat_count, out.stat_accepted, out.stat_dropped, ws.tag, tag);
  return hipGetLastError();
}

}  // namespace sffn
