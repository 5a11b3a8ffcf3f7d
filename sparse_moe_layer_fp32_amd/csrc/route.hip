// Routing metadata (expert histogram -> prefix scan -> stable permutation and
// GEMM tile tables) and the weighted combine.
//
// "GPT-OSS on day 0", section "MoE": the dispatcher selects the tokens routed
// to each expert and the combine is a weighted accumulation of the expert
// outputs.  "Hosting Qwen on Blackwell", section "Expert Parallel": dispatch
// aggregates the routing information and stages tokens into the buffer the
// MoE GEMM reads; combine first accumulates locally.  On one GPU that is a
// counting sort of the (token, slot) pairs by expert, stable in token order,
// and a gather-sum over the k rows of each token in slot order.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// Exclusive scan of n <= 256 ints in LDS by one wave (4 per lane); returns the total.
__device__ int wave0_exclusive_scan(int* s, int n) {
  const int lane = threadIdx.x & 63;
  int v[4], run = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane * 4 + q;
    v[q] = i < n ? s[i] : 0;
    run += v[q];
  }
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  int pre = incl - run;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane * 4 + q;
    if (i < n) s[i] = pre;
    pre += v[q];
  }
  return __shfl(incl, 63);
}

// Cost of an expert's row blocks in one column tile of a prefill GEMM:
// `full` per row block, `part` for a last block of at most bm/2 rows (the
// waves of the empty half skip their MFMAs and stores; every weight load
// runs).  Fitted to the finishing times of the eight XCDs on the skewed
// prefill layer: such a tile takes 0.67 of a full one in the gate/up GEMM,
// 0.50 in the down GEMM (whose fp32 output stores halve too).
__device__ __forceinline__ int tile_cost(int c, int bm, int full_cost, int part_cost) {
  const int full = c / bm, tail = c - full * bm;
  return full_cost * full + (tail == 0 ? 0 : 2 * tail <= bm ? part_cost : full_cost);
}

// One workgroup.  hist[nt][E] holds the expert counts of every router tile.
__global__ __launch_bounds__(1024) void route_scan_kernel(const int32_t* __restrict__ hist, int nt,
                                                          int E, int bm0, int ntile0, int bm1,
                                                          int ntile1, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tile_base,
                                                          int32_t* __restrict__ tile_off0,
                                                          int32_t* __restrict__ tile_off1) {
  __shared__ int spart[1024];
  __shared__ int scnt[256], soff[256], st0[256], st1[256];
  const int tid = threadIdx.x;
  int EP = 1;
  while (EP < E) EP <<= 1;
  const int P = 1024 / EP;               // threads per expert
  const int e = tid % EP, p = tid / EP;
  const int ch = ceil_div(nt, P);
  const int lo = min(nt, p * ch), hi = min(nt, lo + ch);
  // the thread's chunk of its expert's column, 16 loads in flight at a time
  constexpr int kBatch = 16;
  int s = 0;
  if (e < E)
    for (int t0 = lo; t0 < hi; t0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = t0 + j < hi ? hist[(size_t)(t0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) s += v[j];
    }
  spart[tid] = s;
  __syncthreads();
  if (p == 0 && e < E) {                 // exclusive scan over this expert's chunks
    int run = 0;
    for (int q = 0; q < P; ++q) {
      const int v = spart[q * EP + e];
      spart[q * EP + e] = run;
      run += v;
    }
    scnt[e] = run;
  }
  __syncthreads();
  if (tid < E) {
    const int c = scnt[tid];
    counts[tid] = c;
    soff[tid] = c;
    st0[tid] = ceil_div(c, bm0) * ntile0;
    st1[tid] = ceil_div(c, bm1) * ntile1;
  }
  __syncthreads();
  if (tid < 64) {
    const int tot = wave0_exclusive_scan(soff, E);
    const int t0 = wave0_exclusive_scan(st0, E);
    const int t1 = wave0_exclusive_scan(st1, E);
    if (tid == 0) {
      offsets[E] = tot;
      tile_off0[E] = t0;
      tile_off1[E] = t1;
    }
  }
  __syncthreads();
  if (tid < E) {
    offsets[tid] = soff[tid];
    tile_off0[tid] = st0[tid];
    tile_off1[tid] = st1[tid];
  }
  if (e < E) {                           // absolute first row of every (tile, expert)
    int run = soff[e] + spart[tid];
    for (int t0 = lo; t0 < hi; t0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = t0 + j < hi ? hist[(size_t)(t0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (t0 + j < hi) {
          tile_base[(size_t)(t0 + j) * E + e] = run;
          run += v[j];
        }
    }
  }
}

// Rank of every (token, slot) pair of router tile tl among the earlier pairs
// of the tile with the same expert (a token never picks an expert twice, so
// this is the token order), and its row.
__device__ void place_tile(const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ tile_base,
                           int tl, int T, int E, int k, int32_t* __restrict__ row_of,
                           int32_t* __restrict__ row_token, int* se) {
  const int t0 = tl * RT_TT;
  const int n = min(RT_TT, T - t0) * k;
  const int p = threadIdx.x;
  if (p < n) se[p] = topk_idx[(size_t)t0 * k + p];
  __syncthreads();
  if (p < n) {
    const int e = se[p];
    int rank = 0;
    for (int q = 0; q < p; ++q) rank += (se[q] == e);
    const int row = tile_base[(size_t)tl * E + e] + rank;
    row_of[(size_t)t0 * k + p] = row;
    row_token[row] = t0 + p / k;
  }
}

// Entries L = first, first + stride, ... of a GEMM's tile list: the expert
// whose tiles hold L (binary search of the tile offsets), then inside the
// expert the order (column group of kTileGroup tiles, row block, column
// tile), so that consecutive tiles share one slice of the expert's weights.
__device__ void tile_entries(const int32_t* __restrict__ tile_off, const int32_t* __restrict__ counts,
                             const int32_t* __restrict__ offsets, int E, int bm, int n_tiles,
                             int max_tiles, int4* __restrict__ tiles, int first, int stride) {
  const int total = min(tile_off[E], max_tiles);
  for (int L = first; L < total; L += stride) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_off[mid] <= L) lo = mid; else hi = mid;
    }
    const int cnt = counts[lo];
    const int local = L - tile_off[lo];
    if (cnt <= bm) {  // one row block: the entries are the column tiles in order
      tiles[L] = make_int4(lo, offsets[lo], cnt, local);
      continue;
    }
    const int mt = ceil_div(cnt, bm);
    const int ng = local / (mt * kTileGroup);
    const int rem = local - ng * mt * kTileGroup;
    const int gw = min(kTileGroup, n_tiles - ng * kTileGroup);
    const int m = rem / gw;
    tiles[L] = make_int4(lo, offsets[lo] + m * bm, min(bm, cnt - m * bm), ng * kTileGroup + rem % gw);
  }
}

// The XCD ranges of both GEMMs' tile lists (sched, kSchedInts ints per
// GEMM): range x starts at the tile where the cost before it reaches x/8 of
// the total, inside an expert in proportion to its tiles; and the tile
// counters zeroed.  One workgroup of >= 256 threads; sc: 512 ints of LDS.
__device__ void xcd_ranges(const int32_t* __restrict__ counts, const int32_t* __restrict__ tile_off0,
                           int bm0, int nt0, const int32_t* __restrict__ tile_off1, int bm1, int nt1,
                           int E, int32_t* __restrict__ sched, int* sc) {
  __shared__ int sbound[2][9], scost[2];
  const int tid = threadIdx.x;
  if (tid < 2 * kSchedCounters)
    sched[(tid / kSchedCounters) * kSchedInts + tid % kSchedCounters] = 0;
  if (tid < E) {
    const int c = counts[tid];
    sc[tid] = tile_cost(c, bm0, 3, 2) * nt0;
    sc[256 + tid] = tile_cost(c, bm1, 2, 1) * nt1;
  }
  __syncthreads();
  if (tid < 128) {  // one cost scan per wave
    const int g = tid >> 6;
    const int total = wave0_exclusive_scan(sc + 256 * g, E);
    if ((tid & 63) == 0) {
      scost[g] = total;
      for (int x = 0; x < 8; ++x) sbound[g][x] = 0;  // empty lists
      sbound[g][8] = (g == 0 ? tile_off0 : tile_off1)[E];
    }
  }
  __syncthreads();
  if (tid < E) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int32_t* toff = g == 0 ? tile_off0 : tile_off1;
      const int total = scost[g];
      const int c0 = sc[256 * g + tid];
      const int ce = (tid + 1 < E ? sc[256 * g + tid + 1] : total) - c0;
      const int first = toff[tid], n = toff[tid + 1] - first;
      for (int x = 1; x < 8; ++x) {
        const int target = x * (total >> 3) + ((x * (total & 7)) >> 3);  // x * total / 8
        // in float: a range start needs no more than tile precision, and any
        // start inside the expert's tiles keeps every tile in one range
        if (ce > 0 && c0 <= target && target < c0 + ce)
          sbound[g][x] = first + min(n - 1, (int)((float)(target - c0) * (float)n / (float)ce));
      }
    }
  }
  __syncthreads();
  if (tid < 18) sched[(tid / 9) * kSchedInts + kSchedBounds + tid % 9] = sbound[tid / 9][tid % 9];
}

// After the scan, in one launch: workgroups [0, nt) place router tile
// blockIdx.x, the next g0 build the gate/up GEMM's tile list, the next g1 the
// down GEMM's, and the last one the GEMMs' XCD ranges (all only read the
// scan's results).
__global__ __launch_bounds__(RT_TT * kMaxTopK) void route_place_tables_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ tile_base, int T, int E, int k,
    int32_t* __restrict__ row_of, int32_t* __restrict__ row_token, int nt,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off0, int bm0, int n_tiles0, int max0, int4* __restrict__ tiles0,
    int g0, const int32_t* __restrict__ tile_off1, int bm1, int n_tiles1, int max1,
    int4* __restrict__ tiles1, int g1, int32_t* __restrict__ sched) {
  __shared__ int se[RT_TT * kMaxTopK];
  constexpr int NTH = RT_TT * kMaxTopK;
  static_assert(2 * kSchedCounters <= NTH && NTH >= kMaxExperts && NTH >= 512, "xcd_ranges");
  const int b = blockIdx.x;
  if (b < nt) {
    place_tile(topk_idx, tile_base, b, T, E, k, row_of, row_token, se);
  } else if (b < nt + g0) {
    tile_entries(tile_off0, counts, offsets, E, bm0, n_tiles0, max0, tiles0, (b - nt) * NTH + threadIdx.x,
                 g0 * NTH);
  } else if (b < nt + g0 + g1) {
    tile_entries(tile_off1, counts, offsets, E, bm1, n_tiles1, max1, tiles1,
                 (b - nt - g0) * NTH + threadIdx.x, g1 * NTH);
  } else {
    xcd_ranges(counts, tile_off0, bm0, n_tiles0, tile_off1, bm1, n_tiles1, E, sched, se);
  }
}

// out[t, :] = bf16( sum_j w[t,j] * Y[row_of[t,j], :] ), fp32 in slot order.
// Workgroup (t, y) takes columns 1024 y.. of token t (one pass per thread for
// hidden sizes up to 1024 * gridDim.y).  Every Y row is read once: the loads
// carry the non-temporal policy.
typedef float v4f_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4f_nt load_once(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4f_nt*>(p));
}
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Y,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ topk_w, int T,
                                                      int d, int k, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  int rows[kMaxTopK];
  float ws[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    rows[j] = j < k ? row_of[(size_t)t * k + j] : 0;
    ws[j] = j < k ? topk_w[(size_t)t * k + j] : 0.f;
  }
  for (int c = (blockIdx.y * 256 + threadIdx.x) * 4; c < d; c += 1024 * gridDim.y) {
    const v4f_nt y0 = load_once(Y + (size_t)rows[0] * d + c);
    float4 acc = make_float4(y0[0] * ws[0], y0[1] * ws[0], y0[2] * ws[0], y0[3] * ws[0]);
#pragma unroll
    for (int j = 1; j < kMaxTopK; ++j) {
      if (j < k) {
        const v4f_nt y = load_once(Y + (size_t)rows[j] * d + c);
        acc.x = fmaf(ws[j], y[0], acc.x);
        acc.y = fmaf(ws[j], y[1], acc.y);
        acc.z = fmaf(ws[j], y[2], acc.z);
        acc.w = fmaf(ws[j], y[3], acc.w);
      }
    }
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
    o.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2*>(out + (size_t)t * d + c) = o;
  }
}

}  // namespace

hipError_t launch_route_scan(const int32_t* hist, int ntiles, int E, int bm0, int nt0, int bm1,
                             int nt1, int32_t* counts, int32_t* offsets, int32_t* tile_base,
                             int32_t* tile_off0, int32_t* tile_off1, hipStream_t stream) {
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, hist, ntiles, E, bm0, nt0,
                     bm1, nt1, counts, offsets, tile_base, tile_off0, tile_off1);
  return hipGetLastError();
}

hipError_t launch_route_place_tables(const int32_t* topk_idx, const int32_t* tile_base, int T, int E,
                                     int k, int32_t* row_of, int32_t* row_token, const int32_t* counts,
                                     const int32_t* offsets, const int32_t* tile_off0, int bm0,
                                     int nt0, int max0, int32_t* tiles0, const int32_t* tile_off1,
                                     int bm1, int nt1, int max1, int32_t* tiles1, int32_t* sched,
                                     hipStream_t stream) {
  constexpr int NTH = RT_TT * kMaxTopK;
  const int nt = ceil_div(T, RT_TT);
  const int g0 = max0 > 0 ? std::min(1024, ceil_div(max0, NTH)) : 0;
  const int g1 = max1 > 0 ? std::min(1024, ceil_div(max1, NTH)) : 0;
  hipLaunchKernelGGL(route_place_tables_kernel, dim3(nt + g0 + g1 + 1), dim3(NTH), 0, stream, topk_idx,
                     tile_base, T, E, k, row_of, row_token, nt, counts, offsets, tile_off0, bm0, nt0,
                     max0, reinterpret_cast<int4*>(tiles0), g0, tile_off1, bm1, nt1, max1,
                     reinterpret_cast<int4*>(tiles1), g1, sched);
  return hipGetLastError();
}

hipError_t launch_combine(const float* Y, const int32_t* row_of, const float* topk_w, int T, int d,
                          int k, uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(T, ceil_div(d, 1024)), dim3(256), 0, stream, Y, row_of, topk_w, T,
                     d, k, out);
  return hipGetLastError();
}

}  // namespace moe
