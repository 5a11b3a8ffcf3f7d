// Router + top-k + softmax, fused with the per-token 1x128 e4m3 activation
// quantisation (both read x once).
//
// "GPT-OSS on day 0", section "MoE": the routing kernel scores the experts,
// keeps the top-k and takes the softmax over the selected experts only (the
// max-subtracted form of section "Sink attention").  Section "GPT-OSS on
// Hopper" fixes FP8 with 128x128 block scaling; activations are quantised per
// token per 128 columns so that every 128-deep K block of the expert GEMMs has
// one activation scale per row.
//
// Design: every wave owns 16 tokens and its own LDS rows (the workgroup
// barriers only order each wave's LDS writes before its cross-lane reads).
// Per 128-column group a wave stages its x rows in LDS, quantises them, and
// accumulates fp32 logits with v_mfma_f32_16x16x4_f32,
// reading W_router [d, E] straight from memory (16 consecutive experts of one
// row are 64 contiguous bytes, exactly the B operand of one lane group).  The
// logits are summed per 128-column group and then across groups (blocked sum).
// Small batches split the K range over workgroups (partial logits in the
// workspace, then router_topk_kernel); large batches finish top-k in place.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int XP = kBlock + 4;  // LDS pitch (floats) of a staged x row

__device__ __forceinline__ uint32_t ordered_key(float v) {
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Logits of 16 tokens x (16*NBW) experts in MFMA accumulator layout: lane l
// holds token 4*(l/16)+i (register i) and expert 16*nb + l%16 (block nb).
// For every token: top-k over 64-bit keys (ordered logit bits, then the
// complemented expert index, so ties go to the lower index; absent experts
// have key 0 below every real key), softmax over the k selected logits,
// writes, and counts the picks into the tile histogram.
template <int NBW>
__device__ void topk_emit(const v4f (&tot)[NBW], const float* __restrict__ br, int t_base, int T,
                          int E, int k, int32_t* __restrict__ topk_idx,
                          float* __restrict__ topk_w, int* shist) {
  const int lane = threadIdx.x & 63;
  float bias[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int e = nb * 16 + (lane & 15);
    bias[nb] = e < E ? br[e] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t_base + 4 * (lane >> 4) + i;
    uint64_t key[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int e = nb * 16 + (lane & 15);
      key[nb] = e < E ? ((uint64_t)ordered_key(tot[nb][i] + bias[nb]) << 32) |
                            (uint64_t)(0xffffffffu - (uint32_t)e)
                      : 0ull;
    }
    float sel_l[kMaxTopK];
    int sel_e[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
      sel_l[s] = 0.f;
      sel_e[s] = 0;
      if (s < k) {
        uint64_t best = key[0];
#pragma unroll
        for (int nb = 1; nb < NBW; ++nb) best = key[nb] > best ? key[nb] : best;
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {  // within the 16 lanes of this token
          const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), o);
          const uint32_t lo = __shfl_xor((uint32_t)best, o);
          const uint64_t other = ((uint64_t)hi << 32) | lo;
          best = other > best ? other : best;
        }
        const int e = (int)(0xffffffffu - (uint32_t)best);
        sel_e[s] = e;
        sel_l[s] = key_value((uint32_t)(best >> 32));
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
          if (nb * 16 + (lane & 15) == e) key[nb] = 0ull;
      }
    }
    float ex[kMaxTopK];
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
      ex[s] = s < k ? expf(sel_l[s] - sel_l[0]) : 0.f;
      sum += ex[s];
    }
    if (t < T) {
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s) {
        if (s < k && (lane & 15) == s) {
          topk_idx[(size_t)t * k + s] = sel_e[s];
          topk_w[(size_t)t * k + s] = ex[s] / sum;
          atomicAdd(&shist[sel_e[s]], 1);
        }
      }
    }
  }
}

// W_router rows staged per step: a whole 128-row group for E <= 128, half a
// group for larger E (keeps the LDS slice at <= 64 KB).
constexpr int wr_rows(int nbw) { return nbw <= 8 ? kBlock : kBlock / 2; }

// grid = (token tiles of RT_TT, K splits); 4 waves x 16 tokens per workgroup.
// Per step the workgroup loads one W_router slice [WR_ROWS][16*NBW] into LDS
// with every load in flight, and prefetches the next slice (and, at a group
// boundary, the next x rows) into registers while the waves compute.
template <int NBW>
__global__ __launch_bounds__(256) void router_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ Wr, const float* __restrict__ br,
    int T, int d, int E, int k, int groups_per_split, float* __restrict__ partial,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ hist,
    uint8_t* __restrict__ xq, float* __restrict__ xs) {
  constexpr int EP = NBW * 16;                 // experts padded to 16
  constexpr int WP = EP + 16;                  // LDS pitch (floats) of a staged W_router row
  constexpr int WR = wr_rows(NBW);             // rows per step
  constexpr int STEPS = kBlock / WR;           // steps per 128-column group
  constexpr int WV = WR * EP / 4 / 256;        // float4 per thread per step
  static_assert(WR * EP % 1024 == 0, "slice divides over 256 threads");
  __shared__ float sxw[4][16 * XP];
  __shared__ __attribute__((aligned(16))) float sw[WR * WP];
  __shared__ int shist[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT_TT + wave * 16;  // this wave's first token
  const int ngroups = d / kBlock;
  const int g0 = blockIdx.y * groups_per_split;
  const int g1 = min(ngroups, g0 + groups_per_split);
  const bool fused = gridDim.y == 1;
  float* sx = sxw[wave];
  if (fused)
    for (int i = tid; i < E; i += 256) shist[i] = 0;

  // x rows of this wave: lane -> row lane/4, 32 columns
  const int xr = lane >> 2, xc = (lane & 3) * 32;
  const uint16_t* xrow = (t0 + xr) < T ? x + (size_t)(t0 + xr) * d + xc : nullptr;
  uint4 xv[4];
  auto load_x = [&](int g) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xv[q] = xrow ? *reinterpret_cast<const uint4*>(xrow + g * kBlock + 8 * q)
                   : make_uint4(0u, 0u, 0u, 0u);
  };
  // W_router slice: thread -> float4 number tid + 256*j of the [WR][EP] slice
  float4 wv[WV];
  auto load_w = [&](int g, int step) {
#pragma unroll
    for (int j = 0; j < WV; ++j) {
      const int f4 = tid + 256 * j;
      const int r = f4 / (EP / 4), c = (f4 % (EP / 4)) * 4;
      const size_t row = (size_t)g * kBlock + step * WR + r;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c + 3 < E && (E & 3) == 0) {  // 16-byte aligned rows
        v = *reinterpret_cast<const float4*>(Wr + row * E + c);
      } else if (c < E) {
        if (c + 3 < E) v.w = Wr[row * E + c + 3];
        v.x = Wr[row * E + c];
        if (c + 1 < E) v.y = Wr[row * E + c + 1];
        if (c + 2 < E) v.z = Wr[row * E + c + 2];
      }
      wv[j] = v;
    }
  };

  v4f tot[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) tot[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  v4f part[NBW];

  if (g0 < g1) {
    load_x(g0);
    load_w(g0, 0);
  }
  for (int g = g0; g < g1; ++g) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) part[nb] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int step = 0; step < STEPS; ++step) {
      __syncthreads();  // previous step's LDS readers are done
      if (step == 0) {  // x rows of group g as fp32
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w4[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            sx[xr * XP + xc + 8 * q + 2 * j] = bf16_to_f32(static_cast<uint16_t>(w4[j] & 0xffffu));
            sx[xr * XP + xc + 8 * q + 2 * j + 1] = bf16_to_f32(static_cast<uint16_t>(w4[j] >> 16));
          }
        }
      }
#pragma unroll
      for (int j = 0; j < WV; ++j) {
        const int f4 = tid + 256 * j;
        const int r = f4 / (EP / 4), c = (f4 % (EP / 4)) * 4;
        *reinterpret_cast<float4*>(sw + r * WP + c) = wv[j];
      }
      __syncthreads();
      // prefetch the next slice (and the next x rows) while computing this one
      if (step + 1 < STEPS) {
        load_w(g, step + 1);
      } else if (g + 1 < g1) {
        load_w(g + 1, 0);
        load_x(g + 1);
      }
      if (step == 0) {
        // quantisation of group g: s = amax/448 (1 for an all-zero group), q = e4m3(x/s)
        for (int r = 0; r < 16; ++r) {
          const int t = t0 + r;
          const float a = sx[r * XP + 2 * lane], b = sx[r * XP + 2 * lane + 1];
          const float amax = wave_max(fmaxf(fabsf(a), fabsf(b)));
          const float s = amax > 0.f ? amax / kFp8Max : 1.0f;
          const float qa = fminf(fmaxf(a / s, -kFp8Max), kFp8Max);
          const float qb = fminf(fmaxf(b / s, -kFp8Max), kFp8Max);
          if (t < T) {
            reinterpret_cast<uint16_t*>(xq + (size_t)t * d + g * kBlock)[lane] =
                static_cast<uint16_t>(f32x2_to_e4m3(qa, qb));
            if (lane == 0) xs[(size_t)t * ngroups + g] = s;
          }
        }
      }
      // logits: K = 4 per MFMA
#pragma unroll 4
      for (int k4 = 0; k4 < WR / 4; ++k4) {
        const float a = sx[(lane & 15) * XP + step * WR + 4 * k4 + (lane >> 4)];
        const float* wrow = sw + (4 * k4 + (lane >> 4)) * WP + (lane & 15);
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
          part[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, wrow[nb * 16], part[nb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) tot[nb] += part[nb];
  }

  if (!fused) {
    // partial logits [split][T][E]
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int e = nb * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * (lane >> 4) + i;
        if (t < T && e < E) partial[((size_t)blockIdx.y * T + t) * E + e] = tot[nb][i];
      }
    }
    return;
  }
  __syncthreads();  // shist cleared
  topk_emit<NBW>(tot, br, t0, T, E, k, topk_idx, topk_w, shist);
  __syncthreads();
  for (int e = tid; e < E; e += 256) hist[(size_t)blockIdx.x * E + e] = shist[e];
}

// Split-K finish: sum the partial logits of every split in split order, then
// top-k + softmax + tile histogram.  Same token mapping as router_kernel.
template <int NBW>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ partial,
                                                          int nsplit, const float* __restrict__ br,
                                                          int T, int E, int k,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w,
                                                          int32_t* __restrict__ hist) {
  __shared__ int shist[kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * RT_TT + wave * 16;
  for (int i = threadIdx.x; i < E; i += 256) shist[i] = 0;
  v4f tot[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int e = nb * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * (lane >> 4) + i;
      float s = 0.f;
      if (t < T && e < E) {
        const float* p = partial + (size_t)t * E + e;
        const size_t stride = (size_t)T * E;
        int sp = 0;
        for (; sp + 8 <= nsplit; sp += 8) {  // 8 loads in flight, summed in split order
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = p[(size_t)(sp + u) * stride];
#pragma unroll
          for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; sp < nsplit; ++sp) s += p[(size_t)sp * stride];
      }
      tot[nb][i] = s;
    }
  }
  __syncthreads();
  topk_emit<NBW>(tot, br, t0, T, E, k, topk_idx, topk_w, shist);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(size_t)blockIdx.x * E + e] = shist[e];
}

template <int NBW>
hipError_t launch_router_nbw(const uint16_t* x, const float* Wr, const float* br, int T, int d,
                             int E, int k, int nsplit, float* partial, int32_t* topk_idx,
                             float* topk_w, int32_t* hist, uint8_t* xq, float* xs,
                             hipStream_t stream) {
  const int tiles = ceil_div(T, RT_TT);
  const int ngroups = d / kBlock;
  const int gps = ceil_div(ngroups, nsplit);
  const int ns = ceil_div(ngroups, gps);
  hipLaunchKernelGGL((router_kernel<NBW>), dim3(tiles, ns), dim3(256), 0, stream, x, Wr, br, T, d,
                     E, k, gps, partial, topk_idx, topk_w, hist, xq, xs);
  if (ns > 1)
    hipLaunchKernelGGL((router_topk_kernel<NBW>), dim3(tiles), dim3(256), 0, stream, partial, ns,
                       br, T, E, k, topk_idx, topk_w, hist);
  return hipGetLastError();
}

}  // namespace

int router_splits(int T, int d) {
  if (T <= 0) return 1;
  const int waves = 4 * ceil_div(T, RT_TT);
  const int ngroups = d / kBlock;
  const int want = ceil_div(1024, waves);
  const int ns = want < ngroups ? want : ngroups;
  if (ns <= 1) return 1;
  const int gps = ceil_div(ngroups, ns);
  return ceil_div(ngroups, gps);
}

hipError_t launch_router(const uint16_t* x, const float* Wr, const float* br, int T, int d, int E,
                         int k, float* partial, int32_t* topk_idx, float* topk_w, int32_t* hist,
                         uint8_t* xq, float* xs, hipStream_t stream) {
  const int nsplit = router_splits(T, d);
  switch (ceil_div(E, 16)) {
#define MOE_ROUTER_CASE(n)                                                                     \
  case n:                                                                                      \
    return launch_router_nbw<n>(x, Wr, br, T, d, E, k, nsplit, partial, topk_idx, topk_w, hist, \
                                xq, xs, stream);
    MOE_ROUTER_CASE(1)
    MOE_ROUTER_CASE(2)
    MOE_ROUTER_CASE(3)
    MOE_ROUTER_CASE(4)
    MOE_ROUTER_CASE(5)
    MOE_ROUTER_CASE(6)
    MOE_ROUTER_CASE(7)
    MOE_ROUTER_CASE(8)
    MOE_ROUTER_CASE(9)
    MOE_ROUTER_CASE(10)
    MOE_ROUTER_CASE(11)
    MOE_ROUTER_CASE(12)
    MOE_ROUTER_CASE(13)
    MOE_ROUTER_CASE(14)
    MOE_ROUTER_CASE(15)
    MOE_ROUTER_CASE(16)
#undef MOE_ROUTER_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
