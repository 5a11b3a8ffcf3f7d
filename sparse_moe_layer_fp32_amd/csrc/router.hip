// Router + top-k + softmax, fused with the per-token 1x128 e4m3 activation
// quantisation (both read x once).
//
// "GPT-OSS on day 0", section "MoE": the routing kernel scores the experts,
// keeps the top-k and takes the softmax over the selected experts only (the
// max-subtracted form of section "Sink attention").  Section "GPT-OSS on
// Hopper" fixes FP8 with 128x128 block scaling; activations are quantised per
// token per 128 columns so that every 128-long K block of the expert GEMMs has
// one activation scale per row.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int RT_KC = 32;  // router rows staged in LDS per step

__device__ __forceinline__ uint32_t ordered_key(float v) {
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// One workgroup = RT_TT tokens, 4 waves; wave w owns tokens 4w..4w+3 of the
// tile for quantisation, logits and top-k.  Lane l owns experts l + 64*j.
template <int EJ>
__global__ __launch_bounds__(256) void router_quant_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ Wr, const float* __restrict__ br,
    int T, int d, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ hist, uint8_t* __restrict__ xq, float* __restrict__ xs) {
  constexpr int EP = EJ * 64;
  __shared__ float sx[RT_TT][kBlock + 4];
  __shared__ float sw[RT_KC][EP];
  __shared__ int shist[EP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT_TT;
  const int ngroups = d / kBlock;
  for (int i = tid; i < EP; i += 256) shist[i] = 0;

  float total[4][EJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < EJ; ++j) total[i][j] = 0.f;

  for (int c = 0; c < ngroups; ++c) {
    __syncthreads();
    {  // x chunk [16 tokens][128] -> fp32 in LDS
      const int tt = tid >> 4, cc = (tid & 15) * 8, t = t0 + tt;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (t < T) v = *reinterpret_cast<const uint4*>(x + (size_t)t * d + c * kBlock + cc);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sx[tt][cc + 2 * q] = bf16_to_f32(static_cast<uint16_t>(w4[q] & 0xffffu));
        sx[tt][cc + 2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(w4[q] >> 16));
      }
    }
    __syncthreads();
    // activation quantisation of this 128-column group: s = amax/448, q = e4m3(x/s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = wave * 4 + i, t = t0 + tt;
      const float a = sx[tt][2 * lane], b = sx[tt][2 * lane + 1];
      const float amax = wave_max(fmaxf(fabsf(a), fabsf(b)));
      const float s = amax > 0.f ? amax / kFp8Max : 1.0f;
      const float qa = fminf(fmaxf(a / s, -kFp8Max), kFp8Max);
      const float qb = fminf(fmaxf(b / s, -kFp8Max), kFp8Max);
      if (t < T) {
        reinterpret_cast<uint16_t*>(xq + (size_t)t * d + c * kBlock)[lane] =
            static_cast<uint16_t>(f32x2_to_e4m3(qa, qb));
        if (lane == 0) xs[(size_t)t * ngroups + c] = s;
      }
    }
    // router logits: blocked sum, one partial per 128-column group
    float part[4][EJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < EJ; ++j) part[i][j] = 0.f;
    for (int sub = 0; sub < kBlock / RT_KC; ++sub) {
      __syncthreads();
      const size_t r0 = (size_t)c * kBlock + sub * RT_KC;
      for (int i = tid; i < RT_KC * EP; i += 256) {
        const int r = i / EP, e = i - r * EP;
        sw[r][e] = e < E ? Wr[(r0 + r) * E + e] : 0.f;
      }
      __syncthreads();
#pragma unroll 4
      for (int kk = 0; kk < RT_KC; ++kk) {
        float xv[4], wv[EJ];
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[i] = sx[wave * 4 + i][sub * RT_KC + kk];
#pragma unroll
        for (int j = 0; j < EJ; ++j) wv[j] = sw[kk][lane + 64 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < EJ; ++j) part[i][j] = fmaf(xv[i], wv[j], part[i][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < EJ; ++j) total[i][j] += part[i][j];
  }

  // top-k per token: k rounds of a wave-wide argmax over 64-bit keys
  // (ordered logit bits, then the complement of the expert index so that ties
  // go to the lower index).  Removed or absent experts have key 0, below every
  // real key, so every pick is a valid, distinct expert.
  float bias[EJ];
#pragma unroll
  for (int j = 0; j < EJ; ++j) bias[j] = (lane + 64 * j) < E ? br[lane + 64 * j] : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + wave * 4 + i;
    uint64_t key[EJ];
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
      const int e = lane + 64 * j;
      key[j] = e < E ? ((uint64_t)ordered_key(total[i][j] + bias[j]) << 32) |
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
        for (int j = 1; j < EJ; ++j) best = key[j] > best ? key[j] : best;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), o);
          const uint32_t lo = __shfl_xor((uint32_t)best, o);
          const uint64_t other = ((uint64_t)hi << 32) | lo;
          best = other > best ? other : best;
        }
        const int e = (int)(0xffffffffu - (uint32_t)best);
        sel_e[s] = e;
        sel_l[s] = key_value((uint32_t)(best >> 32));
#pragma unroll
        for (int j = 0; j < EJ; ++j)
          if (lane + 64 * j == e) key[j] = 0ull;
      }
    }
    // softmax over the selected logits (descending, so sel_l[0] is the max)
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
        if (s < k && lane == s) {
          topk_idx[(size_t)t * k + s] = sel_e[s];
          topk_w[(size_t)t * k + s] = ex[s] / sum;
          atomicAdd(&shist[sel_e[s]], 1);
        }
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) hist[(size_t)blockIdx.x * E + e] = shist[e];
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const float* Wr, const float* br, int T, int d, int E,
                         int k, int32_t* topk_idx, float* topk_w, int32_t* hist, uint8_t* xq,
                         float* xs, hipStream_t stream) {
  const int nt = ceil_div(T, RT_TT);
  const int ej = ceil_div(E, 64);
  switch (ej) {
    case 1:
      hipLaunchKernelGGL(router_quant_kernel<1>, dim3(nt), dim3(256), 0, stream, x, Wr, br, T, d, E,
                         k, topk_idx, topk_w, hist, xq, xs);
      break;
    case 2:
      hipLaunchKernelGGL(router_quant_kernel<2>, dim3(nt), dim3(256), 0, stream, x, Wr, br, T, d, E,
                         k, topk_idx, topk_w, hist, xq, xs);
      break;
    case 3:
      hipLaunchKernelGGL(router_quant_kernel<3>, dim3(nt), dim3(256), 0, stream, x, Wr, br, T, d, E,
                         k, topk_idx, topk_w, hist, xq, xs);
      break;
    default:
      hipLaunchKernelGGL(router_quant_kernel<4>, dim3(nt), dim3(256), 0, stream, x, Wr, br, T, d, E,
                         k, topk_idx, topk_w, hist, xq, xs);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
