// Router + top-k + softmax, fused with the per-token e4m3 activation
// quantisation, 1x128 fp32-scaled or 1x32 MX (both read x once).
//
// "GPT-OSS on day 0", section "MoE": the routing kernel scores the experts,
// keeps the top-k and takes the softmax over the selected experts only (the
// max-subtracted form of section "Sink attention").  Section "GPT-OSS on
// Hopper" fixes FP8 with 128x128 block scaling; activations are quantised per
// token per 128 columns so that every 128-deep K block of the expert GEMMs has
// one activation scale per row.  "Hosting Qwen on Blackwell", section
// "Quantization", serves the experts in MXFP8 microscaling on Blackwell:
// there every 32 columns get an E8M0 scale.
//
// Design: every wave owns 16 tokens.  The logits run on the bf16 matrix
// cores with each fp32 router weight split into three exact bf16 parts, so
// they carry fp32 accumulation error only (see router_kernel).  Small
// batches split the K range over workgroups (partial logits in the
// workspace, summed in split order by router_finish_kernel); large batches
// finish top-k in place.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

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
// Gate weight of pick s from ex[s] = exp(l_s - l_max) and the normaliser
// (the selected logits' sum, or all logits' for kGateSoftmaxAll), optionally
// rounded to bf16.
__device__ __forceinline__ float gate_weight(float ex, float sum, int gate_mode) {
  const float w = ex / sum;
  return (gate_mode & kGateBf16) ? bf16_to_f32(f32_to_bf16(w)) : w;
}

template <int NBW>
__device__ void topk_emit(const v4f (&tot)[NBW], const float* __restrict__ br, int t_base, int T,
                          int E, int k, int gate_mode, int32_t* __restrict__ topk_idx,
                          float* __restrict__ topk_w, int* shist, int* spick = nullptr,
                          int spick_base = 0) {
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
    if (gate_mode & kGateSoftmaxAll) {  // normaliser over all E logits (xor tree: same in every lane)
      float part = 0.f;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int e = nb * 16 + (lane & 15);
        if (e < E) part += expf(tot[nb][i] + bias[nb] - sel_l[0]);
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) part += __shfl_xor(part, o);
      sum = part;
    }
    if (t < T) {
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s) {
        if (s < k && (lane & 15) == s) {
          topk_idx[(size_t)t * k + s] = sel_e[s];
          topk_w[(size_t)t * k + s] = gate_weight(ex[s], sum, gate_mode);
          atomicAdd(&shist[sel_e[s]], 1);
          if (spick) spick[(t - spick_base) * k + s] = sel_e[s];
        }
      }
    }
  }
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// fp32 -> three bf16 parts whose sum is exactly w: each part keeps the top 8
// significant bits of what the previous parts left (truncation), and a
// float's 24-bit significand splits into three such pieces.
__device__ __forceinline__ void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t b0 = __float_as_uint(w) & 0xffff0000u;
  const float r1 = w - __uint_as_float(b0);  // exact
  const uint32_t b1 = __float_as_uint(r1) & 0xffff0000u;
  const float r2 = r1 - __uint_as_float(b1);  // exact, at most 8 significant bits
  hi = b0 >> 16;
  mid = b1 >> 16;
  lo = __float_as_uint(r2) >> 16;
}

// W_router rows converted per LDS fill: a whole 128-column group for up to 64
// experts, fewer rows for more experts (the three planes stay <= 61 KB).
constexpr int w_fill(int nbw) { return nbw <= 4 ? kBlock : nbw <= 8 ? kBlock / 2 : kBlock / 4; }

// grid = (token blocks of 16 WAVES tokens, K splits); WAVES waves x 16 tokens
// per workgroup (4: one router tile; 8: two, for large batches, so that every
// converted W_router fill serves twice the tokens).
//
// Logits l = x . W_router run on v_mfma_f32_16x16x32_bf16: x is bf16 and each
// fp32 router weight is split into three bf16 parts (hi + mid + lo, exact),
// so every product x * part is exact in fp32 and the MFMA sums them in fp32:
// the logits carry fp32 accumulation error only (summed per 128-column group,
// then across groups).  The workgroup converts the W_router rows of its K
// range into three K-contiguous bf16 planes in LDS (the MFMA's B operand);
// the x fragments (A operand, 8 consecutive bf16 per lane) come straight from
// memory.  The same registers feed the per-token e4m3 quantisation of x.
// One split: top-k + softmax + tile histogram in place; several: partial
// logits [split][T][E] for router_finish_kernel.
template <int NBW, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void router_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ Wr, const float* __restrict__ br,
    int T, int d, int E, int k, int gate_mode, int mx, int groups_per_split,
    float* __restrict__ partial, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ hist, uint8_t* __restrict__ xq, void* __restrict__ xs) {
  static_assert(WAVES == 4 || WAVES == 8, "one or two router tiles per workgroup");
  constexpr int EP = NBW * 16;                   // experts padded to 16
  constexpr int KC = w_fill(NBW);                // W rows per fill
  constexpr int PITCH = 2 * KC + 16;             // bytes per expert row of a plane
  constexpr int UNITS = EP * KC / 8;             // (expert, 8 rows) conversion units
  constexpr int NTH = 64 * WAVES;                // threads
  constexpr int TPW = WAVES / 4;                 // router tiles per workgroup
  constexpr int UPT = (UNITS + NTH - 1) / NTH;   // units per thread
  constexpr int FILLS = kBlock / KC;             // fills per group
  __shared__ __attribute__((aligned(16))) uint8_t wl[3 * EP * PITCH];
  __shared__ int shist[TPW][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, gq = lane >> 4;
  const int t0 = blockIdx.x * (16 * WAVES) + wave * 16;  // this wave's first token
  const int ngroups = d / kBlock;
  const int g0 = blockIdx.y * groups_per_split;
  const int g1 = min(ngroups, g0 + groups_per_split);
  const bool fused = gridDim.y == 1;
  if (fused)
    for (int i = tid; i < TPW * kMaxExperts; i += NTH) shist[i / kMaxExperts][i % kMaxExperts] = 0;

  // x: lane holds token t0 + l16, the 8 bf16 at columns 32 c + 8 gq of a group
  const int xt = t0 + l16;
  const uint16_t* xrow = xt < T ? x + (size_t)xt * d + 8 * gq : nullptr;
  uint4 xa[4], xn[4];
  auto load_x = [&](int g, uint4 (&dst)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      dst[c] = xrow ? *reinterpret_cast<const uint4*>(xrow + g * kBlock + 32 * c)
                    : make_uint4(0u, 0u, 0u, 0u);
  };
  // W fill: unit u -> expert u % EP, rows 8 (u / EP) .. + 7 of the fill
  float wv[UPT][8];
  auto load_w = [&](int row0) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + NTH * j;
      const int e = u % EP, r8 = u / EP;
      const bool ok = u < UNITS && e < E;
#pragma unroll
      for (int i = 0; i < 8; ++i) wv[j][i] = ok ? Wr[(size_t)(row0 + 8 * r8 + i) * E + e] : 0.f;
    }
  };
  auto store_w = [&]() {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + NTH * j;
      if (u >= UNITS) continue;
      const int e = u % EP, r8 = u / EP;
      uint32_t h[8], m[8], l[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) split3(wv[j][i], h[i], m[i], l[i]);
      uint8_t* dst = wl + e * PITCH + 16 * r8;
      *reinterpret_cast<uint4*>(dst) = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16,
                                                  h[4] | h[5] << 16, h[6] | h[7] << 16);
      *reinterpret_cast<uint4*>(dst + EP * PITCH) = make_uint4(
          m[0] | m[1] << 16, m[2] | m[3] << 16, m[4] | m[5] << 16, m[6] | m[7] << 16);
      *reinterpret_cast<uint4*>(dst + 2 * EP * PITCH) = make_uint4(
          l[0] | l[1] << 16, l[2] | l[3] << 16, l[4] | l[5] << 16, l[6] | l[7] << 16);
    }
  };

  v4f tot[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) tot[nb] = v4f{0.f, 0.f, 0.f, 0.f};

  if (g0 < g1) {
    load_x(g0, xa);
    load_w(g0 * kBlock);
  }
  for (int g = g0; g < g1; ++g) {
    // ---- quantisation of x for the wave's 16 tokens: row l16's 128
    // values sit in the four lanes l16 + 16 gq
    {
      float v[32];
      float am = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w4[4] = {xa[c].x, xa[c].y, xa[c].z, xa[c].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[8 * c + 2 * q] = bf16_to_f32(static_cast<uint16_t>(w4[q] & 0xffffu));
          v[8 * c + 2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(w4[q] >> 16));
        }
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) am = nan_max(am, fabsf(v[i]));
      am = nan_max(am, __shfl_xor(am, 16));
      am = nan_max(am, __shfl_xor(am, 32));
      const float s = group_scale(am);
      if (mx) {
        // MXFP8: columns 32c..32c+31 of the group are one block, held 8 per
        // lane by the four lanes l16 + 16 gq; E8M0 codes of the 4 blocks -> one dword
        uint32_t codes = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float bm = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) bm = nan_max(bm, fabsf(v[8 * c + i]));
          bm = nan_max(bm, __shfl_xor(bm, 16));
          bm = nan_max(bm, __shfl_xor(bm, 32));
          const uint32_t code = mx_code(bm);
          const float inv = mx_inv_scale(code);
          if (xt < T)
            *reinterpret_cast<uint2*>(xq + (size_t)xt * d + g * kBlock + 32 * c + 8 * gq) = make_uint2(
                f32x4_to_e4m3(v[8 * c] * inv, v[8 * c + 1] * inv, v[8 * c + 2] * inv, v[8 * c + 3] * inv),
                f32x4_to_e4m3(v[8 * c + 4] * inv, v[8 * c + 5] * inv, v[8 * c + 6] * inv,
                              v[8 * c + 7] * inv));
          codes |= code << (8 * c);
        }
        if (xt < T && gq == 0)
          reinterpret_cast<uint32_t*>(xs)[(size_t)xt * ngroups + g] = codes;
      } else {
        // v / s for the 32 values of one scale.  With the correctly rounded
        // reciprocal y, q0 = v y and the residual v - q0 s (exact by fma),
        // q0 + residual * y is the IEEE quotient wherever |v / s| >= 2^-10,
        // and smaller quotients get the same e4m3 code (a zero of v's sign):
        // checked exhaustively over every bf16 group maximum with
        // s >= 2^-64 and every bf16 value up to it.  A wave with a smaller,
        // an infinite or a NaN scale divides.
        const bool quick = __all(xt >= T || (s >= 0x1p-64f && s < __builtin_inff()));
        const float y = 1.0f / s;
        auto put = [&](int c, const float (&q)[8]) {
          *reinterpret_cast<uint2*>(xq + (size_t)xt * d + g * kBlock + 32 * c + 8 * gq) =
              make_uint2(f32x4_to_e4m3(q[0], q[1], q[2], q[3]), f32x4_to_e4m3(q[4], q[5], q[6], q[7]));
        };
        if (xt < T) {
          if (quick) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              float q[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                const float a = v[8 * c + i], q0 = a * y;
                q[i] = clamp_fp8(copysignf(fmaf(fmaf(-q0, s, a), y, q0), a));
              }
              put(c, q);
            }
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              float q[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) q[i] = clamp_fp8(v[8 * c + i] / s);
              put(c, q);
            }
          }
          if (gq == 0) reinterpret_cast<float*>(xs)[(size_t)xt * ngroups + g] = s;
        }
      }
    }
    v4f part[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) part[nb] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int f = 0; f < FILLS; ++f) {
      __syncthreads();  // the previous fill's readers are done
      store_w();
      __syncthreads();
      // prefetch the next fill (and, at the group's first fill, the next group's x)
      if (f + 1 < FILLS) load_w(g * kBlock + (f + 1) * KC);
      else if (g + 1 < g1) load_w((g + 1) * kBlock);
      if (f == 0 && g + 1 < g1) load_x(g + 1, xn);
#pragma unroll
      for (int sc = 0; sc < KC / 32; ++sc) {
        const v8bf a = __builtin_bit_cast(v8bf, xa[f * (KC / 32) + sc]);
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const uint8_t* pb = wl + (16 * nb + l16) * PITCH + 64 * sc + 16 * gq;
#pragma unroll
          for (int pl = 0; pl < 3; ++pl) {
            const v8bf b = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(pb + pl * EP * PITCH));
            part[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, part[nb], 0, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) tot[nb] += part[nb];
#pragma unroll
    for (int c = 0; c < 4; ++c) xa[c] = xn[c];
  }

  if (!fused) {
    // partial logits [split][T][EP] (padded experts hold 0): lane holds tokens
    // 4 gq + i, expert 16 nb + l16
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int e = nb * 16 + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * gq + i;
        if (t < T) partial[((size_t)blockIdx.y * T + t) * EP + e] = tot[nb][i];
      }
    }
    // the finish kernel adds its token blocks' picks into the tile histogram
    if (blockIdx.y == 0)
      for (int i = tid; i < TPW * E; i += NTH) {
        const int rt = blockIdx.x * TPW + i / E;  // router tile
        if (rt * RT_TT < T) hist[(size_t)rt * E + i % E] = 0;
      }
    return;
  }
  __syncthreads();  // shist cleared
  topk_emit<NBW>(tot, br, t0, T, E, k, gate_mode, topk_idx, topk_w, shist[wave >> 2]);
  __syncthreads();
  for (int i = tid; i < TPW * E; i += NTH) {
    const int rt = blockIdx.x * TPW + i / E;  // router tile
    if (rt * RT_TT < T) hist[(size_t)rt * E + i % E] = shist[i / E][i % E];
  }
}

// Lane exchanges inside the aligned group of eight lanes (half a DPP row):
// swap neighbours, swap pairs, then mirror the half row, so after the three
// steps every lane of the group has combined all eight values.  DPP moves
// read the other lane's register directly (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
constexpr int kDppSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i of a half row reads lane 7 - i

template <int CTRL>
__device__ __forceinline__ uint64_t max_step(uint64_t v) {
  const uint64_t o = ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
  return o > v ? o : v;
}
__device__ __forceinline__ uint64_t max8(uint64_t v) {
  return max_step<kDppHalfMirror>(max_step<kDppSwap2>(max_step<kDppSwap1>(v)));
}
// Sum over the group; the same value in all eight lanes (each step adds a
// pair of values that the partner lane adds in the other order).
template <int CTRL>
__device__ __forceinline__ float sum_step(float v) {
  return v + __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
__device__ __forceinline__ float sum8(float v) {
  return sum_step<kDppHalfMirror>(sum_step<kDppSwap2>(sum_step<kDppSwap1>(v)));
}

// Top-k + softmax of the RT_TT tokens tt0.. of a router tile with eight lanes
// per token (all 512 threads of the workgroup), from their logits in LDS (sl
// [RT_TT][EP + 8]: the eight tokens of a wave start 8 banks apart, so a
// wave's 64 reads of one round hit 64 distinct banks).
// Lane j of a token's group holds the 64-bit keys of experts j, j + 8, ...
// (ordered logit bits, then the complemented expert index, so ties go to the
// lower index and every pick is a valid, distinct expert); each of the k
// rounds takes the group maximum with three register exchanges (max8) and
// clears the winner.  Lane s < k of the group writes pick s and its weight (softmax over
// the selected logits, or over all E for kGateSoftmaxAll), counts it in the
// tile histogram and, when given, records it in spick and the token's bit in
// the expert's token mask.
template <int EP>
__device__ __forceinline__ void topk_group8(const float* sl, const float* sbr, int tt0, int T, int E, int k,
                            int gate_mode, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                            int* shist, int* spick, uint32_t* smask_lo, uint32_t* smask_hi) {
  constexpr int KPL = EP / 8;  // keys per lane
  const int tl = threadIdx.x >> 3, sub = threadIdx.x & 7;
  const int t = tt0 + tl;
  const float* row = sl + tl * (EP + 8);
  uint64_t key[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {  // reads stay inside sl and sbr for every lane: no branch
    const int e = 8 * j + sub;
    const uint64_t kv = ((uint64_t)ordered_key(row[e] + sbr[e]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
    key[j] = (t < T && e < E) ? kv : 0ull;
  }
  // round s: the group maximum (the same in all eight lanes) is pick s; lane
  // s of the group keeps it, so each lane < k then finishes one pick
  uint64_t first = 0ull, mine = 0ull;
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) {
    if (s < k) {
      uint64_t best = key[0];
#pragma unroll
      for (int j = 1; j < KPL; ++j) best = key[j] > best ? key[j] : best;
      best = max8(best);
      if (s == 0) first = best;
      if (sub == s) mine = best;
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        if (key[j] == best) key[j] = 0ull;
    }
  }
  if (t >= T) return;
  const float l0 = key_value((uint32_t)(first >> 32));
  const bool owner = sub < k;
  const float ex = owner ? expf(key_value((uint32_t)(mine >> 32)) - l0) : 0.f;
  float sum = sum8(ex);  // sum of the k selected exponentials (0 from lanes >= k)
  if (gate_mode & kGateSoftmaxAll) {  // normaliser over all E logits (lane sums, then the group sum)
    float part = 0.f;
    for (int e = sub; e < E; e += 8) part += expf(row[e] + sbr[e] - l0);
    sum = sum8(part);
  }
  if (owner) {
    const int e = (int)(0xffffffffu - (uint32_t)mine);
    topk_idx[(size_t)t * k + sub] = e;
    topk_w[(size_t)t * k + sub] = gate_weight(ex, sum, gate_mode);
    atomicAdd(&shist[e], 1);
    if (spick) spick[tl * k + sub] = e;
    if (smask_lo) atomicOr(tl < 32 ? &smask_lo[e] : &smask_hi[e], 1u << (tl & 31));
  }
}

// Logits of ntok (<= RT_TT) tokens from tt0 into sl [RT_TT][EP + 8] (the
// pitch of topk_group8): the sum of every (token, expert) partial in split
// order.  A
// thread takes 4 experts of one token (one float4 per split); up to 24 splits
// are in flight at once, so a K range of up to 24 splits costs one memory
// round trip.
template <int EP>
__device__ void sum_partials(const float* __restrict__ partial, int nsplit, int T, int tt0,
                             float* sl, int nthreads, int ntok = RT_TT) {
  constexpr int Q = EP / 4;
  constexpr int kInFlight = 24;
  const size_t stride = (size_t)T * EP;
  for (int q = threadIdx.x; q < ntok * Q; q += nthreads) {
    const int tl = q / Q, e4 = 4 * (q % Q);
    const int t = tt0 + tl;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < T) {
      const float* p = partial + (size_t)t * EP + e4;
      for (int s0 = 0; s0 < nsplit; s0 += kInFlight) {
        float4 v[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j)
          v[j] = s0 + j < nsplit ? *reinterpret_cast<const float4*>(p + (s0 + j) * stride)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
        // selects rather than a skipped add: every loaded register is consumed
        // on every path, so no load stays in flight past this loop (on this
        // chip a wait for loads also waits for the stores issued before it)
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
          const bool in = s0 + j < nsplit;
          s.x = in ? s.x + v[j].x : s.x;
          s.y = in ? s.y + v[j].y : s.y;
          s.z = in ? s.z + v[j].z : s.z;
          s.w = in ? s.w + v[j].w : s.w;
        }
      }
    }
    float* dst = sl + tl * (EP + 8) + e4;
    dst[0] = s.x;
    dst[1] = s.y;
    dst[2] = s.z;
    dst[3] = s.w;
  }
}

// Split-K finish for a block of ntok tokens (a whole router tile, or a
// quarter of one when the batch has few tiles, so that a tile's partial
// reads spread over four CUs): the logit of every (token, expert) is the sum
// of its partials in split order; then top-k + softmax, and the block's
// picks are added to its router tile's histogram (integer atomics: the
// counts do not depend on the order; the router kernel zeroed the row).
template <int NBW>
__global__ __launch_bounds__(512) void router_finish_kernel(const float* __restrict__ partial,
                                                             int nsplit, const float* __restrict__ br,
                                                             int T, int E, int k, int gate_mode,
                                                             int32_t* __restrict__ topk_idx,
                                                             float* __restrict__ topk_w,
                                                             int32_t* __restrict__ hist, int ntok) {
  constexpr int EP = NBW * 16;
  __shared__ float sl[RT_TT * (EP + 8)];
  __shared__ int shist[kMaxExperts];
  __shared__ float sbr[512];  // entries >= E are written but never read
  const int tid = threadIdx.x;
  const int tt0 = blockIdx.x * ntok;
  const int tend = min(T, tt0 + ntok);
  const float brv = tid < E ? br[tid] : 0.f;
  if (tid < E) shist[tid] = 0;
  sum_partials<EP>(partial, nsplit, T, tt0, sl, 512, ntok);
  sbr[tid] = brv;
  __syncthreads();  // the sums are in LDS, shist and sbr are set
  topk_group8<EP>(sl, sbr, tt0, tend, E, k, gate_mode, topk_idx, topk_w, shist, nullptr, nullptr,
                  nullptr);
  __syncthreads();  // the histogram atomics are done
  if (tid < E && shist[tid] != 0) atomicAdd(&hist[(size_t)(tt0 / RT_TT) * E + tid], shist[tid]);
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts scan each
// 16-lane row, then the row totals (lanes 15, 31, 47) are added to the rows
// above them.  Integer adds, so the order does not matter.
__device__ __forceinline__ int scan64(int v) {
  v += (int)__builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr 1
  v += (int)__builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr 2
  v += (int)__builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr 4
  v += (int)__builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr 8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// All routing of a batch that fits one router tile (T <= RT_TT, the decode
// regime) in one workgroup: the split partials are summed in split order,
// then top-k + softmax, the expert counts and offsets (exclusive scan), the
// stable placement of every (token, slot) pair, and the tile lists of both
// GEMMs (the same entries as route_place_tables_kernel writes).  With one split the router
// already chose the experts (have_topk) and only the rest runs here.
template <int NBW>
__global__ __launch_bounds__(512) void route_small_kernel(
    const float* __restrict__ partial, int nsplit, bool have_topk, const float* __restrict__ br,
    int T, int E, int k, int gate_mode, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ tile_off0,
    int32_t* __restrict__ tile_off1, int4* __restrict__ tiles0, int4* __restrict__ tiles1, int bm0,
    int nt0, int max0, int bm1, int nt1, int max1, int32_t* __restrict__ row_of,
    int32_t* __restrict__ row_token) {
  constexpr int EP = NBW * 16;
  static_assert(RT_TT * 8 == 512, "the top-k takes eight lanes per token");
  __shared__ float sl[RT_TT * (EP + 8)];
  __shared__ int spick[RT_TT * kMaxTopK];
  __shared__ int scnt[kMaxExperts], soff[kMaxExperts + 1], so0[kMaxExperts + 1], so1[kMaxExperts + 1];
  __shared__ uint32_t smask[2][kMaxExperts];  // tokens (bits) that chose each expert
  const int tid = threadIdx.x;
  const int R = T * k;
  __shared__ float sbr[512];  // entries >= E are written but never read
  static_assert(kMaxExperts <= 512, "one bias per thread");
  // the bias load is issued before the partial loads, so both share one
  // round trip to memory; every thread stores its value (0 past E), so the
  // load is consumed on every path and no later wait has to cover it
  const float brv = tid < E ? br[tid] : 0.f;
  if (tid < E) {
    scnt[tid] = 0;
    smask[0][tid] = smask[1][tid] = 0u;
  }
  if (!have_topk) {
    sum_partials<EP>(partial, nsplit, T, 0, sl, 512);
  } else {
    for (int p = tid; p < R; p += 512) spick[p] = topk_idx[p];
  }
  sbr[tid] = brv;
  __syncthreads();
  if (!have_topk) {
    topk_group8<EP>(sl, sbr, 0, T, E, k, gate_mode, topk_idx, topk_w, scnt, spick, smask[0], smask[1]);
  } else {
    for (int p = tid; p < R; p += 512) {
      const int t = p / k;
      atomicAdd(&scnt[spick[p]], 1);
      atomicOr(&smask[t >> 5][spick[p]], 1u << (t & 31));
    }
  }
  __syncthreads();
  // exclusive scans, one per wave: wave 0 the counts (row offsets), waves 1
  // and 2 the two GEMMs' tiles per expert (tile offsets); lane l takes
  // experts 4l .. 4l + 3
  if (tid < 192) {
    const int w = tid >> 6, l = tid & 63;
    const int bm = w == 1 ? bm0 : bm1, ntl = w == 1 ? nt0 : nt1;
    int v[4], r = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * l + q;
      const int c = e < E ? scnt[e] : 0;
      v[q] = w == 0 ? c : ceil_div(c, bm) * ntl;
      r += v[q];
    }
    const int inc = scan64(r);
    int pre = inc - r;
    int* dst = w == 0 ? soff : w == 1 ? so0 : so1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * l + q;
      if (e < E) dst[e] = pre;
      pre += v[q];
    }
    if (l == 63) dst[E] = inc;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += 512) {
    if (e < E) counts[e] = scnt[e];
    offsets[e] = soff[e];
    tile_off0[e] = so0[e];
    tile_off1[e] = so1[e];
  }
  // stable placement: the rank of pair (t, j) within its expert is the number
  // of earlier tokens that chose the expert (a token picks an expert once)
  for (int p = tid; p < R; p += 512) {
    const int e = spick[p], t = p / k;
    const uint32_t below = (1u << (t & 31)) - 1u;
    const int rank = t < 32 ? __popc(smask[0][e] & below)
                            : __popc(smask[0][e]) + __popc(smask[1][e] & below);
    const int row = soff[e] + rank;
    row_of[p] = row;
    row_token[row] = t;
  }
  // tile lists: tpe threads per expert, thread j of an expert's team writes
  // the expert's tiles j, j + tpe, ... (inside the expert: column group of
  // kTileGroup tiles, row block, column tile); all experts at once, so the
  // LDS reads of every expert share one round trip
  const int tpe = E < 512 ? 512 / E : 1;
  const int e = tid / tpe, j0 = tid - e * tpe;
  if (e < E) {
    const int cnt = scnt[e], row0 = soff[e];
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int* so = pass == 0 ? so0 : so1;
      const int bm = pass == 0 ? bm0 : bm1, n_tiles = pass == 0 ? nt0 : nt1;
      const int max_tiles = pass == 0 ? max0 : max1;
      int4* tiles = pass == 0 ? tiles0 : tiles1;
      const int first = so[e];
      const int n = min(so[e + 1], max_tiles) - first;
      const int mt = ceil_div(cnt, bm);
      for (int local = j0; local < n; local += tpe) {
        if (cnt <= bm) {  // one row block: the entries are the column tiles in order
          tiles[first + local] = make_int4(e, row0, cnt, local);
          continue;
        }
        const int ng = local / (mt * kTileGroup);
        const int rem = local - ng * mt * kTileGroup;
        const int gw = min(kTileGroup, n_tiles - ng * kTileGroup);
        const int m = rem / gw;
        tiles[first + local] =
            make_int4(e, row0 + m * bm, min(bm, cnt - m * bm), ng * kTileGroup + rem % gw);
      }
    }
  }
}

template <int NBW>
hipError_t launch_router_nbw(const uint16_t* x, const float* Wr, const float* br, int T, int d,
                             int E, int k, int gate_mode, bool mx, int nsplit, float* partial,
                             int32_t* topk_idx, float* topk_w, int32_t* hist, uint8_t* xq, void* xs,
                             const SmallRoute* sr, hipStream_t stream) {
  const int tiles = ceil_div(T, RT_TT);
  const int ngroups = d / kBlock;
  const int gps = ceil_div(ngroups, nsplit);
  const int ns = ceil_div(ngroups, gps);
  const int waves = router_waves(T, E);
  if constexpr (NBW <= 8) {
    if (waves == 8) {
      hipLaunchKernelGGL((router_kernel<NBW, 8>), dim3(ceil_div(T, 16 * 8), ns), dim3(64 * 8), 0, stream,
                         x, Wr, br, T, d, E, k, gate_mode, mx ? 1 : 0, gps, partial, topk_idx, topk_w,
                         hist, xq, xs);
    }
  }
  if (waves == 4)
    hipLaunchKernelGGL((router_kernel<NBW, 4>), dim3(tiles, ns), dim3(64 * 4), 0, stream, x, Wr, br, T,
                       d, E, k, gate_mode, mx ? 1 : 0, gps, partial, topk_idx, topk_w, hist, xq, xs);
  if (sr != nullptr)
    hipLaunchKernelGGL((route_small_kernel<NBW>), dim3(1), dim3(512), 0, stream, partial, ns, ns == 1,
                       br, T, E, k, gate_mode, topk_idx, topk_w, sr->counts, sr->offsets, sr->tile_off0,
                       sr->tile_off1, reinterpret_cast<int4*>(sr->tiles0),
                       reinterpret_cast<int4*>(sr->tiles1), sr->bm0, sr->nt0, sr->max0, sr->bm1,
                       sr->nt1, sr->max1, sr->row_of, sr->row_token);
  else if (ns > 1) {
    // quarter tiles while the batch has fewer tiles than half the CUs
    const int ntok = tiles < 128 ? RT_TT / 4 : RT_TT;
    hipLaunchKernelGGL((router_finish_kernel<NBW>), dim3(ceil_div(T, ntok)), dim3(512), 0, stream,
                       partial, ns, br, T, E, k, gate_mode, topk_idx, topk_w, hist, ntok);
  }
  return hipGetLastError();
}

}  // namespace

int router_waves(int T, int E) { return (T >= 2048 && ceil_div(E, 16) <= 8) ? 8 : 4; }

int router_splits(int T, int d, int E) {
  if (T <= 0) return 1;
  const int ngroups = d / kBlock;
  // about two 4-wave or one 8-wave workgroup per CU
  const int want = router_waves(T, E) == 8 ? ceil_div(256, ceil_div(T, 16 * 8)) : ceil_div(512, ceil_div(T, RT_TT));
  const int ns = want < ngroups ? want : ngroups;
  if (ns <= 1) return 1;
  const int gps = ceil_div(ngroups, ns);
  return ceil_div(ngroups, gps);
}

hipError_t launch_router(const uint16_t* x, const float* Wr, const float* br, int T, int d, int E,
                         int k, int gate_mode, bool mx, float* partial, int32_t* topk_idx,
                         float* topk_w, int32_t* hist, uint8_t* xq, void* xs, const SmallRoute* sr,
                         hipStream_t stream) {
  const int nsplit = router_splits(T, d, E);
  switch (ceil_div(E, 16)) {
#define MOE_ROUTER_CASE(n)                                                                     \
  case n:                                                                                      \
    return launch_router_nbw<n>(x, Wr, br, T, d, E, k, gate_mode, mx, nsplit, partial, topk_idx, \
                                topk_w, hist, xq, xs, sr, stream);
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
