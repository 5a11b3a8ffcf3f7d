// Grouped FP8 GEMMs of the experts on the gfx950 matrix cores.
//
// "GPT-OSS on day 0": section "GPT-OSS on Hopper" serves the experts in FP8
// with 128x128 block scaling and gives them SwiGLU and biases; section "MoE"
// puts the bias into the GEMM by initialising the accumulators from it once
// per output tile; section "Performance optimizations" notes that the launch
// grid has to be chosen for the 2880-wide hidden size.  "Hosting Qwen on
// Blackwell", sections "Prefiller" and "Decoder": prefill batches make the
// MoE GEMM dense and compute-bound, decode batches are bound by loading the
// weights from HBM.  "Disaggregated prefill and decode", section "Prefill vs
// decode performance": small token batches leave a single M block.
//
// Design (MI355X): one workgroup = 4 waves computes a BM x BNP tile of one
// expert.  Per 128-deep K block it stages A (gathered activation rows, K
// contiguous) and B (weights, stored K x N with N contiguous, transposed to
// K-contiguous columns through registers) in LDS, then every wave runs
// v_mfma_f32_16x16x128_f8f6f4 on 16x16 blocks.  Each MFMA covers exactly one
// scale block, so its fp32 result is promoted into the accumulator with the
// product of the row's activation scale and the block's weight scale.
// Tiles are taken from a device-side table (expert, row block, column block),
// grouped so that tiles sharing weights run together on one XCD (L2).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int KP = 144;      // LDS pitch (bytes) of a staged row/column: 128 + 16
constexpr int B_COLQ = 16;   // extra bytes after every 16 staged B columns (bank spread)
constexpr int GN = 4;        // column tiles per group in the tile order

template <int BM, int BNP, int WAVES_M, int WAVES_N, bool GATED>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs g) {
  constexpr int WM = BM / WAVES_M;
  constexpr int WN = BNP / WAVES_N;
  constexpr int MB = WM / 16;
  constexpr int NB = WN / 16;
  constexpr int A_LOADS = BM * 8 / 256;
  constexpr int B_GROUPS = BNP / 16;
  constexpr int KR = 128 * B_GROUPS / 256;
  constexpr int SA_BYTES = BM * KP;
  constexpr int SB_BYTES = BNP * KP + B_GROUPS * B_COLQ;
  static_assert(WAVES_M * WAVES_N == 4, "4 waves");
  static_assert(KR == 4 || KR == 8, "B staging rows");
  static_assert(A_LOADS >= 1, "A staging");
  static_assert(!GATED || BNP == 256, "gated tile = 128 gate + 128 up columns");
  static_assert(GATED || WN <= 128, "one weight-scale block per wave");
  static_assert(!GATED || NB % 2 == 0, "gate/up pairs");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SA_BYTES + SB_BYTES + BM * 4];
  uint8_t* sA = smem;
  uint8_t* sB = smem + SA_BYTES;
  float* sAs = reinterpret_cast<float*>(smem + SA_BYTES + SB_BYTES);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int K = g.K, N = g.N, nkb = K / kBlock, nsb = N / kBlock;

  // ---- which tile: XCD-contiguous slice of the tile table
  const int total = g.tile_off[g.E];
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  if (slot >= chunk) return;
  const int L = xcd * chunk + slot;
  if (L >= total) return;
  int lo = 0, hi = g.E;  // tile_off[lo] <= L < tile_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.tile_off[mid] <= L) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int cnt = g.counts[e];
  const int mt = ceil_div(cnt, BM);
  const int local = L - g.tile_off[e];
  const int ng = local / (mt * GN);
  const int rem = local - ng * mt * GN;
  const int gw = min(GN, g.n_tiles - ng * GN);
  const int m = rem / gw, nt = ng * GN + rem % gw;
  const int row0 = g.offsets[e] + m * BM;
  const int valid = min(BM, cnt - m * BM);
  const int n0 = nt * (GATED ? kBlock : BNP);  // gated: first h column; plain: first column

  // global column of tile column p
  auto gcol_of = [&](int p) -> int {
    if (GATED) return p < BNP / 2 ? n0 + p : g.f + n0 + (p - BNP / 2);
    return n0 + p;
  };

  // ---- staging sources (fixed for the tile)
  const uint8_t* a_src[A_LOADS];
  int a_lds[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int idx = tid + 256 * i, r = idx >> 3, seg = idx & 7;
    a_lds[i] = r * KP + seg * 16;
    a_src[i] = nullptr;
    if (r < valid) {
      const int arow = GATED ? g.row_token[row0 + r] : row0 + r;
      a_src[i] = g.A + (size_t)arow * K + seg * 16;
    }
  }
  const float* as_src = nullptr;
  if (tid < valid) {
    const int arow = GATED ? g.row_token[row0 + tid] : row0 + tid;
    as_src = g.As + (size_t)arow * nkb;
  }
  const int bgrp = tid % B_GROUPS, kgrp = tid / B_GROUPS;
  const int bgcol = gcol_of(bgrp * 16);
  const uint8_t* b_src =
      bgcol < N ? g.B + (size_t)e * K * N + (size_t)(kgrp * KR) * N + bgcol : nullptr;
  const int b_lds = bgrp * 16 * KP + bgrp * B_COLQ + kgrp * KR;

  uint4 ra[A_LOADS];
  uint4 rb[KR];
  float ras = 0.f;
  auto stage_load = [&](int kb) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      ra[i] = a_src[i] ? *reinterpret_cast<const uint4*>(a_src[i] + kb * kBlock)
                       : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int r = 0; r < KR; ++r)
      rb[r] = b_src ? *reinterpret_cast<const uint4*>(b_src + (size_t)(kb * kBlock + r) * N)
                    : make_uint4(0u, 0u, 0u, 0u);
    ras = as_src ? as_src[kb] : 0.f;
  };
  auto stage_store = [&]() {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) *reinterpret_cast<uint4*>(sA + a_lds[i]) = ra[i];
    if (tid < BM) sAs[tid] = ras;
    // KR rows x 16 columns (bytes) -> 16 columns x KR rows
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w0 = q == 0 ? rb[0].x : q == 1 ? rb[0].y : q == 2 ? rb[0].z : rb[0].w;
      const uint32_t w1 = q == 0 ? rb[1].x : q == 1 ? rb[1].y : q == 2 ? rb[1].z : rb[1].w;
      const uint32_t w2 = q == 0 ? rb[2].x : q == 1 ? rb[2].y : q == 2 ? rb[2].z : rb[2].w;
      const uint32_t w3 = q == 0 ? rb[3].x : q == 1 ? rb[3].y : q == 2 ? rb[3].z : rb[3].w;
      uint32_t c0, c1, c2, c3;
      transpose4x4(w0, w1, w2, w3, c0, c1, c2, c3);
      if constexpr (KR == 8) {
        const uint32_t w4 = q == 0 ? rb[4].x : q == 1 ? rb[4].y : q == 2 ? rb[4].z : rb[4].w;
        const uint32_t w5 = q == 0 ? rb[5].x : q == 1 ? rb[5].y : q == 2 ? rb[5].z : rb[5].w;
        const uint32_t w6 = q == 0 ? rb[6].x : q == 1 ? rb[6].y : q == 2 ? rb[6].z : rb[6].w;
        const uint32_t w7 = q == 0 ? rb[7].x : q == 1 ? rb[7].y : q == 2 ? rb[7].z : rb[7].w;
        uint32_t d0, d1, d2, d3;
        transpose4x4(w4, w5, w6, w7, d0, d1, d2, d3);
        *reinterpret_cast<uint2*>(sB + b_lds + (4 * q + 0) * KP) = make_uint2(c0, d0);
        *reinterpret_cast<uint2*>(sB + b_lds + (4 * q + 1) * KP) = make_uint2(c1, d1);
        *reinterpret_cast<uint2*>(sB + b_lds + (4 * q + 2) * KP) = make_uint2(c2, d2);
        *reinterpret_cast<uint2*>(sB + b_lds + (4 * q + 3) * KP) = make_uint2(c3, d3);
      } else {
        *reinterpret_cast<uint32_t*>(sB + b_lds + (4 * q + 0) * KP) = c0;
        *reinterpret_cast<uint32_t*>(sB + b_lds + (4 * q + 1) * KP) = c1;
        *reinterpret_cast<uint32_t*>(sB + b_lds + (4 * q + 2) * KP) = c2;
        *reinterpret_cast<uint32_t*>(sB + b_lds + (4 * q + 3) * KP) = c3;
      }
    }
  };

  // ---- wave's column blocks (tile columns) and their weight-scale block
  auto colbase = [&](int nb) -> int {
    if (GATED)
      return nb < NB / 2 ? wn * (WN / 2) + nb * 16 : BNP / 2 + wn * (WN / 2) + (nb - NB / 2) * 16;
    return wn * WN + nb * 16;
  };
  // scale-block column index for the gate (0) and up (1) halves, or the plain block
  int sblk[2];
  sblk[0] = gcol_of(colbase(0)) / kBlock;
  sblk[1] = GATED ? gcol_of(colbase(NB / 2)) / kBlock : sblk[0];
  const float* bs_e = g.Bs + (size_t)e * nkb * nsb;

  // ---- accumulators start at the bias (once per output tile)
  v4f acc[MB][NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int gc = gcol_of(colbase(nb) + (lane & 15));
    const float bv = gc < N ? bf16_to_f32(g.bias[(size_t)e * N + gc]) : 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = v4f{bv, bv, bv, bv};
  }

  stage_load(0);
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    stage_store();
    __syncthreads();
    if (kb + 1 < nkb) stage_load(kb + 1);

    const float sb0 = sblk[0] < nsb ? bs_e[(size_t)kb * nsb + sblk[0]] : 0.f;
    const float sb1 = sblk[1] < nsb ? bs_e[(size_t)kb * nsb + sblk[1]] : 0.f;
    v8i af[MB];
    v4f rs0[MB], rs1[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = wm * WM + mb * 16;
      const uint8_t* pa = sA + (r + (lane & 15)) * KP + 32 * (lane >> 4);
      const v4i lo4 = *reinterpret_cast<const v4i*>(pa);
      const v4i hi4 = *reinterpret_cast<const v4i*>(pa + 16);
      af[mb] = v8i{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      const v4f rsv = *reinterpret_cast<const v4f*>(sAs + r + 4 * (lane >> 4));
      rs0[mb] = rsv * sb0;
      rs1[mb] = rsv * sb1;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int cb = colbase(nb);
      const uint8_t* pb = sB + (cb + (lane & 15)) * KP + (cb >> 4) * B_COLQ + 32 * (lane >> 4);
      const v4i lo4 = *reinterpret_cast<const v4i*>(pb);
      const v4i hi4 = *reinterpret_cast<const v4i*>(pb + 16);
      const v8i bf = v8i{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const v4f p = mfma_fp8_16x16x128(af[mb], bf, v4f{0.f, 0.f, 0.f, 0.f});
        const v4f sc = (GATED && nb >= NB / 2) ? rs1[mb] : rs0[mb];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(p[i], sc[i], acc[mb][nb][i]);
      }
    }
  }

  if constexpr (GATED) {
    // ---- SwiGLU, then per-row 1x128 e4m3 quantisation of h over the tile's
    // 128 h columns (spread over WAVES_N waves)
    constexpr int NH = NB / 2;
    float* sRed = reinterpret_cast<float*>(sB);           // [WAVES_N][BM] row maxima
    uint8_t* sQ = sA;                                      // [BM][128] h codes
    float h[MB][NH][4];
    float rmax[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = 0.f;
#pragma unroll
        for (int nb = 0; nb < NH; ++nb) {
          const float gv = acc[mb][nb][i], uv = acc[mb][nb + NH][i];
          const float hv = gv / (1.0f + expf(-gv)) * uv;
          h[mb][nb][i] = hv;
          mx = fmaxf(mx, fabsf(hv));
        }
        rmax[mb][i] = max16(mx);
      }
    __syncthreads();  // all waves are done with sA / sB
    if ((lane & 15) == 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sRed[wn * BM + wm * WM + mb * 16 + 4 * (lane >> 4) + i] = rmax[mb][i];
    }
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * WM + mb * 16 + 4 * (lane >> 4) + i;
        float amax = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES_N; ++w) amax = fmaxf(amax, sRed[w * BM + r]);
        const float s = amax > 0.f ? amax / kFp8Max : 1.0f;
#pragma unroll
        for (int nb = 0; nb < NH; ++nb) {
          const float y = fminf(fmaxf(h[mb][nb][i] / s, -kFp8Max), kFp8Max);
          sQ[r * kBlock + wn * (WN / 2) + nb * 16 + (lane & 15)] =
              static_cast<uint8_t>(f32x2_to_e4m3(y, 0.f) & 0xffu);
        }
        if (wn == 0 && (lane & 15) == 0 && r < valid)
          g.Hs[(size_t)(row0 + r) * (g.f / kBlock) + nt] = s;
      }
    __syncthreads();
    for (int idx = tid; idx < BM * 8; idx += 256) {
      const int r = idx >> 3, seg = idx & 7;
      if (r < valid)
        *reinterpret_cast<uint4*>(g.Hq + (size_t)(row0 + r) * g.f + n0 + seg * 16) =
            *reinterpret_cast<const uint4*>(sQ + r * kBlock + seg * 16);
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int gc = gcol_of(colbase(nb) + (lane & 15));
        if (gc >= N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * WM + mb * 16 + 4 * (lane >> 4) + i;
          if (r < valid) g.Y[(size_t)(row0 + r) * N + gc] = acc[mb][nb][i];
        }
      }
  }
}

int grid_for(int max_tiles) { return 8 * ceil_div(max_tiles, 8); }

}  // namespace

hipError_t launch_gemm_gated(const GemmArgs& a, bool decode, int max_tiles, hipStream_t stream) {
  if (max_tiles <= 0) return hipSuccess;
  const dim3 grid(grid_for(max_tiles));
  if (decode)
    hipLaunchKernelGGL((grouped_gemm_kernel<kGatedDecode.bm, kGatedDecode.bnp, 1, 4, true>), grid,
                       dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<kGatedPrefill.bm, kGatedPrefill.bnp, 2, 2, true>),
                       grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm_plain(const GemmArgs& a, bool decode, int max_tiles, hipStream_t stream) {
  if (max_tiles <= 0) return hipSuccess;
  const dim3 grid(grid_for(max_tiles));
  if (decode)
    hipLaunchKernelGGL((grouped_gemm_kernel<kPlainDecode.bm, kPlainDecode.bnp, 1, 4, false>), grid,
                       dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<kPlainPrefill.bm, kPlainPrefill.bnp, 2, 2, false>),
                       grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
