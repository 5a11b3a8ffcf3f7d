// GQA attention with per-head sinks on the gfx950 matrix cores.
//
// "GPT-OSS on day 0", section "Sink attention": every head has a learned sink
// value that joins the scaled scores inside the softmax; the softmax runs
// online (the max-subtracted form, with the running maximum seeded by the
// sink and the running sum by its term), and when the keys are split into
// several parts the sink must be counted in the first part only.  Section
// "GPT-OSS on Hopper": the attention is GQA.  The sink has no value vector:
// it only adds exp(sink - M) to the denominator.
//
// Both kernels compute S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys are
// the MFMA rows, queries its columns), so a query's scores sit in one lane
// column: lane (l16, g) holds keys 4g..4g+3 of every 16-key tile for query
// l16, and the softmax reductions are in-lane plus two shuffles.  P stays in
// registers as the B operand of O^T = V^T P^T: for 32 keys 32p.. the lane's
// eight values are keys 32p + 4g + j and 32p + 16 + 4g + j (j < 4), and the
// matching A operand (V^T) comes from two ds_read_b64_tr_b16 reads of V rows
// 32p + 4g.. and 32p + 16 + 4g.. (lane i of a 16-lane group receives column
// i of the four rows its group addressed).  Scores are scaled by
// sm_scale * log2(e) and exponentiated with exp2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "attention.hpp"
#include "common.hpp"

namespace moe {

namespace {

constexpr int AD = 64;          // head dim
constexpr int ABK = 64;         // keys per block
constexpr int APITCH = 144;     // LDS bytes per key row (128 + 16: rows on distinct banks)
constexpr float kLog2e = 1.44269504088896341f;
constexpr int kAttnQt = 2;      // prefill query tiles (16 rows) per wave: 16 waves of 32 rows
constexpr uint32_t kOnes2 = 0x3f803f80u;  // two bf16 ones

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_bf16(uint4 a, uint4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b),
                                                 c, 0, 0, 0);
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32: round to nearest even), low half first
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

// IEEE maximum (v_maximum3_f32): unlike fmaxf it needs no quieting of its
// operands first, which the compiler otherwise adds for values that come out
// of lane swaps (two extra VALU operations per maximum)
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max / sum over the four lanes l, l^16, l^32, l^48 (one query column of an
// S^T tile) with the VALU lane swaps (no LDS round trip)
__device__ __forceinline__ float max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x with the hardware exp (arguments here are <= 0; results below 2^-126 flush to 0)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint2 tr16(const uint8_t* p) {
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
  return __builtin_bit_cast(uint2, r);
}

// ---------------------------------------------------------------------------
// Prefill: one workgroup = HW query heads sharing one key/value head times
// 64 * (8 / HW) query rows, in NW = 32 / QT waves of 16 QT rows (wave w: head
// h0 + w % HW).  The K and V blocks of 64 keys go through LDS once for all
// waves (double buffered: the next block is loaded to registers while the
// current one is used).  With QT = 2 a wave needs at most 128 VGPRs, so four
// waves share a SIMD and hide each other's MFMA, LDS and exp latencies.
// Causal: a block is used by the waves whose rows reach it; the block on the
// diagonal masks key > query.
template <int HW, int QT>
__global__ __launch_bounds__(64 * (32 / QT)) void attn_prefill_kernel(const uint16_t* __restrict__ q,
                                                                      const uint16_t* __restrict__ k,
                                                                      const uint16_t* __restrict__ v,
                                                                      const float* __restrict__ sinks,
                                                                      uint16_t* __restrict__ out, int S,
                                                                      int Hq, int Hkv, float scale2) {
  constexpr int NW = 32 / QT;                        // waves
  constexpr int RW = 16 * QT;                        // query rows per wave
  constexpr int QB = RW * (NW / HW);                 // query rows per workgroup: 64 * (8 / HW)
  constexpr int IPT = 2 * ABK * 8 / (64 * NW);       // 16-byte K/V pieces per thread and block
  __shared__ __attribute__((aligned(16))) uint8_t kl[2][ABK * APITCH];
  __shared__ __attribute__((aligned(16))) uint8_t vl[2][ABK * APITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int G = Hq / Hkv;
  // 1-D grid, longest work first across every head group: workgroup i takes
  // head group i % (Hq / HW) and query block nqb - 1 - i / (Hq / HW)
  const int ngrp = Hq / HW;
  const int nqb = gridDim.x / ngrp;
  const int qb = nqb - 1 - (int)blockIdx.x / ngrp;
  const int h0 = ((int)blockIdx.x % ngrp) * HW;
  const int kvh = h0 / G;
  const int h = h0 + wave % HW;
  const int row0 = qb * QB + RW * (wave / HW);      // this wave's first query row
  const int wg_last = min(S, (qb + 1) * QB) - 1;    // last query row of the workgroup
  const int nblk = wg_last / ABK + 1;               // key blocks the workgroup needs

  // Q^T fragments (B operand): query row0 + 16 qt + l16, dims 32 c + 8 g .. + 7
  uint4 qf[QT][2];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = row0 + 16 * qt + l16;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      qf[qt][c] = r < S ? *reinterpret_cast<const uint4*>(q + ((size_t)r * Hq + h) * AD + 32 * c + 8 * g)
                        : make_uint4(0u, 0u, 0u, 0u);
  }
  // running max (log2 domain) per query column, the sink's term of the sum,
  // O^T, and the sum of the probabilities: an MFMA of an all-ones A operand
  // with P^T, whose 16 rows all hold the column sums (one MFMA instead of
  // eight adds per lane and qt; it sums the bf16 P that the P V product uses)
  float m[QT], sterm[QT];
  v4f lsum[QT];
  v4f o[4][QT];  // [dt][qt]: dims 16 dt + 4 g + i, query 16 qt + l16
  const float sink2 = sinks[h] * kLog2e;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = sink2;     // the sink seeds the running maximum ...
    sterm[qt] = 1.0f;  // ... and contributes exp2(0) = 1 to the sum
    lsum[qt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt][qt] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  // block loader: piece it = tid + 64 NW j: K (it < 512) or V, key (it % 512) / 8,
  // bytes 16 (it % 8) of its row.  Blocks are loaded two iterations ahead into
  // two register sets (block b in set b % 2) and written to LDS one ahead.
  uint4 lr0[IPT], lr1[IPT];
  auto load = [&](int kb, uint4 (&lr)[IPT]) {
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int it = tid + 64 * NW * j;
      const int key = kb * ABK + ((it & 511) >> 3);
      const uint16_t* src = it < 512 ? k : v;
      lr[j] = key < S ? *reinterpret_cast<const uint4*>(src + ((size_t)key * Hkv + kvh) * AD + 8 * (it & 7))
                      : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store = [&](int buf, const uint4 (&lr)[IPT]) {
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int it = tid + 64 * NW * j;
      uint8_t* dst = (it < 512 ? kl[buf] : vl[buf]) + ((it & 511) >> 3) * APITCH + 16 * (it & 7);
      *reinterpret_cast<uint4*>(dst) = lr[j];
    }
  };

  load(0, lr0);
  if (nblk > 1) load(1, lr1);
  store(0, lr0);
  __syncthreads();
  // one key block; block kb's registers (set kb % 2) are free again, so they take block kb + 2
  auto block = [&](int kb, uint4 (&cur)[IPT], uint4 (&nxt)[IPT]) {
    const int buf = kb & 1;
    if (kb + 2 < nblk) load(kb + 2, cur);
    const int key0 = kb * ABK;
    if (key0 <= row0 + RW - 1 && row0 < S) {  // some of this wave's rows see the block
      const uint8_t* kb_l = kl[buf];
      const uint8_t* vb_l = vl[buf];
      // two 32-key halves, each its own online-softmax step (fewer live scores)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int kh0 = key0 + 32 * p;
        if (kh0 > row0 + RW - 1) break;  // the wave's rows see none of this half
        // S^T tiles: keys kh0 + 16 kt + 4 g + i, query 16 qt + l16
        v4f s[2][QT];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const uint8_t* pk = kb_l + (32 * p + 16 * kt + l16) * APITCH + 16 * g;
          const uint4 a0 = *reinterpret_cast<const uint4*>(pk);
          const uint4 a1 = *reinterpret_cast<const uint4*>(pk + 64);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            s[kt][qt] = mfma_bf16(a0, qf[qt][0], v4f{0.f, 0.f, 0.f, 0.f});
            s[kt][qt] = mfma_bf16(a1, qf[qt][1], s[kt][qt]);
          }
        }
        // causal mask on the diagonal only (a uniform branch): key > query -> -inf
        if (kh0 + 31 > row0) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (kh0 + 16 * kt + 4 * g + i > row0 + 16 * qt + l16) s[kt][qt][i] = -INFINITY;
        }
        uint4 pb[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          // the maximum on raw scores (scale2 > 0 keeps the order), then p = 2^(s scale2 - m)
          float bm = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) bm = fmaxf(bm, s[kt][qt][i]);
          const float mn = vmax(m[qt], max4(bm) * scale2);
          // O and the sum are rescaled only when some query's maximum moved
          // (rare once it settles); the factor's exp2 is skipped otherwise
          const bool moved = __builtin_amdgcn_ballot_w64(mn != m[qt]) != 0;
          const float alpha = moved ? ex2(m[qt] - mn) : 1.0f;
          m[qt] = mn;
          float pr[2][4];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[kt][i] = ex2(fmaf(s[kt][qt][i], scale2, -mn));
          if (moved) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt][qt] *= alpha;
            lsum[qt] *= alpha;
            sterm[qt] *= alpha;
          }
          // B operand of the PV MFMA: keys kh0 + 4 g + j, then kh0 + 16 + 4 g + j
          pb[qt] = make_uint4(pack_bf16(pr[0][0], pr[0][1]), pack_bf16(pr[0][2], pr[0][3]),
                              pack_bf16(pr[1][0], pr[1][1]), pack_bf16(pr[1][2], pr[1][3]));
          lsum[qt] = mfma_bf16(make_uint4(kOnes2, kOnes2, kOnes2, kOnes2), pb[qt], lsum[qt]);
        }
        // O^T += V^T P^T: lanes of group g address key rows 32p + 4g + i/4 (and +16),
        // dims 16 dt + 4 (i % 4)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const uint8_t* pv = vb_l + (32 * p + 4 * g + (l16 >> 2)) * APITCH + 2 * (16 * dt + 4 * (l16 & 3));
          const uint2 lo = tr16(pv);
          const uint2 hi = tr16(pv + 16 * APITCH);
          const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) o[dt][qt] = mfma_bf16(a, pb[qt], o[dt][qt]);
        }
      }
    }
    if (kb + 1 < nblk) {
      // buffer buf ^ 1 was last read for block kb - 1, before the previous barrier
      store(buf ^ 1, nxt);
      __syncthreads();
    }
  };
  for (int kb = 0; kb < nblk; kb += 2) {
    block(kb, lr0, lr1);
    if (kb + 1 < nblk) block(kb + 1, lr1, lr0);
  }

  // out[query][h][d] = O^T[d][query] / sum
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float inv = 1.0f / (lsum[qt][0] + sterm[qt]);
    const int r = row0 + 16 * qt + l16;
    if (r >= S) continue;
    uint16_t* po = out + ((size_t)r * Hq + h) * AD + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      *reinterpret_cast<uint2*>(po + 16 * dt) =
          make_uint2(pack_bf16(o[dt][qt][0] * inv, o[dt][qt][1] * inv),
                     pack_bf16(o[dt][qt][2] * inv, o[dt][qt][3] * inv));
  }
}

// ---------------------------------------------------------------------------
// Decode, balanced over the waves: for each key/value head the cached keys of
// all sequences, taken one sequence after the other (offset P_b for sequence
// b), are cut into wk ranges of Q = max(kMinSplitKeys, ceil(total / wk)) keys,
// one per wave, so every wave streams the same amount whatever the length mix.
// A range can hold pieces of several sequences; each piece (b, keys k0..k1 of
// b) is a segment with its own running max, sum and O, written to record slot
// base_b + (its index among b's segments); the segment that starts at key 0
// of b also carries the sink (max = sink, sum = 1), the others start from an
// empty softmax.  Every wave derives P_b, the segment counts and base_b from
// kv_len itself (wave scans over chunks of 64 sequences); wave (0, 0) stores
// P_b and base_b for the combine.
//
// A segment: the G <= 16 query heads of the key/value head are the 16 MFMA
// columns (the rest are zero); K fragments come straight from the cache (a
// lane reads 16 bytes of one key row); each 64-key block of V is staged in the
// wave's own LDS slice for the transposing reads; both are loaded to
// registers one block ahead.
__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  return incl - v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(256, 2) void attn_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ kv_len, const float* __restrict__ sinks, float* __restrict__ part,
    int32_t* __restrict__ plan, int B, int Hq, int Hkv, int Lmax, int wk, int slots, float scale2) {
  __shared__ __attribute__((aligned(16))) uint8_t vl[4][ABK * APITCH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int wid = blockIdx.x * 4 + wave;
  const int kvh = wid / wk, wi = wid % wk;
  if (kvh >= Hkv) return;
  const bool planner = wid == 0;                    // stores P_b and base_b
  const int G = Hq / Hkv;
  const int h = kvh * G + l16;                      // query head of column l16
  const bool hv = l16 < G;
  const float sink2 = hv ? sinks[h] * kLog2e : 0.f;

  // total keys per key/value head, then this wave's range [lo, hi); the
  // lengths of the first 64 sequences are kept for the walk below
  const int len0 = lane < B ? min(max(kv_len[lane], 0), Lmax) : 0;
  int tot = len0;
  for (int c = 64; c < B; c += 64) {
    const int bb = c + lane;
    tot += bb < B ? min(max(kv_len[bb], 0), Lmax) : 0;
  }
  const int total = wave_sum(tot);
  const int Q = max(kMinSplitKeys, ceil_div(total, wk));
  const int64_t lo = (int64_t)wi * Q, hi = lo + Q;
  if (lo >= total && !planner) return;

  uint8_t* vw = vl[wave];
  // every cached key and value row is read once per call: non-temporal loads
  auto load_once = [](const uint16_t* p) -> uint4 {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  size_t cache_base = 0;
  int k1 = 0;
  // block registers: V rows 8 j + lane / 8 (16 bytes each) and the K fragments
  // of rows 16 kt + l16; the next block is fetched while the current one is used
  uint4 kA[8], vA[8], kB[8], vB[8];
  auto fetch = [&](int key0, uint4 (&kr)[8], uint4 (&vr)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = key0 + 8 * j + (lane >> 3);
      vr[j] = key < k1 ? load_once(vc + cache_base + (size_t)key * AD + 8 * (lane & 7))
                       : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = key0 + 16 * kt + l16;
      const uint16_t* pk = kc + cache_base + (size_t)key * AD + 8 * g;
      kr[2 * kt] = key < k1 ? load_once(pk) : make_uint4(0u, 0u, 0u, 0u);
      kr[2 * kt + 1] = key < k1 ? load_once(pk + 32) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  uint4 qf[2];
  float m = 0.f, l = 0.f;
  v4f o[4];
  auto block = [&](int key0, const uint4 (&kr)[8], const uint4 (&vr)[8], uint4 (&kn)[8], uint4 (&vn)[8]) {
    if (key0 + ABK < k1) fetch(key0 + ABK, kn, vn);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint4*>(vw + (8 * j + (lane >> 3)) * APITCH + 16 * (lane & 7)) = vr[j];
    // S^T: keys key0 + 16 kt + 4 g + i, query column l16
    v4f s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = mfma_bf16(kr[2 * kt], qf[0], v4f{0.f, 0.f, 0.f, 0.f});
      s[kt] = mfma_bf16(kr[2 * kt + 1], qf[1], s[kt]);
    }
    float bm = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (key0 + 16 * kt + 4 * g + i >= k1) s[kt][i] = -INFINITY;  // past the segment
        bm = fmaxf(bm, s[kt][i]);
      }
    const float mn = vmax(m, max4(bm) * scale2);  // finite: the block has a valid key
    const float alpha = ex2(m - mn);
    m = mn;
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = ex2(fmaf(s[kt][i], scale2, -mn));
        s[kt][i] = p;
        sum += p;
      }
    l = fmaf(l, alpha, sum);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    __builtin_amdgcn_s_waitcnt(0xc07f);             // lgkmcnt(0): this wave's V rows are in LDS
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint4 pb = make_uint4(pack_bf16(s[2 * p][0], s[2 * p][1]), pack_bf16(s[2 * p][2], s[2 * p][3]),
                                  pack_bf16(s[2 * p + 1][0], s[2 * p + 1][1]),
                                  pack_bf16(s[2 * p + 1][2], s[2 * p + 1][3]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint8_t* pv = vw + (32 * p + 4 * g + (l16 >> 2)) * APITCH + 2 * (16 * dt + 4 * (l16 & 3));
        const uint2 lo2 = tr16(pv);
        const uint2 hi2 = tr16(pv + 16 * APITCH);
        o[dt] = mfma_bf16(make_uint4(lo2.x, lo2.y, hi2.x, hi2.y), pb, o[dt]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);             // the reads are done before the next block's writes
  };
  // one segment: keys k0 .. k1 - 1 of sequence b into record slot `slot`
  auto segment = [&](int b, int k0, int kend, int slot) {
    k1 = kend;
    cache_base = ((size_t)b * Hkv + kvh) * (size_t)Lmax * AD;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      qf[c] = hv ? *reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + h) * AD + 32 * c + 8 * g)
                 : make_uint4(0u, 0u, 0u, 0u);
    m = k0 == 0 ? sink2 : -INFINITY;
    l = (k0 == 0 && g == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = v4f{0.f, 0.f, 0.f, 0.f};
    if (k0 < k1) fetch(k0, kA, vA);
    for (int key0 = k0; key0 < k1; key0 += 2 * ABK) {
      block(key0, kA, vA, kB, vB);
      if (key0 + ABK < k1) block(key0 + ABK, kB, vB, kA, vA);
    }
    // record [slot][h] = {O[64], m, l, -, -}; the four lanes of a head add their sums
    const float lt = sum4(l);
    if (!hv || slot < 0 || slot >= slots) return;
    float* pp = part + ((size_t)slot * Hq + h) * kPartFloats;
    if (g == 0) {
      pp[AD] = m;
      pp[AD + 1] = lt;
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      *reinterpret_cast<v4f*>(pp + 16 * dt + 4 * g) = o[dt];
  };

  // walk the sequences 64 at a time: P_b, segment counts, base_b; run the
  // segments of this wave's range in sequence order
  int prun = 0, brun = 0;
  for (int c = 0; c < B && (prun < hi || planner); c += 64) {
    const int bb = c + lane;
    const int len = c == 0 ? len0 : bb < B ? min(max(kv_len[bb], 0), Lmax) : 0;
    const int P = prun + wave_excl_scan(len, lane);
    const int cnt = len > 0 ? (P + len - 1) / Q - P / Q + 1 : 0;
    const int base = brun + wave_excl_scan(cnt, lane);
    if (planner && bb < B) {
      plan[bb] = P;
      plan[B + 1 + bb] = base;
    }
    uint64_t mine = __builtin_amdgcn_ballot_w64(bb < B && len > 0 && P < hi && P + len > lo);
    while (mine) {
      const int j = __builtin_ctzll(mine);
      mine &= mine - 1;
      const int b = c + j;
      const int Pj = __shfl(P, j), lenj = __shfl(len, j), basej = __shfl(base, j);
      const int k0 = (int)max((int64_t)0, lo - Pj);
      const int kend = (int)min((int64_t)lenj, hi - Pj);
      segment(b, k0, kend, basej + wi - Pj / Q);
    }
    prun += wave_sum(len);
    brun += wave_sum(cnt);
  }
  if (planner && lane == 0) {
    plan[B] = total;
    plan[2 * B + 1] = brun;
  }
}

// out[b][h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the segments
// of sequence b (M = max_s m_s, finite: the first segment carries the sink);
// a sequence without keys has the sink alone and a zero output.  One
// workgroup of W waves per (b, h): wave w takes records w, w + W, ... and the
// waves add their sums through LDS (W = 4 where a sequence can have tens to
// hundreds of records, 1 where it has at most 32).
template <int W>
__global__ __launch_bounds__(64 * W) void attn_combine_kernel(const float* __restrict__ part,
                                                              const int32_t* __restrict__ kv_len,
                                                              const int32_t* __restrict__ plan,
                                                              uint16_t* __restrict__ out, int B, int Hq,
                                                              int Lmax, int wk, int slots) {
  __shared__ float red[W][AD + 1];
  const int bh = blockIdx.x, t = threadIdx.x, d = t & 63, w = t >> 6;
  const int b = bh / Hq, h = bh % Hq;
  const int len = min(max(kv_len[b], 0), Lmax);
  if (len == 0) {
    if (w == 0) out[(size_t)bh * AD + d] = 0;
    return;
  }
  const int total = plan[B], P = plan[b], base = plan[B + 1 + b];
  const int Q = max(kMinSplitKeys, ceil_div(total, wk));
  const int n = max(0, min((P + len - 1) / Q - P / Q + 1, slots - base));
  const float* rec = part + ((size_t)base * Hq + h) * kPartFloats;
  const size_t stride = (size_t)Hq * kPartFloats;  // between consecutive slots
  float M = -INFINITY;
  for (int s = t; s < n; s += 64 * W) M = fmaxf(M, rec[s * stride + AD]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if constexpr (W > 1) {
    if (d == 0) red[w][0] = M;
    __syncthreads();
    M = red[0][0];
#pragma unroll
    for (int i = 1; i < W; ++i) M = fmaxf(M, red[i][0]);
    __syncthreads();
  }
  float num = 0.f, den = 0.f;
#pragma unroll 4
  for (int s = w; s < n; s += W) {
    const float* pp = rec + s * stride;
    const float wt = exp2f(pp[AD] - M);
    den = fmaf(wt, pp[AD + 1], den);
    num = fmaf(wt, pp[d], num);
  }
  if constexpr (W > 1) {
    red[w][d] = num;
    if (d == 0) red[w][AD] = den;
    __syncthreads();
    if (w != 0) return;
    num = red[0][d];
    den = red[0][AD];
#pragma unroll
    for (int i = 1; i < W; ++i) {
      num += red[i][d];
      den += red[i][AD];
    }
  }
  out[(size_t)bh * AD + d] = f32_to_bf16(num / den);
}

}  // namespace

int attn_decode_waves(int Hkv) { return std::max(1, kResidentWaves / std::max(1, Hkv)); }

int64_t attn_decode_slots(int B, int Lmax) {
  // segments of all sequences: at most total / Q + 2 B with total / Q <= the
  // waves per head (<= kResidentWaves), and at most B (Lmax / kMinSplitKeys + 2)
  const int64_t by_waves = (int64_t)kResidentWaves + 2 * (int64_t)B;
  const int64_t by_len = (int64_t)B * (ceil_div(std::max(Lmax, 1), kMinSplitKeys) + 2);
  return std::min(by_waves, by_len);
}

hipError_t launch_attn_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const float* sinks, uint16_t* out, int S, int Hq, int Hkv,
                               float sm_scale, hipStream_t stream) {
  const int G = Hq / Hkv;
  const int HW = G >= 8 ? 8 : G;                    // heads per workgroup
  const int QB = 64 * (8 / HW);
  constexpr int QT = kAttnQt;
  const dim3 grid(ceil_div(S, QB) * (Hq / HW)), block(64 * (32 / QT));
  const float scale2 = sm_scale * kLog2e;
  switch (HW) {
    case 8: hipLaunchKernelGGL((attn_prefill_kernel<8, QT>), grid, block, 0, stream, q, k, v, sinks, out, S, Hq, Hkv, scale2); break;
    case 4: hipLaunchKernelGGL((attn_prefill_kernel<4, QT>), grid, block, 0, stream, q, k, v, sinks, out, S, Hq, Hkv, scale2); break;
    case 2: hipLaunchKernelGGL((attn_prefill_kernel<2, QT>), grid, block, 0, stream, q, k, v, sinks, out, S, Hq, Hkv, scale2); break;
    case 1: hipLaunchKernelGGL((attn_prefill_kernel<1, QT>), grid, block, 0, stream, q, k, v, sinks, out, S, Hq, Hkv, scale2); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                              const int32_t* kv_len, const float* sinks, uint16_t* out, float* part,
                              int32_t* plan, int B, int Hq, int Hkv, int Lmax, float sm_scale,
                              hipStream_t stream) {
  const int wk = attn_decode_waves(Hkv);
  const int slots = (int)attn_decode_slots(B, Lmax);
  hipLaunchKernelGGL(attn_decode_kernel, dim3(ceil_div(Hkv * wk, 4)), dim3(256), 0, stream, q, kc, vc, kv_len,
                     sinks, part, plan, B, Hq, Hkv, Lmax, wk, slots, sm_scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // a sequence has at most ceil(Lmax / kMinSplitKeys) + 1 records
  if (ceil_div(std::max(Lmax, 1), kMinSplitKeys) + 1 > 32)
    hipLaunchKernelGGL(attn_combine_kernel<4>, dim3(B * Hq), dim3(256), 0, stream, part, kv_len, plan, out, B,
                       Hq, Lmax, wk, slots);
  else
    hipLaunchKernelGGL(attn_combine_kernel<1>, dim3(B * Hq), dim3(64), 0, stream, part, kv_len, plan, out, B,
                       Hq, Lmax, wk, slots);
  return hipGetLastError();
}

}  // namespace moe
