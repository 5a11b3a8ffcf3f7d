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
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// ---------------------------------------------------------------------------
// Prefill kernel: persistent, direct global->LDS loads into a 3-stage ring,
// 8 waves.
//
// Tile 128 rows x 256 B columns, K block 128.  Per stage: A [128][128] e4m3
// with the 16-byte segments of row r stored at position seg ^ (r & 7);
// B [128 K][256 N] in its global K x N orientation with the 16-byte segments
// of K row kr at seg ^ swz_b(kr); a 2 KB side area where wave w's load lands
// at 256w: the A row scales of the K block (waves 0, 1), the tile's bias
// (waves 2, 3), the two weight-block scales of the K block (wave 4, lanes
// 0-1) and zeros (waves 5-7).  Loads are buffer_load ... lds: lane i of a
// load writes bytes [s*i, s*i+s) of the LDS destination; rows outside the
// tile or columns outside N read offsets past the buffer end and land as
// zeros.
//
// Eight waves (two per SIMD, so one wave's LDS waits and barrier hide under
// the other's MFMAs) in a 2 x 4 grid each own 64 rows x 64 columns.  The
// weights are the first MFMA operand and the activations the second, so a
// lane's four outputs are four consecutive columns of one row: the row scale
// is one scalar per lane and the epilogue writes whole dwords / float4s.
// The weight operand is read with ds_read_b64_tr_b8: in each group of 16
// lanes, lanes 2j and 2j+1 address the two 8-byte halves of one 16-column
// segment of K row j, and lane i receives column i of those 8 rows.
// Gated tiles hold 128 gate and the matching 128 up columns; wave column
// wn owns h columns 32wn..32wn+31 as two gate and two up blocks, so SwiGLU
// and the per-row h quantisation run on registers.
//
// Persistent: one workgroup per CU walks the tiles L = lo + slot + i * nslots
// of its XCD's contiguous slice of the tile list with one continuous K-block
// stream, so the next tile's first stages load while the current tile ends.
// Inside that stream the only vector-memory operations are the stage loads,
// the row-token loads of the gated kernel and the epilogue stores, all with a
// fixed count per wave; tile descriptors come through the scalar cache and
// bias and weight scales through the stages.  So every wait is a vmcnt the
// kernel states itself, and nothing drains the ring at a tile boundary.
constexpr int DMA_WAVES = 8;
constexpr int DMA_SS = DMA_WAVES * 256;              // side area: wave w's load lands at 256w
constexpr int SIDE_AS = 0, SIDE_BIAS = 512, SIDE_BS = 1024;
// MX side area: the E8M0 weight scales of the K block's four 32-deep groups,
// group g (loaded by wave 4 + g) at SIDE_BS + MX_PITCH g.  A wave's load
// always lands 256 bytes; the extra 16 put the groups on distinct LDS banks.
constexpr int MX_PITCH = 272;
// Tiles: 128 rows (prefill: waves of 64 rows) or 32 rows (decode, bound by
// streaming the weights: waves of 16 rows), by 256 B columns (waves of 64)
// or, for the decode down projection, 128 (waves of 32).  A stage is
// A [BM][128], B [128][BNP] and the side area: 50 KB for prefill.
template <int BM, int BNP, bool MX, bool FP4>
struct DmaShape {
  static constexpr int MB = BM / 32;                 // 16-row blocks per wave
  static constexpr int NB = BNP / 64;                // 16-column blocks per wave
  static constexpr int KR = FP4 ? kBlock / 2 : kBlock;  // stored weight rows per K block
  static constexpr int SA = BM * kBlock;
  static constexpr int SB = KR * BNP;
  static constexpr int SS = MX ? SIDE_BS + 4 * MX_PITCH : DMA_SS;
  static constexpr int STAGE = SA + SB + SS;
  static constexpr int A_PER = BM >= 64 ? BM / 64 : 1;        // A chunks (1 KB) per loading wave
  static constexpr int A_WAVES = BM / 8 / A_PER;              // waves that load A
  static constexpr int B_PER = SB / 1024 / DMA_WAVES;         // B chunks per wave
  static constexpr int SEGS = BNP / 16;                       // 16-byte segments per K row
  static constexpr int LOADS_MIN = (A_WAVES == DMA_WAVES ? A_PER : 0) + B_PER + 1;  // fewest per wave
  static_assert(BM == 32 || BM == 128, "row tile");
  static_assert(BNP == 128 || BNP == 256, "column tile");
};
constexpr uint32_t kOob = 0x80000000u;               // buffer offset that reads as zero
constexpr int kRsrcWord3 = 0x00020000;               // raw buffer, gfx9 family

typedef __attribute__((address_space(4))) int32_t const_i32;

// A row r keeps its 16-byte segment s at position s ^ swz_a(r), with the
// XOR key built from row bits 2, 0, 1 (in that order).  The fragment reads
// (16 rows x 2 segments per lane group) then run without LDS bank conflicts;
// measured on gfx950 with the SQ_LDS_BANK_CONFLICT counter, where the keys
// r & 7 and (r >> 1) & 7 cost one extra cycle per read cycle.
__device__ __forceinline__ int swz_a(int r) { return ((r >> 2) & 1) | ((r & 3) << 1); }
// With 16 segments per K row the key's bit 3 comes from the K-row bit that
// tells the lane groups 0 and 1 apart in the fragment reads: bit 5 for K rows
// 32g + 8r + j, bit 4 for the MX order 64(r/2) + 16g + 8(r%2) + j.
template <int SEGS, bool MX = false>
__device__ __forceinline__ int swz_b(int kr) {
  if (SEGS != 16) return kr & 7;
  return MX ? (kr & 7) | (((kr >> 4) & 1) << 3) : (kr & 7) | (((kr >> 5) & 1) << 3);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | vmcnt[5:4] << 14)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// Raw buffer resource (gfx9: base, stride 0, byte size, raw-buffer word 3) in SGPRs.
__device__ __forceinline__ v4i dma_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = kRsrcWord3;
  return r;
}

// Global -> LDS loads (buffer_load ... lds): lane i writes bytes [s*i, s*i+s)
// at LDS address `lds` (uniform); offsets past the resource size read zeros.
// Inline asm, which the compiler does not track, for the decode kernel: its
// own s_waitcnt + s_barrier pairs order these loads against the reads, and a
// wait the compiler adds for its own memory operations only waits longer.
// (The prefill kernel uses the compiler's builtin instead; see lds_load.)  M0
// is restored.
// PIN: the descriptor is uniform, but in some kernels the register allocator
// copies it to VGPRs, which the scalar asm operand cannot take; readfirstlane
// pins it to SGPRs there (elsewhere it would only perturb the allocation).
template <bool PIN>
__device__ __forceinline__ v4i sgpr4(v4i r) {
  if constexpr (PIN) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
  }
  return r;
}
// NT: the non-temporal policy, for data read once (decode weights): the
// stream then does not displace what the caches still serve.
template <bool PIN = false, bool NT = false>
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds, uint32_t voff) {
  rsrc = sgpr4<PIN>(rsrc);
  int saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(rsrc)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(rsrc)
        : "memory");
}
template <bool PIN = false>
__device__ __forceinline__ void dma4(v4i rsrc, uint32_t lds, uint32_t voff) {
  rsrc = sgpr4<PIN>(rsrc);
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
      static_cast<int>(reinterpret_cast<uintptr_t>(p))));
}

// One output tile: {expert, first row, rows, column tile} from the tile list,
// and the K blocks [kb0, kb1) it covers: all of them, or with split K the
// range of split sp.
struct DmaTile {
  int e, row0, valid, nt, kb0, kb1, sp;
};

__device__ __forceinline__ DmaTile dma_tile(const GemmArgs& g, int L) {
  const const_i32* v = (const const_i32*)g.tiles + 4 * L;  // uniform: scalar loads
  return DmaTile{v[0], v[1], v[2], v[3], 0, 0, 0};
}

// Split K: work item V is split V % ksplit of tile V / ksplit, K blocks
// [sp * kper, min(nkb, (sp + 1) * kper)); the splits of one tile are
// consecutive items, so they run on one XCD and share its L2.
template <bool SPLIT>
__device__ __forceinline__ DmaTile dma_vtile(const GemmArgs& g, int V, int nkb) {
  if constexpr (SPLIT) {
    const int S = g.ksplit;
    DmaTile t = dma_tile(g, V / S);
    t.sp = V - (V / S) * S;
    t.kb0 = t.sp * g.kper;
    t.kb1 = min(nkb, t.kb0 + g.kper);
    return t;
  } else {
    DmaTile t = dma_tile(g, V);
    t.kb1 = nkb;
    return t;
  }
}

// FP4 (with MX): E2M1 weights packed two per byte along K, K/2 stored rows.
// SPLIT: every tile is cut into g.ksplit K ranges, and a work item stores
// its promoted fp32 sums (no bias, no epilogue) into its split's slice of
// g.part [ksplit][R][N]; a finish kernel adds the slices in split order.
template <bool GATED, int BM, int BNP, bool MX, bool FP4, bool SPLIT>
__global__ __launch_bounds__(DMA_WAVES * 64, 1) void grouped_gemm_dma_kernel(GemmArgs g) {
  using S = DmaShape<BM, BNP, MX, FP4>;
  static_assert(MX || !FP4, "FP4 weights come with E8M0 scales");
  static_assert(!GATED || BNP == 256, "gated tiles: 128 gate + 128 up columns");
  static_assert(!MX || BM == 32, "MX decode tiles: one 16-row block per wave");
  constexpr int DMA_SA = S::SA, DMA_SB = S::SB, DMA_STAGE = S::STAGE;
  constexpr int MB = S::MB, NB = S::NB;             // 16x16 blocks per wave
  constexpr int WR = 16 * MB;                       // rows per wave
  constexpr int RT = GATED ? 1 : 0;                 // row-token loads per cursor move
  constexpr int ST = (GATED && !SPLIT) ? MB * 3 : MB * NB;  // epilogue stores per wave
  __shared__ __attribute__((aligned(1024))) uint8_t st0[DMA_STAGE];  // the three ring stages
  __shared__ __attribute__((aligned(1024))) uint8_t st1[DMA_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[DMA_STAGE];
  __shared__ float smax[(GATED && !MX) ? 4 * BM : 1];  // gated epilogue: row maxima per wave column
  __shared__ int32_t rtok[GATED ? 2 : 1][GATED ? DMA_WAVES * 64 : 1];  // row tokens, 2 tiles

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addressing
  const int wm = wave >> 2, wn = wave & 3;
  const int gq = lane >> 4, l16 = lane & 15;
  const int K = g.K, N = g.N, nkb = K / kBlock, nsb = N / kBlock;

  // ---- this workgroup's work items: L = lo + slot + i * nslots < hi
  const int total = ((const const_i32*)g.tile_off)[g.E] * (SPLIT ? g.ksplit : 1);
  const int nslots = gridDim.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int lo = (blockIdx.x & 7) * chunk;
  const int hi = min(total, lo + chunk);
  const int L0 = lo + (blockIdx.x >> 3);
  if (L0 >= hi) return;

  const v4i rA = dma_rsrc(g.A, g.A_bytes);
  // side-area load of this wave: A row scales, bias, weight scales or zeros.
  // MX: waves 4-7 load the E8M0 weight scales of K groups 0-3 (rows 4 kb + g
  // of [E][K/32][N]); block-scaled: wave 4 the two block scales of the K block.
  const uint32_t bs_bytes = MX ? (uint32_t)g.E * (uint32_t)(K / 32) * (uint32_t)N
                               : 4u * (uint32_t)g.E * nkb * nsb;
  const v4i rSide = wave < 2   ? dma_rsrc(g.As, g.As_bytes)
                    : wave < 4 ? dma_rsrc(g.bias, 2u * (uint32_t)g.E * (uint32_t)N)
                               : dma_rsrc(g.Bs, bs_bytes);
  const int side_step = wave < 2 ? 4 : wave < 4 ? 0 : MX ? 4 * N : (wave == 4 ? 4 * nsb : 0);
  const uint32_t side_dst = (MX && wave >= 4) ? SIDE_BS + MX_PITCH * (wave - 4) : 256 * wave;

  // ---- load cursor: tile tl (index Ll), K block kbl; the next tile prefetched
  int Ll = L0, rb = 0;
  int Lln = Ll + nslots;
  DmaTile tl = dma_vtile<SPLIT>(g, Ll, nkb), tln = tl;
  int kbl = tl.kb0;
  if (Lln < hi) tln = dma_vtile<SPLIT>(g, Lln, nkb);
  uint32_t aoff[S::A_PER], boff[S::B_PER], soff;
  auto no_loads = [&]() {
    aoff[0] = aoff[S::A_PER - 1] = soff = kOob;
#pragma unroll
    for (int q = 0; q < S::B_PER; ++q) boff[q] = kOob;
  };

  // gated: tokens of the tile's 128 rows -> rtok[buf] (waves 0, 1; the
  // others load zeros into their own slots)
  auto rt_load = [&](const DmaTile& t, bool live, int buf) {
    if constexpr (GATED) {
      const int r = 64 * wave + lane;
      const uint32_t o = (live && wave < 2 && r < t.valid) ? 4u * (uint32_t)(t.row0 + r) : kOob;
      dma4(dma_rsrc(g.row_token, g.rows_bytes), lds_addr(&rtok[buf][64 * wave]), o);
    }
  };
  // per-lane load offsets of tile t (row tokens in rtok[buf] for the gated kernel);
  // loads that must read zeros get an offset past the buffer, which stays past
  // it when the K-block stride is added
  v4i rB;
  // weights read once (the expert's rows fit one row block) stream with the
  // non-temporal policy; an expert with more row blocks keeps them cacheable
  // for its other tiles, which read the same weight slices
  bool b_once = true;
  auto setup = [&](const DmaTile& t, int buf) {
    const int n0 = t.nt * (GATED ? kBlock : BNP);
    b_once = ((const const_i32*)g.counts)[t.e] <= BM;
    rB = dma_rsrc(g.B + (size_t)t.e * S::KR * nkb * N, (uint32_t)(S::KR * nkb) * (uint32_t)N);
#pragma unroll
    for (int q = 0; q < S::A_PER; ++q) {  // A: 1 KB chunk c = rows 8c..8c+7; wave w: A_PER chunks
      const int r = 8 * (S::A_PER * wave + q) + (lane >> 3);
      const int sgm = (lane & 7) ^ swz_a(r);
      aoff[q] = kOob;
      if (r < t.valid) aoff[q] = (uint32_t)(GATED ? rtok[buf][r] : t.row0 + r) * (uint32_t)K + 16u * sgm;
    }
    // B: 1 KB chunk c = K rows (1024 / BNP) c..; wave w: chunks B_PER w..; lane ->
    // K row of the chunk lane / SEGS, the 16 bytes of segment (lane % SEGS) ^ swz_b(kr)
#pragma unroll
    for (int q = 0; q < S::B_PER; ++q) {
      const int kr = (1024 / BNP) * (S::B_PER * wave + q) + lane / S::SEGS;
      const int s = (lane % S::SEGS) ^ swz_b<S::SEGS, MX>(kr);
      const int gc = GATED ? (s < 8 ? n0 + 16 * s : g.f + n0 + 16 * (s - 8)) : n0 + 16 * s;
      boff[q] = gc < N ? (uint32_t)kr * (uint32_t)N + (uint32_t)gc : kOob;
    }
    soff = kOob;
    if (wave < 2) {  // A row scales in the order [row % 16][row / 16] of each 64-row half
      const int r = 64 * wave + 16 * (lane & 3) + (lane >> 2);
      if (r < t.valid) soff = (uint32_t)(GATED ? rtok[buf][r] : t.row0 + r) * (uint32_t)nkb * 4u;
    } else if (wave < 4) {  // bias: 128 columns (bf16 pairs) per wave
      const int c = (GATED ? (wave == 2 ? n0 : g.f + n0) : n0 + 128 * (wave - 2)) + 2 * lane;
      if (c < N) soff = 2u * ((uint32_t)t.e * (uint32_t)N + (uint32_t)c);
    } else if constexpr (MX) {  // wave 4 + q: E8M0 scales of K group q, tile columns 4 lane..
      const int c = 4 * lane;
      const int gc = GATED ? (c < 128 ? n0 + c : g.f + n0 + c - 128) : n0 + c;
      if (c < BNP && gc < N)
        soff = ((uint32_t)t.e * (uint32_t)(K / 32) + (uint32_t)(wave - 4)) * (uint32_t)N + (uint32_t)gc;
    } else if (wave == 4 && lane < 2) {  // the two weight-block scales of the K block
      const int sb = GATED ? (lane == 0 ? n0 : g.f + n0) / kBlock : n0 / kBlock + lane;
      if (sb < nsb) soff = 4u * ((uint32_t)t.e * (uint32_t)nkb * (uint32_t)nsb + (uint32_t)sb);
    }
  };

  // Every call issues the same loads per wave, also past the last tile (they
  // then read offsets past the buffers and land as zeros in a stage no one
  // reads): the in-flight count is the same on every path.
  auto issue = [&](uint8_t* base) {
    const uint32_t sbase = lds_addr(base);
    const uint32_t ka = (uint32_t)kbl * kBlock, kb = (uint32_t)kbl * S::KR * (uint32_t)N;
    if (S::A_WAVES == DMA_WAVES || wave < S::A_WAVES)
#pragma unroll
      for (int q = 0; q < S::A_PER; ++q)
        dma16<MX>(rA, sbase + (S::A_PER * wave + q) * 1024, aoff[q] + ka);
#pragma unroll
    for (int q = 0; q < S::B_PER; ++q)
      if (b_once) dma16<MX, true>(rB, sbase + DMA_SA + (S::B_PER * wave + q) * 1024, boff[q] + kb);
      else dma16<MX, false>(rB, sbase + DMA_SA + (S::B_PER * wave + q) * 1024, boff[q] + kb);
    dma4<MX>(rSide, sbase + DMA_SA + DMA_SB + side_dst, soff + (uint32_t)(kbl * side_step));
    ++kbl;
  };
  // After a tile's last K block has been issued the cursor moves to its next
  // tile, whose row tokens were loaded one move earlier; returns the number
  // of loads it issued.
  auto advance = [&]() -> int {
    if (kbl < tl.kb1) return 0;
    Ll = Lln;
    tl = tln;
    kbl = tl.kb0;
    rb ^= 1;
    Lln += nslots;
    if (Lln < hi) tln = dma_vtile<SPLIT>(g, Lln, nkb);
    if (nkb == 1) {  // the row tokens were loaded one K block ago: wait for them
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    if (Ll < hi) setup(tl, rb);
    else no_loads();
    // the previous readers of rtok[rb ^ 1] are past a ring barrier
    rt_load(tln, Lln < hi, rb ^ 1);
    return RT;
  };

  // ---- per-lane LDS read offsets (stage-relative)
  // activations: row 64*wm + 16*mb + l16, 32 bytes = segments 2gq, 2gq+1
  // (MX K order: gq, gq + 4), swizzled
  const int a_row = (wm * WR + l16) * kBlock;
  const int a_pos0 = 16 * ((MX ? gq : 2 * gq) ^ swz_a(l16));
  const int a_pos1 = 16 * ((MX ? gq + 4 : 2 * gq + 1) ^ swz_a(l16));
  // weights: transposing reads r = 0..3 of K rows b_kr(r) + b_kg, half l16 & 1
  // of a segment: K rows 8r + 32gq + l16/2 (MX: 64(r/2) + 8(r%2) + 16gq + l16/2)
  const int b_kg = (MX ? 16 : 32) * gq + (l16 >> 1);
  const int b_row = b_kg * BNP + 8 * (l16 & 1);
  const int b_swz = swz_b<S::SEGS, MX>(b_kg);  // the same for the 4 reads
  // tile segment of column block nb: gated 2wn + nb (gate) and 8 + 2wn + nb - 2 (up),
  // plain NB wn + nb; stored at segment ^ b_swz
  const int b_base = 16 * ((GATED ? 2 * wn : NB * wn) ^ b_swz);
  auto b_seg = [&](int nb) -> int { return GATED ? ((nb & 1) | ((nb >> 1) << 3)) : nb; };
  // row scale of row r at float 64 (r / 64) + 4 (r % 16) + (r % 64) / 16
  const int s_pos = DMA_SA + DMA_SB + SIDE_AS + (MB == 4 ? (wm * 64 + 4 * l16) : (4 * l16 + wm)) * 4;
  // bias of block nb: 4 bf16 at columns 4gq.. of the block
  auto bias_pos = [&](int nb) -> int {
    return DMA_SA + DMA_SB + SIDE_BIAS +
           2 * (GATED ? (nb < 2 ? 32 * wn + 16 * nb : 128 + 32 * wn + 16 * (nb - 2))
                      : 16 * NB * wn + 16 * nb) + 8 * gq;
  };

  // ---- compute side: tile tc, K block kbc; the next tile prefetched
  DmaTile tc = tl, tcn = tln;
  int Lcn = Lln, kbc = 0;
  // block-scaled: promoted sums, scalars (no register-quad constraint in the loop);
  // MX: the matrix cores accumulate in macc, copied to acc for the epilogue
  float acc[MB][NB][4];
  v4f macc[MX ? MB : 1][MX ? NB : 1];

  auto compute_mx = [&](const uint8_t* base) {
    const uint8_t* sA = base;
    const uint8_t* sB = base + DMA_SA;
    if (kbc == 0) {  // accumulators start from the bias (split K: from zero)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint2 w = *reinterpret_cast<const uint2*>(base + bias_pos(nb));
        const v4f bv = SPLIT ? v4f{0.f, 0.f, 0.f, 0.f}
                             : v4f{bf16_to_f32(w.x & 0xffffu), bf16_to_f32(w.x >> 16),
                                   bf16_to_f32(w.y & 0xffffu), bf16_to_f32(w.y >> 16)};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) macc[mb][nb] = bv;
      }
    }
    // E8M0 scales: byte gq (K group) of row 16 wm + l16's dword; weight column
    // 16 seg + l16 of K group gq
    const int xsc = static_cast<int>(*reinterpret_cast<const uint32_t*>(base + s_pos) >> (8 * gq));
    const uint8_t* wsc = base + DMA_SA + DMA_SB + SIDE_BS + MX_PITCH * gq + l16;
    const v4i lo4 = *reinterpret_cast<const v4i*>(sA + a_row + a_pos0);
    const v4i hi4 = *reinterpret_cast<const v4i*>(sA + a_row + a_pos1);
    const v8i xf = v8i{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // FP4: two reads, stored rows 16gq + 8r + l16/2 (K 32gq.. in order)
      v8i wf = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < (FP4 ? 2 : 4); ++r) {
        const int rr = FP4 ? 8 * r : 64 * (r >> 1) + 8 * (r & 1);
        const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(sB + b_row + rr * BNP + (b_base ^ (16 * b_seg(nb)))));
        wf[2 * r] = t[0];
        wf[2 * r + 1] = t[1];
      }
      const int ws = wsc[16 * ((GATED ? 2 * wn : NB * wn) + b_seg(nb))];
      if constexpr (FP4) macc[0][nb] = mfma_fp4_fp8_16x16x128_mx(wf, xf, macc[0][nb], ws, xsc);
      else macc[0][nb] = mfma_fp8_16x16x128_mx(wf, xf, macc[0][nb], ws, xsc);
    }
  };

  auto compute = [&](const uint8_t* base) {
    const uint8_t* sA = base;
    const uint8_t* sB = base + DMA_SA;
    const float* sbs = reinterpret_cast<const float*>(base + DMA_SA + DMA_SB + SIDE_BS);
    const float sb0 = sbs[(GATED || BNP == 128) ? 0 : (wn >> 1)];
    const float sb1 = GATED ? sbs[1] : sb0;
    if (kbc == 0) {  // accumulators start from the bias (split K: from zero)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint2 w = *reinterpret_cast<const uint2*>(base + bias_pos(nb));
        float bv[4] = {bf16_to_f32(w.x & 0xffffu), bf16_to_f32(w.x >> 16),
                       bf16_to_f32(w.y & 0xffffu), bf16_to_f32(w.y >> 16)};
        if constexpr (SPLIT) bv[0] = bv[1] = bv[2] = bv[3] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb][nb][i] = bv[i];
      }
    }
    v4f sa;
    if constexpr (MB == 4) sa = *reinterpret_cast<const v4f*>(base + s_pos);
    else sa[0] = *reinterpret_cast<const float*>(base + s_pos);
    v8i xf[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const v4i lo4 = *reinterpret_cast<const v4i*>(sA + a_row + mb * 16 * kBlock + a_pos0);
      const v4i hi4 = *reinterpret_cast<const v4i*>(sA + a_row + mb * 16 * kBlock + a_pos1);
      xf[mb] = v8i{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      v8i wf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(sB + b_row + r * 8 * BNP +
                                                     (b_base ^ (16 * b_seg(nb)))));
        wf[2 * r] = t[0];
        wf[2 * r + 1] = t[1];
      }
      const float sb = (GATED && nb >= 2) ? sb1 : sb0;
      v4f pn[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) pn[mb] = mfma_fp8_16x16x128(wf, xf[mb], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const float s = sa[mb] * sb;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(pn[mb][i], s, acc[mb][nb][i]);
      }
    }
  };

  // lane -> rows 64wm + 16mb + l16, columns (of block nb) 4gq..4gq+3.  Every
  // wave issues ST stores whatever the tile's shape (rows past the tile and
  // columns past N go to offsets past the buffers, which drops them).
  auto epilogue = [&](const DmaTile& t) {
    const int n0 = t.nt * (GATED ? kBlock : BNP);
    if constexpr (MX) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mb][nb][i] = macc[mb][nb][i];
    }
    if constexpr (SPLIT) {
      // promoted sums of K blocks [kb0, kb1) -> part[sp][row][column]: gated
      // block nb < 2 is gate column n0 + 32wn + 16nb + 4gq.., nb >= 2 the up
      // column f + n0 + 32wn + 16(nb - 2) + 4gq..; plain n0 + 16 NB wn + 16nb + 4gq..
      const __amdgpu_buffer_rsrc_t rP =
          __builtin_amdgcn_make_buffer_rsrc(g.part, (short)0, g.part_bytes, kRsrcWord3);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int gc = GATED ? (nb < 2 ? n0 + 32 * wn + 16 * nb + 4 * gq : g.f + n0 + 32 * wn + 16 * (nb - 2) + 4 * gq)
                             : n0 + 16 * NB * wn + 16 * nb + 4 * gq;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = wm * WR + 16 * mb + l16;
          const uint32_t o = 4u * (((uint32_t)t.sp * (uint32_t)g.R + (uint32_t)(t.row0 + r)) * (uint32_t)N +
                                   (uint32_t)gc);
          const v4u d = v4u{__builtin_bit_cast(uint32_t, acc[mb][nb][0]),
                            __builtin_bit_cast(uint32_t, acc[mb][nb][1]),
                            __builtin_bit_cast(uint32_t, acc[mb][nb][2]),
                            __builtin_bit_cast(uint32_t, acc[mb][nb][3])};
          __builtin_amdgcn_raw_buffer_store_b128(d, rP, (r < t.valid && gc < N) ? (int)o : (int)kOob, 0, 0);
        }
      }
    } else if constexpr (GATED) {
      // h = silu(gate) * up on registers: h column 32wn + 16j + 4gq + i
      float h[MB][2][4];
      float pmax[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float mx = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gv = acc[mb][j][i], uv = acc[mb][2 + j][i];
            // silu with the hardware exp2 and reciprocal (relative error ~1e-7,
            // far below the e4m3 spacing h is rounded to)
            const float ex = __builtin_amdgcn_exp2f(-gv * 1.44269504088896341f);
            h[mb][j][i] = gv * __builtin_amdgcn_rcpf(1.0f + ex) * uv;
            mx = nan_max(mx, fabsf(h[mb][j][i]));
          }
        mx = nan_max(mx, __shfl_xor(mx, 16));
        pmax[mb] = nan_max(mx, __shfl_xor(mx, 32));
      }
      if constexpr (MX) {
        // the wave's 32 h columns of a row are one MX block: no exchange
        const __amdgpu_buffer_rsrc_t rH =
            __builtin_amdgcn_make_buffer_rsrc(g.Hq, (short)0, g.out_bytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rHs =
            __builtin_amdgcn_make_buffer_rsrc(g.Hs, (short)0, g.out2_bytes, kRsrcWord3);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = wm * WR + 16 * mb + l16;
          const uint32_t code = mx_code(pmax[mb]);
          const float inv = mx_inv_scale(code);
          const bool ok = r < t.valid;
          const uint32_t hrow = (uint32_t)(t.row0 + r) * (uint32_t)g.f + n0 + 32 * wn + 4 * gq;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(
                f32x4_to_e4m3(h[mb][j][0] * inv, h[mb][j][1] * inv, h[mb][j][2] * inv, h[mb][j][3] * inv),
                rH, ok ? (int)(hrow + 16 * j) : (int)kOob, 0, 0);
          const uint32_t so = (uint32_t)(t.row0 + r) * (uint32_t)(g.f / 32) + 4 * t.nt + wn;
          __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(code), rHs,
                                               (ok && gq == 0) ? (int)so : (int)kOob, 0, 0);
        }
      } else {
        // row maxima over the four wave columns through LDS.  The previous
        // tile's readers are past at least one ring barrier; a bare s_barrier
        // (no memory fence) leaves the next tile's stage loads in flight.
        if (gq == 0)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) smax[wn * BM + wm * WR + 16 * mb + l16] = pmax[mb];
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the smax writes are done
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const __amdgpu_buffer_rsrc_t rH =
            __builtin_amdgcn_make_buffer_rsrc(g.Hq, (short)0, g.out_bytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rHs =
            __builtin_amdgcn_make_buffer_rsrc(g.Hs, (short)0, g.out2_bytes, kRsrcWord3);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = wm * WR + 16 * mb + l16;
          const float amax =
              nan_max(nan_max(smax[r], smax[BM + r]), nan_max(smax[2 * BM + r], smax[3 * BM + r]));
          const float s = group_scale(amax);
          const float inv = 1.0f / s;
          const bool ok = r < t.valid;
          const uint32_t hrow = (uint32_t)(t.row0 + r) * (uint32_t)g.f + n0 + 32 * wn + 4 * gq;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float q[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) q[i] = clamp_fp8(h[mb][j][i] * inv);
            __builtin_amdgcn_raw_buffer_store_b32(f32x4_to_e4m3(q[0], q[1], q[2], q[3]), rH,
                                                  ok ? (int)(hrow + 16 * j) : (int)kOob, 0, 0);
          }
          const uint32_t so = 4u * ((uint32_t)(t.row0 + r) * (uint32_t)(g.f / kBlock) + t.nt);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, s), rHs,
                                                (ok && wn == 0 && gq == 0) ? (int)so : (int)kOob, 0, 0);
        }
      }
    } else {
      const __amdgpu_buffer_rsrc_t rY =
          __builtin_amdgcn_make_buffer_rsrc(g.Y, (short)0, g.out_bytes, kRsrcWord3);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int gc = n0 + 16 * NB * wn + 16 * nb + 4 * gq;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = wm * WR + 16 * mb + l16;
          const uint32_t o = 4u * ((uint32_t)(t.row0 + r) * (uint32_t)N + (uint32_t)gc);
          const v4u d = v4u{__builtin_bit_cast(uint32_t, acc[mb][nb][0]),
                            __builtin_bit_cast(uint32_t, acc[mb][nb][1]),
                            __builtin_bit_cast(uint32_t, acc[mb][nb][2]),
                            __builtin_bit_cast(uint32_t, acc[mb][nb][3])};
          __builtin_amdgcn_raw_buffer_store_b128(d, rY, (r < t.valid && gc < N) ? (int)o : (int)kOob,
                                                 0, 0);
        }
      }
    }
  };

  // Ring synchronisation: wait for this wave's loads of the stage about to be
  // read.  Younger than them are the next stage's 7 loads and `pend` more
  // operations (row tokens, epilogue stores), which may stay in flight.
  // Then a bare s_barrier (a __syncthreads fence would wait for everything).
  auto wait_stage = [&](int pend) {
    constexpr int NL = S::LOADS_MIN;  // waves that issue more wait for a little more
    if (pend == 0) wait_vmcnt<NL>();
    else if (pend == RT) wait_vmcnt<NL + RT>();
    else if (pend == ST) wait_vmcnt<NL + ST>();
    else if (pend == RT + ST) wait_vmcnt<NL + RT + ST>();
    else wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- prologue: row tokens of the first two tiles, offsets of the first
  rt_load(tl, true, 0);
  rt_load(tln, Lln < hi, 1);
  if constexpr (GATED) {
    wait_vmcnt<0>();
    __syncthreads();
  }
  setup(tl, 0);
  if constexpr (GATED) {
    // every wave has read rtok[0] before a tile move inside the prologue (K of
    // one or two blocks) loads the tile after next into it
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // One K block; returns false after the workgroup's last tile.
  int pend = 0;
  auto step = [&](const uint8_t* cur, uint8_t* next2) -> bool {
    wait_stage(pend);
    issue(next2);
    if constexpr (MX) compute_mx(cur);
    else compute(cur);
    pend = advance();
    if (++kbc < tc.kb1 - tc.kb0) return true;
    epilogue(tc);
    pend += ST;
    if (Lcn >= hi) return false;
    kbc = 0;
    tc = tcn;
    Lcn += nslots;
    if (Lcn < hi) tcn = dma_vtile<SPLIT>(g, Lcn, nkb);
    return true;
  };

  issue(st0);
  pend = advance();
  issue(st1);
  pend = advance();
  while (step(st0, st2) && step(st1, st0) && step(st2, st1)) {
  }
  wait_vmcnt<0>();  // the loads past the last tile land before the workgroup ends
}

// ---------------------------------------------------------------------------
// Wide prefill kernel: 192 x 256 tiles, 8 waves of 96 x 64, weights three K
// blocks deep and activations two.
//
// A wave owning 96 rows x 64 columns reads 28 fragments from LDS per 24 MFMAs
// (the 64 x 64 waves of the kernel above read 24 per 16), which keeps the
// LDS read rate below the FP8 MFMA rate with room for the stage writes.  The
// promotion of each 128-deep MFMA result (4 FMAs per lane) is issued two
// MFMAs after it, so the VALU work of one wave runs under the MFMAs of the
// other wave on its SIMD.
//
// LDS: activation stages A [192][128] (segment s of row r at s ^ swz_a(r))
// with a 2 KB side area each, two deep; weight stages B [128 K][256 N]
// (segment s of K row kr at s ^ swz_b<16>(kr)), three deep, so a weight
// slice is requested two K blocks before it is read: the tiles that share a
// slice all request it at about the same time, and the first of them waits
// for HBM.  Side area: [0, 1 KB) the A row scales of the K block, row
// 96 wm + 16 mb + l16 at float 128 wm + 8 l16 + mb (waves 0-3); [1 KB,
// 1.5 KB) the tile's 256 bias values (waves 4, 5); [1.5 KB, +8) the two
// weight-block scales of the K block (wave 6).  The bias is added in the
// epilogue (the accumulator initialisation, reordered; equal up to fp32
// rounding).
//
// Rows: waves wm = 0 / 1 own tile rows 0-95 / 96-191; a wave whose half has
// no valid row skips its MFMAs and its epilogue, so a ragged tail tile of
// <= 96 rows costs about half a tile.  Persistent over the tile list; the
// loads run ahead across tile boundaries (the next tile's first blocks load
// while the current tile ends).
//
// Schedule: XCD x (workgroups b with b % 8 == x) owns the x-th of eight
// ranges of the tile list, and workgroup b takes its slot's first two tiles
// lo + b / 8 and lo + b / 8 + slots.  With g.sched the ranges have equal cost
// (the place stage sets them; a tile of at most 96 rows costs 2/3 of a full
// one in the gate/up GEMM, 1/2 in the down GEMM) instead of equal length,
// and, with at least 3 K blocks per tile, the rest of a range is handed out
// in order by an integer counter of its XCD.
// Tiles take 29-44 us on the skewed prefill layer, and a fixed round robin
// over equal lengths left the workgroups of an XCD up to five tiles apart at
// the end and the XCDs up to 150 us apart (the range that holds only full
// tiles of the hottest expert against one with 329 short tiles).  A tile
// index is fetched two tiles ahead, only where a cursor changes tiles (no
// per-step state): wave 0 adds to the counter as the compute cursor enters a
// tile, stores the index in LDS as the weight cursor leaves it and every wave
// reads it as the activation cursor does.  Which workgroup computes a tile
// does not change any result.  The last
// workgroup to finish zeroes the counters again.
// Global -> LDS loads through the compiler's builtin (the instruction of
// dma16 / dma4), for the kernel below.  Every ring stage there is a
// __shared__ array of its own, so the compiler's wait analysis tells the
// stages apart and adds no wait inside a step; and it sees every load in
// flight, so a value that an atomic returns is known to have arrived once
// the ring wait that covers the atomic has passed.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}
template <int SIZE>
__device__ __forceinline__ void lds_load(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff) {
  static_assert(SIZE == 4 || SIZE == 16, "dword or dwordx4 loads");
  if constexpr (SIZE == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, 0, 0, 0);
}

constexpr int WM_ROWS = 192, WN_COLS = 256, W_HALF = WM_ROWS / 2;
constexpr int W_SA = WM_ROWS * kBlock, W_SIDE = 2048;
constexpr int W_ASTAGE = W_SA + W_SIDE;
constexpr int W_SIDE_BIAS = 1024, W_SIDE_BS = 1536;
constexpr int W_AQ = W_SA / 1024 / DMA_WAVES;       // A chunks (1 KB) per wave: 3

template <bool GATED, bool MX, bool FP4>
__global__ __launch_bounds__(DMA_WAVES * 64, 1) void grouped_gemm_wide_kernel(GemmArgs g) {
  static_assert(MX || !FP4, "FP4 weights come with E8M0 scales");
  constexpr int KR = FP4 ? kBlock / 2 : kBlock;      // stored weight rows per K block
  constexpr int SB = KR * WN_COLS;
  constexpr int BQ = SB / 1024 / DMA_WAVES;          // B chunks (1 KB) per wave
  constexpr int MB = W_HALF / 16, NB = 4;            // 16 x 16 blocks per wave: 6 x 4
  constexpr int RT = GATED ? 1 : 0;                  // row-token loads per A-cursor tile move
  constexpr int ST = GATED ? MB * 3 : MB * NB;       // epilogue stores per wave with rows
  constexpr int ASTAGE = MX ? W_SA + W_SIDE_BS + 4 * MX_PITCH : W_ASTAGE;
  __shared__ __attribute__((aligned(1024))) uint8_t sa0[ASTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sa1[ASTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sb0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sb1[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sb2[SB];
  __shared__ float smax[(GATED && !MX) ? 4 * WM_ROWS : 1];  // row maxima per wave column
  __shared__ int32_t rtok[GATED ? 2 : 1][GATED ? DMA_WAVES * 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int gq = lane >> 4, l16 = lane & 15;
  const int K = g.K, N = g.N, nkb = K / kBlock, nsb = N / kBlock;

  const int total = ((const const_i32*)g.tile_off)[g.E];
  const int nslots = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7;
  int32_t* const sched = g.sched;
  int lo, hi;
  if (sched != nullptr) {  // ranges of equal cost (clamped into the list)
    const const_i32* bd = (const const_i32*)(sched + kSchedBounds);
    lo = min(max(bd[xcd], 0), total);
    hi = min(max(bd[xcd + 1], lo), total);
  } else {
    const int c = (total + 7) >> 3;
    lo = min(xcd * c, total);
    hi = min(total, lo + c);
  }
  const int chunk = hi - lo;
  const int L0 = lo + (blockIdx.x >> 3);
  const bool dyn = sched != nullptr && nkb >= 3;
  // the last workgroup to finish (every fetch of every workgroup has returned
  // by then) zeroes the counters for the next launch
  auto finish = [&]() {
    if (sched != nullptr && tid == 0 && atomicAdd(&sched[8], 1) == (int)gridDim.x - 1) {
#pragma unroll
      for (int i = 0; i < 9; ++i) atomicExch(&sched[i], 0);
    }
  };
  if (L0 >= hi) {
    finish();
    return;
  }

  const __amdgpu_buffer_rsrc_t rA = buf_rsrc(g.A, g.A_bytes);
  // side loads: waves 0-3 the A row scales; block-scaled: waves 4, 5 the bias,
  // wave 6 the two weight-block scales; MX: waves 4-7 the E8M0 weight scales
  // of K groups 0-3 and waves 4, 5 the bias with a second load
  const __amdgpu_buffer_rsrc_t rBias = buf_rsrc(g.bias, 2u * (uint32_t)g.E * (uint32_t)N);
  const uint32_t bs_bytes = MX ? (uint32_t)g.E * (uint32_t)(K / 32) * (uint32_t)N
                               : 4u * (uint32_t)g.E * nkb * nsb;
  const __amdgpu_buffer_rsrc_t rSide = wave < 4 ? buf_rsrc(g.As, g.As_bytes)
                                        : (wave < 6 && !MX) ? rBias : buf_rsrc(g.Bs, bs_bytes);
  const int side_step = wave < 4 ? 4 : MX ? 4 * N : (wave == 6 ? 4 * nsb : 0);
  const uint32_t side_dst = (MX && wave >= 4) ? W_SIDE_BS + MX_PITCH * (wave - 4) : 256 * wave;

  // ---- A cursor (activations + side area, one K block ahead of compute)
  int La = L0, kba = 0, rb = 0;
  int Lan = La + nslots;
  DmaTile ta = dma_tile(g, La), tan = ta;
  if (Lan < hi) tan = dma_tile(g, Lan);
  uint32_t aoff[W_AQ], soff, soff2 = kOob;
  // ---- B cursor (weights, two K blocks ahead of compute)
  int Lb = L0, kbb = 0;
  DmaTile tb = ta;
  uint32_t boff[BQ];
  __amdgpu_buffer_rsrc_t rB;
  // ---- dynamic schedule, in the cursors' tile moves only.  When the compute
  // cursor enters tile Y (in the prologue: the first tile) and Y's successor
  // Z is a tile, wave 0 adds to its XCD's counter for the tile after Z.  When
  // the B cursor moves from Y to Z, at least one step later (nkb >= 3), wave 0
  // stores the index in snext: the compiler's wait for the atomic there asks
  // less than the ring wait that follows (the atomic is older than the step's
  // own loads).  One step later, past a ring barrier, the A cursor moves from
  // Y to Z and every wave reads snext as the tile after Z.
  __shared__ int32_t snext;
  int tkt = 0;
  auto fetch = [&]() {
    if (dyn && Lan < hi && wave == 0 && lane == 0) tkt = atomicAdd(&sched[xcd], 1);
  };
  auto fetch_store = [&]() {
    if (dyn && Lan < hi && wave == 0) {
      // a count outside [0, chunk) (counters not zeroed) reads as the end
      if (lane == 0) snext = (tkt >= 0 && tkt < chunk) ? lo + 2 * nslots + tkt : hi;
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the store is done before the barrier
    }
  };

  auto rt_load = [&](const DmaTile& t, bool live, int buf) {
    if constexpr (GATED) {
      const int r = 64 * wave + lane;
      const uint32_t o = (live && wave < 3 && r < t.valid) ? 4u * (uint32_t)(t.row0 + r) : kOob;
      lds_load<4>(buf_rsrc(g.row_token, g.rows_bytes), reinterpret_cast<uint8_t*>(&rtok[buf][64 * wave]), o);
    }
  };
  auto setup_a = [&](const DmaTile& t, int buf) {
#pragma unroll
    for (int q = 0; q < W_AQ; ++q) {  // chunk W_AQ wave + q: rows 8 chunk + lane / 8
      const int r = 8 * (W_AQ * wave + q) + (lane >> 3);
      const int sgm = (lane & 7) ^ swz_a(r);
      aoff[q] = kOob;
      if (r < t.valid)
        aoff[q] = (uint32_t)(GATED ? rtok[buf][r] : t.row0 + r) * (uint32_t)K + 16u * sgm;
    }
    const int n0 = t.nt * (GATED ? kBlock : WN_COLS);
    soff = kOob;
    if (wave < 4) {  // the scale of row 96 wm + 16 mb + l16 lands at float 128 wm + 8 l16 + mb
      const int i = 64 * wave + lane;
      const int mb = i & 7;
      const int r = W_HALF * (i >> 7) + 16 * mb + ((i >> 3) & 15);
      if (mb < MB && r < t.valid)
        soff = (uint32_t)(GATED ? rtok[buf][r] : t.row0 + r) * (uint32_t)nkb * 4u;
    } else if (MX || wave < 6) {
      if (wave < 6) {  // bias: 128 tile columns (bf16 pairs) per wave
        const int c = (GATED ? (wave == 4 ? n0 : g.f + n0) : n0 + 128 * (wave - 4)) + 2 * lane;
        uint32_t& o = MX ? soff2 : soff;
        o = kOob;
        if (c < N) o = 2u * ((uint32_t)t.e * (uint32_t)N + (uint32_t)c);
      }
      if constexpr (MX) {  // wave 4 + q: E8M0 scales of K group q, tile columns 4 lane..
        const int c = 4 * lane;
        const int gc = GATED ? (c < 128 ? n0 + c : g.f + n0 + c - 128) : n0 + c;
        if (gc < N)
          soff = ((uint32_t)t.e * (uint32_t)(K / 32) + (uint32_t)(wave - 4)) * (uint32_t)N + (uint32_t)gc;
      }
    } else if (wave == 6 && lane < 2) {
      const int sb = GATED ? (lane == 0 ? n0 : g.f + n0) / kBlock : n0 / kBlock + lane;
      if (sb < nsb) soff = 4u * ((uint32_t)t.e * (uint32_t)nkb * (uint32_t)nsb + (uint32_t)sb);
    }
  };
  auto setup_b = [&](const DmaTile& t) {
    const int n0 = t.nt * (GATED ? kBlock : WN_COLS);
    rB = buf_rsrc(g.B + (size_t)t.e * KR * nkb * N, (uint32_t)(KR * nkb) * (uint32_t)N);
#pragma unroll
    for (int q = 0; q < BQ; ++q) {  // chunk BQ wave + q: stored rows 4 chunk + lane / 16
      const int kr = 4 * (BQ * wave + q) + (lane >> 4);
      const int s = (lane & 15) ^ swz_b<16, MX>(kr);
      const int gc = GATED ? (s < 8 ? n0 + 16 * s : g.f + n0 + 16 * (s - 8)) : n0 + 16 * s;
      boff[q] = gc < N ? (uint32_t)kr * (uint32_t)N + (uint32_t)gc : kOob;
    }
  };
  // The loads of one step: A chunks and the side area of block kba into the
  // next A stage before the compute, B chunks of block kbb into the next B
  // stage after it.  Issued in one burst after the barrier, the 64 loads of
  // a step fill the address queues and stall every wave's instruction stream
  // (MFMAs included) until they drain; two bursts of 32, one at each end of
  // the compute, do not.  Every load is issued on every path, also past the
  // last tile (the offsets then point past the buffers and the loads land as
  // zeros in a stage no one reads), so the in-flight count is the same on
  // every path.
  // The ring waits count this wave's loads in issue order (activation group,
  // weight group, row tokens, epilogue stores): a scheduling barrier after
  // each group keeps the compiler from moving loads across groups.
  auto a_load = [&](uint8_t* base, int q) {
    lds_load<16>(rA, base + (W_AQ * wave + q) * 1024, aoff[q] + (uint32_t)kba * kBlock);
  };
  auto side_load = [&](uint8_t* base) {
    lds_load<4>(rSide, base + W_SA + side_dst, soff + (uint32_t)(kba * side_step));
    if (MX && (wave == 4 || wave == 5)) lds_load<4>(rBias, base + W_SA + W_SIDE_BIAS + 256 * (wave - 4), soff2);
  };
  auto b_load = [&](uint8_t* base, int q) {
    lds_load<16>(rB, base + (BQ * wave + q) * 1024, boff[q] + (uint32_t)kbb * KR * (uint32_t)N);
  };
  auto issue_a = [&](uint8_t* base) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < W_AQ; ++q) a_load(base, q);
    side_load(base);
    __builtin_amdgcn_sched_barrier(0);
    ++kba;
  };
  auto issue_b = [&](uint8_t* base) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < BQ; ++q) b_load(base, q);
    __builtin_amdgcn_sched_barrier(0);
    ++kbb;
  };
  // Cursor moves after a tile's last K block has been issued.
  auto advance_b = [&]() {
    if (kbb < nkb) return;
    kbb = 0;
    fetch_store();
    Lb = dyn ? Lan : Lb + nslots;  // the A cursor is one K block behind: its next tile
    if (Lb < hi) {
      tb = dma_tile(g, Lb);
      setup_b(tb);
    } else {
#pragma unroll
      for (int q = 0; q < BQ; ++q) boff[q] = kOob;
    }
  };
  auto advance_a = [&]() -> int {
    if (kba < nkb) return 0;
    kba = 0;
    La = Lan;
    ta = tan;
    rb ^= 1;
    Lan = __builtin_amdgcn_readfirstlane(!dyn ? Lan + nslots : La < hi ? snext : hi);
    if (Lan < hi) tan = dma_tile(g, Lan);
    if (nkb == 1) {  // the row tokens were loaded one K block ago: wait for them
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    if (La < hi) {
      setup_a(ta, rb);
    } else {
#pragma unroll
      for (int q = 0; q < W_AQ; ++q) aoff[q] = kOob;
      soff = soff2 = kOob;
    }
    // the previous readers of rtok[rb ^ 1] are past a ring barrier
    rt_load(tan, Lan < hi, rb ^ 1);
    return RT;
  };

  // ---- per-lane LDS read offsets
  // (the MX K order reads segments gq, gq + 4 and K rows 64(r/2) + 8(r%2) + 16gq + l16/2)
  const int a_row = (wm * W_HALF + l16) * kBlock;
  const int a_pos0 = 16 * ((MX ? gq : 2 * gq) ^ swz_a(l16));
  const int a_pos1 = 16 * ((MX ? gq + 4 : 2 * gq + 1) ^ swz_a(l16));
  const int b_kg = (MX ? 16 : 32) * gq + (l16 >> 1);
  const int b_row = b_kg * WN_COLS + 8 * (l16 & 1);
  const int b_swz = swz_b<16, MX>(b_kg);
  // tile B segment of block nb: gated gate 2wn + nb, up 8 + 2wn + nb - 2; plain 4wn + nb
  auto b_tseg = [&](int nb) -> int {
    return GATED ? (nb < 2 ? 2 * wn + nb : 8 + 2 * wn + nb - 2) : 4 * wn + nb;
  };
  auto b_off = [&](int nb) -> int { return b_row + 16 * (b_tseg(nb) ^ b_swz); };
  const int s_pos = W_SA + (wm * 128 + 8 * l16) * 4;

  DmaTile tc = ta;
  int Lc = L0, kbc = 0;
  // block-scaled: promoted sums; MX: the matrix cores accumulate in macc
  // (copied to acc for the epilogue)
  float acc[MB][NB][4];
  v4f macc[MX ? MB : 1][MX ? NB : 1];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (MX) macc[mb][nb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mb][nb][i] = 0.f;
    }

  // activation fragment of row block mb (rows 96 wm + 16 mb + l16)
  auto a_frag = [&](const uint8_t* abase, int mb) -> v8i {
    const uint8_t* pa = abase + a_row + mb * 16 * kBlock;
    const v4i lo4 = *reinterpret_cast<const v4i*>(pa + a_pos0);
    const v4i hi4 = *reinterpret_cast<const v4i*>(pa + a_pos1);
    return v8i{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  };

  // LDS reads in the order of first use (LDS data returns in order), and the
  // activation fragment of row block mb + 1 read right after the first MFMA
  // of block mb, three MFMAs before its use (two buffers)
  auto compute_mx = [&](const uint8_t* abase, const uint8_t* bbase) {
    if (wm == 1 && tc.valid <= W_HALF) return;  // no rows in this wave's half
    // E8M0 scales: byte gq (K group) of the dwords of rows 96 wm + 16 mb + l16,
    // stored at dword 128 wm + 8 l16 + mb; weight column 16 seg + l16 of group gq
    const v4u sl = *reinterpret_cast<const v4u*>(abase + s_pos);
    const uint2 sh = *reinterpret_cast<const uint2*>(abase + s_pos + 16);
    int xsc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      xsc[mb] = static_cast<int>((mb < 4 ? sl[mb] : (mb == 4 ? sh.x : sh.y)) >> (8 * gq));
    v8i xf[2];
    xf[0] = a_frag(abase, 0);
    int wsv[NB];
    v8i wf[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      {  // the byte through its aligned dword: byte loads lost their LDS alias scope
         // in code generation, and with it the compiler waited for every stage load
        const int o = 16 * b_tseg(nb) + (int)(MX_PITCH * gq + l16);
        const uint32_t w = *reinterpret_cast<const uint32_t*>(abase + W_SA + W_SIDE_BS + (o & ~3));
        wsv[nb] = (int)((w >> (8 * (o & 3))) & 0xffu);
      }
      wf[nb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < (FP4 ? 2 : 4); ++r) {  // FP4: stored rows 16gq + 8r + l16/2
        const int rr = FP4 ? 8 * r : 64 * (r >> 1) + 8 * (r & 1);
        const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(bbase + b_off(nb) + rr * WN_COLS));
        wf[nb][2 * r] = t[0];
        wf[nb][2 * r + 1] = t[1];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (FP4) macc[mb][nb] = mfma_fp4_fp8_16x16x128_mx(wf[nb], xf[mb & 1], macc[mb][nb], wsv[nb], xsc[mb]);
        else macc[mb][nb] = mfma_fp8_16x16x128_mx(wf[nb], xf[mb & 1], macc[mb][nb], wsv[nb], xsc[mb]);
        if (nb == 0 && mb + 1 < MB) xf[(mb + 1) & 1] = a_frag(abase, mb + 1);
        __builtin_amdgcn_sched_barrier(0);  // keeps the read ahead of its use
      }
    }
  };

  auto compute = [&](const uint8_t* abase, const uint8_t* bbase) {
    if (wm == 1 && tc.valid <= W_HALF) return;  // no rows in this wave's half
    // the first MFMA waits for its own two operands only; the scales come
    // last (the first promotion follows the fourth MFMA)
    v8i xf[2];
    xf[0] = a_frag(abase, 0);
    v8i wf[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(bbase + b_off(nb) + r * 8 * WN_COLS));
        wf[nb][2 * r] = t[0];
        wf[nb][2 * r + 1] = t[1];
      }
    __builtin_amdgcn_sched_barrier(0);
    const float* sbs = reinterpret_cast<const float*>(abase + W_SA + W_SIDE_BS);
    const v4f sl = *reinterpret_cast<const v4f*>(abase + s_pos);
    const v2f sh = *reinterpret_cast<const v2f*>(abase + s_pos + 16);
    const float sb0 = GATED ? sbs[0] : sbs[wn >> 1];
    const float sb1 = GATED ? sbs[1] : sb0;
    __builtin_amdgcn_sched_barrier(0);
    // MB * NB MFMAs j = 4 mb + nb; the FMAs of MFMA j follow MFMA j + 3, by
    // when its result is ready (two behind measured 1.4 % slower)
    v4f pp[MB * NB];
#pragma unroll
    for (int j = 0; j < MB * NB + 3; ++j) {
      if (j < MB * NB) {
        const int mb = j >> 2, nb = j & 3;
        pp[j] = mfma_fp8_16x16x128(wf[nb], xf[mb & 1], v4f{0.f, 0.f, 0.f, 0.f});
        if (nb == 0 && mb + 1 < MB) xf[(mb + 1) & 1] = a_frag(abase, mb + 1);
      }
      if (j >= 3) {
        const int q = j - 3, mb = q >> 2, nb = q & 3;
        const float sa = mb < 4 ? sl[mb] : sh[mb - 4];
        const float s = sa * ((GATED && nb >= 2) ? sb1 : sb0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(pp[q][i], s, acc[mb][nb][i]);
      }
      // keep each MFMA ahead of the promotions that follow it in this order:
      // left free, the scheduler pulls them next to the MFMA whose result
      // they read and stalls on it
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // lane -> rows 96 wm + 16 mb + l16, columns 4 gq.. of each 16-column block
  // Returns the number of stores issued (the ring waits count them).
  auto epilogue = [&](const DmaTile& t, const uint8_t* abase) -> int {
    // A wave whose row half holds no valid row (a tile of at most 96 rows)
    // has nothing to write: its MFMAs were skipped, so its accumulators are
    // still zero.  It only joins the row-maximum barrier of the block-scaled
    // gated epilogue, which every wave passes once per tile.
    if (wm == 1 && t.valid <= W_HALF) {
      if constexpr (GATED && !MX) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      return 0;
    }
    const int n0 = t.nt * (GATED ? kBlock : WN_COLS);
    const uint8_t* sbias = abase + W_SA + W_SIDE_BIAS;
    if constexpr (MX) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mb][nb][i] = macc[mb][nb][i];
    }
    if constexpr (GATED) {
      float bg[2][4], bu[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint2 wg = *reinterpret_cast<const uint2*>(sbias + 2 * (32 * wn + 16 * j + 4 * gq));
        const uint2 wu = *reinterpret_cast<const uint2*>(sbias + 2 * (128 + 32 * wn + 16 * j + 4 * gq));
        bg[j][0] = bf16_to_f32(wg.x & 0xffffu); bg[j][1] = bf16_to_f32(wg.x >> 16);
        bg[j][2] = bf16_to_f32(wg.y & 0xffffu); bg[j][3] = bf16_to_f32(wg.y >> 16);
        bu[j][0] = bf16_to_f32(wu.x & 0xffffu); bu[j][1] = bf16_to_f32(wu.x >> 16);
        bu[j][2] = bf16_to_f32(wu.y & 0xffffu); bu[j][3] = bf16_to_f32(wu.y >> 16);
      }
      float pmax[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float mx = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gv = acc[mb][j][i] + bg[j][i], uv = acc[mb][2 + j][i] + bu[j][i];
            // silu with the hardware exp2 and reciprocal (relative error ~1e-7,
            // far below the e4m3 spacing h is rounded to)
            const float ex = __builtin_amdgcn_exp2f(-gv * 1.44269504088896341f);
            const float hv = gv * __builtin_amdgcn_rcpf(1.0f + ex) * uv;
            acc[mb][j][i] = hv;
            mx = nan_max(mx, fabsf(hv));
          }
        mx = nan_max(mx, __shfl_xor(mx, 16));
        pmax[mb] = nan_max(mx, __shfl_xor(mx, 32));
      }
      if constexpr (MX) {
        // the wave's 32 h columns of a row are one MX block: no exchange, no barrier
        const __amdgpu_buffer_rsrc_t rH =
            __builtin_amdgcn_make_buffer_rsrc(g.Hq, (short)0, g.out_bytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rHs =
            __builtin_amdgcn_make_buffer_rsrc(g.Hs, (short)0, g.out2_bytes, kRsrcWord3);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = wm * W_HALF + 16 * mb + l16;
          const uint32_t code = mx_code(pmax[mb]);
          const float inv = mx_inv_scale(code);
          const bool ok = r < t.valid;
          const uint32_t hrow = (uint32_t)(t.row0 + r) * (uint32_t)g.f + n0 + 32 * wn + 4 * gq;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(
                f32x4_to_e4m3(acc[mb][j][0] * inv, acc[mb][j][1] * inv, acc[mb][j][2] * inv,
                              acc[mb][j][3] * inv),
                rH, ok ? (int)(hrow + 16 * j) : (int)kOob, 0, 0);
          const uint32_t so = (uint32_t)(t.row0 + r) * (uint32_t)(g.f / 32) + 4 * t.nt + wn;
          __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(code), rHs,
                                               (ok && gq == 0) ? (int)so : (int)kOob, 0, 0);
        }
      } else {
        // row maxima over the four wave columns through LDS.  The previous
        // tile's readers are past at least one ring barrier; a bare s_barrier
        // (no memory fence) leaves the stage loads in flight.
        if (gq == 0)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) smax[wn * WM_ROWS + wm * W_HALF + 16 * mb + l16] = pmax[mb];
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the smax writes are done
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const __amdgpu_buffer_rsrc_t rH =
            __builtin_amdgcn_make_buffer_rsrc(g.Hq, (short)0, g.out_bytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rHs =
            __builtin_amdgcn_make_buffer_rsrc(g.Hs, (short)0, g.out2_bytes, kRsrcWord3);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = wm * W_HALF + 16 * mb + l16;
          const float amax = nan_max(nan_max(smax[r], smax[WM_ROWS + r]),
                                     nan_max(smax[2 * WM_ROWS + r], smax[3 * WM_ROWS + r]));
          const float s = group_scale(amax);
          const float inv = 1.0f / s;
          const bool ok = r < t.valid;
          const uint32_t hrow = (uint32_t)(t.row0 + r) * (uint32_t)g.f + n0 + 32 * wn + 4 * gq;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float q[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) q[i] = clamp_fp8(acc[mb][j][i] * inv);
            __builtin_amdgcn_raw_buffer_store_b32(f32x4_to_e4m3(q[0], q[1], q[2], q[3]), rH,
                                                  ok ? (int)(hrow + 16 * j) : (int)kOob, 0, 0);
          }
          const uint32_t so = 4u * ((uint32_t)(t.row0 + r) * (uint32_t)(g.f / kBlock) + t.nt);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, s), rHs,
                                                (ok && wn == 0 && gq == 0) ? (int)so : (int)kOob, 0, 0);
        }
      }
    } else {
      const __amdgpu_buffer_rsrc_t rY =
          __builtin_amdgcn_make_buffer_rsrc(g.Y, (short)0, g.out_bytes, kRsrcWord3);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int cl = 64 * wn + 16 * nb + 4 * gq;  // tile column
        const uint2 wb = *reinterpret_cast<const uint2*>(sbias + 2 * cl);
        const float b4[4] = {bf16_to_f32(wb.x & 0xffffu), bf16_to_f32(wb.x >> 16),
                             bf16_to_f32(wb.y & 0xffffu), bf16_to_f32(wb.y >> 16)};
        const int gc = n0 + cl;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = wm * W_HALF + 16 * mb + l16;
          const uint32_t o = 4u * ((uint32_t)(t.row0 + r) * (uint32_t)N + (uint32_t)gc);
          const v4u d = v4u{__builtin_bit_cast(uint32_t, acc[mb][nb][0] + b4[0]),
                            __builtin_bit_cast(uint32_t, acc[mb][nb][1] + b4[1]),
                            __builtin_bit_cast(uint32_t, acc[mb][nb][2] + b4[2]),
                            __builtin_bit_cast(uint32_t, acc[mb][nb][3] + b4[3])};
          __builtin_amdgcn_raw_buffer_store_b128(d, rY, (r < t.valid && gc < N) ? (int)o : (int)kOob,
                                                 0, 0);
        }
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (MX) {
          macc[mb][nb] = v4f{0.f, 0.f, 0.f, 0.f};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mb][nb][i] = 0.f;
        }
      }
    return ST;
  };

  // Ring wait: this wave's loads of the A stage about to be read (and, older,
  // of the B stage) are done; younger are the next B stage's BQ loads and
  // `pend` row-token loads and epilogue stores (none from a wave without
  // rows in the tile).  Then a bare s_barrier.
  auto wait_stage = [&](int pend) {
    if (pend == 0) wait_vmcnt<BQ>();
    else if (pend == RT) wait_vmcnt<BQ + RT>();
    else if (pend == ST) wait_vmcnt<BQ + ST>();
    else if (pend == RT + ST) wait_vmcnt<BQ + RT + ST>();
    else wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- prologue: the successor of the second tile, row tokens of the first
  // two tiles, then B of K blocks 0 and 1 and A of K block 0 (the B stages
  // are older than the A stage)
  fetch();
  rt_load(ta, true, 0);
  rt_load(tan, Lan < hi, 1);
  if constexpr (GATED) {
    wait_vmcnt<0>();
    __syncthreads();
  }
  setup_a(ta, 0);
  setup_b(tb);
  issue_b(sb0);
  advance_b();
  int pend = 0;
  issue_a(sa0);
  pend = advance_a();
  issue_b(sb1);
  advance_b();

  // One K block: compute reads A stage i % 2 and B stage i % 3; loads A of
  // block i + 1 and B of block i + 2.  Returns false after the last tile.
  auto step = [&](const uint8_t* ca, uint8_t* na, const uint8_t* cb, uint8_t* nb2) -> bool {
    wait_stage(pend);
    issue_a(na);
    if constexpr (MX) compute_mx(ca, cb);
    else compute(ca, cb);
    issue_b(nb2);
    pend = advance_a();
    advance_b();
    if (++kbc < nkb) return true;
    pend += epilogue(tc, ca);
    Lc = dyn ? La : Lc + nslots;  // the A cursor moved to the next tile one step ago
    if (Lc >= hi) return false;
    fetch();
    kbc = 0;
    tc = dma_tile(g, Lc);
    return true;
  };
  while (step(sa0, sa1, sb0, sb2) && step(sa1, sa0, sb1, sb0) && step(sa0, sa1, sb2, sb1) &&
         step(sa1, sa0, sb0, sb2) && step(sa0, sa1, sb1, sb0) && step(sa1, sa0, sb2, sb1)) {
  }
  wait_vmcnt<0>();  // the loads past the last tile land before the workgroup ends
  finish();
}

// ---------------------------------------------------------------------------
// Split-K finish kernels (decode path): the K splits' fp32 partial sums
// [ksplit][R][N] are added in split order, then the fused epilogue of the
// unsplit GEMM follows: bias, SwiGLU and h quantisation (gated), or bias (plain).

// Expert of permuted row r: the last e with offsets[e] <= r (offsets[E] = R > r).
__device__ __forceinline__ int row_expert(const int32_t* __restrict__ offsets, int E, int r) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

// One wave per (row, 128 h columns); lane l holds h columns 2l, 2l + 1 of the
// group.  h = silu(gate) * up with the same arithmetic as the fused epilogue,
// quantised per 128 columns (fp32 scale) or, with MX, per 32 (E8M0).
template <bool MX>
__global__ __launch_bounds__(256) void splitk_gated_finish(GemmArgs g) {
  const int lane = threadIdx.x & 63;
  const int groups = g.f / kBlock;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= g.R * groups) return;
  const int r = item / groups, gi = item - (item / groups) * groups;
  const int e = row_expert(g.offsets, g.E, r);
  const int N = 2 * g.f;
  const int c = gi * kBlock + 2 * lane;
  float h[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float gs = 0.f, us = 0.f;
    for (int s = 0; s < g.ksplit; ++s) {
      const float* p = g.part + ((size_t)s * g.R + r) * N;
      gs += p[c + i];
      us += p[g.f + c + i];
    }
    const float gv = gs + bf16_to_f32(g.bias[(size_t)e * N + c + i]);
    const float uv = us + bf16_to_f32(g.bias[(size_t)e * N + g.f + c + i]);
    const float ex = __builtin_amdgcn_exp2f(-gv * 1.44269504088896341f);
    h[i] = gv * __builtin_amdgcn_rcpf(1.0f + ex) * uv;
  }
  float mx = nan_max(fabsf(h[0]), fabsf(h[1]));
  uint8_t* hq = g.Hq + (size_t)r * g.f + c;
  if constexpr (MX) {
    // a 32-column block is 16 lanes
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) mx = nan_max(mx, __shfl_xor(mx, o));
    const uint32_t code = mx_code(mx);
    const float inv = mx_inv_scale(code);
    *reinterpret_cast<uint16_t*>(hq) = static_cast<uint16_t>(f32x2_to_e4m3(h[0] * inv, h[1] * inv));
    if ((lane & 15) == 0)
      static_cast<uint8_t*>(g.Hs)[(size_t)r * (g.f / 32) + 4 * gi + (lane >> 4)] = static_cast<uint8_t>(code);
  } else {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = nan_max(mx, __shfl_xor(mx, o));
    const float sc = group_scale(mx);
    const float inv = 1.0f / sc;
    *reinterpret_cast<uint16_t*>(hq) =
        static_cast<uint16_t>(f32x2_to_e4m3(clamp_fp8(h[0] * inv), clamp_fp8(h[1] * inv)));
    if (lane == 0) static_cast<float*>(g.Hs)[(size_t)r * groups + gi] = sc;
  }
}

// Y[r][n..n+3] = sum over splits + bias, one thread per 4 columns.
__global__ __launch_bounds__(256) void splitk_plain_finish(GemmArgs g) {
  const int q = g.N / 4;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= g.R * q) return;
  const int r = idx / q, c = 4 * (idx - (idx / q) * q);
  const int e = row_expert(g.offsets, g.E, r);
  v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < g.ksplit; ++s)
    sum += *reinterpret_cast<const v4f*>(g.part + ((size_t)s * g.R + r) * g.N + c);
  const uint16_t* b = g.bias + (size_t)e * g.N + c;
  *reinterpret_cast<v4f*>(g.Y + (size_t)r * g.N + c) =
      v4f{sum[0] + bf16_to_f32(b[0]), sum[1] + bf16_to_f32(b[1]), sum[2] + bf16_to_f32(b[2]),
          sum[3] + bf16_to_f32(b[3])};
}

int grid_for(int max_tiles) { return 8 * ceil_div(max_tiles, 8); }

// Launch facts of a device, looked up once per device and then read without
// a lock: std::call_once orders the first lookup before every later read, so
// concurrent callers on several host threads see a complete value.
constexpr int kMaxDevices = 64;

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  return dev;
}

// Compute units of the current device, rounded up to a multiple of 8 (one
// slice per XCD).
int device_cus() {
  auto lookup = [](int dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return 8 * ceil_div(n, 8);
  };
  const int dev = current_device();
  if (dev >= kMaxDevices) return lookup(dev);
  static std::once_flag once[kMaxDevices];
  static int cus[kMaxDevices];
  std::call_once(once[dev], [&] { cus[dev] = lookup(dev); });
  return cus[dev];
}

// Persistent prefill grid: one workgroup per CU (a multiple of 8, one slice
// per XCD), fewer when the tile list cannot fill them.
int grid_persistent(int max_tiles) { return std::min(device_cus(), grid_for(max_tiles)); }

// Persistent decode grid: as many workgroups per CU as the kernel's registers
// and LDS allow, at most two (a second workgroup keeps a second ring of weight
// loads in flight on the CU), fewer when the tile list cannot fill them.  The
// occupancy is looked up once per kernel instance and device.
template <bool GATED, int DBM, int DBN, bool MX, bool FP4, bool SPLIT>
dim3 grid_decode(int max_tiles) {
  auto lookup = [] {
    int n = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, grouped_gemm_dma_kernel<GATED, DBM, DBN, MX, FP4, SPLIT>, DMA_WAVES * 64, 0) != hipSuccess ||
        n < 1)
      n = 1;
    return std::min(n, 2);
  };
  const int dev = current_device();
  int per;
  if (dev >= kMaxDevices) {
    per = lookup();
  } else {
    static std::once_flag once[kMaxDevices];
    static int per_dev[kMaxDevices];
    std::call_once(once[dev], [&] { per_dev[dev] = lookup(); });
    per = per_dev[dev];
  }
  return dim3(std::min(per * device_cus(), grid_for(max_tiles)));
}

template <bool GATED, int DBM, int DBN, bool MX, bool FP4>
hipError_t launch_decode(const GemmArgs& a, int max_tiles, hipStream_t stream) {
  const dim3 block(DMA_WAVES * 64);
  if (a.ksplit <= 1) {
    hipLaunchKernelGGL((grouped_gemm_dma_kernel<GATED, DBM, DBN, MX, FP4, false>),
                       (grid_decode<GATED, DBM, DBN, MX, FP4, false>(max_tiles)), block, 0, stream, a);
    return hipGetLastError();
  }
  const int items = max_tiles * a.ksplit;
  hipLaunchKernelGGL((grouped_gemm_dma_kernel<GATED, DBM, DBN, MX, FP4, true>),
                     (grid_decode<GATED, DBM, DBN, MX, FP4, true>(items)), block, 0, stream, a);
  if (GATED)
    hipLaunchKernelGGL((splitk_gated_finish<MX>), dim3(ceil_div(a.R * (a.f / kBlock), 4)), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(splitk_plain_finish, dim3(ceil_div(a.R * (a.N / 4), 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <bool GATED, int DBM, int DBN>
hipError_t launch_gemm(const GemmArgs& a, bool decode, int fmt, int max_tiles, hipStream_t stream) {
  if (max_tiles <= 0) return hipSuccess;
  const dim3 grid(grid_persistent(max_tiles)), block(DMA_WAVES * 64);
  if (decode) {
    if (fmt == kFmtMxFp4) return launch_decode<GATED, DBM, DBN, true, true>(a, max_tiles, stream);
    if (fmt == kFmtMx) return launch_decode<GATED, DBM, DBN, true, false>(a, max_tiles, stream);
    return launch_decode<GATED, DBM, DBN, false, false>(a, max_tiles, stream);
  }
  if (fmt == kFmtMxFp4)
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<GATED, true, true>), grid, block, 0, stream, a);
  else if (fmt == kFmtMx)
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<GATED, true, false>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<GATED, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_gated(const GemmArgs& a, bool decode, int fmt, int max_tiles,
                             hipStream_t stream) {
  static_assert(kGatedPrefill.bm == WM_ROWS && kGatedPrefill.bnp == WN_COLS, "wide tile");
  return launch_gemm<true, kGatedDecode.bm, kGatedDecode.bnp>(a, decode, fmt, max_tiles, stream);
}

hipError_t launch_gemm_plain(const GemmArgs& a, bool decode, int fmt, int max_tiles,
                             hipStream_t stream) {
  static_assert(kPlainPrefill.bm == WM_ROWS && kPlainPrefill.bnp == WN_COLS, "wide tile");
  return launch_gemm<false, kPlainDecode.bm, kPlainDecode.bnp>(a, decode, fmt, max_tiles, stream);
}

}  // namespace moe
