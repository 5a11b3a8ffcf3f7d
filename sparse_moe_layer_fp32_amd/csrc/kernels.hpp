// Host-side launchers of the MoE kernels (one translation unit per kernel family).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

constexpr int RT_TT = 64;     // tokens per router / placement workgroup (histogram tile)
constexpr int kTileGroup = 4; // column tiles per group in a GEMM's tile order
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 256;

// GEMM tile shapes.  "Gated" is gate/up + bias + SwiGLU + h quantisation,
// "plain" is down + bias.  Prefill tiles are MFMA-bound, decode tiles stream
// the weights with few rows.
struct GemmShape {
  int bm;       // rows per tile
  int bnp;      // B columns per tile (gate+up columns for the gated kernel)
};
constexpr GemmShape kGatedPrefill{192, 256};
constexpr GemmShape kGatedDecode{32, 256};
constexpr GemmShape kPlainPrefill{192, 256};
constexpr GemmShape kPlainDecode{32, 128};

// Scales: block-scaled fp32 (As [rows, K/128], Bs [E, K/128, N/128], Hs
// [R, f/128]) or MX E8M0 bytes (As [rows, K/32], Bs [E, K/32, N], Hs [R, f/32]).
struct GemmArgs {
  const uint8_t* A;            // e4m3 activations: x codes [T,K] (gated) or h codes [R,K] (plain)
  const void* As;              // their scales
  const int32_t* row_token;    // gated: token of each permuted row
  const uint8_t* B;            // weights [E, K, N] e4m3 (FP4: [E, K/2, N], two E2M1 per byte)
  const void* Bs;              // weight scales
  const uint16_t* bias;        // bf16 [E, N]
  const int32_t* counts;       // rows per expert [E]
  const int32_t* offsets;      // first row per expert [E+1]
  const int32_t* tile_off;     // first tile per expert [E+1] (this kernel's tiling)
  const int32_t* tiles;        // prefill: tile list [tiles][4] = {expert, first row, rows, column tile}
  int K, N, f, n_tiles, E;
  int A_bytes, As_bytes;       // sizes of A and As (buffer bounds; reads past them give 0)
  int rows_bytes;              // 4 * R: size of row_token
  int out_bytes, out2_bytes;   // gated: sizes of Hq and Hs; plain: size of Y
  uint8_t* Hq;                 // gated outputs: h codes [R, f] and their scales
  void* Hs;
  float* Y;                    // plain output [R, N]
  // split K (decode path only; ksplit = 1 otherwise): K blocks per split,
  // the routed rows R, and the fp32 partial sums [ksplit][R][N] in the workspace
  int ksplit, kper, R;
  float* part;
  int part_bytes;
  // prefill: the schedule block of this GEMM (kSchedInts ints, see below);
  // nullptr: eight equal ranges of the tile list and a fixed round robin
  int32_t* sched;
};
// Schedule block of a prefill GEMM: ints [0, 8) the tile counters of the
// XCDs, [8] the count of finished workgroups (both zero before the launch
// and zero again after it), [kSchedBounds, kSchedBounds + 9) the first tile
// of every XCD's range of the tile list (ranges of equal cost) and the end.
constexpr int kSchedInts = 32;
constexpr int kSchedCounters = 16;  // the leading ints the place stage zeroes
constexpr int kSchedBounds = 16;

// K splits of a decode-path GEMM with at most max_tiles tiles of nkb K
// blocks: with fewer tiles than the chip has workgroup slots (two per CU of
// the 256-CU part), each tile is cut into K ranges of at least 4 blocks so
// that about 512 (tile, split) items run, and every range keeps at least two
// blocks.  Host-only arithmetic on the sizes, so the workspace can be sized
// without a device query.
inline int decode_ksplits(int max_tiles, int nkb) {
  if (max_tiles <= 0 || max_tiles >= 256) return 1;
  int s = 512 / max_tiles;
  if (s > nkb / 4) s = nkb / 4;
  if (s > 8) s = 8;
  while (s > 1) {
    const int kper = (nkb + s - 1) / s;
    if (nkb - (s - 1) * kper >= 2) break;
    --s;
  }
  return s < 1 ? 1 : s;
}
inline int decode_kper(int nkb, int ksplit) { return (nkb + ksplit - 1) / ksplit; }

// Waves per router workgroup (4: 64 tokens; 8: 128 tokens, for large batches
// with at most 128 experts) and K splits of the router for T tokens (1: top-k
// fused into the router kernel; >1: partial logits [splits][T][E] fp32 in
// `partial`, then a top-k kernel).
int router_waves(int T, int E);
int router_splits(int T, int d, int E);

// Outputs of the whole-batch routing path (T <= RT_TT): the router stage then
// also writes counts, offsets, both tile lists and the placement.
struct SmallRoute {
  int32_t *counts, *offsets, *tile_off0, *tile_off1, *tiles0, *tiles1, *row_of, *row_token;
  int bm0, nt0, max0, bm1, nt1, max1;
};

// sr == nullptr: top-k + histogram per router tile (scan and placement follow
// as their own stages); otherwise the whole routing of a one-tile batch.
// Gate-weight rule (bits of gate_mode): softmax over all E logits instead of
// the selected k; round the weights to bf16.
constexpr int kGateSoftmaxAll = 1;
constexpr int kGateBf16 = 2;

// mx: x is quantised per 32 columns with E8M0 scales (xs bytes [T, d/32]);
// otherwise per 128 columns with fp32 scales (xs floats [T, d/128]).
hipError_t launch_router(const uint16_t* x, const float* Wr, const float* br, int T, int d, int E,
                         int k, int gate_mode, bool mx, float* partial, int32_t* topk_idx,
                         float* topk_w, int32_t* hist, uint8_t* xq, void* xs, const SmallRoute* sr,
                         hipStream_t stream);

hipError_t launch_route_scan(const int32_t* hist, int ntiles, int E, int bm0, int nt0, int bm1,
                             int nt1, int32_t* counts, int32_t* offsets, int32_t* tile_base,
                             int32_t* tile_off0, int32_t* tile_off1, hipStream_t stream);

// After the scan: the row of every (token, slot) pair (rank among the earlier
// pairs of its router tile with the same expert), and the tile lists of both
// grouped GEMMs from their per-expert tile offsets (row blocks of bm rows,
// nt column tiles, grouped kTileGroup column tiles at a time), in one launch.
// Also, in one more workgroup, both GEMMs' schedule blocks at sched: the
// counters zeroed, and the XCD ranges, eight ranges of the tile list of equal
// cost, a tile whose rows fill at most half of its row block counting 2/3
// (gate/up) or 1/2 (down) of a full tile (half the row waves idle, all the
// weight loads run).
hipError_t launch_route_place_tables(const int32_t* topk_idx, const int32_t* tile_base, int T, int E,
                                     int k, int32_t* row_of, int32_t* row_token, const int32_t* counts,
                                     const int32_t* offsets, const int32_t* tile_off0, int bm0,
                                     int nt0, int max0, int32_t* tiles0, const int32_t* tile_off1,
                                     int bm1, int nt1, int max1, int32_t* tiles1, int32_t* sched,
                                     hipStream_t stream);

hipError_t launch_combine(const float* Y, const int32_t* row_of, const float* topk_w, int T, int d,
                          int k, uint16_t* out, hipStream_t stream);

// Weight formats of the grouped GEMMs: 128x128 block-scaled FP8, MXFP8 (E8M0
// scales applied by the matrix cores), MXFP4 (E2M1 weights packed two per
// byte along K with E8M0 scales, MXFP8 activations).
constexpr int kFmtBlock = 0, kFmtMx = 1, kFmtMxFp4 = 2;

// max_tiles bounds the tile count so the grid covers every tile.
hipError_t launch_gemm_gated(const GemmArgs& a, bool decode, int fmt, int max_tiles,
                             hipStream_t stream);
hipError_t launch_gemm_plain(const GemmArgs& a, bool decode, int fmt, int max_tiles,
                             hipStream_t stream);

}  // namespace moe
