// C ABI of the MoE block forward: argument checks, workspace carving and the
// launch sequence on the caller's stream.  No allocation, no host sync.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "kernels.hpp"
#include "moe.h"

namespace {

using moe::ceil_div;

constexpr int64_t kMaxRows = int64_t(1) << 28;  // T*k bound (row indices are int32)
constexpr int64_t kMaxBuffer = int64_t(1) << 31;

struct Layout {
  size_t partial, topk_idx, topk_w, hist, counts, offsets, tile_base, tile_off0, tile_off1, tiles0,
      tiles1, row_of, row_token, xq, xs, hq, hs, y, kpart, sched, total;
};

// Decode-path GEMM shapes for T*k = R rows: tile-count bounds and K splits
// (the same numbers the launch uses, so the workspace holds the partials).
struct DecodeSplit {
  int max_g, max_p, sg, sp;
};
DecodeSplit decode_split(int64_t R, int64_t d, int64_t f, int64_t E) {
  const int nz = (int)(E < R ? E : R);
  DecodeSplit s{};
  s.max_g = (ceil_div((int)R, moe::kGatedDecode.bm) + nz) * (int)(f / moe::kBlock);
  s.max_p = (ceil_div((int)R, moe::kPlainDecode.bm) + nz) * ceil_div((int)d, moe::kPlainDecode.bnp);
  s.sg = moe::decode_ksplits(s.max_g, (int)(d / moe::kBlock));
  s.sp = moe::decode_ksplits(s.max_p, (int)(f / moe::kBlock));
  return s;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

Layout make_layout(int64_t T, int64_t d, int64_t f, int64_t E, int64_t k) {
  const int64_t R = T * k, NT = ceil_div((int)T, moe::RT_TT);
  Layout l{};
  size_t o = 0;
  auto put = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const int64_t ns = moe::router_splits((int)T, (int)d, (int)E);
  l.partial = put(ns > 1 ? 4 * ns * T * (16 * ceil_div((int)E, 16)) : 0);  // experts padded to 16
  l.topk_idx = put(4 * R);
  l.topk_w = put(4 * R);
  l.hist = put(4 * NT * E);
  l.counts = put(4 * E);
  l.offsets = put(4 * (E + 1));
  l.tile_base = put(4 * NT * E);
  l.tile_off0 = put(4 * (E + 1));
  l.tile_off1 = put(4 * (E + 1));
  // tile lists, sized for the shorter (decode) row tiles
  const int64_t mtiles = ceil_div((int)R, moe::kGatedDecode.bm) + (E < R ? E : R);
  l.tiles0 = put(16 * mtiles * (f / moe::kBlock));
  l.tiles1 = put(16 * mtiles * ceil_div((int)d, moe::kPlainDecode.bnp));
  l.row_of = put(4 * R);
  l.row_token = put(4 * R);
  l.xq = put(T * d);
  l.xs = put(4 * T * (d / moe::kBlock));
  l.hq = put(R * f);
  l.hs = put(4 * R * (f / moe::kBlock));
  l.y = put(4 * R * d);
  // split-K partial sums of the decode-path GEMMs [splits][R][N], fp32
  const DecodeSplit ds = decode_split(R, d, f, E);
  const int64_t kp = ds.sg > 1 || ds.sp > 1 ? std::max<int64_t>(ds.sg * 2 * f, ds.sp * d) : 0;
  l.kpart = put(4 * R * kp);
  // tile counters of the prefill GEMMs' dynamic schedule (gate/up, down)
  l.sched = put(4 * 2 * moe::kSchedInts);
  l.total = o;
  return l;
}

moe_status check_sizes(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k) {
  if (T < 0 || d <= 0 || f <= 0 || E < 1 || d % MOE_BLOCK || f % MOE_BLOCK) return MOE_ERR_SHAPE;
  if (k < 1 || k > E || k > MOE_MAX_TOPK || E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  // the GEMMs keep one weight scale per K block in one lane: at most 64 blocks
  if ((int64_t)T * k > kMaxRows || d > 64 * MOE_BLOCK || f > 64 * MOE_BLOCK)
    return MOE_ERR_UNSUPPORTED;
  // The GEMMs address their loads and stores through 32-bit buffer offsets,
  // and a masked lane stores at offset 2^31, which the buffer's size must
  // exclude: every buffer they touch stays below 2^31 bytes (x codes, h
  // codes, one expert's weights, the activation scales and the fp32 expert
  // outputs Y, 4*R*d bytes).
  const int64_t R = (int64_t)T * k;
  if ((int64_t)T * d >= kMaxBuffer || R * f >= kMaxBuffer || 2 * (int64_t)d * f >= kMaxBuffer ||
      4 * R * (d / MOE_BLOCK + f / MOE_BLOCK) >= kMaxBuffer || 4 * R * d >= kMaxBuffer)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The workspace of moe_forward_noalloc: a device array of the library, one
// copy per GPU, alive until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels and copies get the address
// that hipGetSymbolAddress returns for the current device instead.
constexpr size_t kScratchBytes = MOE_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup failed.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  static std::once_flag once[kMaxScratchDevices];
  static void* ptr[kMaxScratchDevices];
  std::call_once(once[dev], [&] {
    void* p = nullptr;
    ptr[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
  });
  return ptr[dev];
}

bool valid_flags(uint32_t flags) {
  return (flags & ~(MOE_PATH_MASK | MOE_ROUTE_SOFTMAX_ALL | MOE_GATE_BF16 | MOE_FORMAT_MX |
                    MOE_WEIGHTS_FP4)) == 0u &&
         (flags & MOE_PATH_MASK) != MOE_PATH_MASK &&
         !((flags & MOE_WEIGHTS_FP4) != 0u && (flags & MOE_FORMAT_MX) == 0u);
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k) {
  if (check_sizes(T, d, f, E, k) != MOE_OK) return 0;
  return make_layout(T, d, f, E, k).total;
}

const char* moe_status_string(int32_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "invalid shape (T < 0, or d/f not a positive multiple of 128, or E < 1)";
    case MOE_ERR_UNSUPPORTED: return "unsupported sizes (k outside [1, min(E, 8)], E > 256, d or f > 8192, or a buffer of 2^31 bytes or more)";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MOE_ERR_HIP: return "a HIP kernel launch failed";
    case MOE_ERR_FLAGS: return "unknown flags";
    case MOE_ERR_SCRATCH: return "these sizes need more workspace than the library's static scratch (MOE_SCRATCH_BYTES); pass a workspace to moe_forward_ex instead";
    default: return "unknown status";
  }
}

moe_status moe_forward_stages(const void* x, const float* W_router, const float* b_router,
                              int32_t k, const uint8_t* W_gateup, const float* S_gateup,
                              const void* b_gateup, const uint8_t* W_down, const float* S_down,
                              const void* b_down, void* out, int32_t T, int32_t d, int32_t f,
                              int32_t E, void* workspace, size_t workspace_bytes, uint32_t flags,
                              int32_t first_stage, int32_t last_stage, hipStream_t stream) {
  const moe_status sz = check_sizes(T, d, f, E, k);
  if (sz != MOE_OK) return sz;
  if (!valid_flags(flags)) return MOE_ERR_FLAGS;
  const uint32_t path = flags & MOE_PATH_MASK;
  const bool mx = (flags & MOE_FORMAT_MX) != 0u;
  const int fmt = (flags & MOE_WEIGHTS_FP4) ? moe::kFmtMxFp4 : mx ? moe::kFmtMx : moe::kFmtBlock;
  const int gate_mode = ((flags & MOE_ROUTE_SOFTMAX_ALL) ? moe::kGateSoftmaxAll : 0) |
                        ((flags & MOE_GATE_BF16) ? moe::kGateBf16 : 0);
  if (first_stage < 0 || last_stage >= MOE_NUM_STAGES || first_stage > last_stage)
    return MOE_ERR_FLAGS;
  if (T == 0) return MOE_OK;
  const void* ptrs[] = {x, W_router, b_router, W_gateup, S_gateup, b_gateup,
                        W_down, S_down, b_down, out, workspace};
  for (const void* p : ptrs)
    if (p == nullptr) return MOE_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  const Layout l = make_layout(T, d, f, E, k);
  if (workspace_bytes < l.total) return MOE_ERR_WORKSPACE;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  auto at = [&](size_t off) { return ws + off; };
  float* partial = reinterpret_cast<float*>(at(l.partial));
  int32_t* topk_idx = reinterpret_cast<int32_t*>(at(l.topk_idx));
  float* topk_w = reinterpret_cast<float*>(at(l.topk_w));
  int32_t* hist = reinterpret_cast<int32_t*>(at(l.hist));
  int32_t* counts = reinterpret_cast<int32_t*>(at(l.counts));
  int32_t* offsets = reinterpret_cast<int32_t*>(at(l.offsets));
  int32_t* tile_base = reinterpret_cast<int32_t*>(at(l.tile_base));
  int32_t* tile_off0 = reinterpret_cast<int32_t*>(at(l.tile_off0));
  int32_t* tile_off1 = reinterpret_cast<int32_t*>(at(l.tile_off1));
  int32_t* tiles0 = reinterpret_cast<int32_t*>(at(l.tiles0));
  int32_t* tiles1 = reinterpret_cast<int32_t*>(at(l.tiles1));
  int32_t* row_of = reinterpret_cast<int32_t*>(at(l.row_of));
  int32_t* row_token = reinterpret_cast<int32_t*>(at(l.row_token));
  uint8_t* xq = at(l.xq);
  void* xs = at(l.xs);  // fp32 [T, d/128] or E8M0 [T, d/32]: the same bytes
  uint8_t* hq = at(l.hq);
  void* hs = at(l.hs);
  float* y = reinterpret_cast<float*>(at(l.y));
  float* kpart = reinterpret_cast<float*>(at(l.kpart));
  int32_t* sched = reinterpret_cast<int32_t*>(at(l.sched));

  const int R = T * k;
  const int NT = ceil_div(T, moe::RT_TT);
  bool decode;
  if (path == MOE_PATH_AUTO) decode = (int64_t)R <= 32 * (int64_t)E;
  else decode = path == MOE_PATH_DECODE;
  const moe::GemmShape gs = decode ? moe::kGatedDecode : moe::kGatedPrefill;
  const moe::GemmShape ps = decode ? moe::kPlainDecode : moe::kPlainPrefill;
  const int nt_g = f / moe::kBlock;
  const int nt_p = ceil_div(d, ps.bnp);
  const int nz = E < R ? E : R;  // experts that can hold rows
  const int max_g = (ceil_div(R, gs.bm) + nz) * nt_g;
  const int max_p = (ceil_div(R, ps.bm) + nz) * nt_p;
  // split K for decode batches with few tiles (prefill tiles are never split)
  const DecodeSplit dsp = decode_split(R, d, f, E);
  const int ks_g = decode ? dsp.sg : 1, ks_p = decode ? dsp.sp : 1;
  const bool small = NT == 1;  // the whole routing runs in the router stage

  for (int stage = first_stage; stage <= last_stage; ++stage) {
    hipError_t err = hipSuccess;
    switch (stage) {
      case MOE_STAGE_ROUTER: {
        const moe::SmallRoute sr{counts,  offsets, tile_off0, tile_off1, tiles0, tiles1, row_of,
                                 row_token, gs.bm,   nt_g,      max_g,     ps.bm,  nt_p,   max_p};
        err = moe::launch_router(static_cast<const uint16_t*>(x), W_router, b_router, T, d, E, k,
                                 gate_mode, mx, partial, topk_idx, topk_w, hist, xq, xs,
                                 small ? &sr : nullptr, stream);
        break;
      }
      case MOE_STAGE_SCAN:
        if (small) break;  // done by the router stage
        err = moe::launch_route_scan(hist, NT, E, gs.bm, nt_g, ps.bm, nt_p, counts, offsets,
                                     tile_base, tile_off0, tile_off1, stream);
        break;
      case MOE_STAGE_PLACE:
        if (small) break;  // done by the router stage
        err = moe::launch_route_place_tables(topk_idx, tile_base, T, E, k, row_of, row_token, counts,
                                             offsets, tile_off0, gs.bm, nt_g, max_g, tiles0, tile_off1,
                                             ps.bm, nt_p, max_p, tiles1, sched, stream);
        break;
      case MOE_STAGE_GATEUP: {
        moe::GemmArgs g{};
        g.A = xq;
        g.As = xs;
        g.row_token = row_token;
        g.B = W_gateup;
        g.Bs = S_gateup;
        g.bias = static_cast<const uint16_t*>(b_gateup);
        g.counts = counts;
        g.offsets = offsets;
        g.tile_off = tile_off0;
        g.tiles = tiles0;
        g.rows_bytes = (int)(4 * (int64_t)R);
        g.out_bytes = (int)((int64_t)R * f);
        g.out2_bytes = (int)(4 * (int64_t)R * (f / moe::kBlock));
        g.K = d;
        g.N = 2 * f;
        g.f = f;
        g.n_tiles = nt_g;
        g.E = E;
        g.Hq = hq;
        g.Hs = hs;
        g.A_bytes = (int)((int64_t)T * d);
        g.As_bytes = (int)(4 * (int64_t)T * (d / moe::kBlock));
        g.ksplit = ks_g;
        g.kper = moe::decode_kper(d / moe::kBlock, ks_g);
        g.R = R;
        g.part = kpart;
        g.part_bytes = (int)(4 * (int64_t)ks_g * R * 2 * f);
        // the place stage wrote the XCD ranges and zeroed the counters
        // (batches of one router tile keep the static schedule: no place stage)
        g.sched = small ? nullptr : sched;
        err = moe::launch_gemm_gated(g, decode, fmt, max_g, stream);
        break;
      }
      case MOE_STAGE_DOWN: {
        moe::GemmArgs p{};
        p.A = hq;
        p.As = hs;
        p.B = W_down;
        p.Bs = S_down;
        p.bias = static_cast<const uint16_t*>(b_down);
        p.counts = counts;
        p.offsets = offsets;
        p.tile_off = tile_off1;
        p.tiles = tiles1;
        p.rows_bytes = (int)(4 * (int64_t)R);
        p.out_bytes = (int)(4 * (int64_t)R * d);
        p.K = f;
        p.N = d;
        p.f = f;
        p.n_tiles = nt_p;
        p.E = E;
        p.Y = y;
        p.A_bytes = (int)((int64_t)R * f);
        p.As_bytes = (int)(4 * (int64_t)R * (f / moe::kBlock));
        p.ksplit = ks_p;
        p.kper = moe::decode_kper(f / moe::kBlock, ks_p);
        p.R = R;
        p.part = kpart;
        p.part_bytes = (int)(4 * (int64_t)ks_p * R * d);
        p.sched = small ? nullptr : sched + moe::kSchedInts;
        err = moe::launch_gemm_plain(p, decode, fmt, max_p, stream);
        break;
      }
      case MOE_STAGE_COMBINE:
        err = moe::launch_combine(y, row_of, topk_w, T, d, k, static_cast<uint16_t*>(out), stream);
        break;
    }
    if (err != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_status moe_forward_ex(const void* x, const float* W_router, const float* b_router, int32_t k,
                          const uint8_t* W_gateup, const float* S_gateup, const void* b_gateup,
                          const uint8_t* W_down, const float* S_down, const void* b_down,
                          void* out, int32_t T, int32_t d, int32_t f, int32_t E, void* workspace,
                          size_t workspace_bytes, uint32_t flags, hipStream_t stream) {
  return moe_forward_stages(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down, S_down,
                            b_down, out, T, d, f, E, workspace, workspace_bytes, flags, 0,
                            MOE_NUM_STAGES - 1, stream);
}

moe_status moe_forward(const void* x, const float* W_router, const float* b_router, int32_t k,
                       const uint8_t* W_gateup, const float* S_gateup, const void* b_gateup,
                       const uint8_t* W_down, const float* S_down, const void* b_down, void* out,
                       int32_t T, int32_t d, int32_t f, int32_t E, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return moe_forward_ex(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down, S_down,
                        b_down, out, T, d, f, E, workspace, workspace_bytes, MOE_PATH_AUTO, stream);
}

moe_status moe_forward_mx(const void* x, const float* W_router, const float* b_router, int32_t k,
                          const uint8_t* W_gateup, const uint8_t* X_gateup, const void* b_gateup,
                          const uint8_t* W_down, const uint8_t* X_down, const void* b_down,
                          void* out, int32_t T, int32_t d, int32_t f, int32_t E, void* workspace,
                          size_t workspace_bytes, uint32_t flags, hipStream_t stream) {
  return moe_forward_stages(x, W_router, b_router, k, W_gateup,
                            reinterpret_cast<const float*>(X_gateup), b_gateup, W_down,
                            reinterpret_cast<const float*>(X_down), b_down, out, T, d, f, E,
                            workspace, workspace_bytes, flags | MOE_FORMAT_MX, 0,
                            MOE_NUM_STAGES - 1, stream);
}

moe_status moe_forward_noalloc(const void* x, const float* W_router, const float* b_router,
                               int32_t k, const uint8_t* W_gateup, const float* S_gateup,
                               const void* b_gateup, const uint8_t* W_down, const float* S_down,
                               const void* b_down, void* out, int32_t T, int32_t d, int32_t f,
                               int32_t E, uint32_t flags, hipStream_t stream) {
  const moe_status sz = check_sizes(T, d, f, E, k);
  if (sz != MOE_OK) return sz;
  if (make_layout(T, d, f, E, k).total > kScratchBytes) return MOE_ERR_SCRATCH;
  if (!valid_flags(flags)) return MOE_ERR_FLAGS;
  if (T == 0) return MOE_OK;
  const void* ptrs[] = {x, W_router, b_router, W_gateup, S_gateup, b_gateup, W_down, S_down, b_down, out};
  for (const void* p : ptrs)
    if (p == nullptr) return MOE_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  void* ws = scratch_address();
  if (ws == nullptr) return MOE_ERR_HIP;
  // Nothing in the workspace has to start at zero: every stage writes what
  // the later stages read before they read it.
  return moe_forward_stages(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down, S_down,
                            b_down, out, T, d, f, E, ws, kScratchBytes, flags, 0,
                            MOE_NUM_STAGES - 1, stream);
}

moe_status moe_forward_debug(const void* x, const float* W_router, const float* b_router,
                             int32_t k, const uint8_t* W_gateup, const float* S_gateup,
                             const void* b_gateup, const uint8_t* W_down, const float* S_down,
                             const void* b_down, void* out, int32_t T, int32_t d, int32_t f,
                             int32_t E, void* workspace, size_t workspace_bytes, uint32_t flags,
                             hipStream_t stream, int32_t* topk_idx, float* topk_w, int32_t* offsets,
                             int32_t* row_token, int32_t* row_of, uint8_t* xq, float* xs,
                             uint8_t* hq, float* hs, float* y) {
  const moe_status st =
      moe_forward_ex(x, W_router, b_router, k, W_gateup, S_gateup, b_gateup, W_down, S_down,
                     b_down, out, T, d, f, E, workspace, workspace_bytes, flags, stream);
  if (st != MOE_OK || T == 0) return st;
  const Layout l = make_layout(T, d, f, E, k);
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  const size_t R = (size_t)T * k;
  struct Copy {
    void* dst;
    size_t off, bytes;
  } copies[] = {
      {topk_idx, l.topk_idx, 4 * R},
      {topk_w, l.topk_w, 4 * R},
      {offsets, l.offsets, 4 * ((size_t)E + 1)},
      {row_token, l.row_token, 4 * R},
      {row_of, l.row_of, 4 * R},
      {xq, l.xq, (size_t)T * d},
      {xs, l.xs, 4 * (size_t)T * (d / MOE_BLOCK)},
      {hq, l.hq, R * f},
      {hs, l.hs, 4 * R * (f / MOE_BLOCK)},
      {y, l.y, 4 * R * d},
  };
  for (const Copy& c : copies) {
    if (c.dst == nullptr) continue;
    if (hipMemcpyAsync(c.dst, ws + c.off, c.bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return MOE_ERR_HIP;
  }
  return MOE_OK;
}

}  // extern "C"
