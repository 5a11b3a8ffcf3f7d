// C ABI of the sink-attention kernels: argument checks and launches.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attention.h"
#include "attention.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_heads(int32_t Hq, int32_t Hkv, int32_t D) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return MOE_ERR_SHAPE;
  if (D != 64) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

constexpr int64_t kMaxElems = int64_t(1) << 40;  // sanity bound on tensor sizes

}  // namespace

extern "C" {

moe_status attn_sink_prefill(const void* q, const void* k, const void* v, const float* sinks,
                             void* out, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                             float sm_scale, hipStream_t stream) {
  if (S < 0) return MOE_ERR_SHAPE;
  const moe_status hs = check_heads(Hq, Hkv, D);
  if (hs != MOE_OK) return hs;
  const int G = Hq / Hkv;
  if (!(G == 1 || G == 2 || G == 4 || G % 8 == 0)) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)S * Hq * D >= kMaxElems ||
      (int64_t)((S + 63) / 64 + 1) * 8 * (Hq / (G >= 8 ? 8 : G)) >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  if (S == 0) return MOE_OK;
  const void* ptrs[] = {q, k, v, sinks, out};
  for (const void* p : ptrs)
    if (p == nullptr) return MOE_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  const hipError_t e = moe::launch_attn_prefill(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      sinks, static_cast<uint16_t*>(out), S, Hq, Hkv, sm_scale, stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

namespace {
// segment records, then the plan (2 B + 2 int32, rounded to 16 bytes)
size_t decode_records_bytes(int32_t B, int32_t Hq, int32_t Lmax) {
  return (size_t)moe::attn_decode_slots(B, Lmax) * Hq * moe::kPartFloats * sizeof(float);
}
}  // namespace

size_t attn_sink_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Lmax) {
  if (B < 0 || Hq < 1 || Lmax < 1) return 0;
  return decode_records_bytes(B, Hq, Lmax) + (((size_t)2 * B + 2) * sizeof(int32_t) + 15) / 16 * 16;
}

moe_status attn_sink_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* kv_len, const float* sinks, void* out, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax, float sm_scale,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || Lmax < 1) return MOE_ERR_SHAPE;
  const moe_status hs = check_heads(Hq, Hkv, D);
  if (hs != MOE_OK) return hs;
  if (Hq / Hkv > 16) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv * Lmax * D >= kMaxElems ||
      moe::attn_decode_slots(B, Lmax) * Hq * moe::kPartFloats >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  if (B == 0) return MOE_OK;
  const void* ptrs[] = {q, k_cache, v_cache, kv_len, sinks, out, workspace};
  for (const void* p : ptrs)
    if (p == nullptr) return MOE_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  if (workspace_bytes < attn_sink_decode_workspace_bytes(B, Hq, Lmax)) return MOE_ERR_WORKSPACE;
  const hipError_t e = moe::launch_attn_decode(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
      static_cast<const uint16_t*>(v_cache), kv_len, sinks, static_cast<uint16_t*>(out),
      static_cast<float*>(workspace),
      reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + decode_records_bytes(B, Hq, Lmax)), B,
      Hq, Hkv, Lmax, sm_scale, stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
