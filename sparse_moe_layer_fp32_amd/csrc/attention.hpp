// Host-side launchers of the sink-attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMinSplitKeys = 256;    // shortest decode range per wave
constexpr int kResidentWaves = 1024;  // decode waves: one per SIMD
constexpr int kPartFloats = 68;       // per (segment, head): O[64], max, sum, 2 pad (16-byte records)

// Decode waves per key/value head (the keys of all sequences of one head are
// cut into this many equal ranges), and the segment record slots a call can
// need for B sequences of at most Lmax tokens (times Hq records each).
int attn_decode_waves(int Hkv);
int64_t attn_decode_slots(int B, int Lmax);

// q [S, Hq, 64], k and v [S, Hkv, 64] bf16 (token major), sinks [Hq] fp32, out [S, Hq, 64] bf16.
// Hq / Hkv must be 1, 2, 4 or a multiple of 8.
hipError_t launch_attn_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const float* sinks, uint16_t* out, int S, int Hq, int Hkv,
                               float sm_scale, hipStream_t stream);

// q [B, Hq, 64]; caches [B, Hkv, Lmax, 64] bf16; kv_len [B]; part:
// attn_decode_slots(B, Lmax) * Hq * kPartFloats fp32; plan: 2 B + 2 int32.
// Hq / Hkv <= 16.
hipError_t launch_attn_decode(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                              const int32_t* kv_len, const float* sinks, uint16_t* out, float* part,
                              int32_t* plan, int B, int Hq, int Hkv, int Lmax, float sm_scale,
                              hipStream_t stream);

}  // namespace moe
