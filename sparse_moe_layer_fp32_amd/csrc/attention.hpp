// Host-side launchers of the sink-attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMinSplitKeys = 256;    // smallest decode split
constexpr int kResidentWaves = 1024;  // decode waves: one per SIMD
constexpr int kPartFloats = 68;       // per (sequence, head, split): O[64], max, sum, 2 pad (16-byte records)

// Keys per decode split: the smallest 256 * 2^j that keeps B * Hkv * splits
// within one wave per SIMD (a wave streams its split with two blocks in
// flight; more, shorter splits measured slower at every batch shape tried).
int attn_decode_split_keys(int B, int Hkv, int Lmax);
// splits of a decode call, and the most any (B, Hkv) can need for Lmax
int attn_decode_splits(int B, int Hkv, int Lmax);
int attn_decode_max_splits(int Lmax);

// q [S, Hq, 64], k and v [S, Hkv, 64] bf16 (token major), sinks [Hq] fp32, out [S, Hq, 64] bf16.
// Hq / Hkv must be 1, 2, 4 or a multiple of 8.
hipError_t launch_attn_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const float* sinks, uint16_t* out, int S, int Hq, int Hkv,
                               float sm_scale, hipStream_t stream);

// q [B, Hq, 64]; caches [B, Hkv, Lmax, 64] bf16; kv_len [B]; part: B * Hq * splits * kPartFloats fp32.
// Hq / Hkv <= 16.
hipError_t launch_attn_decode(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                              const int32_t* kv_len, const float* sinks, uint16_t* out, float* part,
                              int B, int Hq, int Hkv, int Lmax, float sm_scale, hipStream_t stream);

}  // namespace moe
