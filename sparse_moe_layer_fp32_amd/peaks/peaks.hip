// Ceilings of the MI355X (gfx950) that the MoE kernels are measured against:
// the FP8 matrix-core issue rate and the clock it settles at, the HBM read
// rate, and the LDS read rates of the two fragment reads the grouped GEMMs
// use.  A measurement library (libmoe_peaks.so), not part of the block's
// C ABI; bench.py --workload peaks drives it.
//
// Every entry point enqueues one kernel on `stream` and returns the launch
// status (0 = success); the caller times it with events.  Per-wave cycle
// counts come from clock64() (the shader clock) and wall_clock64() (the
// constant-rate wall clock), so the host can derive the clock the waves ran
// at.  Each kernel reads and writes only the buffers it is given, inside the
// bounds the caller passes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wave

// Each wave runs `iters` rounds of kChains independent 16x16x128 FP8 MFMAs.
// timing[wave] = {clock64 delta, wall_clock64 delta}; sink gets one float per
// wave so the work cannot be dropped.
__global__ __launch_bounds__(256) void mfma_fp8_loop(int iters, float* sink, long long* timing) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ (lane + i);   // small e4m3 values: no overflow over the loop
    b[i] = 0x30303030 ^ (lane * 3 + i);
  }
  v4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
  const long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  const long long c1 = clock64(), w1 = wall_clock64();
  if (lane == 0) {
    sink[wave] = s;
    timing[2 * wave] = c1 - c0;
    timing[2 * wave + 1] = w1 - w0;
  }
}

// Streaming read of `n16` 16-byte words: grid-stride, XOR-reduced per thread.
__global__ __launch_bounds__(256) void hbm_read(const v4i* __restrict__ src, long long n16,
                                                int* __restrict__ sink) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  v4i x = v4i{0, 0, 0, 0};
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) x ^= src[i];
  const int r = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (r == 0x12345678) sink[blockIdx.x] = r;  // practically never taken; keeps the loads
}

// LDS read rate: every wave of the workgroup reads `iters` x 8 fragments of
// its LDS buffer (64 KB, filled first) with ds_read_b128 (tr = 0) or with the
// transposing ds_read_b64_tr_b8 (tr = 1), at addresses that are bank-conflict
// free for each read.  timing[wave] as above; bytes per wave = iters * 8 *
// 64 lanes * (16 or 8).
template <int TR>
__global__ __launch_bounds__(512) void lds_read(int iters, int* sink, long long* timing) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[65536];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 65536 / 4; i += blockDim.x) reinterpret_cast<int*>(lds)[i] = i * 2654435761u;
  __syncthreads();
  v4i acc = v4i{0, 0, 0, 0};
  const int base = (wave * 8192) & 0xffff;  // ds_read_b128: a distinct 8 KB per wave
  const long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if constexpr (TR) {
        // the grouped GEMMs' weight-fragment read: in each group of 16 lanes,
        // lanes 2j and 2j+1 read the two 8-byte halves of one 16-byte segment
        // of K row 32 (lane / 16) + j (rows of 256 bytes, segment s of row kr
        // stored at s ^ ((kr & 7) | (bit 5 of kr) << 3), the GEMMs' key, so the
        // rows of a read hit distinct banks)
        const int l16 = lane & 15, gq = lane >> 4;
        const int row = (32 * gq + (l16 >> 1) + 8 * r + 128 * (wave & 1)) & 255;
        const int seg = ((it + wave) & 15) ^ ((row & 7) | (((row >> 5) & 1) << 3));
        const int off = row * 256 + seg * 16 + 8 * (l16 & 1);
        const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(lds + off));
        acc[0] ^= t[0];
        acc[1] ^= t[1];
      } else {
        const int off = (base + r * 1024 + lane * 16 + ((it & 7) << 10)) & 0xfff0;
        acc ^= *reinterpret_cast<const v4i*>(lds + off);
      }
    }
  }
  const long long c1 = clock64(), w1 = wall_clock64();
  const int gw = blockIdx.x * (blockDim.x >> 6) + wave;
  const int r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == 0x12345678) sink[gw] = r;
  if (lane == 0) {
    timing[2 * gw] = c1 - c0;
    timing[2 * gw + 1] = w1 - w0;
  }
}

// The grouped GEMMs' per-K-block MFMA sequence in isolation (fragments in
// registers, no memory traffic): 6 x 4 blocks of 16x16x128 per wave per
// step, `steps` steps.  MODE 0: each MFMA starts from zero and its result is
// promoted (4 FMAs with a per-row-block scale) three MFMAs later, with a
// scheduling barrier per MFMA (the block-scaled kernel's order); 1: the same
// without the scheduling barriers; 2: the MFMAs accumulate in place (the MX
// kernels' form, no promotion).  timing[wave] as above.
template <int MODE>
__global__ __launch_bounds__(512) void mfma_seq(int steps, float* sink, long long* timing) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  v8i wf[4], xf[6];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int n = 0; n < 4; ++n) wf[n][i] = 0x38383838 ^ (lane + i + 7 * n);
#pragma unroll
    for (int m = 0; m < 6; ++m) xf[m][i] = 0x30303030 ^ (lane * 3 + i + 5 * m);
  }
  float acc[6][4][4];
  v4f macc[6][4];
#pragma unroll
  for (int m = 0; m < 6; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      macc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][n][i] = 0.f;
    }
  float sa[6];
#pragma unroll
  for (int m = 0; m < 6; ++m) sa[m] = 1.0f + 1e-3f * (lane + m);
  const long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < steps; ++it) {
    const float sb = 1.0f + 1e-4f * it;
    if constexpr (MODE == 2) {
#pragma unroll
      for (int j = 0; j < 24; ++j)
        macc[j >> 2][j & 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            wf[j & 3], xf[j >> 2], macc[j >> 2][j & 3], 0, 0, 0, 0, 0, 0);
    } else {
      v4f pp[24];
#pragma unroll
      for (int j = 0; j < 27; ++j) {
        if (j < 24)
          pp[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j & 3], xf[j >> 2],
                                                                   v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        if (j >= 3) {
          const int q = j - 3;
          const float s = sa[q >> 2] * sb;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[q >> 2][q & 3][i] = fmaf(pp[q][i], s, acc[q >> 2][q & 3][i]);
        }
        if constexpr (MODE == 0) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 6; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) s += acc[m][n][0] + acc[m][n][3] + macc[m][n][0] + macc[m][n][3];
  const long long c1 = clock64(), w1 = wall_clock64();
  if (lane == 0) {
    sink[wave] = s;
    timing[2 * wave] = c1 - c0;
    timing[2 * wave + 1] = w1 - w0;
  }
}

// Global -> LDS rate: each wave of a workgroup of `waves` waves issues
// `iters` x 8 loads of 1 KB (64 lanes x 16 bytes) from its workgroup's
// region of `src` (region_bytes per workgroup, read cyclically, so a small
// region stays in L2) into its own 8 KB of LDS.  DMA = 1: buffer_load_dwordx4
// ... lds (the GEMMs' stage loads); DMA = 0: buffer_load_dwordx4 to registers
// followed by ds_write_b128.  Every read offset is below region_bytes (the
// buffer resource also bounds it) and every LDS write lies in the 64 KB array.
template <int DMA>
__global__ __launch_bounds__(512) void lds_fill(const uint8_t* src, int region_bytes, int iters, int* sink,
                                                long long* timing) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[65536];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t base = reinterpret_cast<uint64_t>(src) + (uint64_t)blockIdx.x * (uint64_t)region_bytes;
  v4i rsrc;
  rsrc[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(base)));
  rsrc[1] = __builtin_amdgcn_readfirstlane(static_cast<int>((base >> 32) & 0xffffu));
  rsrc[2] = region_bytes;
  rsrc[3] = 0x00020000;
  const uint32_t dst = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
      static_cast<int>(reinterpret_cast<uintptr_t>(lds + (wave & 7) * 8192))));
  const int chunks = region_bytes / 1024;
  v4i acc = v4i{0, 0, 0, 0};
  const long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int chunk = (it * 8 + r + wave * 13) % chunks;
      const uint32_t voff = (uint32_t)chunk * 1024u + 16u * lane;
      if constexpr (DMA) {
        int saved;
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(dst + 1024u * r), "v"(voff), "s"(rsrc)
            : "memory");
      } else {
        const v4i v = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src) + (size_t)blockIdx.x * region_bytes,
                                              (short)0, region_bytes, 0x00020000),
            (int)voff, 0, 0));
        acc ^= v;
      }
    }
    if constexpr (DMA) __builtin_amdgcn_s_waitcnt(0x0f70 | (48 & 15) | ((48 >> 4) << 14));  // vmcnt(48): <= 56 in flight
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (DMA) acc = *reinterpret_cast<const v4i*>(lds + (threadIdx.x * 16) % 65536);
  const long long c1 = clock64(), w1 = wall_clock64();
  const int gw = blockIdx.x * (blockDim.x >> 6) + wave;
  const int rr = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (rr == 0x12345678) sink[gw] = rr;
  if (lane == 0) {
    timing[2 * gw] = c1 - c0;
    timing[2 * gw + 1] = w1 - w0;
  }
}

}  // namespace

extern "C" {

// blocks x `waves` (<= 8) waves; src must hold blocks * region_bytes bytes,
// region_bytes a multiple of 1024 (at most 2^30); dma: 1 = global->LDS DMA,
// 0 = loads to registers (XOR-reduced, no LDS).  sink: blocks*waves ints, timing:
// blocks*waves*2 int64.
int peak_lds_fill(const void* src, int blocks, int waves, int region_bytes, int iters, int dma, int* sink,
                  long long* timing, hipStream_t stream) {
  if (!src || blocks <= 0 || waves <= 0 || waves > 8 || region_bytes < 1024 || (region_bytes & 1023) ||
      region_bytes > (1 << 30) || iters <= 0 || !sink || !timing)
    return -1;
  const auto s = static_cast<const uint8_t*>(src);
  if (dma)
    hipLaunchKernelGGL(lds_fill<1>, dim3(blocks), dim3(64 * waves), 0, stream, s, region_bytes, iters, sink, timing);
  else
    hipLaunchKernelGGL(lds_fill<0>, dim3(blocks), dim3(64 * waves), 0, stream, s, region_bytes, iters, sink, timing);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// blocks x `waves` waves (4 or 8) running the GEMM MFMA sequence `mode` (0-2);
// sink: blocks*waves floats, timing: blocks*waves*2 int64.
int peak_mfma_sequence(int blocks, int waves, int steps, int mode, float* sink, long long* timing,
                       hipStream_t stream) {
  if (blocks <= 0 || (waves != 4 && waves != 8) || steps <= 0 || mode < 0 || mode > 2 || !sink || !timing)
    return -1;
  const dim3 grid(blocks), block(64 * waves);
  if (mode == 0) hipLaunchKernelGGL(mfma_seq<0>, grid, block, 0, stream, steps, sink, timing);
  else if (mode == 1) hipLaunchKernelGGL(mfma_seq<1>, grid, block, 0, stream, steps, sink, timing);
  else hipLaunchKernelGGL(mfma_seq<2>, grid, block, 0, stream, steps, sink, timing);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// blocks x 4 waves; sink: blocks*4 floats, timing: blocks*4*2 int64.
int peak_mfma_fp8(int blocks, int iters, float* sink, long long* timing, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || !sink || !timing) return -1;
  hipLaunchKernelGGL(mfma_fp8_loop, dim3(blocks), dim3(256), 0, stream, iters, sink, timing);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// reads `bytes` (a multiple of 16) from src; sink: `blocks` ints.
int peak_hbm_read(const void* src, long long bytes, int blocks, int* sink, hipStream_t stream) {
  if (!src || !sink || bytes <= 0 || (bytes & 15) || blocks <= 0) return -1;
  hipLaunchKernelGGL(hbm_read, dim3(blocks), dim3(256), 0, stream, static_cast<const v4i*>(src),
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// blocks x `waves` waves (at most 8); tr: 0 = ds_read_b128, 1 = ds_read_b64_tr_b8.
// sink: blocks*waves ints, timing: blocks*waves*2 int64.
int peak_lds_read(int blocks, int waves, int iters, int tr, int* sink, long long* timing,
                  hipStream_t stream) {
  if (blocks <= 0 || waves <= 0 || waves > 8 || iters <= 0 || !sink || !timing) return -1;
  if (tr)
    hipLaunchKernelGGL(lds_read<1>, dim3(blocks), dim3(64 * waves), 0, stream, iters, sink, timing);
  else
    hipLaunchKernelGGL(lds_read<0>, dim3(blocks), dim3(64 * waves), 0, stream, iters, sink, timing);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
