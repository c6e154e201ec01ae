// Rate probes of the device.  The attention kernels are reported against the
// vendor peaks (8 TB/s HBM, 2.5 PFLOP/s dense bf16) and also against what a
// kernel with nothing else to do reaches on the same chip: a gather cannot
// read HBM faster than a plain streaming read, and a fused attention kernel
// cannot issue bf16 products faster than a loop of independent ones.
#include "spa_internal.h"

namespace spa {

namespace {

constexpr int kProbeThreads = 256;  // four waves
constexpr int kReadInFlight = 4;    // 16-byte loads a lane keeps in flight

// Read-only stream over n_vec 16-byte vectors: non-temporal loads (the policy
// the decode gather uses), kReadInFlight per lane in flight, striding by the
// whole grid so each wave instruction reads 1 KiB contiguous.  The XOR of all
// data read decides a store that practically never happens, so no load can be
// dropped.
__global__ void __launch_bounds__(kProbeThreads) probe_read_kernel(const u32x4* __restrict__ src, size_t n_vec,
                                                                   unsigned* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kReadInFlight - 1) * stride < n_vec; i += kReadInFlight * stride) {
    u32x4 v[kReadInFlight];
#pragma unroll
    for (int u = 0; u < kReadInFlight; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadInFlight; ++u) acc ^= v[u];
  }
  for (; i < n_vec; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9E3779B9u) sink[0] = x;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave,
// iters rounds (the attention kernels interleave two or more chains the same
// way).  The operands are positive bf16 values built from the lane index, so
// nothing folds and every sum is positive: the store never happens, but the
// compiler cannot know that.  One round is 4 x 2 x 32 x 32 x 16 = 131,072
// flops per wave.
__global__ void __launch_bounds__(kProbeThreads) probe_mfma_kernel(int iters, float* __restrict__ sink) {
  const unsigned lane = threadIdx.x & (kWave - 1);
  const unsigned pa = 0x3F803F80u + (lane & 7u) * 0x00010001u;         // 1.0 .. 1.05 in both halves
  const unsigned pb = 0x3F003F00u + ((lane >> 3) & 7u) * 0x00010001u;  // 0.5 .. 0.53
  const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{pa, pa, pa, pa});
  const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{pb, pb, pb, pb});
  f32x16 c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) c[j][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  if (s < 0.f) sink[0] = s;
}

}  // namespace

hipError_t launch_probe_read(const void* buf, size_t bytes, int workgroups, unsigned* sink, hipStream_t s) {
  probe_read_kernel<<<workgroups, kProbeThreads, 0, s>>>(reinterpret_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma_bf16(int workgroups, int iters, float* sink, hipStream_t s) {
  probe_mfma_kernel<<<workgroups, kProbeThreads, 0, s>>>(iters, sink);
  return hipGetLastError();
}

}  // namespace spa
