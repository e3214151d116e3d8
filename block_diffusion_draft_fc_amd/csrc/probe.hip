// A plain streaming read of device memory: the reference against which the
// attention kernel's HBM throughput is read.  Each lane loads 16-byte words,
// four per pass of a grid-stride loop, so that a launch keeps the memory
// system as busy as a pure read can; the words are folded into one value that
// is stored only when it equals a constant no input produces in practice, so
// the loads cannot be removed and the launch writes nothing.
#include "kernels.hpp"

namespace dflash {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  uint32_t x = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 * 4 + threadIdx.x; i < n16; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t j = i + 256 * k;
      v[k] = j < n16 ? src[j] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) x ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  if (x == 0x9e3779b9u && sink != nullptr) sink[0] = x;
}

// Back-to-back bf16 16x16x32 MFMAs on register operands: the matrix-core rate
// this GPU sustains at its clocks under load, against which the projections'
// TFLOP/s are read beside the published peak.  Every wave runs eight
// independent accumulator chains of `iters` steps; the operands come from the
// lane index, and the accumulators are stored only when they sum to a value
// no run produces, so nothing can be folded away and the launch writes nothing.
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  // distinct operands per chain: identical chains could be merged
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[i][e] = static_cast<bf16>(0.001f * (float)(lane + e + 3 * i));
      b[i][e] = static_cast<bf16>(0.002f * (float)(lane - e + 5 * i));
    }
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = mma32(a[i], b[i], acc[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  if (s == 1234567.f && sink != nullptr) sink[0] = s;
}

hipError_t launch_mfma_peak(int iters, int64_t workgroups, float* sink, hipStream_t s) {
  if (workgroups <= 0 || iters <= 0) return hipSuccess;
  launch(mfma_peak_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(8192, (n16 + 1023) / 1024);
  launch(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace dflash
