// Draft head ("DFlash KV Injection Walkthrough" Step 5): the stack's block
// outputs go through a final RMSNorm over d, the last B-1 rows of every
// request's block (row 0 is the known token, whose prediction is dropped) go
// through lm_head, and greedy sampling keeps the argmax of each row's logits.
// The lm_head product itself is one of the weight-streaming / tile GEMMs
// (fp32 split-K partials [split][M][vocab]); this file holds the norm in front
// of it and the argmax behind it.
#include "kernels.hpp"

namespace dflash {

// x[m] = h[r*B + 1 + j] / sqrt(mean(h^2) + eps) * gamma for m = r*(B-1) + j:
// one workgroup per output row; each thread holds eight consecutive columns
// per pass (d <= 16384: at most four passes), loaded once for both the sum of
// squares and the output.
template <typename T>
__global__ __launch_bounds__(512) void head_norm_kernel(const T* __restrict__ h, int B, int64_t d,
                                                        const T* __restrict__ gamma, float eps,
                                                        T* __restrict__ x) {
  constexpr int PASSES = 4;
  __shared__ float red[8];
  const int64_t m = blockIdx.x;
  const int64_t src_row = (m / (B - 1)) * B + 1 + m % (B - 1);
  const T* row = h + src_row * d;
  vec8_t<T> v[PASSES];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int64_t c = ((int64_t)p * 512 + threadIdx.x) * 8;
    v[p] = c < d ? load8(row + c) : zero8<T>();
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += to_f32(v[p][e]) * to_f32(v[p][e]);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) tot += red[w];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int64_t c = ((int64_t)p * 512 + threadIdx.x) * 8;
    if (c < d) {
      const vec8_t<T> g = load8(gamma + c);
      f32x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = to_f32(v[p][e]) * r * to_f32(g[e]);
      store8(x + m * d + c, cvt8<T>(o));
    }
  }
}

hipError_t launch_head_norm(int dtype, const void* h, int64_t rows, int B, int64_t d, const void* gamma,
                            float eps, void* x, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  // d % 8 == 0 and d <= 16384 (checked by the caller)
  if (dtype == 1)
    launch(head_norm_kernel<bf16>, dim3((unsigned)rows), dim3(512), 0, s, static_cast<const bf16*>(h), B, d,
           static_cast<const bf16*>(gamma), eps, static_cast<bf16*>(x));
  else
    launch(head_norm_kernel<float>, dim3((unsigned)rows), dim3(512), 0, s, static_cast<const float*>(h), B, d,
           static_cast<const float*>(gamma), eps, static_cast<float*>(x));
  return hipGetLastError();
}

// (value, index) pairs: the larger value wins, the lower index on a tie - the
// first maximum, as an argmax over the row reports it.
__device__ __forceinline__ void arg_better(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(v, o, kWave);
    const int i2 = __shfl_xor(i, o, kWave);
    arg_better(v, i, v2, i2);
  }
}

// Stage 1: workgroup (segment, row) sums the split-K partials of its
// kHeadSeg-wide slice of the row's logits and keeps the slice's first maximum.
__global__ __launch_bounds__(256) void head_argmax_seg_kernel(const float* __restrict__ part, int splits,
                                                              int64_t M, int64_t vocab,
                                                              float* __restrict__ seg_val,
                                                              int32_t* __restrict__ seg_idx) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int seg = blockIdx.x, nseg = gridDim.x;
  const int64_t m = blockIdx.y;
  const int64_t c0 = (int64_t)seg * kHeadSeg, c1 = min<int64_t>(vocab, c0 + kHeadSeg);
  const int64_t stride = M * vocab;
  float best = -INFINITY;
  int bi = INT32_MAX;
  // vocab % 4 == 0: four whole columns per thread and pass; the segment's
  // kHeadSeg / 1024 passes are unrolled so that their loads are in flight
  // together (columns past the vocabulary are skipped)
  constexpr int PASSES = kHeadSeg / 1024;
  f32x4 u[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int64_t c = c0 + 4 * threadIdx.x + 1024 * i;
    u[i] = c < c1 ? *reinterpret_cast<const f32x4*>(part + m * vocab + c) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int sp = 1; sp < splits; ++sp) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int64_t c = c0 + 4 * threadIdx.x + 1024 * i;
      if (c < c1) u[i] += *reinterpret_cast<const f32x4*>(part + sp * stride + m * vocab + c);
    }
  }
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int64_t c = c0 + 4 * threadIdx.x + 1024 * i;
    if (c < c1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) arg_better(best, bi, u[i][e], (int)(c + e));
    }
  }
  wave_argmax(best, bi);
  if ((threadIdx.x & 63) == 0) {
    sv[threadIdx.x >> 6] = best;
    si[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) arg_better(best, bi, sv[w], si[w]);
    seg_val[m * nseg + seg] = best;
    seg_idx[m * nseg + seg] = bi;
  }
}

// Stage 2: one wave per row reduces the segments' maxima.
__global__ __launch_bounds__(256) void head_argmax_final_kernel(const float* __restrict__ seg_val,
                                                                const int32_t* __restrict__ seg_idx, int nseg,
                                                                int64_t M, int32_t* __restrict__ ids,
                                                                float* __restrict__ max_logit) {
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;
  float best = -INFINITY;
  int bi = INT32_MAX;
  for (int s = lane; s < nseg; s += 64) arg_better(best, bi, seg_val[m * nseg + s], seg_idx[m * nseg + s]);
  wave_argmax(best, bi);
  if (lane == 0) {
    ids[m] = bi;
    if (max_logit != nullptr) max_logit[m] = best;
  }
}

hipError_t launch_head_argmax(const float* part, int splits, int64_t M, int64_t vocab, float* seg_val,
                              int32_t* seg_idx, int32_t* ids, float* max_logit, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int nseg = (int)((vocab + kHeadSeg - 1) / kHeadSeg);
  launch(head_argmax_seg_kernel, dim3(nseg, (unsigned)M), dim3(256), 0, s, part, splits, M, vocab, seg_val,
         seg_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch(head_argmax_final_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, seg_val, seg_idx, nseg, M, ids,
         max_logit);
  return hipGetLastError();
}

// ---------------------------------------------------------------- acceptance
// "DFlash KV Injection Walkthrough" Step 6 and Step 7, per request r: the
// draft token of block position j+1 is checked against the target's
// prediction from position j; acc = the number of leading matches (the
// cumulative product of the matches, summed), the next round injects acc + 1
// context rows and opens its block with the target's token at the first
// position not accepted, posterior[acc].
// One wave per request: lanes compare 64 positions at a time and a ballot
// of the mismatches gives the first one.
__global__ __launch_bounds__(256) void accept_kernel(const int32_t* __restrict__ draft,
                                                     const int32_t* __restrict__ post, int64_t R, int B,
                                                     int32_t* __restrict__ acc, int32_t* __restrict__ next_rows,
                                                     int32_t* __restrict__ next_anchor) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= R) return;
  const int nd = B - 1;
  const int32_t* dr = draft + r * nd;
  const int32_t* pr = post + r * B;
  int a = nd;
  for (int j0 = 0; j0 < nd; j0 += 64) {
    const int j = j0 + lane;
    const bool miss = j < nd && dr[j] != pr[j];
    const unsigned long long bal = __ballot(miss);
    if (bal != 0ull) {
      a = j0 + __ffsll(bal) - 1;
      break;
    }
  }
  if (lane == 0) {
    acc[r] = a;
    if (next_rows != nullptr) next_rows[r] = a + 1;
    if (next_anchor != nullptr) next_anchor[r] = pr[a];
  }
}

hipError_t launch_accept(const int32_t* draft, const int32_t* post, int64_t R, int B, int32_t* acc,
                         int32_t* next_rows, int32_t* next_anchor, hipStream_t s) {
  if (R == 0) return hipSuccess;
  launch(accept_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s, draft, post, R, B, acc, next_rows,
         next_anchor);
  return hipGetLastError();
}

}  // namespace dflash
