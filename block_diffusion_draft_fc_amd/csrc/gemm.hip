// Weight-streaming GEMM for the few-row projections of a draft round, plus the
// split-K reduction and the row RMSNorm epilogue.
//
// The projections of a decode round multiply at most a few dozen activation
// rows by weight matrices of tens to hundreds of MB (fc: the context rows
// against W_fc, "DFlash KV Injection Walkthrough" Step 2; q/k/v and o: Step 4.1,
// 4.2, 4.5).  They are bound by streaming the weight from HBM once.  Each
// workgroup owns 64 weight rows (output columns) and one K-split; the
// workgroup's activation slice sits in LDS, every wave streams 16 weight rows
// straight into the B operand of 16x16x32 MFMAs with 16-byte loads, and fp32
// partial sums go to a [split][M][N] buffer.
#include "kernels.hpp"

namespace dflash {

template <typename T, int MTMAX>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs args) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* xs = reinterpret_cast<T*>(smem_raw);
  using V8 = vec8_t<T>;

  int b = blockIdx.x;
  int pi = 0;
  if (args.nprob > 1 && b >= args.p[0].blocks) {
    b -= args.p[0].blocks;
    pi = 1;
  }
  const GemmProb p = args.p[pi];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_tile = b % p.n_tiles, split = b / p.n_tiles;
  const int k_begin = split * p.k_chunk;
  const int k_end = min(p.K, k_begin + p.k_chunk);
  const int klen = k_end - k_begin;                 // multiple of 8
  const int kpad = (klen + 255) & ~255;
  const int M = p.m0 + p.m1;
  const int rows = p.mt * 16;
  const int ld = kpad + 8;                          // LDS row stride (elements)

  // Stage the activation slice [rows][kpad] (zero padded) in LDS.
  const int c8n = kpad >> 3;
  for (int idx = tid; idx < rows * c8n; idx += 256) {
    const int r = idx / c8n;
    const int c = (idx - r * c8n) << 3;
    const int k = k_begin + c;
    V8 v = zero8<T>();
    if (r < M && k < k_end) {
      const T* src = (r < p.m0) ? static_cast<const T*>(p.x0) + (int64_t)r * p.K
                                : static_cast<const T*>(p.x1) + (int64_t)(r - p.m0) * p.K;
      v = load8(src + k);
    }
    store8(xs + r * ld + c, v);
  }
  __syncthreads();

  const int n = n_tile * 64 + wave * 16 + (lane & 15);
  const int q8 = (lane >> 4) * 8;
  const bool nvalid = n < p.N;
  const T* wrow = static_cast<const T*>(p.w) + (int64_t)(nvalid ? n : 0) * p.K + k_begin;
  const T* xrow = xs + (lane & 15) * ld + q8;

  f32x4 acc[MTMAX];
#pragma unroll
  for (int t = 0; t < MTMAX; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  V8 wa[8], wb[8];
  auto fetch = [&](V8* dst, int kk) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = kk + 32 * j + q8;
      dst[j] = (nvalid && k < klen) ? load8(wrow + k) : zero8<T>();
    }
  };
  auto compute = [&](const V8* wv, int kk) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int t = 0; t < MTMAX; ++t) {
        if (t < p.mt) {
          const V8 a = load8(xrow + t * 16 * ld + kk + 32 * j);
          acc[t] = mma32(a, wv[j], acc[t]);
        }
      }
    }
  };

  fetch(wa, 0);
  for (int kk = 0; kk < kpad; kk += 512) {
    if (kk + 256 < kpad) fetch(wb, kk + 256);
    compute(wa, kk);
    if (kk + 256 >= kpad) break;
    if (kk + 512 < kpad) fetch(wa, kk + 512);
    compute(wb, kk + 256);
  }

  if (nvalid) {
    float* out = p.part + ((int64_t)split * p.m_out + p.row_off) * p.N + n;
    const int m_lane = (lane >> 4) * 4;
#pragma unroll
    for (int t = 0; t < MTMAX; ++t) {
      if (t < p.mt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = t * 16 + m_lane + e;
          if (m < M) out[(int64_t)m * p.N] = acc[t][e];
        }
      }
    }
  }
}

template <typename T>
static hipError_t launch_skinny_t(const GemmArgs& a, int max_mt, size_t lds, hipStream_t s) {
  const int blocks = a.p[0].blocks + (a.nprob > 1 ? a.p[1].blocks : 0);
  if (blocks == 0) return hipSuccess;
  switch (max_mt) {
    case 1: hipLaunchKernelGGL((gemm_skinny_kernel<T, 1>), dim3(blocks), dim3(256), lds, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_skinny_kernel<T, 2>), dim3(blocks), dim3(256), lds, s, a); break;
    case 3: hipLaunchKernelGGL((gemm_skinny_kernel<T, 3>), dim3(blocks), dim3(256), lds, s, a); break;
    case 4: hipLaunchKernelGGL((gemm_skinny_kernel<T, 4>), dim3(blocks), dim3(256), lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(int dtype, const GemmArgs& a, int max_mt, size_t lds, hipStream_t s) {
  return dtype == 1 ? launch_skinny_t<bf16>(a, max_mt, lds, s) : launch_skinny_t<float>(a, max_mt, lds, s);
}

// ---------------------------------------------------------------- split-K reduction

template <typename Tout>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                            int64_t MN, Tout* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + i);
  for (int sp = 1; sp < splits; ++sp) s += *reinterpret_cast<const f32x4*>(part + (int64_t)sp * MN + i);
#pragma unroll
  for (int e = 0; e < 4; ++e) out[i + e] = from_f32<Tout>(s[e]);
}

hipError_t launch_splitk_reduce(int out_dtype, const float* part, int splits, int64_t M, int64_t N,
                                void* out, hipStream_t s) {
  const int64_t MN = M * N;
  if (MN == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((MN / 4 + 255) / 256);
  if (out_dtype == 1)
    hipLaunchKernelGGL(splitk_reduce_kernel<bf16>, dim3(blocks), dim3(256), 0, s, part, splits, MN,
                       static_cast<bf16*>(out));
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<float>, dim3(blocks), dim3(256), 0, s, part, splits, MN,
                       static_cast<float*>(out));
  return hipGetLastError();
}

// ---------------------------------------------------------------- RMSNorm over rows
// hidden_norm of "DFlash KV Injection Walkthrough" Step 2: each context row is
// divided by the root of its mean square (plus eps) and scaled by the gain.

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float* __restrict__ u, int64_t d,
                                                           const T* __restrict__ gamma, float eps,
                                                           T* __restrict__ out) {
  __shared__ float red[4];
  const float* ur = u + (int64_t)blockIdx.x * d;
  float ss = 0.f;
  for (int64_t i = threadIdx.x; i < d; i += 256) ss += ur[i] * ur[i];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  T* orow = out + (int64_t)blockIdx.x * d;
  for (int64_t i = threadIdx.x; i < d; i += 256) orow[i] = from_f32<T>(ur[i] * r * to_f32(gamma[i]));
}

hipError_t launch_rmsnorm_rows(int dtype, const float* u, int64_t T, int64_t d, const void* gamma,
                               float eps, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(rmsnorm_rows_kernel<bf16>, dim3((unsigned)T), dim3(256), 0, s, u, d,
                       static_cast<const bf16*>(gamma), eps, static_cast<bf16*>(out));
  else
    hipLaunchKernelGGL(rmsnorm_rows_kernel<float>, dim3((unsigned)T), dim3(256), 0, s, u, d,
                       static_cast<const float*>(gamma), eps, static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace dflash
