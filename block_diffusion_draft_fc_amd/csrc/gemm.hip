// Weight-streaming GEMMs for the few-row projections of a draft round, plus
// the split-K reduction and the row RMSNorm epilogue.
//
// The projections of a decode round multiply at most a few dozen activation
// rows by weight matrices of tens to hundreds of MB (fc: the context rows
// against W_fc, "DFlash KV Injection Walkthrough" Step 2; q/k/v and o: Step 4.1,
// 4.2, 4.5).  They are bound by streaming the weight from HBM once, with fp32
// split-K partial sums going to a [split][M][N] buffer.  Two kernels:
//
//  * gemm_lds_kernel - a workgroup owns 64 weight rows (output columns) and one
//    K-chunk; the chunk's activation slice is staged in LDS once, then each wave
//    streams 16 weight rows straight into the B operand of 16x16x32 MFMAs
//    (16-byte loads, double-buffered).  Short chunks and many workgroups: the
//    right shape for 4096-wide inputs, where the time is mostly latency.
//  * gemm_wide_kernel - for long inputs (the 20480-wide fc): each wave streams
//    64 weight rows and reads the activation rows straight from L2 into the A
//    operand, one activation load feeding four weight tiles; no LDS, no
//    barrier, and long per-wave streams.
#include <algorithm>

#include "kernels.hpp"

namespace dflash {

template <typename T, int MTMAX>
__global__ __launch_bounds__(256) void gemm_lds_kernel(GemmArgs args) {
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
static hipError_t launch_lds_t(const GemmArgs& a, int max_mt, size_t lds, hipStream_t s) {
  const int blocks = a.p[0].blocks + (a.nprob > 1 ? a.p[1].blocks : 0);
  if (blocks == 0) return hipSuccess;
  switch (max_mt) {
    case 1: launch((gemm_lds_kernel<T, 1>), dim3(blocks), dim3(256), lds, s, a); break;
    case 2: launch((gemm_lds_kernel<T, 2>), dim3(blocks), dim3(256), lds, s, a); break;
    case 3: launch((gemm_lds_kernel<T, 3>), dim3(blocks), dim3(256), lds, s, a); break;
    case 4: launch((gemm_lds_kernel<T, 4>), dim3(blocks), dim3(256), lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_lds(int dtype, const GemmArgs& a, int max_mt, size_t lds, hipStream_t s) {
  return dtype == 1 ? launch_lds_t<bf16>(a, max_mt, lds, s) : launch_lds_t<float>(a, max_mt, lds, s);
}

// ---------------------------------------------------------------- wide (bf16)
// Workgroup tile: 256 output columns (wave w: columns 64w .. 64w+63 of the tile,
// as four 16-column MFMA tiles) x one K-chunk.  A stage is 4 K-steps of 32;
// loads go out one stage ahead of the MFMAs that use them.

template <int MT>
__global__ __launch_bounds__(256) void gemm_wide_kernel(GemmProb p) {
  constexpr int C = 4;   // 16-column tiles per wave
  constexpr int U = 4;   // K-steps per stage
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, q8 = (lane >> 4) * 8;
  const int n_tile = blockIdx.x % p.n_tiles, split = blockIdx.x / p.n_tiles;
  const int k_begin = split * p.k_chunk;
  const int k_end = min(p.K, k_begin + p.k_chunk);
  const int M = p.m0 + p.m1;
  const int nbase = n_tile * 256 + wave * 64;

  const bf16* wp[C];
  bool nvalid[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int n = nbase + 16 * c + l16;
    nvalid[c] = n < p.N;
    wp[c] = static_cast<const bf16*>(p.w) + (int64_t)(nvalid[c] ? n : 0) * p.K + k_begin + q8;
  }
  // activation rows; rows past M read row 0 and are never stored
  const bf16* xp[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    int m = t * 16 + l16;
    m = m < M ? m : 0;
    const bf16* base = m < p.m0 ? static_cast<const bf16*>(p.x0) + (int64_t)m * p.K
                                : static_cast<const bf16*>(p.x1) + (int64_t)(m - p.m0) * p.K;
    xp[t] = base + k_begin + q8;
  }

  f32x4 acc[C][MT];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (k_end - k_begin + 31) >> 5;
  const int nfull = nsteps / U;

  auto fetch = [&](bf16x8 (&w)[U][C], bf16x8 (&x)[U][MT], int stage) {
    const int k = stage * U * 32;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < C; ++c) w[u][c] = load8(wp[c] + k + 32 * u);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t) x[u][t] = load8(xp[t] + k + 32 * u);
    // keep the loads here: otherwise the compiler sinks them to their use
    asm volatile("" ::: "memory");
  };
  auto compute = [&](const bf16x8 (&w)[U][C], const bf16x8 (&x)[U][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[c][t] = mma32(x[u][t], w[u][c], acc[c][t]);
  };

  if (nfull > 0) {
    // double-buffered; every prefetch is unconditional (past the last stage it
    // re-reads that stage, an L2 hit) so that the wait counts stay exact
    bf16x8 wa[U][C], xa[U][MT], wb[U][C], xb[U][MT];
    fetch(wa, xa, 0);
    for (int st = 0;; st += 2) {
      fetch(wb, xb, min(st + 1, nfull - 1));
      compute(wa, xa);
      if (st + 1 >= nfull) break;
      fetch(wa, xa, min(st + 2, nfull - 1));
      compute(wb, xb);
      if (st + 2 >= nfull) break;
    }
  }
  // K-steps past the last whole stage: guarded loads
  for (int step = nfull * U; step < nsteps; ++step) {
    const int k = step * 32;
    const bool kin = k_begin + k + q8 < k_end;
    bf16x8 x[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) x[t] = kin ? load8(xp[t] + k) : zero8<bf16>();
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bf16x8 w = kin ? load8(wp[c] + k) : zero8<bf16>();
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[c][t] = mma32(x[t], w, acc[c][t]);
    }
  }

  const int m_lane = (lane >> 4) * 4;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    if (!nvalid[c]) continue;
    float* out = p.part + ((int64_t)split * p.m_out + p.row_off) * p.N + nbase + 16 * c + l16;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = t * 16 + m_lane + e;
        if (m < M) out[(int64_t)m * p.N] = acc[c][t][e];
      }
  }
}

hipError_t launch_gemm_wide(const GemmProb& p, hipStream_t s) {
  if (p.blocks == 0) return hipSuccess;
  switch (p.mt) {
    case 1: launch((gemm_wide_kernel<1>), dim3(p.blocks), dim3(256), 0, s, p); break;
    case 2: launch((gemm_wide_kernel<2>), dim3(p.blocks), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- split-K reduction
// out[m][n] = sum_s part[s][m][n] (+ add[m][n] when add is given); one thread
// per 4 outputs, the split loop unrolled so that its loads are in flight
// together.

template <typename Tout>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                            int64_t MN, const Tout* __restrict__ add,
                                                            Tout* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + i);
#pragma unroll 8
  for (int sp = 1; sp < splits; ++sp) s += *reinterpret_cast<const f32x4*>(part + (int64_t)sp * MN + i);
  if (add != nullptr) {
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += to_f32(add[i + e]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) out[i + e] = from_f32<Tout>(s[e]);
}

hipError_t launch_splitk_reduce(int out_dtype, const float* part, int splits, int64_t M, int64_t N,
                                const void* add, void* out, hipStream_t s) {
  const int64_t MN = M * N;
  if (MN == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((MN / 4 + 255) / 256);
  if (out_dtype == 1)
    launch(splitk_reduce_kernel<bf16>, dim3(blocks), dim3(256), 0, s, part, splits, MN,
           static_cast<const bf16*>(add), static_cast<bf16*>(out));
  else
    launch(splitk_reduce_kernel<float>, dim3(blocks), dim3(256), 0, s, part, splits, MN,
           static_cast<const float*>(add), static_cast<float*>(out));
  return hipGetLastError();
}

// ---------------------------------------------------------------- split-K reduction + RMSNorm
// hidden_norm of "DFlash KV Injection Walkthrough" Step 2 fused with the fc
// split-K sum: one workgroup per context row; each thread sums the partials of
// four columns (all splits' loads in flight together), the row's sum of
// squares is reduced through LDS, then C[t] = u / sqrt(mean(u^2) + eps) * gamma.

template <typename T>
__global__ __launch_bounds__(1024) void reduce_rmsnorm_kernel(const float* __restrict__ part, int splits,
                                                              int64_t T_rows, int64_t d,
                                                              const T* __restrict__ gamma, float eps,
                                                              T* __restrict__ out) {
  constexpr int MAXC = 4;   // column quads per thread: d <= 4 * 1024 * MAXC
  __shared__ float red[16];
  const int64_t t = blockIdx.x;
  const int64_t stride = T_rows * d;
  f32x4 u[MAXC];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int64_t col = ((int64_t)c * blockDim.x + threadIdx.x) * 4;
    u[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (col < d) {
      const float* src = part + t * d + col;
#pragma unroll 8
      for (int sp = 0; sp < splits; ++sp) u[c] += *reinterpret_cast<const f32x4*>(src + sp * stride);
      ss += u[c][0] * u[c][0] + u[c][1] * u[c][1] + u[c][2] * u[c][2] + u[c][3] * u[c][3];
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  const int nw = blockDim.x >> 6;
  for (int w = 0; w < nw; ++w) tot += red[w];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int64_t col = ((int64_t)c * blockDim.x + threadIdx.x) * 4;
    if (col < d) {
#pragma unroll
      for (int e = 0; e < 4; ++e) out[t * d + col + e] = from_f32<T>(u[c][e] * r * to_f32(gamma[col + e]));
    }
  }
}

hipError_t launch_reduce_rmsnorm(int dtype, const float* part, int splits, int64_t T, int64_t d,
                                 const void* gamma, float eps, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // d % 4 == 0 and d <= 16384 (checked by the caller); threads: one per column quad, at most 1024
  const int64_t quads = d / 4;
  const unsigned threads = (unsigned)std::min<int64_t>(1024, ((quads + 63) / 64) * 64);
  if (dtype == 1)
    launch(reduce_rmsnorm_kernel<bf16>, dim3((unsigned)T), dim3(threads), 0, s, part, splits, T, d,
                       static_cast<const bf16*>(gamma), eps, static_cast<bf16*>(out));
  else
    launch(reduce_rmsnorm_kernel<float>, dim3((unsigned)T), dim3(threads), 0, s, part, splits, T, d,
                       static_cast<const float*>(gamma), eps, static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace dflash
