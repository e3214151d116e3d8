// The GEMMs of a draft round's projections, plus the split-K reduction and
// the row RMSNorm epilogue.
//
// The projections multiply a few to a few thousand activation rows by weight
// matrices of tens to hundreds of MB (fc: the context rows against W_fc,
// "DFlash KV Injection Walkthrough" Step 2; q/k/v and o: Step 4.1, 4.2, 4.5;
// lm_head: Step 5).  With few rows they are bound by streaming the weight
// from HBM once; with many, by the MFMAs.  Results are fp32, either split-K
// partial sums in a [split][M][N] buffer or the finished product.  Kernels,
// by rows (the host planner picks one per product):
//
//  * gemm_fullk_kernel (<= 16 rows) - one workgroup per 16 output columns
//    over the whole K, no partials;
//  * gemm_resident_kernel (<= 16 rows, a vocabulary of columns) - the rows
//    kept in LDS, whole-K weight tiles streamed per wave;
//  * gemm_stream_kernel (<= 64 rows, K < 8192) - per-wave weight rings of 64-wide
//    K-steps, 512-wide chunks;
//  * gemm_wide_kernel (<= 32 rows, K >= 8192) - each wave streams 64 weight
//    rows and reads the activation rows straight from L2;
//  * gemm_slab_kernel (65..128 rows, or 33..64 with K >= 8192; K a multiple
//    of 512) - the chunk's
//    activation slice staged by direct copies in up to 160 KB of LDS, waves
//    stream 16 weight rows each;
//  * gemm_lds_kernel (fp32, and bf16 with other K) - the same scheme within
//    64 KB of LDS, staged through registers;
//  * gemm_tile_kernel (many rows) - 256 x 256/128/64 MFMA tiles through a
//    two-stage LDS ring.
#include <algorithm>
#include <atomic>
#include <cstdlib>

#include <type_traits>

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

// ---------------------------------------------------------------- slab (bf16, up to 128 rows)
// gemm_lds_kernel's scheme with the activation slice [rows][k_chunk] staged
// by direct-to-LDS copies (1 KB of one row each, all issued before the first
// weight loads and waited for once) into up to 160 KB of LDS: a 64-row
// problem over a 4096-wide input takes four 1024-wide splits instead of
// sixteen 256-wide ones, a 128-row problem eight 512-wide ones, which cuts the
// fp32 partial traffic written here and read by the consumer 2-4 times.
// LDS row stride k_chunk + 8 elements: the 16-byte pad moves the 16 rows of an
// operand read onto different banks.
// Requirements (checked by the planner): bf16, K and k_chunk multiples of 512,
// exactly MT 16-row tiles (the problems of one launch share MT), and
// MT * 16 * (k_chunk + 8) * 2 bytes within kSlabLdsBytes.
template <int MT>
__global__ __launch_bounds__(256) void gemm_slab_kernel(GemmArgs args) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const bf16* xs = reinterpret_cast<const bf16*>(smem_raw);

  int b = blockIdx.x;
  int pi = 0;
  if (args.nprob > 1 && b >= args.p[0].blocks) {
    b -= args.p[0].blocks;
    pi = 1;
  }
  const GemmProb p = args.p[pi];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_tile = b % p.n_tiles, split = b / p.n_tiles;
  const int k_begin = split * p.k_chunk;
  const int klen = min(p.K, k_begin + p.k_chunk) - k_begin;   // a multiple of 512
  const int M = p.m0 + p.m1;
  const int ld = klen + 8;
  const bf16* x0 = static_cast<const bf16*>(p.x0);
  const bf16* x1 = static_cast<const bf16*>(p.x1);

  // copy i: row i / segs, elements 512 (i % segs) .. + 511 of the chunk; rows
  // past M read row 0 (their results are never stored)
  const int segs = klen >> 9;
  const int ncopies = MT * 16 * segs;
  for (int i = wave; i < ncopies; i += 4) {
    const int r = i / segs, seg = i - r * segs;
    const int m = r < M ? r : 0;
    const bf16* src = (m < p.m0 ? x0 + (int64_t)m * p.K : x1 + (int64_t)(m - p.m0) * p.K) + k_begin + 512 * seg + 8 * lane;
    lds_copy16(src, smem_raw + 2 * (r * ld + 512 * seg));
  }

  // columns past N stream row 0 (finite values, never stored)
  const int n = n_tile * 64 + wave * 16 + (lane & 15);
  const int q8 = (lane >> 4) * 8;
  const bool nvalid = n < p.N;
  const bf16* wrow = static_cast<const bf16*>(p.w) + (int64_t)(nvalid ? n : 0) * p.K + k_begin + q8;
  const bf16* xrow = xs + (lane & 15) * ld + q8;

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 wa[8], wb[8];
  auto fetch = [&](bf16x8* dst, int kk) {
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = load8(wrow + kk + 32 * j);
    // keep the loads here: otherwise the compiler sinks them below the
    // MFMAs of the other buffer, and only one buffer is ever in flight
    asm volatile("" ::: "memory");
  };
  auto compute = [&](const bf16x8* wv, int kk) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = mma32(load8(xrow + t * 16 * ld + kk + 32 * j), wv[j], acc[t]);
  };

  fetch(wa, 0);
  // the copies went out before these eight weight loads: this wave's have
  // landed when at most eight loads remain; after the barrier, every wave's
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  asm volatile("s_barrier" ::: "memory");
  for (int kk = 0; kk < klen; kk += 512) {
    fetch(wb, kk + 256);
    compute(wa, kk);
    // unconditional (the last step re-reads its own K-values, an L2 hit): a
    // branch here makes the compiler wait for these loads inside compute(wb)
    fetch(wa, kk + 512 < klen ? kk + 512 : kk);
    compute(wb, kk + 256);
  }

  if (nvalid) {
    float* out = p.part + ((int64_t)split * p.m_out + p.row_off) * p.N + n;
    const int m_lane = (lane >> 4) * 4;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = t * 16 + m_lane + e;
        if (m < M) out[(int64_t)m * p.N] = acc[t][e];
      }
  }
}

template <int MT>
static hipError_t launch_slab_t(const GemmArgs& a, int blocks, size_t lds, hipStream_t s) {
  // dynamic LDS above the default limit, allowed once per kernel and device
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> allowed[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!allowed[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_slab_kernel<MT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kSlabLdsBytes);
    if (e != hipSuccess) return e;
    allowed[dev].store(true, std::memory_order_release);
  }
  launch((gemm_slab_kernel<MT>), dim3(blocks), dim3(256), (uint32_t)lds, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_slab(const GemmArgs& a, size_t lds, hipStream_t s) {
  const int blocks = a.p[0].blocks + (a.nprob > 1 ? a.p[1].blocks : 0);
  if (blocks == 0) return hipSuccess;
  const int mt = a.p[0].mt;
  if (lds > (size_t)kSlabLdsBytes) return hipErrorInvalidValue;
  for (int i = 0; i < a.nprob; ++i) {
    const GemmProb& p = a.p[i];
    if (p.mt != mt || p.K % 512 != 0 || p.k_chunk % 512 != 0 || p.m0 + p.m1 > 16 * mt ||
        (size_t)mt * 16 * (p.k_chunk + 8) * 2 > lds)
      return hipErrorInvalidValue;
  }
  switch (mt) {
    case 1: return launch_slab_t<1>(a, blocks, lds, s);
    case 2: return launch_slab_t<2>(a, blocks, lds, s);
    case 3: return launch_slab_t<3>(a, blocks, lds, s);
    case 4: return launch_slab_t<4>(a, blocks, lds, s);
    case 5: return launch_slab_t<5>(a, blocks, lds, s);
    case 6: return launch_slab_t<6>(a, blocks, lds, s);
    case 7: return launch_slab_t<7>(a, blocks, lds, s);
    case 8: return launch_slab_t<8>(a, blocks, lds, s);
    default: return hipErrorInvalidValue;
  }
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

// ---------------------------------------------------------------- tiled (bf16, many rows)
// For the fresh-context projections (hundreds to thousands of rows), where the
// product is MFMA-bound: a workgroup computes a 256xBN output tile over one
// K-chunk with eight waves.  BN = 256: each wave owns a 128x64 block, i.e. 8x4
// tiles of 16x16x32 MFMAs, 128 fp32 accumulators per lane (two waves per
// SIMD).  BN = 128 / 64 (a few hundred rows, where 256-wide tiles would need
// many K-splits to fill the CUs, and their partials cost more than the
// product): 64x64 / 32x64 blocks per wave.
//
// The K loop steps by 64 through LDS stages: two of 64 KB for BN = 256 (a
// third would not fit), the copies of step s + 1 issued right after the
// barrier of step s and landing while step s computes; three of 48 / 40 KB for
// BN = 128 / 64, the copies of step s + 2 issued after the barrier of step s,
// so that they have two steps to land (the 16-request batch's 256-row q/k/v
// and o products 39 -> 36 us and 20 -> 17 us).  Operands reach LDS by direct-to-LDS copies that each move 8 rows
// x 128 bytes (whole cache lines: copies of half lines run at well under half
// the rate), so a stage holds each tile row's 64 K-values contiguously, in
// 1 KB blocks of 8 rows.  An MFMA fragment read (16 rows, one 16-byte chunk of
// each) would then hit the same banks from many rows, so chunk c of tile row R
// is stored at position c ^ (R % 8) ^ ((R / 8) % 2) of its row - the copy
// picks, for each lane, the chunk its LDS slot must hold - which makes every
// 16-lane group of a ds_read_b128 cover all 64 banks once.  An A fragment
// feeds 4 MFMAs, a B fragment 8.  One barrier per step: after it, every
// wave's copies of the step have landed and every wave is done with the
// previous step, whose stage is the one refilled.
//
// Workgroups are ordered for the L2 of each XCD: consecutive block indices go
// to different XCDs, so the block index is remapped so that each XCD's share
// is a contiguous run of tiles of one split, in groups of kTileGroupM row
// tiles - the XCD's workgroups then read the same activation and weight rows.
// Requirements (checked by the planner): bf16, K and the K-chunk multiples of
// 64, N a multiple of 4, 16-byte aligned rows.

namespace {
constexpr int kTileBM = 256, kTileBK = 64;
constexpr int kTileWaves = 8;
constexpr int kTileBlocks = kTileBM / 8;   // 1 KB blocks (8 rows x 128 B) of A per stage
constexpr int kTileGroupM = 4;
constexpr int kXcds = 8;
}

template <int BN>
__global__ __launch_bounds__(512, 1) void gemm_tile_kernel(TileProb p) {
  constexpr int NST = BN == 256 ? 2 : 3;   // LDS stages
  constexpr int BBLOCKS = BN / 8;          // 1 KB blocks of B per stage
  constexpr int WN = BN / 64;              // waves along N
  constexpr int WM = kTileWaves / WN;      // waves along M
  constexpr int RM = kTileBM / WM;         // rows per wave
  constexpr int FM = RM / 16;              // 16-row fragments per wave
  // stage arrays, always indexed by a compile-time stage number
  __shared__ __align__(16) unsigned char sa[NST][kTileBlocks * 1024];
  __shared__ __align__(16) unsigned char sb[NST][BBLOCKS * 1024];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // XCD-aware order: block b runs on XCD b % 8; give XCD x the run
  // [x * per, (x + 1) * per) of virtual indices (the remainder keeps its own)
  int v = blockIdx.x;
  const int per = gridDim.x / kXcds;
  if (v < per * kXcds) v = (v % kXcds) * per + v / kXcds;
  const int tiles = p.m_tiles * p.n_tiles;
  const int split = v / tiles;
  const int t = v - split * tiles;
  const int band = kTileGroupM * p.n_tiles;
  const int first_m = (t / band) * kTileGroupM;
  const int gsz = min(p.m_tiles - first_m, kTileGroupM);
  const int mt = first_m + (t % band) % gsz, nt = (t % band) / gsz;
  const int m_base = mt * kTileBM, n_base = nt * BN;
  const int k_begin = split * p.k_chunk;
  const int k_end = min(p.K, k_begin + p.k_chunk);
  const int nsteps = (k_end - k_begin) / kTileBK;   // >= 1: K and chunks are multiples of 64
  const int M = p.m0 + p.m1;

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;

  // Copies of one K-step: block b of a stage holds tile rows 8 b .. 8 b + 7;
  // wave w copies blocks w, w + 8, w + 16, w + 24 of A and w, w + 8, .. of B.
  // Lane l fills row 8 b + l / 8, slot l % 8, with the chunk that the swizzle
  // puts there.  Rows past M (columns past N) read row 0 and are never stored.
  constexpr int PER_WAVE = kTileBlocks / kTileWaves;
  constexpr int PER_WAVE_B = BBLOCKS / kTileWaves;
  const int crow = lane >> 3;
  const int cchunk = (lane & 7) ^ crow ^ (wave & 1);   // blocks w + 8 i all have parity w & 1
  auto issue = [&](int step, auto st) {
    unsigned char* da = sa[st.value];
    unsigned char* db = sb[st.value];
    const int k = k_begin + step * kTileBK + 8 * cchunk;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int b = wave + kTileWaves * i;
      int m = m_base + 8 * b + crow;
      m = m < M ? m : 0;
      const bf16* xa = m < p.m0 ? p.x0 + (int64_t)m * p.K : p.x1 + (int64_t)(m - p.m0) * p.K;
      lds_copy16(xa + k, da + b * 1024);
      if (i < PER_WAVE_B) {
        int n = n_base + 8 * b + crow;
        n = n < p.N ? n : 0;
        lds_copy16(p.w + (int64_t)n * p.K + k, db + b * 1024);
      }
    }
  };

  // wave (wm, wn) owns rows RM wm .. +RM-1 and columns 64 wn .. +63 of the tile
  const int wm = wave / WN, wn = wave % WN;
  f32x4 acc[FM][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragment reads: lane l takes row R = l % 16 of a 16-row group (2 blocks)
  // and chunk 4 kk + l / 16 of the step's 64 K-values, found at its swizzled
  // position.
  const int fr = lane & 15;
  const int fkey = (fr & 7) ^ (fr >> 3);
  const int frow_off = (fr >> 3) * 1024 + (fr & 7) * 128;
  const int foff0 = frow_off + (((lane >> 4)) ^ fkey) * 16;
  const int foff1 = frow_off + ((4 + (lane >> 4)) ^ fkey) * 16;

  // The products are taken as W x^T (B fragments in the MFMA's first operand)
  // so that each lane ends up with four consecutive output columns of a row.
  auto compute = [&](auto st) {
    const unsigned char* ga = sa[st.value] + (FM * wm) * 2048;
    const unsigned char* gb = sb[st.value] + (4 * wn) * 2048;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int off = kk ? foff1 : foff0;
      bf16x8 af[FM], bfr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(gb + j * 2048 + off);
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(ga + i * 2048 + off);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma32(bfr[j], af[i], acc[i][j]);
    }
  };

  // Step s: wait for this wave's copies of step s, barrier, refill the stage
  // of step s - 1 with step s + NST - 1, compute.  The barrier is s_barrier in
  // asm, a compiler memory barrier as well; __syncthreads() would add a
  // release fence that waits for every copy.
  if constexpr (NST == 2) {
    // the copies of step s are the only ones in flight
    auto step = [&](int s, auto st, auto st_next) {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (s + 1 < nsteps) issue(s + 1, st_next);
      compute(st);
    };
    issue(0, S0{});
    for (int s = 0; s < nsteps; s += 2) {
      step(s, S0{}, S1{});
      if (s + 1 < nsteps) step(s + 1, S1{}, S0{});
    }
  } else {
    // those of step s + 1 (PER_WAVE + PER_WAVE_B per wave) may still be
    constexpr int CPS = PER_WAVE + PER_WAVE_B;
    auto step = [&](int s, auto st, auto st_issue) {
      wait_vm_blocks<CPS>(s + 1 < nsteps ? 1 : 0);
      asm volatile("s_barrier" ::: "memory");
      if (s + 2 < nsteps) issue(s + 2, st_issue);
      compute(st);
    };
    issue(0, S0{});
    if (nsteps > 1) issue(1, S1{});
    for (int s = 0; s < nsteps; s += 3) {
      step(s, S0{}, S2{});
      if (s + 1 < nsteps) step(s + 1, S1{}, S0{});
      if (s + 2 < nsteps) step(s + 2, S2{}, S1{});
    }
  }

  // lane l holds, for row m = 16 i + l % 16 of the wave's block, the four
  // consecutive columns 16 j + 4 (l / 16) .. +3: one 16-byte store each
  float* out = p.part + (int64_t)split * M * p.N;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m_base + RM * wm + 16 * i + (lane & 15);
    if (m >= M) continue;
    float* row = out + (int64_t)m * p.N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n_base + 64 * wn + 16 * j + 4 * (lane >> 4);
      if (n < p.N) *reinterpret_cast<f32x4*>(row + n) = acc[i][j];
    }
  }
}

hipError_t launch_gemm_tile(const TileProb& p, int bn, hipStream_t s) {
  const int blocks = p.m_tiles * p.n_tiles * p.splits;
  if (blocks == 0) return hipSuccess;
  if (p.n_tiles != (p.N + bn - 1) / bn) return hipErrorInvalidValue;
  switch (bn) {
    case 256: launch(gemm_tile_kernel<256>, dim3(blocks), dim3(64 * kTileWaves), 0, s, p); break;
    case 128: launch(gemm_tile_kernel<128>, dim3(blocks), dim3(64 * kTileWaves), 0, s, p); break;
    case 64: launch(gemm_tile_kernel<64>, dim3(blocks), dim3(64 * kTileWaves), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- weight streaming (bf16, at most 64 rows)
// part[split][m][n] = sum over the split's K-chunk of x[m][k] w[n][k], for the
// q/k/v and o projections of a draft round (16..64 rows): the product is the
// weight stream, so each wave owns 16 weight rows and streams them through its
// own direct-to-LDS ring of 64-wide K-steps - 16 rows x 128 bytes per step,
// two copies of 8 whole rows (whole cache lines), chunks XOR-swizzled so that
// the MFMA fragment reads are conflict free - with no barrier in the loop.  The
// workgroup's activation chunk (at most 64 rows x 512) is staged once in LDS in
// MFMA operand order by direct copies issued together with the first weight
// steps, so its latency overlaps theirs.  Products are taken as W x^T, so each
// lane ends with four consecutive columns of one row (16-byte partial stores).
// Requirements (checked by the planner): bf16, K a multiple of 64, N of 4.
constexpr int kStreamKC = 512;   // K-chunk per workgroup

template <int MT, int WAVES, int NST>
__global__ __launch_bounds__(64 * WAVES) void gemm_stream_kernel(TileProb p) {
  constexpr int XS = kStreamKC / 32;                         // activation slabs per 16-row tile
  __shared__ __align__(16) unsigned char sx[MT * XS * 1024];
  __shared__ __align__(16) unsigned char ring[WAVES][NST * 2048];
  // the operand pointers in the same batch of argument reads as the sizes
  asm volatile("" ::"s"(p.x0), "s"(p.x1), "s"(p.w));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nt = blockIdx.x % p.n_tiles, split = blockIdx.x / p.n_tiles;
  const int k0 = split * p.k_chunk;
  const int kc = min(p.k_chunk, p.K - k0);                   // a multiple of 64
  const int nsteps = kc / 64;
  const int n0 = nt * (16 * WAVES) + 16 * wave;               // this wave's 16 weight rows
  const int M = p.m0 + p.m1;

  // activation chunk in operand order, one direct copy per slab (mt, s): lane
  // l brings row 16 mt + l % 16, k 32 s + 8 (l / 16) .. +7.  Rows past M read
  // row 0: their products are never stored.
  const int slabs = MT * (kc / 32);
  for (int slab = wave; slab < slabs; slab += WAVES) {
    const int mt = slab / (kc / 32), s = slab - mt * (kc / 32);
    int m = 16 * mt + (lane & 15);
    m = m < M ? m : 0;
    const bf16* row = m < p.m0 ? p.x0 + (int64_t)m * p.K : p.x1 + (int64_t)(m - p.m0) * p.K;
    lds_copy16(row + k0 + 32 * s + 8 * (lane >> 4), sx + (mt * XS + s) * 1024);
  }

  // copies of step t into stage t % NST: copy j (0, 1) moves rows 8 j .. 8 j + 7
  // of the wave's 16; lane l fills row 8 j + l / 8, slot l % 8, with chunk
  // (l % 8) ^ key(row), key(R) = (R % 8) ^ (R / 8).  Rows past N read row 0 and
  // are never stored.
  const int crow = lane >> 3;
  unsigned char* my = ring[wave];
  auto issue = [&](int t) {
    unsigned char* st = my + (t % NST) * 2048;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int R = 8 * j + crow;
      const int c = (lane & 7) ^ (R & 7) ^ j;
      int n = n0 + R;
      n = n < p.N ? n : 0;
      lds_copy16(p.w + (int64_t)n * p.K + k0 + 64 * t + 8 * c, st + j * 1024);
    }
  };
  // fragment reads: lane (j16, q4) takes row j16, chunk 4 kk + q4 at its slot
  const int fr = lane & 15, fkey = (fr & 7) ^ (fr >> 3);
  const int foff0 = fr * 128 + ((lane >> 4) ^ fkey) * 16;
  const int foff1 = fr * 128 + ((4 + (lane >> 4)) ^ fkey) * 16;

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int AHEAD = NST - 1;   // steps in flight
  for (int t = 0; t < min(AHEAD, nsteps); ++t) issue(t);
  // the activation copies went out before the weight steps: once step 0 has
  // landed, so have this wave's; after the barrier, every wave's
  wait_vm_blocks<2>(min(nsteps - 1, AHEAD - 1));
  asm volatile("s_barrier" ::: "memory");
  for (int t = 0; t < nsteps; ++t) {
    // this wave's copies of step t have landed when at most those of the
    // later steps already issued remain (two copies per step)
    wait_vm_blocks<2>(min(nsteps - 1 - t, AHEAD - 1));
    const unsigned char* st = my + (t % NST) * 2048;
    const bf16x8 w0 = *reinterpret_cast<const bf16x8*>(st + foff0);
    const bf16x8 w1 = *reinterpret_cast<const bf16x8*>(st + foff1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 x0 = *reinterpret_cast<const bf16x8*>(sx + (mt * XS + 2 * t) * 1024 + 16 * lane);
      const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(sx + (mt * XS + 2 * t + 1) * 1024 + 16 * lane);
      acc[mt] = mma32(w0, x0, acc[mt]);
      acc[mt] = mma32(w1, x1, acc[mt]);
    }
    // every LDS read of this stage has returned before it is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (t + AHEAD < nsteps) issue(t + AHEAD);
  }

  // lane (j16, q4): row m = 16 mt + j16, columns n0 + 4 q4 .. +3
  float* out = p.part + (int64_t)split * M * p.N;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + (lane & 15);
    const int n = n0 + 4 * (lane >> 4);
    if (m < M && n < p.N) *reinterpret_cast<f32x4*>(out + (int64_t)m * p.N + n) = acc[mt];
  }
}

// Configurations (measured): one 16-row tile: 8 waves, 4 stages; two tiles:
// 12 waves, 4 stages (the 8K round's q/k/v product: 32 column tiles x 8
// splits = 256 workgroups, one per CU; 16 waves and 3 stages gave 192
// workgroups, 12.6 us against 12.0 on average); three or four tiles: 8
// waves, 4 stages, 128 KB of LDS (a 64-row 4096 x 4096 product: 32 x 8
// workgroups, 10.5 us against 12.4 for the slab kernel; at 128 rows, 4 waves
// and 160 KB took 12.9 us against the slab kernel's 11.0).  p.n_tiles must be
// ceil(N / (16 * waves)).
int gemm_stream_waves(int mt) { return mt == 2 ? 12 : 8; }

hipError_t launch_gemm_stream(const TileProb& p, int mt, hipStream_t s) {
  const int blocks = p.n_tiles * p.splits;
  if (blocks == 0) return hipSuccess;
  if (p.k_chunk != kStreamKC || mt < 1 || mt > 4) return hipErrorInvalidValue;
  if (mt == 1)
    launch((gemm_stream_kernel<1, 8, 4>), dim3(blocks), dim3(64 * 8), 0, s, p);
  else if (mt == 2)
    launch((gemm_stream_kernel<2, 12, 4>), dim3(blocks), dim3(64 * 12), 0, s, p);
  else
    launch((gemm_stream_kernel<4, 8, 4>), dim3(blocks), dim3(64 * 8), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- full-K weight streaming (bf16, at most 16 rows)
// One workgroup per 16 output columns; its eight waves split K (wave w takes
// K/8 .. ) and stream, per 64-wide step, their 16 weight rows and the 16
// activation rows (whole 128-byte lines, XOR-swizzled chunks) into their own
// direct-to-LDS rings; the waves' accumulators are summed in LDS at the end.
// No split-K partials: the result is written once, either as fp32 [M][N] (a
// single "split" for the reductions that follow) or, for the o projection, as
// the storage type with the residual added (out may alias add: each element
// is read and written by the same lane).
// Requirements (checked by the planner): bf16, K a multiple of 512, N of 4.
constexpr int kFullkWaves = 8, kFullkStages = 5;

__global__ __launch_bounds__(64 * kFullkWaves) void gemm_fullk_kernel(FullkArgs p) {
  constexpr int STAGE = 4 * 1024;   // 16 weight rows + 16 activation rows, 128 bytes each
  // the rings fill the CU's 160 KB; the waves' sums meet in the first ring
  // once every wave is past its last step
  __shared__ __align__(16) unsigned char ring[kFullkWaves][kFullkStages * STAGE];
  static_assert(kFullkWaves * 64 * sizeof(f32x4) <= kFullkStages * STAGE, "the reduction fits one wave's ring");
  f32x4 (*red)[64] = reinterpret_cast<f32x4 (*)[64]>(&ring[0][0]);
  // the operand pointers in the same batch of argument reads as the sizes
  // (read where they are first used, they would add a round trip before the
  // first copies)
  asm volatile("" ::"s"(p.x0), "s"(p.x1), "s"(p.w));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16;
  const int M = p.m0 + p.m1;
  const int kw = p.K / kFullkWaves;   // a multiple of 64
  const int k0 = wave * kw;
  const int nsteps = kw / 64;

  // copies of step t into stage t % kFullkStages: copies 0-1 move weight rows
  // 8 j .. 8 j + 7, copies 2-3 activation rows; lane l fills row 8 j + l / 8,
  // slot l % 8, with chunk (l % 8) ^ key(row), key(R) = (R % 8) ^ (R / 8).
  // Rows past N (past M) read row 0; they are never stored.
  const int crow = lane >> 3;
  unsigned char* my = ring[wave];
  auto issue = [&](int t) {
    unsigned char* st = my + (t % kFullkStages) * STAGE;
    const int k = k0 + 64 * t;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int R = 8 * j + crow;
      const int c = (lane & 7) ^ (R & 7) ^ j;
      int n = n0 + R;
      n = n < p.N ? n : 0;
      lds_copy16(p.w + (int64_t)n * p.K + k + 8 * c, st + j * 1024);
      int m = R < M ? R : 0;
      const bf16* xr = m < p.m0 ? p.x0 + (int64_t)m * p.K : p.x1 + (int64_t)(m - p.m0) * p.K;
      lds_copy16(xr + k + 8 * c, st + (2 + j) * 1024);
    }
  };
  const int fr = lane & 15, fkey = (fr & 7) ^ (fr >> 3);
  const int foff0 = fr * 128 + ((lane >> 4) ^ fkey) * 16;
  const int foff1 = fr * 128 + ((4 + (lane >> 4)) ^ fkey) * 16;

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int AHEAD = kFullkStages - 1;
  for (int t = 0; t < min(AHEAD, nsteps); ++t) issue(t);
  for (int t = 0; t < nsteps; ++t) {
    wait_vm_blocks<4>(min(nsteps - 1 - t, AHEAD - 1));   // four copies per step
    const unsigned char* st = my + (t % kFullkStages) * STAGE;
    const bf16x8 w0 = *reinterpret_cast<const bf16x8*>(st + foff0);
    const bf16x8 w1 = *reinterpret_cast<const bf16x8*>(st + foff1);
    const bf16x8 x0 = *reinterpret_cast<const bf16x8*>(st + 2048 + foff0);
    const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(st + 2048 + foff1);
    acc = mma32(w0, x0, acc);
    acc = mma32(w1, x1, acc);
    // every LDS read of this stage has returned before it is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (t + AHEAD < nsteps) issue(t + AHEAD);
  }
  __syncthreads();   // every wave's ring reads are done before ring 0 takes the sums
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  // lane (j16, q4): row m = j16, columns n0 + 4 q4 .. +3
  f32x4 sum = red[0][lane];
#pragma unroll
  for (int w = 1; w < kFullkWaves; ++w) sum += red[w][lane];
  const int m = lane & 15, n = n0 + 4 * (lane >> 4);
  if (m >= M || n >= p.N) return;
  const int64_t o = (int64_t)m * p.N + n;
  if (p.part != nullptr) {
    *reinterpret_cast<f32x4*>(p.part + o) = sum;
  } else {
    const bf16* add = static_cast<const bf16*>(p.add);
    bf16* out = static_cast<bf16*>(p.out);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = add != nullptr ? to_f32(add[o + e]) : 0.f;
      out[o + e] = from_f32<bf16>(sum[e] + a);
    }
  }
}

hipError_t launch_gemm_fullk(const FullkArgs& p, hipStream_t s) {
  if (p.m0 + p.m1 <= 0 || p.N <= 0) return hipSuccess;
  if (p.m0 + p.m1 > 16 || p.K % (64 * kFullkWaves) != 0 || p.N % 4 != 0) return hipErrorInvalidValue;
  if ((p.part == nullptr) == (p.out == nullptr)) return hipErrorInvalidValue;
  launch(gemm_fullk_kernel, dim3((p.N + 15) / 16), dim3(64 * kFullkWaves), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- resident activations (bf16, at most 16 rows, many columns)
// For products with tens of thousands of output columns and at most 16 rows
// (the draft head's lm_head: 15 rows x 4096 -> 151936 columns): each
// workgroup copies the activation rows into LDS once, then every wave streams
// whole 16-column weight tiles over the full K straight into MFMA A operands
// (16-byte loads, kResPf K-steps in flight per wave), reading the activation
// operand from LDS.  Where the full-K kernel re-reads the activation rows for
// every 16 columns (as many bytes as the weights), here each workgroup reads
// them once; there are no split-K partials.  Result: fp32 [M][N].
// LDS layout of the rows: 16-byte granule (row, chunk) at granule index
// row * K/8 + (chunk ^ (row % 8)) - the xor spreads the 16 rows of an operand
// read over the banks.
// Requirements (checked by the planner): bf16, M <= 16, K a multiple of 64 and
// at most kResMaxK, N a multiple of 4.
// kResPf: 8 measured best on the lm_head shape (12 and 16 slower).
constexpr int kResWaves = 8, kResPf = 8;

__global__ __launch_bounds__(64 * kResWaves, 1) void gemm_resident_kernel(FullkArgs p) {
  __shared__ __align__(16) unsigned char xs[16 * kResMaxK * 2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = p.m0 + p.m1;
  const int K = p.K;
  const int gpr = K / 8;   // 16-byte granules per row (a multiple of 8)

  // stage the 16 activation rows (rows past M read row 0; never stored):
  // copy i fills granules 64 i .. 64 i + 63, lane l granule 64 i + l
  for (int i = wave; i < 2 * K / 64; i += kResWaves) {
    const int gi = 64 * i + lane;
    const int row = gi / gpr, slot = gi - row * gpr;
    const int chunk = slot ^ (row & 7);
    const int m = row < M ? row : 0;
    const bf16* xr = m < p.m0 ? p.x0 + (int64_t)m * K : p.x1 + (int64_t)(m - p.m0) * K;
    lds_copy16(xr + 8 * chunk, xs + i * 1024);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // this wave's tiles: first, first + G, ... (G = waves in the grid); its
  // work is the sequence of (tile, K-step) pairs, q = i * S + t
  const int S = K / 64;
  const int n_tiles = (p.N + 15) / 16;
  const int G = gridDim.x * kResWaves;
  const int first = blockIdx.x + gridDim.x * wave;
  const int my_tiles = first < n_tiles ? (n_tiles - first + G - 1) / G : 0;
  const int total = my_tiles * S;
  if (total == 0) return;
  const int j16 = lane & 15, q4 = lane >> 4;
  // weight operand of step q: row tile * 16 + j16 (past N: row 0), K-values
  // 64 t + 8 q4 .. (+ 32 for the second half); the prefetch past the last
  // step re-reads that step (an L2 hit) so that every load is unconditional
  auto wsrc = [&](int q) {
    q = min(q, total - 1);
    const int tile = first + G * (q / S);
    int n = tile * 16 + j16;
    n = n < p.N ? n : 0;
    return p.w + (int64_t)n * K + 64 * (q % S) + 8 * q4;
  };
  const unsigned char* xrow = xs + j16 * gpr * 16;
  const int xkey = j16 & 7;

  bf16x8 ra[kResPf], rb[kResPf];
#pragma unroll
  for (int u = 0; u < kResPf; ++u) {
    const bf16* src = wsrc(u);
    ra[u] = load8(src);
    rb[u] = load8(src + 32);
  }
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < total; base += kResPf) {
#pragma unroll
    for (int u = 0; u < kResPf; ++u) {
      const int q = base + u;
      if (q < total) {
        const int t = q % S;
        const bf16x8 x0 = *reinterpret_cast<const bf16x8*>(xrow + (8 * t + (q4 ^ xkey)) * 16);
        const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(xrow + (8 * t + ((4 + q4) ^ xkey)) * 16);
        acc = mma32(ra[u], x0, acc);
        acc = mma32(rb[u], x1, acc);
        if (t == S - 1) {
          // lane (j16, q4): row m = j16, columns tile * 16 + 4 q4 .. +3
          const int n = (first + G * (q / S)) * 16 + 4 * q4;
          if (j16 < M && n < p.N) *reinterpret_cast<f32x4*>(p.part + (int64_t)j16 * p.N + n) = acc;
          acc = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      const bf16* src = wsrc(base + u + kResPf);
      ra[u] = load8(src);
      rb[u] = load8(src + 32);
    }
  }
}

hipError_t launch_gemm_resident(const FullkArgs& p, hipStream_t s) {
  if (p.m0 + p.m1 <= 0 || p.N <= 0) return hipSuccess;
  if (p.m0 + p.m1 > 16 || p.K % 64 != 0 || p.K > kResMaxK || p.N % 4 != 0 || p.part == nullptr)
    return hipErrorInvalidValue;
  // one workgroup per CU (the rows take most of the LDS), capped by the tiles
  const int tiles = (p.N + 15) / 16;
  const int blocks = std::min(256, (tiles + kResWaves - 1) / kResWaves);
  launch(gemm_resident_kernel, dim3(blocks), dim3(64 * kResWaves), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- split-K reduction
// out[m][n] = sum_s part[s][m][n] (+ add[m][n] when add is given); one thread
// per 4 outputs, the split loop unrolled so that its loads are in flight
// together.

template <typename Tout>
// add and out carry no __restrict__: a residual layer may write its output over
// the block rows it adds (out == add); each element is read, then written, by
// the same thread.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                            int64_t MN, const Tout* add, Tout* out) {
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
