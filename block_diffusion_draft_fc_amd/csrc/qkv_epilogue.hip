// Epilogue of the fused q/k/v projection: split-K reduction, per-head RMSNorm
// on Q and K, rotary embedding, and the stores (Q to the workspace in GQA
// order, K and V straight into the draft cache).
//
//   per-head norms: "DFlash源码导读二 Qwen3DFlashAttention注意力实现全解析" section 1
//     (q_norm / k_norm over head_dim); V is not normed ("DFlash KV Injection
//     Walkthrough" Step 4.2).
//   rotary window: Step 4.3 of the walkthrough and section 3 of the article: the
//     n + B new K rows take positions L .. L+n+B-1 (context rows first), the B
//     queries the last B of them; pairs are (i, i + d_h/2) as in rotate_half.
//   cache write: section 4 of the article, the rows enter the cache after the
//     norm and the rotation.  An fp8 cache ("KV Cache + Speculative Decoding
//     面试 Cheat Sheet" 2.1 and 4.5: one byte per element) takes the OCP E4M3
//     byte nearest x / scale.
//
// One wavefront per (row, head); lane l < d_h/2 owns the rotation pair
// (l, l + d_h/2).  Angles p * w_i are formed and reduced in fp64 (positions go
// past 3e4, where an fp32 angle is off by ~1e-3 rad), then rounded to fp32.
#include "kernels.hpp"

namespace dflash {

// The E4M3 byte nearest x (the conversion rounds to nearest even), magnitudes
// beyond 448 clamped first so that they saturate whatever the conversion does
// on overflow; NaN stays NaN.
__device__ __forceinline__ uint8_t to_e4m3(float x) {
  const float c = __builtin_isnan(x) ? x : fminf(fmaxf(x, -448.f), 448.f);
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xff);
}

// Each wave is one short chain of loads, a reduction and stores: at most 64
// VGPRs, so that eight waves per SIMD cover the load latency of the large rounds
// (17152 waves for 1024 fresh context rows).
template <typename T, bool F8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void qkv_epilogue_kernel(QkvEpiArgs a) {
  // the scalar arguments in one batch of reads (left to itself the compiler
  // reads them behind the branches that use them, a round trip each, before
  // the first partial load)
  asm volatile("" ::"s"(a.part_q), "s"(a.part_kv), "s"(a.part_kvh), "s"(a.q_row), "s"(a.q_split), "s"(a.kv_row),
               "s"(a.kv_split), "s"(a.kvh_row), "s"(a.kvh_split));
  asm volatile("" ::"s"(a.sq), "s"(a.skv), "s"(a.skvh), "s"(a.R), "s"(a.B), "s"(a.T), "s"(a.n_h), "s"(a.n_kv),
               "s"(a.d_h), "s"(a.n_sync), "s"(a.attn_sync), "s"(a.d_rows));
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int RB = a.R * a.B;
  const int Mkv = a.T + RB;
  const int half = a.d_h >> 1;
  const int kvd = a.n_kv * a.d_h;
  const int64_t n_q_items = (int64_t)RB * a.n_h;
  const int64_t n_kv_items = (int64_t)Mkv * a.n_kv;
  // the next attention launch's arrival words and flags (plain stores: the
  // kernel boundary makes them visible to that launch)
  if (a.attn_sync != nullptr && blockIdx.x == 0) {
    constexpr int per_head = kAttnSyncWords + kAttnMergeMaxItems;
    for (int t = threadIdx.x; t < a.n_sync * per_head; t += blockDim.x) {
      const int h = t / per_head, wd = t - h * per_head;
      a.attn_sync[kAttnSyncStride * h + (wd < kAttnSyncWords ? wd : kAttnSyncFlags + wd - kAttnSyncWords)] = 0u;
    }
  }
  if (item >= n_q_items + 2 * n_kv_items) return;

  int kind;   // 0 = Q, 1 = K, 2 = V
  int m, head;
  if (item < n_q_items) {
    kind = 0; m = (int)(item / a.n_h); head = (int)(item % a.n_h);
  } else {
    const int64_t k = item - n_q_items;
    kind = k < n_kv_items ? 1 : 2;
    const int64_t kk = kind == 1 ? k : k - n_kv_items;
    m = (int)(kk / a.n_kv); head = (int)(kk % a.n_kv);
  }

  // split-K reduction of the two elements of this lane's rotation pair
  // (block rows' K/V from their own source: sel 2)
  const int sel = kind == 0 ? 0 : m < a.T ? 1 : 2;
  const float* part = sel == 0 ? a.part_q : sel == 1 ? a.part_kv : a.part_kvh;
  const int splits = sel == 0 ? a.sq : sel == 1 ? a.skv : a.skvh;
  const int64_t row_stride = sel == 0 ? a.q_row : sel == 1 ? a.kv_row : a.kvh_row;
  const int64_t stride = sel == 0 ? a.q_split : sel == 1 ? a.kv_split : a.kvh_split;
  const int col = (kind == 2 ? kvd : 0) + head * a.d_h;
  const int pm = sel == 2 ? m - a.T : m;
  const bool act = lane < half;
  float x0 = 0.f, x1 = 0.f;
  if (act) {
    // every split's loads of a group of 8 go out before the first is added
    // (one memory latency per 8 splits), then the sums in split order
    const float* src = part + (int64_t)pm * row_stride + col + lane;
    for (int s0 = 0; s0 < splits; s0 += 8) {
      float v0[8], v1[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sj = min(s0 + j, splits - 1);
        v0[j] = src[sj * stride];
        v1[j] = src[sj * stride + half];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < splits) { x0 += v0[j]; x1 += v1[j]; }
    }
  }

  // sequence and position of this row (device-driven rounds: lengths and new
  // rows from device memory, context rows at a fixed stride n_max, those past
  // a sequence's new rows skipped; the whole wave shares the row)
  int r, pos;
  const bool dev = a.d_rows != nullptr;
  if (kind == 0) {
    r = m / a.B;
    pos = (dev ? a.d_len[r] + dev_rows_of(a.d_rows, r, a.n_max) : a.seq.L[r] + a.seq.n[r]) + (m - r * a.B);
  } else if (m < a.T) {
    if (dev) {
      r = m / a.n_max;
      const int j = m - r * a.n_max;
      if (j >= dev_rows_of(a.d_rows, r, a.n_max)) return;
      pos = a.d_len[r] + j;
    } else {
      r = 0;
      while (r + 1 < a.R && m >= a.seq.cu[r + 1]) ++r;
      pos = a.seq.L[r] + (m - a.seq.cu[r]);
    }
  } else {
    const int bm = m - a.T;
    r = bm / a.B;
    pos = (dev ? a.d_len[r] + dev_rows_of(a.d_rows, r, a.n_max) : a.seq.L[r] + a.seq.n[r]) + (bm - r * a.B);
  }

  if (kind != 2) {
    const T* gam = static_cast<const T*>(kind == 0 ? a.gamma_q : a.gamma_k);
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float rr = 1.0f / sqrtf(ss / (float)a.d_h + a.eps);
    if (act) {
      x0 = x0 * rr * to_f32(gam[lane]);
      x1 = x1 * rr * to_f32(gam[lane + half]);
      // the angle pos * w in fp64 (positions reach tens of thousands: its
      // fp32 rounding alone would shift it by ~1e-3 rad), reduced to
      // [-pi, pi] in fp64 (k * 2pi exact to ~1e-11 rad for any position
      // here), then sine and cosine of the reduced angle in fp32
      const double ang = (double)pos * a.inv_freq[lane];
      const double kr = rint(ang * 0.15915494309189535);   // 1 / (2 pi)
      const float red = (float)fma(-kr, 6.283185307179586, ang);
      float sv, c;
      sincosf(red, &sv, &c);
      const float y0 = x0 * c - x1 * sv;
      const float y1 = x1 * c + x0 * sv;
      x0 = y0; x1 = y1;
    }
  }
  if (!act) return;

  if (kind == 0) {
    const int b = m - r * a.B;
    const int group = a.n_h / a.n_kv;
    const int g = head / group, hl = head - g * group;
    T* dst = static_cast<T*>(a.q_ws) + (((int64_t)r * a.n_kv + g) * a.qrows + hl * a.B + b) * a.d_h;
    dst[lane] = from_f32<T>(x0);
    dst[lane + half] = from_f32<T>(x1);
  } else {
    const int64_t page = cache_page(a.cache, r, pos);
    const int slot = pos % a.cache.page_rows;
    if constexpr (F8) {
      const float sc = kind == 1 ? a.k_scale : a.v_scale;
      const uint8_t c0 = to_e4m3(x0 / sc), c1 = to_e4m3(x1 / sc);
      if (kind == 1) {
        uint8_t* dst = static_cast<uint8_t*>(a.cache.k_pool) + k_offset(a.cache, page, head, slot);
        dst[lane] = c0;
        dst[lane + half] = c1;
      } else {
        uint8_t* dst = static_cast<uint8_t*>(a.cache.v_pool) + v_offset(a.cache, page, head, slot);
        dst[lane * kVTile] = c0;
        dst[(lane + half) * kVTile] = c1;
      }
    } else if (kind == 1) {
      T* dst = static_cast<T*>(a.cache.k_pool) + k_offset(a.cache, page, head, slot);
      dst[lane] = from_f32<T>(x0);
      dst[lane + half] = from_f32<T>(x1);
    } else {
      T* dst = static_cast<T*>(a.cache.v_pool) + v_offset(a.cache, page, head, slot);
      dst[lane * kVTile] = from_f32<T>(x0);
      dst[(lane + half) * kVTile] = from_f32<T>(x1);
    }
  }
}

hipError_t launch_qkv_epilogue(int dtype, const QkvEpiArgs& a, hipStream_t s) {
  const int64_t items = (int64_t)a.R * a.B * a.n_h + 2 * (int64_t)(a.T + a.R * a.B) * a.n_kv;
  if (items == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((items + 3) / 4);
  if (dtype == 1 && a.cache_fp8)
    launch(qkv_epilogue_kernel<bf16, true>, dim3(blocks), dim3(256), 0, s, a);
  else if (dtype == 1)
    launch(qkv_epilogue_kernel<bf16, false>, dim3(blocks), dim3(256), 0, s, a);
  else
    launch(qkv_epilogue_kernel<float, false>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
