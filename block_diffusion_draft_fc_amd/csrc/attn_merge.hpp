// Device helpers shared by the attention kernels (bf16 and fp8 caches): the
// merge of one query row's split partials, and the arrival of a K/V head's
// work items when the split is merged inside the attention launch.
#pragma once
#include "kernels.hpp"

namespace dflash {

// ---------------------------------------------------------------- merge of a row's partials
// One query row's chunk partials merged: m = max_c m_c,
// l = sum_c 2^(m_c - m) l_c, O = sum_c 2^(m_c - m) O_c / l, stored in the
// row-major [R*B][n_h*d_h] order of the attention output (head h at columns
// h*d_h .., "DFlash KV Injection Walkthrough" Step 4.5).  One wave per row,
// lane l owning head dims 2l, 2l+1 (d_h <= 128); the partials are in the
// layer's storage type.  Chunks go in groups of 32: every O load of the group
// and the group's (m, l) loads (lane c % 32 loads chunk c's) are issued before
// any is used, so a row costs one memory latency per 32 chunks; the group
// maximum and weights come from wave reductions and readlane.  A group maximum
// above the running one rescales the accumulators.

__device__ __forceinline__ float2 load2f(const float* p) { return *reinterpret_cast<const float2*>(p); }
__device__ __forceinline__ float2 load2f(const bf16* p) {
  const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
  return float2{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)};
}

// Row qrow of the n items it0 .. it0 + n - 1 (one (sequence, K/V head)):
// returns this lane's two normalised output values.
template <typename T>
__device__ __forceinline__ float2 merge_partials_row(const T* part_o, const float* part_ml, int64_t it0, int n,
                                                     int qrows, int qrow, int d_h, int lane) {
  constexpr int G = 32;
  const float* ml = part_ml + it0 * 2 * qrows + qrow;   // m_c at ml[c * mstride], l_c at + qrows
  const int mstride = 2 * qrows;
  const bool act = 2 * lane < d_h;
  const T* po = part_o + (it0 * qrows + qrow) * d_h + 2 * (act ? lane : 0);
  const int ostride = qrows * d_h;
  float mrun = -INFINITY, lrun = 0.f, o0 = 0.f, o1 = 0.f;
  for (int cb = 0; cb < n; cb += G) {
    float2 oc[G];
    // chunks past n load chunk n - 1 again (their weight is 0): the loads
    // stay unconditional, so all of them go out before the first is used;
    // 32-bit offsets within a group of 32 chunks (qrows * d_h <= 64 * 128)
    const T* pb = po + (int64_t)cb * ostride;
    const int last = n - 1 - cb;
#pragma unroll
    for (int k = 0; k < G; ++k) oc[k] = load2f(pb + min(k, last) * ostride);
    // issue the O loads before the (m, l) loads and their reductions
    asm volatile("" ::: "memory");
    const int c = cb + (lane & (G - 1));
    const float mc = c < n ? ml[(int64_t)c * mstride] : -INFINITY;
    const float lc = c < n ? ml[(int64_t)c * mstride + qrows] : 0.f;
    const float mg = fmaxf(wave_max(mc), mrun);
    const float mu = mg == -INFINITY ? 0.f : mg;
    const float wc = __builtin_amdgcn_exp2f(mc - mu);     // weight of chunk cb + lane % 32 (0 for -inf)
    const float sa = __builtin_amdgcn_exp2f(mrun - mu);   // rescale of the groups before
    // lanes 32..63 repeat lanes 0..31: half the wave sum is the group's
    lrun = lrun * sa + 0.5f * wave_sum(wc * lc);
    o0 *= sa;
    o1 *= sa;
    mrun = mg;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wc), k));
      o0 += w * oc[k].x;
      o1 += w * oc[k].y;
    }
  }
  const float inv = lrun > 0.f ? 1.0f / lrun : 0.f;
  return float2{o0 * inv, o1 * inv};
}

template <typename T>
__device__ __forceinline__ void store_merged_row(T* attn, float2 o, int r, int g, int qrow, int B, int group,
                                                 int n_kv, int d_h, int lane) {
  if (2 * lane >= d_h) return;
  const int hl = qrow / B, b = qrow - hl * B;
  const int h = g * group + hl;
  T* dst = attn + ((int64_t)r * B + b) * (n_kv * group * d_h) + h * d_h + 2 * lane;
  dst[0] = from_f32<T>(o.x);
  dst[1] = from_f32<T>(o.y);
}

// Lines of one item's partial (O rows, then m and l) brought into the XCD's
// L2 before the item writes them, by one line per thread t (t < 132 for 64
// query rows of 128 dims; others load nothing).  A store that misses the L2
// does not leave its line there, so the other items' first reads of a freshly
// written partial would wait on memory (a row merge 1.7 against 1.3 us with
// the lines brought in first).  The word returned is unused; the caller keeps
// it live until its loads may complete in the background.
__device__ __forceinline__ uint32_t attn_partial_preload(const void* part_o, const float* part_ml, int64_t item,
                                                         int qrows, int d_h, int t) {
  const int olines = qrows * d_h * 2 / 128;
  const int mlines = (qrows * 2 * 4 + 127) / 128;
  const unsigned char* p = nullptr;
  if (t >= 0 && t < olines)
    p = static_cast<const unsigned char*>(part_o) + item * qrows * d_h * 2 + 128 * t;
  else if (t >= olines && t < olines + mlines)
    p = reinterpret_cast<const unsigned char*>(part_ml + item * 2 * qrows) + 128 * (t - olines);
  return p != nullptr ? *reinterpret_cast<const uint32_t*>(p) : 0u;
}

// ---------------------------------------------------------------- in-launch merge: a head's arrivals
// The items of one K/V head meet before merging the head's rows from each
// other's partials.  Items of a head whose workgroup indices agree mod 8 sit
// on one XCD, so their partials are in that XCD's L2 and no cache write-back
// is needed.  Each item, once its partial stores are complete, stores a flag
// (1 + its XCD) in its slot of the head's flag line with a plain store, which
// lands in its XCD's L2, and adds 1 << (8 * XCD) to the head's arrival word
// with a system-scope atomic.  The waiting wave polls the flag line with loads
// that miss its CU's L1 and are served by the L2 (one round trip of the L2,
// ~0.4 us from the last arrival to the release): when all n flags carry its
// own XCD, every item ran beside it.  A flag stored on another XCD stays in
// that XCD's L2 and never shows as this XCD's, so a head whose items came
// from several XCDs never completes its flags; every 8th poll therefore also
// reads the arrival word past every cache, and once its bytes count all n
// items without this XCD's byte doing so, every item writes its L2 back,
// meets the others at a second count and invalidates its caches before the
// merge (slow, but exact).  Waits are bounded: a workgroup whose wait runs out
// counts itself in its kernel file's timeout counter (read by
// dflash_attn_sync_timeouts) and writes its rows as NaN rather than hang.

__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}
// loads that miss the CU's L1 and every cache past it, waited for in the same asm block
__device__ __forceinline__ uint64_t load_sync64(const uint64_t* p) {
  uint64_t v;
  asm volatile("global_load_dwordx2 %0, %1, off sc0 sc1\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t load_sync32(const uint32_t* p) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off sc0 sc1\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}
// a load that misses the CU's L1 and is served by the XCD's L2 (device scope)
__device__ __forceinline__ uint32_t load_l2_32(const uint32_t* p) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ int byte_sum(uint64_t v) {
  int s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += (int)((v >> (8 * i)) & 0xff);
  return s;
}

// One wave per workgroup (all 64 lanes), after the workgroup's partial stores
// have completed: item `slot` of its head arrives at head words w (the u64
// arrival word, the fallback count, and the flags at w + kAttnSyncFlags) and
// waits for the head's n items (n <= kAttnMergeMaxItems), giving up after
// `polls` polls of a wait (0: without polling).  Returns, in every lane, 0
// when all n came from this XCD, 1 when they came from several (every item's
// L2 is then written back and this CU's caches invalidated), 2 when a wait
// timed out.
__device__ __forceinline__ int attn_head_arrive(uint32_t* w, int n, int slot, int lane, int polls) {
  const uint32_t x = xcc_id() & 7;
  uint32_t* flags = w + kAttnSyncFlags;
  uint64_t* word = reinterpret_cast<uint64_t*>(w);
  if (lane == 0) {
    flags[slot] = 1u + x;
    __hip_atomic_fetch_add(reinterpret_cast<unsigned long long*>(word), 1ull << (8 * x), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
  }
  for (int i = 0;; ++i) {
    if (i >= polls) return 2;
    const uint32_t f = load_l2_32(flags + (lane < n ? lane : 0));
    if (__all(lane >= n || f == 1u + x)) return 0;
    if ((i & 7) == 7) {
      const uint64_t v = load_sync64(word);
      if (byte_sum(v) >= n && (int)((v >> (8 * x)) & 0xff) != n) break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  if (lane == 0) __hip_atomic_fetch_add(w + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  for (int i = 0; (int)load_sync32(w + 2) < n; ++i) {
    if (i >= polls) return 2;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return 1;
}

}  // namespace dflash
