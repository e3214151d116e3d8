// Shared device-side definitions for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

namespace dflash {

constexpr int kWave = 64;

// Eight consecutive elements of the storage type, the per-lane operand of one
// K=32 matrix step (16 bytes for bf16, 32 bytes for fp32).
template <typename T> struct Vec8;
template <> struct Vec8<bf16> { using type = bf16x8; };
template <> struct Vec8<float> { using type = f32x8; };
template <typename T> using vec8_t = typename Vec8<T>::type;

__device__ __forceinline__ bf16x8 load8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ f32x8 load8(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void store8(bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ __forceinline__ void store8(float* p, f32x8 v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
template <typename T> __device__ __forceinline__ vec8_t<T> zero8() { return vec8_t<T>{}; }
// Four fp32 values stored in the storage type (rounded to nearest even for bf16).
__device__ __forceinline__ void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
  *reinterpret_cast<bf16x4*>(p) = __builtin_convertvector(v, bf16x4);
}

template <typename T> __device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }

__device__ __forceinline__ bf16x8 cvt8_bf16(f32x8 v) { return __builtin_convertvector(v, bf16x8); }
template <typename T> __device__ __forceinline__ vec8_t<T> cvt8(f32x8 v);
template <> __device__ __forceinline__ bf16x8 cvt8<bf16>(f32x8 v) { return cvt8_bf16(v); }
template <> __device__ __forceinline__ f32x8 cvt8<float>(f32x8 v) { return v; }

// One K=32 step of a 16x16 fp32-accumulating matrix product.
// Operand order (both A and B): lane l holds row/column l % 16 and the eight
// k-values 8*(l/16) .. 8*(l/16)+7 of the step.  Result: lane l holds column
// l % 16, rows 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32 inputs: eight 16x16x4 steps.  Step e takes element e of every lane, i.e.
// k-value 8*(l/16)+e for the lane group l/16 - the same k on both operands, so
// the eight steps together cover the 32 k-values exactly once.
__device__ __forceinline__ f32x4 mma32(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

// Cross-lane exchanges without the LDS crossbar (a ds_bpermute shuffle costs
// ~100 clocks of latency per step): v_permlane16_swap / v_permlane32_swap
// with both operands x give each lane {x, x of lane ^ 16} (^ 32) in some
// order, and DPP row_mirror, row_half_mirror and quad_perm pair lanes within
// a row of 16.  Every step pairs lanes symmetrically, so all lanes of a
// reduction end with the same bits.
__device__ __forceinline__ float2 lane_swap16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return float2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float2 lane_swap32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return float2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_xor16(float x) { const float2 s = lane_swap16(x); return fmaxf(s.x, s.y); }
__device__ __forceinline__ float max_xor32(float x) { const float2 s = lane_swap32(x); return fmaxf(s.x, s.y); }
__device__ __forceinline__ float sum_xor16(float x) { const float2 s = lane_swap16(x); return s.x + s.y; }
__device__ __forceinline__ float sum_xor32(float x) { const float2 s = lane_swap32(x); return s.x + s.y; }
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141, kDppXor2 = 0x4e, kDppXor1 = 0xb1;

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppRowMirror>(v);       // lane i + lane 15 - i (row of 16)
  v += dpp_f<kDppRowHalfMirror>(v);   // + lane 7 - i (half row)
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppXor1>(v);            // the row's sum
  return sum_xor32(sum_xor16(v));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  return max_xor32(max_xor16(v));
}

// One direct-to-LDS copy of 16 bytes per lane (lane l's bytes land at
// lds + 16 * l), written in asm so that the compiler does not track it: its
// own tracking of these copies cannot follow LDS stages chosen at run time or
// carried around a loop, and waits for every copy in flight before reading a
// stage.  The kernels order these copies with explicit s_waitcnt vmcnt instead
// (vector memory operations of a wave complete in order); other
// vector-memory waits the compiler emits stay correct, since copies it does
// not count only make a vmcnt wait stricter.  M0 (the LDS base of the copy) is
// a reserved register, so the asm saves and restores it rather than declaring
// it clobbered.
__device__ __forceinline__ void lds_copy16(const void* src, const unsigned char* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(base)
      : "memory");
}

// s_waitcnt vmcnt(blocks * N) for blocks in 0..6 (the count must be an
// immediate): "at most the copies of the `blocks` later steps remain".
template <int N>
__device__ __forceinline__ void wait_vm_blocks(int blocks) {
  switch (blocks) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * N) : "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * N) : "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * N) : "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(5 * N) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * N) : "memory"); break;
  }
}

// Cache addressing shared by the append paths and the attention kernel.
// Contiguous caches are the special case of one "page" of `rows` slots per
// sequence whose physical index is the sequence index.
struct CacheView {
  void* k_pool;
  void* v_pool;
  const int32_t* block_table;  // nullptr for contiguous
  int32_t page_rows;           // page_size, or the capacity of a contiguous cache
  int32_t max_pages;           // page-table row length
  int32_t n_kv, d_h;
};

__device__ __forceinline__ int64_t cache_page(const CacheView& c, int seq, int pos) {
  if (c.block_table == nullptr) return seq;
  return c.block_table[(int64_t)seq * c.max_pages + pos / c.page_rows];
}
// Element offset of K[seq][g][pos][0].
__device__ __forceinline__ int64_t k_offset(const CacheView& c, int64_t page, int g, int slot) {
  return ((page * c.n_kv + g) * (int64_t)c.page_rows + slot) * c.d_h;
}
// V is stored transposed in tiles of kVTile slots: tile t of a (page, head)
// holds d_h rows of kVTile elements, row i = head dim i of slots
// t * kVTile .. t * kVTile + kVTile - 1.  A 64-key block (blocks start at
// multiples of 64) is then one contiguous run of d_h * 64 elements, whatever
// the capacity or page size: the rows of a whole-page transposed layout sit a
// page apart, and at some page strides (capacity 129 * 64, say) the 128 rows
// of every block meet in the same memory channels.
constexpr int kVTile = 64;
// Element offset of V^T head dim 0 of slot `slot`; head dim i is kVTile * i
// further.
__device__ __forceinline__ int64_t v_offset(const CacheView& c, int64_t page, int g, int slot) {
  return (page * c.n_kv + g) * (int64_t)c.d_h * c.page_rows + (int64_t)(slot / kVTile) * c.d_h * kVTile +
         slot % kVTile;
}

}  // namespace dflash
