// Non-causal GQA block attention over the draft KV cache, split over the
// cached context (one workgroup per (sequence, K/V head, key chunk)), with an
// online softmax and a separate combine of the partial (max, sum, O) triples.
//
// What it computes ("DFlash KV Injection Walkthrough" Step 4.4; "DFlash源码导读二
// Qwen3DFlashAttention注意力实现全解析", the non-causal key design and sections
// 1 and 5): every query row of the block attends to every cached key, with
// scale d_h^-0.5 and no mask on full layers; a sliding layer hides keys with
// pos_q - pos_k >= window.  Query head h reads K/V head h / (n_h / n_kv)
// ("KV Cache + Speculative Decoding 面试 Cheat Sheet" 6.3).
//
// Layout of the work on gfx950:
//  * The g = n_h/n_kv query heads that share a K/V head contribute g*B query
//    rows (64 for 32/8 heads and B = 16).  They stay in VGPRs for the whole
//    chunk as the B operand of S^T = K Q^T, so each K/V byte is read from HBM
//    once and feeds all of them.
//  * Keys go through in blocks of 32 per wavefront, the four waves of a
//    workgroup taking every fourth block.  K rows load straight into the A
//    operand of 16x16x32 MFMAs (16-byte loads, 64 contiguous bytes per key per
//    instruction).  The two 16-key tiles of a block use the key order
//    tile kt, row i -> key 8*(i/4) + 4*kt + i%4, so after the S^T products each
//    lane holds the scores of 8 consecutive keys for one query row: exactly the
//    B operand of O^T = V^T P^T.
//  * V is stored key-minor in the cache, so the A operand of that product (16
//    head dims x 32 keys) is 16 contiguous bytes per lane as well.  No LDS and
//    no lane shuffles sit in the key loop; the row max needs two xor shuffles.
//  * The running max, sum and output stay per lane in the log2 domain; the
//    four waves merge through LDS at the end and the workgroup writes one
//    partial (m, l, unnormalised O) per query row.
#include "kernels.hpp"

namespace dflash {

template <typename T, int DH, int NQW, int QS>
__global__ __launch_bounds__(256, 1) void attn_split_kernel(AttnArgs a) {
  using V8 = vec8_t<T>;
  constexpr int DS = DH / 32;      // K=32 steps over the head dim
  constexpr int DT = DH / 16;      // 16-row tiles of the head dim
  constexpr int QW = NQW * 16;     // query rows held by one wave
  constexpr int NS = 4 / QS;       // block streams: waves that share query rows
  constexpr int LDO = DH + 4;      // LDS row stride of the merge buffer

  __shared__ float s_o[4][QW][LDO];
  __shared__ float s_m[4][QW];
  __shared__ float s_l[4][QW];

  const int item = blockIdx.x;
  int r = 0;
  while (r + 1 < a.R && item >= a.item_base[r + 1]) ++r;
  const int local = item - a.item_base[r];
  const int g = local / a.chunks[r];
  const int chunk = local - g * a.chunks[r];
  const int key_hi = a.key_hi[r];
  const int kbeg = (a.key_lo[r] & ~31) + chunk * a.chunk_keys;
  const int kend = min(kbeg + a.chunk_keys, key_hi);
  const int nblk = kend > kbeg ? (kend - kbeg + 31) >> 5 : 0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qg = wave % QS;        // which QW query rows this wave holds
  const int stream = wave / QS;    // which blocks it walks: stream, stream + NS, ...
  const int j16 = lane & 15, q4 = lane >> 4;
  const int valid_q = a.group * a.B;

  // queries: B operand of S^T; lane (j16, q4) holds row qg*QW + 16t + j16,
  // head dims 32s + 8q4 .. +7
  V8 qv[NQW][DS];
  const T* qbase = static_cast<const T*>(a.q_ws) + (int64_t)(r * a.n_kv + g) * a.qrows * DH;
  int qpos[NQW];
  float m_run[NQW], l_run[NQW];
  f32x4 o[NQW][DT];
#pragma unroll
  for (int t = 0; t < NQW; ++t) {
    const int qrow = qg * QW + t * 16 + j16;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qv[t][s] = qrow < valid_q ? load8(qbase + (int64_t)qrow * DH + 32 * s + 8 * q4) : zero8<T>();
    qpos[t] = a.qpos0[r] + qrow % a.B;
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) o[t][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const T* kpool = static_cast<const T*>(a.cache.k_pool);
  const T* vpool = static_cast<const T*>(a.cache.v_pool);
  const int krow_in_tile = 8 * (j16 >> 2) + (j16 & 3);   // + 4*kt

  // One 32-key block: K rows into the A operand of S^T (tile kt, row i holds
  // key 8*(i/4) + 4*kt + i%4), V^T into the A operand of O^T (16 head dims x
  // 8 consecutive keys per lane).  Keys at or beyond key_hi read as zero.
  auto fetch = [&](V8 (&kv)[2][DS], V8 (&vv)[DT], int blk) {
    const int64_t page = cache_page(a.cache, r, blk);
    const int slot = blk % a.cache.page_rows;
    const T* kb = kpool + k_offset(a.cache, page, g, slot);
    const T* vb = vpool + v_offset(a.cache, page, g, slot);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int kr = krow_in_tile + 4 * kt;
      const bool ok = blk + kr < key_hi;
#pragma unroll
      for (int s = 0; s < DS; ++s)
        kv[kt][s] = ok ? load8(kb + (int64_t)kr * DH + 32 * s + 8 * q4) : zero8<T>();
    }
    const int kk0 = blk + 8 * q4;
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      V8 v = kk0 < key_hi ? load8(vb + (int64_t)(16 * d + j16) * a.cache.page_rows + 8 * q4) : zero8<T>();
      if (kk0 + 8 > key_hi) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kk0 + e >= key_hi) v[e] = static_cast<T>(0.f);
      }
      vv[d] = v;
    }
  };

  auto process = [&](const V8 (&kv)[2][DS], const V8 (&vv)[DT], int blk) {
    f32x4 sacc[2][NQW];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int t = 0; t < NQW; ++t) {
        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DS; ++s) c = mma32(kv[kt][s], qv[t][s], c);
        sacc[kt][t] = c;
      }
    const int key0 = blk + 8 * q4;   // this lane's 8 consecutive keys
    V8 pv[NQW];
    float alpha[NQW];
    bool any_need = false;
#pragma unroll
    for (int t = 0; t < NQW; ++t) {
      f32x8 sv;
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = key0 + 4 * kt + e;
          bool vis = key < key_hi;
          if (a.window > 0) vis = vis && (qpos[t] - key < a.window);
          const float x = vis ? sacc[kt][t][e] * a.scale_log2 : -INFINITY;
          sv[4 * kt + e] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      // Lazy rescale: the reference max only moves when the block max exceeds
      // it by more than 8 (log2 units), so every p <= 256, and O is rescaled
      // only on those rare blocks (wave-uniform branch below), which keeps the
      // accumulators out of the VALU path.
      const bool need = mx > m_run[t] + 8.f;
      const float m_new = need ? mx : m_run[t];
      alpha[t] = need ? exp2f(m_run[t] - m_new) : 1.f;
      any_need |= need;
      m_run[t] = m_new;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      f32x8 p;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = exp2f(sv[e] - m_use);
        ps += p[e];
      }
      l_run[t] = l_run[t] * alpha[t] + ps;
      pv[t] = cvt8<T>(p);
    }
    if (__any(any_need)) {
#pragma unroll
      for (int t = 0; t < NQW; ++t)
#pragma unroll
        for (int d = 0; d < DT; ++d) o[t][d] *= alpha[t];
    }
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int t = 0; t < NQW; ++t) o[t][d] = mma32(vv[d], pv[t], o[t][d]);
  };

  // this wave's blocks: stream, stream + NS, ... (double-buffered)
  const int my_n = nblk > stream ? (nblk - stream + NS - 1) / NS : 0;
  constexpr int STEP = 32 * NS;
  V8 kA[2][DS], vA[DT], kB[2][DS], vB[DT];
  if (my_n > 0) fetch(kA, vA, kbeg + 32 * stream);
  for (int i = 0; i < my_n; i += 2) {
    const int blk = kbeg + 32 * stream + STEP * i;
    if (i + 1 < my_n) fetch(kB, vB, blk + STEP);
    process(kA, vA, blk);
    if (i + 1 >= my_n) break;
    if (i + 2 < my_n) fetch(kA, vA, blk + 2 * STEP);
    process(kB, vB, blk + STEP);
  }

  // merge the waves that hold the same query rows, through LDS
#pragma unroll
  for (int t = 0; t < NQW; ++t) {
    float l = l_run[t];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const int row = t * 16 + j16;
    if (q4 == 0) {
      s_m[wave][row] = m_run[t];
      s_l[wave][row] = l;
    }
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_o[wave][row][16 * d + 4 * q4 + e] = o[t][d][e];
  }
  __syncthreads();

  float* po = a.part_o + (int64_t)item * a.qrows * DH;
  const int rows_out = min(a.qrows, QS * QW);
  for (int idx = tid; idx < rows_out * DH; idx += 256) {
    const int qrow = idx / DH, d = idx - qrow * DH;
    const int gq = qrow / QW, row = qrow - gq * QW;
    float mm = -INFINITY;
#pragma unroll
    for (int st = 0; st < NS; ++st) mm = fmaxf(mm, s_m[st * QS + gq][row]);
    const float mu = mm == -INFINITY ? 0.f : mm;
    float acc = 0.f;
#pragma unroll
    for (int st = 0; st < NS; ++st) acc += exp2f(s_m[st * QS + gq][row] - mu) * s_o[st * QS + gq][row][d];
    po[idx] = acc;
  }
  if (tid < rows_out) {
    const int qrow = tid;
    const int gq = qrow / QW, row = qrow - gq * QW;
    float mm = -INFINITY;
#pragma unroll
    for (int st = 0; st < NS; ++st) mm = fmaxf(mm, s_m[st * QS + gq][row]);
    const float mu = mm == -INFINITY ? 0.f : mm;
    float l = 0.f;
#pragma unroll
    for (int st = 0; st < NS; ++st) l += exp2f(s_m[st * QS + gq][row] - mu) * s_l[st * QS + gq][row];
    float* pml = a.part_ml + (int64_t)item * 2 * a.qrows;
    pml[qrow] = mm;
    pml[a.qrows + qrow] = l;
  }
}

template <typename T>
static hipError_t launch_attn_t(const AttnArgs& a, int items, hipStream_t s) {
  const int nqt = (a.qrows + 15) / 16;
#define DFLASH_ATTN_CASE(DH_, NQT_, NQW_, QS_)                                                     \
  if (a.d_h == DH_ && nqt == NQT_) {                                                               \
    hipLaunchKernelGGL((attn_split_kernel<T, DH_, NQW_, QS_>), dim3(items), dim3(256), 0, s, a);    \
    return hipGetLastError();                                                                      \
  }
  DFLASH_ATTN_CASE(64, 1, 1, 1) DFLASH_ATTN_CASE(64, 2, 2, 1) DFLASH_ATTN_CASE(64, 3, 3, 1)
  DFLASH_ATTN_CASE(64, 4, 2, 2)
  if constexpr (sizeof(T) == 2) {
    DFLASH_ATTN_CASE(128, 1, 1, 1) DFLASH_ATTN_CASE(128, 2, 2, 1) DFLASH_ATTN_CASE(128, 3, 3, 1)
    DFLASH_ATTN_CASE(128, 4, 2, 2)
  } else {
    // fp32 operands take twice the registers: one 16-row tile per wave
    DFLASH_ATTN_CASE(128, 1, 1, 1) DFLASH_ATTN_CASE(128, 2, 1, 2) DFLASH_ATTN_CASE(128, 3, 1, 4)
    DFLASH_ATTN_CASE(128, 4, 1, 4)
  }
#undef DFLASH_ATTN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_split(int dtype, const AttnArgs& a, int items, hipStream_t s) {
  if (items == 0) return hipSuccess;
  return dtype == 1 ? launch_attn_t<bf16>(a, items, s) : launch_attn_t<float>(a, items, s);
}

// ---------------------------------------------------------------- combine
// Merges the chunk partials of one query row: m = max_c m_c,
// l = sum_c 2^(m_c - m) l_c, O = sum_c 2^(m_c - m) O_c / l, and stores O in the
// row-major [R*B][n_h*d_h] order of the attention output (head h at columns
// h*d_h .., "DFlash KV Injection Walkthrough" Step 4.5).  One wave per row.

template <typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int per_seq = a.n_kv * a.group * a.B;
  if (row >= (int64_t)a.R * per_seq) return;
  const int r = (int)(row / per_seq);
  const int rem = (int)(row - (int64_t)r * per_seq);
  const int g = rem / (a.group * a.B);
  const int qrow = rem - g * a.group * a.B;
  const int hl = qrow / a.B, b = qrow - hl * a.B;
  const int n = a.chunks[r];
  const int64_t it0 = a.item_base[r] + (int64_t)g * n;

  float mm = -INFINITY;
  for (int c = lane; c < n; c += 64) mm = fmaxf(mm, a.part_ml[(it0 + c) * 2 * a.qrows + qrow]);
  mm = wave_max(mm);
  const float mu = mm == -INFINITY ? 0.f : mm;
  float lsum = 0.f;
  for (int c = lane; c < n; c += 64) {
    const float* pml = a.part_ml + (it0 + c) * 2 * a.qrows;
    lsum += exp2f(pml[qrow] - mu) * pml[a.qrows + qrow];
  }
  lsum = wave_sum(lsum);
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;

  const int h = g * a.group + hl;
  T* dst = static_cast<T*>(a.attn) + ((int64_t)r * a.B + b) * (a.n_kv * a.group * a.d_h) + h * a.d_h;
  for (int d = lane; d < a.d_h; d += 64) {
    float acc = 0.f;
    for (int c = 0; c < n; ++c) {
      const float w = exp2f(a.part_ml[(it0 + c) * 2 * a.qrows + qrow] - mu);
      acc += w * a.part_o[((it0 + c) * a.qrows + qrow) * a.d_h + d];
    }
    dst[d] = from_f32<T>(acc * inv);
  }
}

hipError_t launch_attn_combine(int dtype, const CombineArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.R * a.n_kv * a.group * a.B;
  if (rows == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (dtype == 1)
    hipLaunchKernelGGL(attn_combine_kernel<bf16>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_combine_kernel<float>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
