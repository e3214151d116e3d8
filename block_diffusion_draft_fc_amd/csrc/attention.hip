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
// The kernels (all one workgroup per (sequence, K/V head, key chunk); the g =
// n_h/n_kv query heads that share a K/V head contribute g*B query rows - 64
// for 32/8 heads and B = 16 - which stay resident for the whole chunk, so each
// K/V byte is read from HBM once and feeds all of them):
//  * attn_ring64_kernel (bf16, four 16-row query tiles: the layer shapes of
//    the workloads): 64-key blocks through a ring of LDS stages filled by
//    direct-to-LDS copies, one query tile per wave; two wave groups on
//    alternate blocks where one workgroup holds a CU.  Its own comment below
//    gives the layout.
//  * attn_lds_kernel (bf16, one to three query tiles): 32-key blocks through
//    per-wave LDS rings.
//  * attn_split_kernel (fp32 layers): K and V^T rows loaded straight into
//    MFMA operands (16-byte loads), the four waves of a workgroup on every
//    fourth 32-key block, merged through LDS at the end.
// Every kernel keeps the running max, sum and output per lane in the log2
// domain and writes one partial (m, l, unnormalised O) per query row and item;
// attn_combine_kernel merges the partials of a row.
#include "attn_merge.hpp"

namespace dflash {

// ---------------------------------------------------------------- fp32: register-fed blocks
// Keys go through in blocks of 32 per wavefront, the four waves of a
// workgroup taking every fourth block.  K rows load straight into the A
// operand of 16x16x32 MFMAs (16-byte loads, 64 contiguous bytes per key per
// instruction).  The two 16-key tiles of a block use the key order
// tile kt, row i -> key 8*(i/4) + 4*kt + i%4, so after the S^T = K Q^T
// products each lane holds the scores of 8 consecutive keys for one query row:
// exactly the B operand of O^T = V^T P^T.  V is stored transposed in the cache
// (tiles of 64 slots, head dim-major within a tile), so the A operand of that
// product (16 head dims x 32 keys) is 16 contiguous bytes per lane as well.
// No LDS sits in the key loop; the four waves merge through LDS at the end.
template <typename T, int DH, int NQW, int QS>
__global__ __launch_bounds__(256, 1) void attn_split_kernel(AttnArgs a) {
  using V8 = vec8_t<T>;
  constexpr int DS = DH / 32;      // K=32 steps over the head dim
  constexpr int DT = DH / 16;      // 16-row tiles of the head dim
  constexpr int QW = NQW * 16;     // query rows held by one wave
  constexpr int NS = 4 / QS;       // block streams: waves that share query rows
  constexpr int LDO = DH + 4;      // LDS row stride of the merge buffer

  constexpr int QROWS = QS * QW;   // query rows staged for the workgroup
  constexpr int LDQ = DH + 8;      // LDS row stride of the queries: 16 rows of a
                                   // 16-byte read land on distinct banks

  __shared__ __align__(16) T s_q[QROWS * LDQ];
  __shared__ int32_t s_page[kAttnMaxChunkPages];
  __shared__ float s_o[4][QW][LDO];
  __shared__ float s_m[4][QW];
  __shared__ float s_l[4][QW];

  const int item = blockIdx.x;
  int r = 0;
  while (r + 1 < a.R && item >= a.item_base[r + 1]) ++r;
  const int local = item - a.item_base[r];
  const int g = local / a.chunks[r];
  const int chunk = local - g * a.chunks[r];
  int key_lo, key_hi, qpos0;
  attn_seq_keys(a, r, key_lo, key_hi, qpos0);
  const int kbeg = (key_lo & ~63) + chunk * a.chunk_keys;
  const int kend = min(kbeg + a.chunk_keys, key_hi);
  const int nblk = kend > kbeg ? (kend - kbeg + 31) >> 5 : 0;

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform across the wave; saying so keeps the block loop
  // scalar (a loop the compiler thinks divergent gets exec masking and a
  // full wait for every load at its header)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wave % QS;        // which QW query rows this wave holds
  const int stream = wave / QS;    // which blocks it walks: stream, stream + NS, ...
  const int j16 = lane & 15, q4 = lane >> 4;
  const int valid_q = a.group * a.B;

  // The workgroup's query rows go to LDS (rows past g*B as zeros); every wave
  // reads its B operands of S^T from there, lane (j16, q4) taking row
  // qg*QW + 16t + j16, head dims 32s + 8q4 .. +7.  Their global loads are
  // issued before any K/V load, so waiting for them never waits for K/V.
  constexpr int QV8 = QROWS * DH / 8;
  constexpr int QPT = (QV8 + 255) / 256;
  const T* qbase = static_cast<const T*>(a.q_ws) + (int64_t)(r * a.n_kv + g) * a.qrows * DH;
  V8 qstage[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int idx = tid + 256 * i;
    const int row = idx / (DH / 8);
    qstage[i] = (idx < QV8 && row < valid_q) ? load8(qbase + (int64_t)idx * 8) : zero8<T>();
  }
  // keys visible to query row q are [vlo_q, key_hi): vlo_q = pos_q - window + 1
  // on sliding layers, no lower bound on full ones
  int vlo[NQW];
  float m_run[NQW], l_run[NQW];
  f32x4 o[NQW][DT];
#pragma unroll
  for (int t = 0; t < NQW; ++t) {
    const int qrow = qg * QW + t * 16 + j16;
    vlo[t] = a.window > 0 ? qpos0 + qrow % a.B - a.window + 1 : INT_MIN;
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) o[t][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const T* qlds = s_q + (qg * QW + j16) * LDQ + 8 * q4;
  // the largest lower bound among the rows (the last block row's)
  const int vis_lo_max = qpos0 + a.B - 1 - a.window + 1;

  // physical pages of the chunk, read once: fetches then take their page from
  // LDS and never wait on a global load (vector loads complete in order, so a
  // dependent page-table load would also wait for every K/V load in flight)
  const int pg0 = kbeg / a.cache.page_rows;
  const int npg = nblk > 0 ? (kend - 1) / a.cache.page_rows - pg0 + 1 : 0;
  for (int i = tid; i < npg; i += 256) s_page[i] = (int32_t)cache_page(a.cache, r, (pg0 + i) * a.cache.page_rows);

  const T* kpool = static_cast<const T*>(a.cache.k_pool);
  const T* vpool = static_cast<const T*>(a.cache.v_pool);
  const int krow_in_tile = 8 * (j16 >> 2) + (j16 & 3);   // + 4*kt

  // One 32-key block: K rows into the A operand of S^T (tile kt, row i holds
  // key 8*(i/4) + 4*kt + i%4), V^T into the A operand of O^T (16 head dims x
  // 8 consecutive keys per lane).  The loads are unconditional: a block starts
  // at a multiple of 32 below key_hi and never crosses a page (pages and
  // contiguous capacities are multiples of 64 rows), so rows at or beyond
  // key_hi are stale cache rows inside the allocation.  Their scores are
  // masked and their V entries zeroed in `process`, so no load result is
  // touched here and the next block's loads stay in flight.
  auto fetch = [&](V8 (&kv)[2][DS], V8 (&vv)[DT], int blk) {
    const int64_t page = s_page[blk / a.cache.page_rows - pg0];
    const int slot = blk % a.cache.page_rows;
    const T* kb = kpool + k_offset(a.cache, page, g, slot);
    const T* vb = vpool + v_offset(a.cache, page, g, slot);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int kr = krow_in_tile + 4 * kt;
#pragma unroll
      for (int s = 0; s < DS; ++s) kv[kt][s] = load8(kb + (int64_t)kr * DH + 32 * s + 8 * q4);
    }
#pragma unroll
    for (int d = 0; d < DT; ++d) vv[d] = load8(vb + (16 * d + j16) * kVTile + 8 * q4);
    // keep the loads here: without the barrier the compiler sinks them to
    // their first use, which leaves no block in flight while another computes
    asm volatile("" ::: "memory");
  };

  auto process = [&](const V8 (&kv)[2][DS], V8 (&vv)[DT], int blk) {
    // stale rows past the end of the cache may hold any bits: zero their V
    // entries so that p = 0 cannot meet an Inf or NaN (wave-uniform branch,
    // taken on the last block of a sequence only)
    if (blk + 32 > key_hi) {
      const int kk0 = blk + 8 * q4;
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kk0 + e >= key_hi) vv[d][e] = static_cast<T>(0.f);
    }
    // the queries are re-read from LDS for every block: the empty asm with a
    // memory clobber keeps the compiler from hoisting them into registers
    asm volatile("" ::: "memory");
    const int key0 = blk + 8 * q4;   // this lane's 8 consecutive keys
    // every key of the block is visible to every query row of the workgroup
    // (the usual case): no per-element masking
    const bool all_vis = blk + 32 <= key_hi && (a.window <= 0 || blk >= vis_lo_max);
    // one 16-row query tile at a time: scores, softmax update, then P V
#pragma unroll
    for (int t = 0; t < NQW; ++t) {
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const V8 q = *reinterpret_cast<const V8*>(qlds + t * 16 * LDQ + 32 * s);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sacc[kt] = mma32(kv[kt][s], q, sacc[kt]);
      }
      f32x8 sv;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * kt + e] = sacc[kt][e] * a.scale_log2;
      if (!all_vis) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = key0 + e;
          const bool vis = (key >= vlo[t]) & (key < key_hi);
          sv[e] = vis ? sv[e] : -INFINITY;
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = max_xor32(max_xor16(mx));
      // Lazy rescale: the reference max only moves when the block max exceeds
      // it by more than 8 (log2 units), so every p <= 256, and O is rescaled
      // only on those rare blocks (wave-uniform branch), which keeps the
      // accumulators out of the VALU path.
      const bool need = mx > m_run[t] + 8.f;
      const float m_new = need ? mx : m_run[t];
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run[t] - m_new) : 1.f;
      m_run[t] = m_new;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      f32x8 p;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // raw v_exp_f32: results below the normal range flush to zero, which
        // only drops weights under 2^-126 of the row maximum
        p[e] = __builtin_amdgcn_exp2f(sv[e] - m_use);
        ps += p[e];
      }
      l_run[t] = l_run[t] * alpha + ps;
      const V8 pv = cvt8<T>(p);
      if (__any(need)) {
#pragma unroll
        for (int d = 0; d < DT; ++d) o[t][d] *= alpha;
      }
#pragma unroll
      for (int d = 0; d < DT; ++d) o[t][d] = mma32(vv[d], pv, o[t][d]);
    }
  };

  // this wave's blocks: stream, stream + NS, ... (double-buffered).  Every
  // prefetch in the loop is unconditional (a prefetch past the wave's last
  // block re-reads that block, an L2 hit): with a conditional prefetch the
  // wait-count pass would have to assume it missing and wait for it too.
  const int my_n = nblk > stream ? (nblk - stream + NS - 1) / NS : 0;
  constexpr int STEP = 32 * NS;
  V8 kA[2][DS], vA[DT], kB[2][DS], vB[DT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int idx = tid + 256 * i;
    if (idx < QV8) {
      const int row = idx / (DH / 8), c = idx - row * (DH / 8);
      *reinterpret_cast<V8*>(s_q + row * LDQ + 8 * c) = qstage[i];
    }
  }
  __syncthreads();
  if (my_n > 0) {
    const int first = kbeg + 32 * stream;
    const int last = first + STEP * (my_n - 1);
    fetch(kA, vA, first);
    for (int i = 0;; i += 2) {
      const int blk = first + STEP * i;
      fetch(kB, vB, min(blk + STEP, last));
      process(kA, vA, blk);
      if (i + 1 >= my_n) break;
      fetch(kA, vA, min(blk + 2 * STEP, last));
      process(kB, vB, blk + STEP);
      if (i + 2 >= my_n) break;
    }
  }

  // merge the waves that hold the same query rows, through LDS
#pragma unroll
  for (int t = 0; t < NQW; ++t) {
    float l = l_run[t];
    l = sum_xor32(sum_xor16(l));
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

  T* po = static_cast<T*>(a.part_o) + (int64_t)item * a.qrows * DH;
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
    po[idx] = from_f32<T>(acc);
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

// ---------------------------------------------------------------- bf16: LDS-streamed keys
// The bf16 path streams K/V through LDS instead of registers.  Each wave owns
// two 32-key stages of a ring in LDS and fills them with direct-to-LDS loads
// (global_load_lds_dwordx4, 16 bytes per lane), so the block in flight costs
// no registers; the wave's queries (all g*B rows of its K/V head) stay in
// VGPRs and its output accumulators in AGPRs.
//
// A stage holds the block in MFMA operand order: for K, one 1 KB slab per
// (key tile kt, head-dim step s) whose lane l entry is the 16 bytes that lane l
// feeds to the S^T product; for V^T, one slab per 16-dim tile d.  Reading an
// operand is one ds_read_b128 at slab + 16 * lane (consecutive lanes,
// consecutive 16-byte words: no bank conflicts), and each K/V operand is read
// once per block and reused by every query tile.
//
// The compiler does not order LDS reads after direct-to-LDS loads, so the
// waits are explicit: vector memory operations of a wave complete in order
// and the loop issues nothing else, so "all but the newest block's loads
// done" is s_waitcnt vmcnt(loads per block).  A wave reads only the stages it
// filled itself, so no barrier is needed inside the loop.

template <int DH, int NQT>
__global__ __launch_bounds__(256, 1) void attn_lds_kernel(AttnArgs a) {
  using V8 = bf16x8;
  constexpr int DS = DH / 32;                 // K=32 steps over the head dim
  constexpr int DT = DH / 16;                 // 16-dim tiles of the head dim
  constexpr int QROWS = NQT * 16;
  constexpr int KSLABS = 2 * DS, VSLABS = DT;
  constexpr int LOADS = KSLABS + VSLABS;      // direct-to-LDS loads per block and wave
  constexpr int STAGE = LOADS * 1024;
  constexpr int RING_HALF = 4 * STAGE;        // one stage of each of the four waves
  constexpr int LDO = DH + 4;                 // merge buffer row stride (floats)
  constexpr int MERGE_HALF = 2 * QROWS * LDO * 4;   // two waves' accumulators
  constexpr int HALF = RING_HALF > MERGE_HALF ? RING_HALF : MERGE_HALF;

  // the two ring stages are separate arrays, so that alias analysis can tell a
  // read of one stage from a load in flight into the other
  __shared__ __align__(16) unsigned char lds0[HALF];
  __shared__ __align__(16) unsigned char lds1[HALF];
  // queries in operand order: slab (t, s) holds, at 16 * lane, the 16 bytes lane
  // (j16, q4) feeds to the S^T product: row 16t + j16, head dims 32s + 8q4 ..
  __shared__ __align__(16) unsigned char s_q[NQT * DS * 1024];
  __shared__ float s_ml[2][4][QROWS];
  __shared__ int32_t s_page[kAttnMaxChunkPages];

  const int item = blockIdx.x;
  int r = 0;
  while (r + 1 < a.R && item >= a.item_base[r + 1]) ++r;
  const int local = item - a.item_base[r];
  const int g = local / a.chunks[r];
  const int chunk = local - g * a.chunks[r];
  int key_lo, key_hi, qpos0;
  attn_seq_keys(a, r, key_lo, key_hi, qpos0);
  const int kbeg = (key_lo & ~63) + chunk * a.chunk_keys;
  const int kend = min(kbeg + a.chunk_keys, key_hi);
  const int nblk = kend > kbeg ? (kend - kbeg + 31) >> 5 : 0;

  const int tid = threadIdx.x, lane = tid & 63;
  // uniform across the wave; saying so keeps the block loop scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, q4 = lane >> 4;
  const int valid_q = a.group * a.B;

  // queries of the K/V head (rows past g*B as zeros), staged to s_q below
  const bf16* qbase = static_cast<const bf16*>(a.q_ws) + (int64_t)(r * a.n_kv + g) * a.qrows * DH;
  constexpr int QSLOTS = NQT * DS * 64;       // 16-byte slots of s_q
  constexpr int QPT = (QSLOTS + 255) / 256;   // per thread
  V8 qstage[QPT];
  int vlo[NQT];
  float m_run[NQT], l_run[NQT];
  f32x4 o[NQT][DT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    const int qrow = t * 16 + j16;
    // keys visible to the row: [vlo, key_hi), vlo = pos - window + 1 on sliding layers
    vlo[t] = a.window > 0 ? qpos0 + qrow % a.B - a.window + 1 : INT_MIN;
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) o[t][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int vis_lo_max = qpos0 + a.B - a.window;   // largest row bound (sliding layers)

  // physical pages of the chunk, read once so that no load of the block loop
  // depends on another global load
  const int pg0 = kbeg / a.cache.page_rows;
  // a contiguous or ring cache holds sequence r at page r: no page list, and
  // no barrier before the first copies go out
  const bool paged = a.cache.block_table != nullptr;
  if (paged) {
    const int npg = nblk > 0 ? (kend - 1) / a.cache.page_rows - pg0 + 1 : 0;
    for (int i = tid; i < npg; i += 256) s_page[i] = (int32_t)cache_page(a.cache, r, (pg0 + i) * a.cache.page_rows);
    __syncthreads();
  }

  const bf16* kpool = static_cast<const bf16*>(a.cache.k_pool);
  const bf16* vpool = static_cast<const bf16*>(a.cache.v_pool);
  const int krow = 8 * (j16 >> 2) + (j16 & 3);   // + 4*kt: key of A-operand row j16
  unsigned char* ring0 = lds0 + wave * STAGE;
  unsigned char* ring1 = lds1 + wave * STAGE;

  // direct-to-LDS loads of one 32-key block into stage st.  Blocks start at a
  // multiple of 32 below key_hi and never cross a page (pages and contiguous
  // capacities are multiples of 64 rows): rows past key_hi are stale rows
  // inside the allocation, masked below.
  auto issue = [&](int blk, int st) {
    const int64_t page = paged ? (int64_t)s_page[blk / a.cache.page_rows - pg0] : (int64_t)r;
    const int slot = blk % a.cache.page_rows;
    const bf16* kb = kpool + k_offset(a.cache, page, g, slot);
    const bf16* vb = vpool + v_offset(a.cache, page, g, slot);
    unsigned char* sb = st ? ring1 : ring0;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < DS; ++s)
        __builtin_amdgcn_global_load_lds(kb + (int64_t)(krow + 4 * kt) * DH + 32 * s + 8 * q4,
                                         sb + (kt * DS + s) * 1024, 16, 0, 0);
#pragma unroll
    for (int d = 0; d < DT; ++d)
      __builtin_amdgcn_global_load_lds(vb + (16 * d + j16) * kVTile + 8 * q4,
                                       sb + (KSLABS + d) * 1024, 16, 0, 0);
  };

  // Fast path for one block: every row's reference maximum m_run stays where
  // it was set (by the row's first visible key), weights exp2(s - m_run) may
  // exceed 1, and no VALU instruction touches the accumulators - which lets
  // them live in AGPRs through the loop.  Returns false, having accumulated
  // nothing, if some score exceeds its row's reference by more than 64
  // (weights up to 2^64 keep every sum far from the fp32 range); the block is
  // then redone by `process`, which rescales.
  auto process_fast = [&](int blk, int st) -> bool {
    asm volatile("" ::: "memory");
    const unsigned char* sb = (st ? ring1 : ring0) + 16 * lane;
    const unsigned char* qb = s_q + 16 * lane;
    V8 kv[2][DS], vv[DT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < DS; ++s) kv[kt][s] = *reinterpret_cast<const V8*>(sb + (kt * DS + s) * 1024);
#pragma unroll
    for (int d = 0; d < DT; ++d) vv[d] = *reinterpret_cast<const V8*>(sb + (KSLABS + d) * 1024);
    const int key0 = blk + 8 * q4;
    if (blk + 32 > key_hi) {
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (key0 + e >= key_hi) vv[d][e] = static_cast<bf16>(0.f);
    }
    const bool all_vis = blk + 32 <= key_hi && (a.window <= 0 || blk >= vis_lo_max);
    f32x8 sv[NQT];
    bool over = false;
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const V8 q = *reinterpret_cast<const V8*>(qb + (t * DS + s) * 1024);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sacc[kt] = mma32(kv[kt][s], q, sacc[kt]);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[t][4 * kt + e] = sacc[kt][e] * a.scale_log2;
      if (!all_vis) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = key0 + e;
          sv[t][e] = ((key >= vlo[t]) & (key < key_hi)) ? sv[t][e] : -INFINITY;
        }
      }
      float mx = sv[t][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[t][e]);
      mx = max_xor32(max_xor16(mx));
      // a row's first visible key sets its reference (its sums are still zero)
      if (m_run[t] == -INFINITY) m_run[t] = mx;
      over |= mx > m_run[t] + 64.f;
    }
    if (__any(over)) return false;
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      const float m_use = m_run[t] == -INFINITY ? 0.f : m_run[t];
      f32x8 p;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(sv[t][e] - m_use);
        ps += p[e];
      }
      l_run[t] += ps;
      const V8 pv = cvt8<bf16>(p);
#pragma unroll
      for (int d = 0; d < DT; ++d) o[t][d] = mma32(vv[d], pv, o[t][d]);
    }
    return true;
  };

  // General path for one block: online softmax with a lazily moved maximum.
  auto process = [&](int blk, int st) {
    asm volatile("" ::: "memory");
    const unsigned char* sb = (st ? ring1 : ring0) + 16 * lane;
    const unsigned char* qb = s_q + 16 * lane;
    V8 kv[2][DS], vv[DT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < DS; ++s) kv[kt][s] = *reinterpret_cast<const V8*>(sb + (kt * DS + s) * 1024);
#pragma unroll
    for (int d = 0; d < DT; ++d) vv[d] = *reinterpret_cast<const V8*>(sb + (KSLABS + d) * 1024);
    const int key0 = blk + 8 * q4;   // this lane's 8 consecutive keys
    // stale rows past the end of the cache may hold any bits: zero their V
    // entries so that p = 0 cannot meet an Inf or NaN (last block only)
    if (blk + 32 > key_hi) {
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (key0 + e >= key_hi) vv[d][e] = static_cast<bf16>(0.f);
    }
    // every key of the block visible to every row of the workgroup (the usual
    // case): no per-element masking
    const bool all_vis = blk + 32 <= key_hi && (a.window <= 0 || blk >= vis_lo_max);
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const V8 q = *reinterpret_cast<const V8*>(qb + (t * DS + s) * 1024);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sacc[kt] = mma32(kv[kt][s], q, sacc[kt]);
      }
      // lane holds the scores of keys key0 .. key0+7 for row 16t + j16
      f32x8 sv;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * kt + e] = sacc[kt][e] * a.scale_log2;
      if (!all_vis) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = key0 + e;
          sv[e] = ((key >= vlo[t]) & (key < key_hi)) ? sv[e] : -INFINITY;
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = max_xor32(max_xor16(mx));
      // Lazy rescale: the reference max only moves when the block max exceeds
      // it by more than 8 (log2 units), so every p <= 256 and O is rescaled on
      // those rare blocks only (wave-uniform branch).
      const bool need = mx > m_run[t] + 8.f;
      const float m_new = need ? mx : m_run[t];
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run[t] - m_new) : 1.f;
      m_run[t] = m_new;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      f32x8 p;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // raw v_exp_f32: results below the normal range flush to zero, which
        // only drops weights under 2^-126 of the row maximum
        p[e] = __builtin_amdgcn_exp2f(sv[e] - m_use);
        ps += p[e];
      }
      l_run[t] = l_run[t] * alpha + ps;
      const V8 pv = cvt8<bf16>(p);
      if (__any(need)) {
#pragma unroll
        for (int d = 0; d < DT; ++d) o[t][d] *= alpha;
      }
#pragma unroll
      for (int d = 0; d < DT; ++d) o[t][d] = mma32(vv[d], pv, o[t][d]);
    }
  };

  // this wave's blocks: wave, wave + 4, ...; block i lives in stage i % 2.
  // Block 0's loads go out first, then the query loads, then block 1's: the
  // wait before the queries are stored covers block 0 as well and leaves
  // block 1 in flight.
  const int my_n = nblk > wave ? (nblk - wave + 3) / 4 : 0;
  const int first = kbeg + 32 * wave;
  if (my_n > 0) issue(first, 0);
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int idx = tid + 256 * i;                 // slot: slab idx / 64, lane idx % 64
    const int slab = idx >> 6, L = idx & 63;
    const int row = 16 * (slab / DS) + (L & 15);
    const int col = 32 * (slab % DS) + 8 * (L >> 4);
    qstage[i] = (idx < QSLOTS && row < valid_q) ? load8(qbase + (int64_t)row * DH + col) : zero8<bf16>();
  }
  if (my_n > 1) issue(first + 128, 1);
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int idx = tid + 256 * i;
    if (idx < QSLOTS) *reinterpret_cast<V8*>(s_q + 16 * idx) = qstage[i];
  }
  __syncthreads();
  int i = 0;
  for (; i < my_n; ++i) {
    // outstanding loads: block i and, if it exists, block i+1, issued after it
    if (i + 1 < my_n)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!process_fast(first + 128 * i, i & 1)) break;
    if (i + 2 < my_n) {
      // every LDS read of this stage has returned before it is refilled
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(first + 128 * (i + 2), i & 1);
    }
  }
  // a score far above its row's reference: the rest goes through the
  // rescaling path, starting with the block the fast path gave back
  for (; i < my_n; ++i) {
    if (i + 1 < my_n)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    process(first + 128 * i, i & 1);
    if (i + 2 < my_n) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(first + 128 * (i + 2), i & 1);
    }
  }

  // merge the four waves' (m, l, O) through LDS, which the ring gives up now:
  // every wave rescales its rows to the workgroup maximum (one exponential per
  // row), then the scaled accumulators are summed with 16-byte LDS reads
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // accumulators of waves 0-1 in the first array, 2-3 in the second:
  // wave w's row q at s_ow(w) + q * LDO
  auto s_ow = [&](int w) {
    return reinterpret_cast<float*>(w < 2 ? lds0 : lds1) + (w & 1) * QROWS * LDO;
  };
  float* s_m = &s_ml[0][0][0];                                // [4][QROWS]
  float* s_l = &s_ml[1][0][0];                                // [4][QROWS]
  if (q4 == 0) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) s_m[wave * QROWS + t * 16 + j16] = m_run[t];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    const int row = t * 16 + j16;
    float mm = s_m[row];
#pragma unroll
    for (int w = 1; w < 4; ++w) mm = fmaxf(mm, s_m[w * QROWS + row]);
    const float f = m_run[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[t] - mm);
    float l = l_run[t];
    l = sum_xor32(sum_xor16(l));
    if (q4 == 0) s_l[wave * QROWS + row] = l * f;
#pragma unroll
    for (int d = 0; d < DT; ++d)
      *reinterpret_cast<f32x4*>(s_ow(wave) + row * LDO + 16 * d + 4 * q4) = o[t][d] * f;
  }
  __syncthreads();

  bf16* po = static_cast<bf16*>(a.part_o) + (int64_t)item * a.qrows * DH;
  const int rows_out = min(a.qrows, QROWS);
  constexpr int C4 = DH / 4;
  for (int idx = tid; idx < rows_out * C4; idx += 256) {
    const int row = idx / C4, c = idx - row * C4;
    f32x4 acc = *reinterpret_cast<const f32x4*>(s_ow(0) + row * LDO + 4 * c);
#pragma unroll
    for (int w = 1; w < 4; ++w) acc += *reinterpret_cast<const f32x4*>(s_ow(w) + row * LDO + 4 * c);
    store4(po + (int64_t)row * DH + 4 * c, acc);
  }
  if (tid < rows_out) {
    const int row = tid;
    float mm = s_m[row];
#pragma unroll
    for (int w = 1; w < 4; ++w) mm = fmaxf(mm, s_m[w * QROWS + row]);
    float* pml = a.part_ml + (int64_t)item * 2 * a.qrows;
    pml[row] = mm;
    pml[a.qrows + row] = s_l[row] + s_l[QROWS + row] + s_l[2 * QROWS + row] + s_l[3 * QROWS + row];
  }
}

// Workgroups of this file's kernels whose in-launch merge wait timed out.
__device__ uint32_t g_attn_sync_timeouts = 0;

hipError_t attn_sync_timeouts(uint32_t* count) {
  return hipMemcpyFromSymbol(count, HIP_SYMBOL(g_attn_sync_timeouts), sizeof(uint32_t), 0, hipMemcpyDeviceToHost);
}

// ---------------------------------------------------------------- bf16: shared ring of 64-key blocks
// For work items with four 16-row query tiles (g*B of 49..64 rows): wave t
// owns query tile t, and the four waves share one ring of NST 64-key blocks in
// LDS.  Each block is brought in by all four waves together (a quarter of its
// 1 KB copies each, direct-to-LDS) and read by each wave for its own tile, so
// every wave holds the online-softmax state of 16 rows only and writes its
// rows' partials itself.  One barrier per block, after which the block has
// landed for every wave and the previous block's stage is free to refill.
// 64-key blocks give each wave's dependency chain (K reads -> S -> softmax
// -> PV) 64 keys per barrier, and V^T arrives in whole 128-byte lines (64
// keys of one head dim).  A stage holds
//   K: the block's 64 key rows in key order (2 DH bytes each), the 16-byte
//      chunk c of key j at position c ^ kswz(j) within its row - each copy
//      moves whole rows (1 KB of consecutive keys, contiguous in the cache),
//      picking per lane the chunk its slot holds; an operand read (16 keys,
//      one chunk) then covers all banks;
//   V^T: one 128-byte row per head dim R (the block's 64 keys), in 16-byte
//      chunks of 8 keys, chunk c at position c ^ (R % 8) ^ ((R / 8) % 2) - each
//      copy moves 8 whole rows and picks, per lane, the chunk its slot holds;
//      a fragment read (16 consecutive rows, one chunk) then covers all banks.
// Block starts are multiples of 64, so a block never crosses a page.
// NST stages keep NST - 1 blocks in flight while the waves compute on one.
// The queries travel as direct copies too, ahead of the first blocks', into
// the last stage (free until the loop's first refill of it): their latency
// overlaps the blocks' instead of preceding it.
// NG = 2 doubles the workgroup to two groups of four waves, wave w taking
// query tile w % 4 in group w / 4; group g processes blocks g, g + 2, ..., so
// an item's chain of dependent blocks is half as long, and at the end group 1
// hands its (m, l, O) to group 0 through LDS for an exact merge.  The ring
// then holds the two blocks in work plus NST - 2 in flight.
// MERGE: 0 = partials for the combine launch; 1 = the split merged in the
// launch, item x on K/V head x % n_kv; 2 = the same with a head's items on
// consecutive workgroups (the diagnostic order that spreads a head over XCDs).
template <int DH, int NST, int NG = 1, int MERGE = 0>
__global__ __launch_bounds__(256 * NG, 1) void attn_ring64_kernel(AttnArgs a) {
  using V8 = bf16x8;
  static_assert(NST >= 2 && NST <= 8, "blocks in flight are counted by wait_vm_blocks (up to 6 after the current)");
  static_assert((NG == 1 || NG == 2) && NST >= 2 * NG, "a step's blocks are issued by the end of the step before");
  constexpr int DS = DH / 32;                 // K=32 steps over the head dim
  constexpr int DT = DH / 16;                 // 16-dim tiles of the head dim
  constexpr int KSLABS = DH / 8;              // 1 KB copies of 1024 / (2 DH) key rows
  constexpr int CK = DH / 8;                  // 16-byte chunks per key row
  static_assert(DH == 64 || DH == 128, "key-row swizzle defined for d_h 64 and 128");
  constexpr int VROWS = DH / 8;               // 1 KB copies of 8 V^T rows
  constexpr int COPIES = KSLABS + VROWS;
  constexpr int PER_WAVE = COPIES / (4 * NG);
  static_assert(PER_WAVE * 4 * NG == COPIES, "copies split evenly over the waves");
  constexpr int STAGE = COPIES * 1024;
  static_assert(MERGE == 0 || NG == 2, "the in-launch merge runs on the one-workgroup-per-CU plans");
  __shared__ __align__(16) unsigned char ring[NST * STAGE];
  __shared__ int32_t s_page[kAttnMaxChunkPages];

  const int item = blockIdx.x;
  int r = 0, g, chunk;
  int key_lo, key_hi, qpos0;
  if constexpr (MERGE != 0) {
    // one sequence of a host-driven round: item x is chunk x / n_kv of K/V
    // head x % n_kv.  Every argument the start needs sits at a fixed offset
    // and nothing here branches on an argument, so they are read in one
    // batch (a chain of dependent argument reads, each an L2 round trip on
    // first touch, held back the first K/V copies by ~2 us).
    if constexpr (MERGE == 2) {
      g = item / a.seq0[3];
      chunk = item - g * a.seq0[3];
    } else {
      g = item % a.n_kv;
      chunk = item / a.n_kv;
    }
    key_lo = a.seq0[0];
    key_hi = a.seq0[1];
    qpos0 = a.seq0[2];
    // the cache's head count and head dim in the same batch (the compiler
    // would read them where the first addresses are formed, a wait later)
    asm volatile("" ::"s"(a.cache.n_kv), "s"(a.cache.d_h));
  } else {
    while (r + 1 < a.R && item >= a.item_base[r + 1]) ++r;
    const int local = item - a.item_base[r];
    g = local / a.chunks[r];
    chunk = local - g * a.chunks[r];
    attn_seq_keys(a, r, key_lo, key_hi, qpos0);
  }
  // the partial's slot: items of one (sequence, head) in chunk order
  const int pitem = MERGE != 0 ? g * a.seq0[3] + chunk : a.item_base[r] + g * a.chunks[r] + chunk;
  const int kbeg = (key_lo & ~63) + chunk * a.chunk_keys;
  const int kend = min(kbeg + a.chunk_keys, key_hi);
  const int nblk = kend > kbeg ? (kend - kbeg + 63) >> 6 : 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qt = wave & 3, grp = wave >> 2;   // query tile, wave group
  const int j16 = lane & 15, q4 = lane >> 4;
  const int valid_q = a.group * a.B;

  const int row = 16 * qt + j16;
  const bf16* qbase = static_cast<const bf16*>(a.q_ws) + (int64_t)(r * a.n_kv + g) * a.qrows * DH;
  const int vlo = a.window > 0 ? qpos0 + row % a.B - a.window + 1 : INT_MIN;
  const int vis_lo_max = qpos0 + a.B - a.window;   // largest row bound (sliding layers)
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int pg0 = kbeg / a.cache.page_rows;
  // a contiguous or ring cache holds sequence r at page r: no page list, and
  // no barrier before the first copies go out
  const bool paged = a.cache.block_table != nullptr;
  if (paged) {
    const int npg = nblk > 0 ? (kend - 1) / a.cache.page_rows - pg0 + 1 : 0;
    for (int i = tid; i < npg; i += 256) s_page[i] = (int32_t)cache_page(a.cache, r, (pg0 + i) * a.cache.page_rows);
    __syncthreads();
  }
  // The queries go to LDS by direct copies issued before the first blocks',
  // so the wait for block 0 covers them too and their latency overlaps the
  // blocks' (a register load would be waited for on its own: the compiler
  // cannot see the block copies, so it would wait for everything in flight
  // at the first use, or on every block if that use sits in the loop).  The
  // workspace holds qrows >= 16 * 4 rows, so every copy is in bounds.  They
  // land in the last stage, which the first copies into it (issued after the
  // first barrier of the loop) find read: wave w's operand-order slabs
  // (wave w, s) hold, at 16 * lane, row 16 (w % 4) + j16, head dims 32 s + 8 q4 ..
  static_assert(4 * NG * DS * 1024 <= STAGE, "the queries fit one stage (one copy per wave)");
  unsigned char* my_q = ring + (NST - 1) * STAGE + wave * DS * 1024;
#pragma unroll
  for (int s = 0; s < DS; ++s) lds_copy16(qbase + (int64_t)row * DH + 32 * s + 8 * q4, my_q + s * 1024);
  V8 qv[DS];

  const bf16* kpool = static_cast<const bf16*>(a.cache.k_pool);
  const bf16* vpool = static_cast<const bf16*>(a.cache.v_pool);
  const int krow = 8 * (j16 >> 2) + (j16 & 3);   // + 4 kt + 32 hh: key of A-operand row j16
  // chunk swizzle of key row j: a function of the key bits that krow varies
  // (0, 1, 3, 4), distinct over an operand read's 16 keys in every 256 bytes
  auto kswz = [](int j) { return DH == 128 ? (j & 3) | ((j >> 1) & 12) : ((j >> 1) & 1) | ((j >> 2) & 6); };
  // K copy i: lane l fills key i * (64 / CK) + l / CK, slot l % CK
  const int kkey_in = lane / CK, kslot = lane % CK;
  // K operand reads: key 32 hh + 4 kt + krow (whose swizzle is kswz(krow)),
  // chunk 4 s + q4
  int koff[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) koff[s] = krow * (2 * DH) + (((4 * s + q4) ^ kswz(krow)) * 16);
  // V^T copies: lane l fills row 8 i + l / 8, slot l % 8, with the chunk the swizzle puts there
  const int vrow_in = lane >> 3;
  // V^T fragment reads: row 16 d + j16, chunk 4 kk + q4 at its swizzled position
  const int vkey = (j16 & 7) ^ (j16 >> 3);
  const int voff0 = j16 * 128 + ((q4) ^ vkey) * 16;
  const int voff1 = j16 * 128 + ((4 + q4) ^ vkey) * 16;

  // blocks in a rotated order (the online softmax does not depend on it): the
  // items that run at once then do not all stream the same offsets of their
  // chunks at the same time
  const int rot0 = a.rot > 0 && nblk > 0 ? (int)(((unsigned)pitem * (unsigned)a.rot) % (unsigned)nblk) : 0;
  auto rot_blk = [&](int b) { const int x = b + rot0; return x >= nblk ? x - nblk : x; };
  auto issue = [&](int b) {
    const int blk = kbeg + 64 * rot_blk(b);
    const int64_t page = paged ? (int64_t)s_page[blk / a.cache.page_rows - pg0] : (int64_t)r;
    const int slot = blk % a.cache.page_rows;
    const bf16* kb = kpool + k_offset(a.cache, page, g, slot);
    const bf16* vb = vpool + v_offset(a.cache, page, g, slot);
    unsigned char* sb = ring + (b % NST) * STAGE;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int idx = wave * PER_WAVE + i;
      const bf16* src;
      if (idx < KSLABS) {
        const int key = idx * (64 / CK) + kkey_in;
        src = kb + (int64_t)key * DH + 8 * (kslot ^ kswz(key));
      } else {
        const int R = 8 * (idx - KSLABS) + vrow_in;
        const int c = (lane & 7) ^ (R & 7) ^ ((R >> 3) & 1);
        src = vb + R * kVTile + 8 * c;
      }
      lds_copy16(src, sb + idx * 1024);
    }
  };

  auto process = [&](int b) {
    const unsigned char* sb = ring + (b % NST) * STAGE;
    const unsigned char* kbs = sb;
    const unsigned char* vbs = sb + KSLABS * 1024;
    const int blk = kbeg + 64 * rot_blk(b);
    // scores: lane (j16, q4) holds row j16's keys blk + 32 hh + 8 q4 .. +7 in sv[hh]
    f32x8 sv[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      V8 kv[2][DS];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int s = 0; s < DS; ++s)
          kv[kt][s] = *reinterpret_cast<const V8*>(kbs + (32 * hh + 4 * kt) * (2 * DH) + koff[s]);
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < DS; ++s)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sacc[kt] = mma32(kv[kt][s], qv[s], sacc[kt]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[hh][4 * kt + e] = sacc[kt][e] * a.scale_log2;
    }
    const bool all_vis = blk + 64 <= key_hi && (a.window <= 0 || blk >= vis_lo_max);
    if (!all_vis) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = blk + 32 * hh + 8 * q4 + e;
          sv[hh][e] = ((key >= vlo) & (key < key_hi)) ? sv[hh][e] : -INFINITY;
        }
    }
    float mx = sv[0][0];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sv[hh][e]);
    mx = max_xor32(max_xor16(mx));
    // the reference maximum moves only when the block maximum exceeds it by
    // more than 8 (log2 units): every p <= 256, O rescaled on those blocks only
    const bool need = mx > m_run + 8.f;
    const float m_new = need ? mx : m_run;
    const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    m_run = m_new;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    V8 pv[2];
    float ps = 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(sv[hh][e] - m_use);
        ps += p[e];
      }
      pv[hh] = cvt8<bf16>(p);
    }
    l_run = l_run * alpha + ps;
    if (__any(need)) {
#pragma unroll
      for (int d = 0; d < DT; ++d) o[d] *= alpha;
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      V8 vv[DT];
#pragma unroll
      for (int d = 0; d < DT; ++d) vv[d] = *reinterpret_cast<const V8*>(vbs + d * 2048 + (kk ? voff1 : voff0));
      // stale rows past the end of the cache may hold any bits: zero their V
      // entries so that p = 0 cannot meet an Inf or NaN (last block only)
      const int key0 = blk + 32 * kk + 8 * q4;
      if (key0 + 8 > key_hi) {
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (key0 + e >= key_hi) vv[d][e] = static_cast<bf16>(0.f);
      }
#pragma unroll
      for (int d = 0; d < DT; ++d) o[d] = mma32(vv[d], pv[kk], o[d]);
    }
  };

  // Up to AHEAD = NST - 1 blocks in flight beyond the one being processed.
  // Only INIT of them go out before the first block is waited for: when every
  // CU asks for all of its first AHEAD blocks at once, each one's first block
  // lands later; the ring deepens to AHEAD once computing has begun.
  constexpr int AHEAD = NST - 1;
  constexpr int INIT = NG == 1 ? (AHEAD < 2 ? AHEAD : 2) : AHEAD;
  int issued = 0;
  for (; issued < min(INIT, nblk); ++issued) issue(issued);
  // this wave's queries (rows past g*B as zeros), once its first copies have
  // landed: they went out first
  wait_vm_blocks<PER_WAVE>(max(0, issued - 1));
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    qv[s] = *reinterpret_cast<const V8*>(my_q + s * 1024 + 16 * lane);
    if (row >= valid_q) qv[s] = zero8<bf16>();
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the stage is refilled
  // Step i works on blocks NG i .. NG i + NG - 1 (group g on block NG i + g).
  // This wave's copies of them have landed when at most those of the blocks
  // issued after them remain; after the barrier every wave's have, and every
  // wave is done with the blocks of step i - 1, whose stages (and those
  // before) may be refilled with the blocks up to NG i + NST - 1.
  for (int i = 0; NG * i < nblk; ++i) {
    wait_vm_blocks<PER_WAVE>(issued - min(NG * (i + 1), nblk));
    asm volatile("s_barrier" ::: "memory");
    for (; issued < min(nblk, NG * i + NST); ++issued) issue(issued);
    if (NG * i + grp < nblk) process(NG * i + grp);
  }

  uint32_t pre = 0;   // a preloaded word of the partial (kept until the end)
  if constexpr (NG == 2) {
    // Group 1's state through LDS: lane l of tile t at [t][d][l] for O, then
    // m and l.  The last step works on blocks b0 = 2 ((nblk - 1) / 2) and
    // b0 + 1, in stages b0 % 4 and b0 % 4 + 1 (b0 is even); once past that
    // step's barrier every other block is done with, so the other two
    // stages are free.  Group 1 writes there as soon as it leaves the loop
    // (while group 0 may still be on its last block), and one barrier
    // hands the state to group 0.
    static_assert(NST == 4, "the exchange uses the two stages the last step leaves free");
    constexpr int XB = DT * 1024 + 512;
    static_assert(4 * XB <= 2 * STAGE, "the exchange fits two stages");
    const int b0 = 2 * ((nblk - 1) / 2);
    unsigned char* xb = ring + ((b0 & 3) == 0 ? 2 * STAGE : 0) + qt * XB;
    if (MERGE != 0 && grp == 1) pre = attn_partial_preload(a.part_o, a.part_ml, pitem, a.qrows, DH, tid - 256);
    if (grp == 1) {
#pragma unroll
      for (int d = 0; d < DT; ++d) *reinterpret_cast<f32x4*>(xb + d * 1024 + 16 * lane) = o[d];
      reinterpret_cast<float*>(xb + DT * 1024)[lane] = m_run;
      reinterpret_cast<float*>(xb + DT * 1024 + 256)[lane] = l_run;
    }
    __syncthreads();
    if (grp == 0) {
      // exact merge of two online-softmax states with reference maxima m0, m1
      const float m1 = reinterpret_cast<const float*>(xb + DT * 1024)[lane];
      const float l1 = reinterpret_cast<const float*>(xb + DT * 1024 + 256)[lane];
      const float m = fmaxf(m_run, m1);
      const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
      for (int d = 0; d < DT; ++d)
        o[d] = o[d] * a0 + *reinterpret_cast<const f32x4*>(xb + d * 1024 + 16 * lane) * a1;
      l_run = l_run * a0 + l1 * a1;
      m_run = m;
    }
  }

  if (grp == 0) {
    bf16* po = static_cast<bf16*>(a.part_o) + (int64_t)pitem * a.qrows * DH;
#pragma unroll
    for (int d = 0; d < DT; ++d) store4(po + (int64_t)row * DH + 16 * d + 4 * q4, o[d]);
    const float l = sum_xor32(sum_xor16(l_run));
    if (q4 == 0) {
      float* pml = a.part_ml + (int64_t)pitem * 2 * a.qrows;
      pml[row] = m_run;
      pml[a.qrows + row] = l;
    }
  }

  if constexpr (MERGE != 0) {
    // every partial store of the workgroup has reached L2, then wave 0
    // arrives for the workgroup and waits for the head's other items
    __shared__ int s_status;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int nch = a.seq0[3];
    if (tid < 64) {
      const int st = attn_head_arrive(a.sync + kAttnSyncStride * g, nch, chunk, lane, a.spin_limit);
      if (tid == 0) s_status = st;
    }
    __syncthreads();
    const int status = s_status;
    if (status == 2 && tid == 0) atomicAdd(&g_attn_sync_timeouts, 1u);
    // rows chunk, chunk + nch, ... of the head, one per wave
    const int valid = a.group * a.B;
    for (int qr = chunk + wave * nch; qr < valid; qr += 4 * NG * nch) {
      float2 ov = merge_partials_row(static_cast<const bf16*>(a.part_o), a.part_ml, (int64_t)g * nch, nch, a.qrows,
                                     qr, DH, lane);
      if (status == 2) ov = float2{__builtin_nanf(""), __builtin_nanf("")};
      store_merged_row(static_cast<bf16*>(a.attn), ov, 0, g, qr, a.B, a.group, a.n_kv, DH, lane);
    }
  }
  asm volatile("" ::"v"(pre));
}

template <typename T>
static hipError_t launch_attn_t(const AttnArgs& a, int items, hipStream_t s) {
  const int nqt = (a.qrows + 15) / 16;
#define DFLASH_ATTN_CASE(DH_, NQT_, NQW_, QS_)                                                     \
  if (a.d_h == DH_ && nqt == NQT_) {                                                               \
    launch((attn_split_kernel<T, DH_, NQW_, QS_>), dim3(items), dim3(256), 0, s, a);    \
    return hipGetLastError();                                                                      \
  }
  if constexpr (sizeof(T) == 2) {
    // bf16, four query tiles: the shared ring of 64-key blocks.  Plans of one
    // workgroup per CU (ring depth 3 and more) at d_h 128 take two groups of
    // four waves on alternate blocks with four stages (8K decode cache: 13.5
    // us against 14.2 us for one group of four); plans of several workgroups
    // per CU two stages and one group.
    if (nqt == 4) {
      if (a.d_h == 128 && a.nst >= 3 && a.sync != nullptr && a.merge_spread) {
        launch((attn_ring64_kernel<128, 4, 2, 2>), dim3(items), dim3(512), 0, s, a);
      } else if (a.d_h == 128 && a.nst >= 3 && a.sync != nullptr) {
        launch((attn_ring64_kernel<128, 4, 2, 1>), dim3(items), dim3(512), 0, s, a);
      } else if (a.d_h == 128 && a.nst >= 3) {
        launch((attn_ring64_kernel<128, 4, 2>), dim3(items), dim3(512), 0, s, a);
      } else if (a.d_h == 128) {
        launch((attn_ring64_kernel<128, 2>), dim3(items), dim3(256), 0, s, a);
      } else {
        launch((attn_ring64_kernel<64, 4>), dim3(items), dim3(256), 0, s, a);
      }
      return hipGetLastError();
    }
#define DFLASH_ATTN_LDS_CASE(DH_, NQT_)                                                          \
  if (a.d_h == DH_ && nqt == NQT_) {                                                             \
    launch((attn_lds_kernel<DH_, NQT_>), dim3(items), dim3(256), 0, s, a);           \
    return hipGetLastError();                                                                    \
  }
    DFLASH_ATTN_LDS_CASE(64, 1) DFLASH_ATTN_LDS_CASE(64, 2) DFLASH_ATTN_LDS_CASE(64, 3)
    DFLASH_ATTN_LDS_CASE(128, 1) DFLASH_ATTN_LDS_CASE(128, 2) DFLASH_ATTN_LDS_CASE(128, 3)
#undef DFLASH_ATTN_LDS_CASE
  } else {
    DFLASH_ATTN_CASE(64, 1, 1, 1) DFLASH_ATTN_CASE(64, 2, 2, 1) DFLASH_ATTN_CASE(64, 3, 3, 1)
    DFLASH_ATTN_CASE(64, 4, 2, 2)
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
// The combine launch: one workgroup of one wave per query row (several per
// CU, so that every CU streams a share of the partials).

template <typename T>
__global__ __launch_bounds__(64) void attn_combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x;
  const int per_seq = a.n_kv * a.group * a.B;
  if (row >= a.R * per_seq) return;
  const int r = row / per_seq;
  const int rem = row - r * per_seq;
  const int g = rem / (a.group * a.B);
  const int qrow = rem - g * a.group * a.B;
  const int n = a.chunks[r];
  const int64_t it0 = a.item_base[r] + (int64_t)g * n;
  const float2 o = merge_partials_row(static_cast<const T*>(a.part_o), a.part_ml, it0, n, a.qrows, qrow, a.d_h,
                                      lane);
  // device-driven rounds: the round's rows are now part of every sequence
  if (a.d_len != nullptr && row == 0)
    for (int q = lane; q < a.R; q += 64) a.d_len[q] += dev_rows_of(a.d_rows, q, a.n_max) + a.B;
  store_merged_row(static_cast<T*>(a.attn), o, r, g, qrow, a.B, a.group, a.n_kv, a.d_h, lane);
}

hipError_t launch_attn_combine(int dtype, const CombineArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.R * a.n_kv * a.group * a.B;
  if (rows == 0) return hipSuccess;
  if (dtype == 1)
    launch(attn_combine_kernel<bf16>, dim3((unsigned)rows), dim3(64), 0, s, a);
  else
    launch(attn_combine_kernel<float>, dim3((unsigned)rows), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
