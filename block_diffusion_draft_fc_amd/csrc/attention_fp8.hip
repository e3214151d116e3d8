// Non-causal GQA block attention over an fp8 (OCP E4M3) draft KV cache: the
// split-context attention of attention.hip with one byte per cached element
// ("KV Cache + Speculative Decoding 面试 Cheat Sheet" 2.1 and 4.5), which halves
// the bytes of the bandwidth-bound step.
//
// What it computes is unchanged ("DFlash KV Injection Walkthrough" Step 4.4;
// "DFlash源码导读二 Qwen3DFlashAttention注意力实现全解析", the non-causal key
// design and sections 1 and 5): every query row of the block attends to every
// cached key with scale d_h^-0.5 (sliding layers hide pos_q - pos_k >= window),
// with keys and values read as their E4M3 values times the cache's scales.
// The key scale is folded into the softmax scale by the host, the value scale
// multiplies the partial outputs here.  Queries stay bf16.
//
// Layout of the work on gfx950 (one workgroup of four waves per (sequence,
// K/V head, key chunk), 64-key blocks through a ring of LDS stages filled by
// direct copies, as in the bf16 ring kernel):
//  * Every E4M3 value is a bf16 value, so the fp8 bytes are widened to bf16
//    exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1) as they leave LDS and
//    feed the same bf16 16x16x32 matrix steps; no precision is lost beyond
//    the storage itself.
//  * The head-dim order inside the QK contraction is free (any permutation
//    applied to both operands): lane group q4 takes head dims
//    q4 * d_h/4 .. q4 * d_h/4 + d_h/4 - 1 over the d_h/32 steps, so a lane's
//    share of a key row is one or two 16-byte LDS reads.  The queries are
//    loaded in that order too.
//  * Likewise the key order: A-operand row i of 16-key tile (hh, kt) is key
//    16 (i / 4) + 8 hh + 4 kt + i % 4.  After the S^T products lane group q4
//    then holds keys 16 q4 .. 16 q4 + 15 of its query row, the B operand of
//    both 32-key steps of O^T = V^T P^T, and the V^T operand of those two
//    steps is one 16-byte read of a V^T row.
//  * LDS stage: K as 64 key rows of d_h bytes, 16-byte chunk c of key j at
//    c ^ hk(j); V^T as d_h rows of 64 bytes, chunk c of row R at
//    c ^ ((R / 4) % 4).  Each operand read (16 lanes, 16 bytes each) then
//    covers all 256 bytes of the banks.

#include "attn_merge.hpp"

namespace dflash {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Sixteen E4M3 bytes (byte e of the vector = element e) as two runs of eight
// bf16 values, elements 0..7 and 8..15.
__device__ __forceinline__ void widen16(u32x4 w, bf16x8& lo, bf16x8& hi) {
  bf16x2 p[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
    p[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
  }
  lo = bf16x8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  hi = bf16x8{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}

// the first `n` bytes of w kept, the rest cleared (0 <= n <= 16)
__device__ __forceinline__ u32x4 keep_bytes(u32x4 w, int n) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = min(max(n - 4 * i, 0), 4);
    w[i] &= k >= 4 ? 0xffffffffu : ((1u << (8 * k)) - 1u);
  }
  return w;
}

}  // namespace

// NG = 2: two groups of four waves on alternate blocks with an exact merge of
// their states at the end, as in the bf16 ring kernel; group 0 copies the
// queries (the last stage holds one copy per tile) and group 1 reads them
// after a barrier.  The two-stage one-group form runs four workgroups per CU
// (32 KB of LDS each): at most 128 VGPRs, i.e. four waves per SIMD.
// Workgroups of this file's kernels whose in-launch merge wait timed out.
__device__ uint32_t g_attn_fp8_sync_timeouts = 0;

hipError_t attn_fp8_sync_timeouts(uint32_t* count) {
  return hipMemcpyFromSymbol(count, HIP_SYMBOL(g_attn_fp8_sync_timeouts), sizeof(uint32_t), 0,
                             hipMemcpyDeviceToHost);
}

// MERGE: as in the bf16 ring kernel (0: partials for the combine launch; 1:
// the split merged in the launch, item x on K/V head x % n_kv; 2: the
// diagnostic order with a head's items on consecutive workgroups).
template <int DH, int NST, int NG = 1, int MERGE = 0>
__global__ __launch_bounds__(256 * NG, (NG == 1 && NST == 2) ? 4 : 1) void attn_ring64_fp8_kernel(AttnArgs a) {
  using V8 = bf16x8;
  static_assert(DH == 64 || DH == 128, "layouts defined for d_h 64 and 128");
  static_assert(NST >= 2 && NST <= 7, "blocks in flight are counted by wait_vm_blocks (up to 6 after the current)");
  static_assert((NG == 1 || NG == 2) && NST >= 2 * NG, "a step's blocks are issued by the end of the step before");
  constexpr int DS = DH / 32;          // K=32 steps over the head dim
  constexpr int DT = DH / 16;          // 16-dim tiles of the output
  constexpr int KCH = DH / 16;         // 16-byte chunks per key row
  constexpr int KSLABS = DH / 16;      // 1 KB copies of the block's K (64 rows of DH bytes)
  constexpr int VSLABS = DH / 16;      // 1 KB copies of its V^T (DH rows of 64 bytes)
  constexpr int COPIES = KSLABS + VSLABS;
  constexpr int PER_WAVE = COPIES / (4 * NG);
  static_assert(PER_WAVE * 4 * NG == COPIES, "copies split evenly over the waves");
  constexpr int STAGE = COPIES * 1024;
  constexpr int QSPAN = DH / 4;        // head dims of a lane group in the QK contraction
  static_assert(MERGE == 0 || NG == 2, "the in-launch merge runs on the one-workgroup-per-CU plans");
  __shared__ __align__(16) unsigned char ring[NST * STAGE];
  __shared__ int32_t s_page[kAttnMaxChunkPages];

  const int item = blockIdx.x;
  int r = 0, g, chunk;
  int key_lo, key_hi, qpos0;
  if constexpr (MERGE != 0) {
    // one sequence of a host-driven round, every argument of the start at a
    // fixed offset and read in one batch (as in the bf16 ring kernel)
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
  // query rows of this wave: 16 wave .. 16 wave + 15; the workspace holds
  // qrows (a multiple of 16) rows per (sequence, K/V head), so a wave past
  // them loads and stores nothing
  const bool wave_rows = 16 * qt < a.qrows;

  const int row = 16 * qt + j16;
  const bf16* qbase = static_cast<const bf16*>(a.q_ws) + (int64_t)(r * a.n_kv + g) * a.qrows * DH;
  const int vlo = a.window > 0 ? qpos0 + row % a.B - a.window + 1 : INT_MIN;
  const int vis_lo_max = qpos0 + a.B - a.window;
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
  // Queries: direct copies into the last stage ahead of the first blocks'
  // (as in the bf16 ring kernel); step s of lane (j16, q4) holds head dims
  // QSPAN q4 + 8 s .. + 7 of row 16 wave + j16, at 16 * lane of slab s.
  static_assert(4 * DS * 1024 <= STAGE, "the queries fit one stage");
  unsigned char* my_q = ring + (NST - 1) * STAGE + qt * DS * 1024;
  if (wave_rows && grp == 0) {
#pragma unroll
    for (int s = 0; s < DS; ++s) lds_copy16(qbase + (int64_t)row * DH + QSPAN * q4 + 8 * s, my_q + s * 1024);
  }
  V8 qv[DS];

  const unsigned char* kpool = static_cast<const unsigned char*>(a.cache.k_pool);
  const unsigned char* vpool = static_cast<const unsigned char*>(a.cache.v_pool);
  // chunk swizzle of key row j: distinct over the 16 keys of an operand read
  // together with the key's offset in the 256 bytes of the banks (key bits
  // 0, 1, 4, 5 vary in a read; 128-byte rows take bit 0 from the offset,
  // 64-byte rows bits 0 and 1)
  auto hk = [](int j) { return DH == 128 ? ((j >> 1) & 1) | ((j >> 3) & 6) : (j >> 4) & 3; };
  const int krow = 16 * (j16 >> 2) + (j16 & 3);   // + 8 hh + 4 kt: key of A-operand row j16
  int koff[DS / 2 > 0 ? DS / 2 : 1];
  if constexpr (DH == 128) {
#pragma unroll
    for (int t = 0; t < 2; ++t) koff[t] = krow * DH + (((2 * q4 + t) ^ hk(krow)) * 16);
  } else {
    koff[0] = krow * DH + ((q4 ^ hk(krow)) * 16);
  }
  // V^T operand: row 16 d + j16, chunk q4 (keys 16 q4 .. 16 q4 + 15)
  const int voff = j16 * 64 + ((q4 ^ ((j16 >> 2) & 3)) * 16);
  // copies: K slab i, lane l -> key i * (64 / KCH) + l / KCH, slot l % KCH;
  // V^T slab i, lane l -> row 16 i + l / 4, slot l % 4
  const int kkey_in = lane / KCH, kslot = lane % KCH;
  const int vrow_in = lane >> 2, vslot = lane & 3;

  const int rot0 = a.rot > 0 && nblk > 0 ? (int)(((unsigned)pitem * (unsigned)a.rot) % (unsigned)nblk) : 0;
  auto rot_blk = [&](int b) { const int x = b + rot0; return x >= nblk ? x - nblk : x; };
  auto issue = [&](int b) {
    const int blk = kbeg + 64 * rot_blk(b);
    const int64_t page = paged ? (int64_t)s_page[blk / a.cache.page_rows - pg0] : (int64_t)r;
    const int slot = blk % a.cache.page_rows;
    const unsigned char* kb = kpool + k_offset(a.cache, page, g, slot);
    const unsigned char* vb = vpool + v_offset(a.cache, page, g, slot);
    unsigned char* sb = ring + (b % NST) * STAGE;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int idx = wave * PER_WAVE + i;
      const unsigned char* src;
      if (idx < KSLABS) {
        const int key = idx * (64 / KCH) + kkey_in;
        src = kb + key * DH + 16 * (kslot ^ hk(key));
      } else {
        const int R = 16 * (idx - KSLABS) + vrow_in;
        src = vb + R * kVTile + 16 * (vslot ^ ((R >> 2) & 3));
      }
      lds_copy16(src, sb + idx * 1024);
    }
  };

  auto process = [&](int b) {
    const unsigned char* sb = ring + (b % NST) * STAGE;
    const unsigned char* kbs = sb;
    const unsigned char* vbs = sb + KSLABS * 1024;
    const int blk = kbeg + 64 * rot_blk(b);
    // scores: lane (j16, q4) holds row j16's keys blk + 16 q4 + 8 hh .. + 7 in sv[hh]
    f32x8 sv[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      V8 kv[2][DS];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const unsigned char* kr = kbs + (8 * hh + 4 * kt) * DH;
        if constexpr (DH == 128) {
          widen16(*reinterpret_cast<const u32x4*>(kr + koff[0]), kv[kt][0], kv[kt][1]);
          widen16(*reinterpret_cast<const u32x4*>(kr + koff[1]), kv[kt][2], kv[kt][3]);
        } else {
          widen16(*reinterpret_cast<const u32x4*>(kr + koff[0]), kv[kt][0], kv[kt][1]);
        }
      }
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
          const int key = blk + 16 * q4 + 8 * hh + e;
          sv[hh][e] = ((key >= vlo) & (key < key_hi)) ? sv[hh][e] : -INFINITY;
        }
    }
    float mx = sv[0][0];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sv[hh][e]);
    mx = max_xor32(max_xor16(mx));
    // lazy maximum, as in the bf16 kernels: moved only when the block's
    // exceeds it by more than 8 (log2 units), so every p <= 256
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
    // stale rows past the end of the cache may hold any bytes (NaN codes
    // included): clear them so that p = 0 cannot meet a NaN (last block only)
    const int key0 = blk + 16 * q4;
    const bool stale = key0 + 16 > key_hi;
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      u32x4 w = *reinterpret_cast<const u32x4*>(vbs + d * 1024 + voff);
      if (stale) w = keep_bytes(w, min(max(key_hi - key0, 0), 16));
      V8 lo, hi;
      widen16(w, lo, hi);
      o[d] = mma32(lo, pv[0], o[d]);
      o[d] = mma32(hi, pv[1], o[d]);
    }
  };

  constexpr int AHEAD = NST - 1;
  constexpr int INIT = NG == 1 ? (AHEAD < 2 ? AHEAD : 2) : AHEAD;
  int issued = 0;
  for (; issued < min(INIT, nblk); ++issued) issue(issued);
  // group 0's query copies have landed once its first block has (they went
  // out first); with two groups a barrier shows that to group 1
  wait_vm_blocks<PER_WAVE>(max(0, issued - 1));
  if constexpr (NG == 2) asm volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    qv[s] = *reinterpret_cast<const V8*>(my_q + s * 1024 + 16 * lane);
    if (row >= valid_q) qv[s] = zero8<bf16>();
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the stage is refilled
  // step i: blocks NG i .. NG i + NG - 1 (group g on block NG i + g)
  for (int i = 0; NG * i < nblk; ++i) {
    wait_vm_blocks<PER_WAVE>(issued - min(NG * (i + 1), nblk));
    asm volatile("s_barrier" ::: "memory");
    for (; issued < min(nblk, NG * i + NST); ++issued) issue(issued);
    if (NG * i + grp < nblk) process(NG * i + grp);
  }

  uint32_t pre = 0;   // a preloaded word of the partial (kept until the end)
  if constexpr (NG == 2) {
    // group 1's (m, l, O) to group 0 through LDS, lane l of tile t at
    // [t][d][l] for O, then m and l; exact merge with reference maxima.
    // The last step works on blocks b0 = 2 ((nblk - 1) / 2) and b0 + 1, in
    // the stage pair (b0 % 6) / 2 (b0 is even); once past that step's
    // barrier the other two pairs are free.  Query tiles 0-1 use one of them
    // and 2-3 the other, so group 1 writes as soon as it leaves the loop
    // and one barrier hands the state to group 0.
    static_assert(NST == 6, "the exchange uses the two stage pairs the last step leaves free");
    constexpr int XB = DT * 1024 + 512;
    static_assert(2 * XB <= 2 * STAGE, "two query tiles fit a stage pair");
    const int busy = (2 * ((nblk - 1) / 2) % 6) / 2;
    const int pair = (busy + (qt < 2 ? 1 : 2)) % 3;
    unsigned char* xb = ring + pair * 2 * STAGE + (qt & 1) * XB;
    if (MERGE != 0 && grp == 1) pre = attn_partial_preload(a.part_o, a.part_ml, pitem, a.qrows, DH, tid - 256);
    if (grp == 1) {
#pragma unroll
      for (int d = 0; d < DT; ++d) *reinterpret_cast<f32x4*>(xb + d * 1024 + 16 * lane) = o[d];
      reinterpret_cast<float*>(xb + DT * 1024)[lane] = m_run;
      reinterpret_cast<float*>(xb + DT * 1024 + 256)[lane] = l_run;
    }
    __syncthreads();
    if (grp == 0) {
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

  if (wave_rows && grp == 0) {
    bf16* po = static_cast<bf16*>(a.part_o) + (int64_t)pitem * a.qrows * DH;
#pragma unroll
    for (int d = 0; d < DT; ++d) store4(po + (int64_t)row * DH + 16 * d + 4 * q4, o[d] * a.v_scale);
    float l = l_run;
    l = sum_xor32(sum_xor16(l));
    if (q4 == 0) {
      float* pml = a.part_ml + (int64_t)pitem * 2 * a.qrows;
      pml[row] = m_run;
      pml[a.qrows + row] = l;
    }
  }

  if constexpr (MERGE != 0) {
    // every partial store of the workgroup has reached L2, then wave 0
    // arrives for the workgroup and waits for the head's other items; then
    // rows chunk, chunk + nch, ... of the head, one per wave
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
    if (status == 2 && tid == 0) atomicAdd(&g_attn_fp8_sync_timeouts, 1u);
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

// Ring depth: the host plans for the bf16 kernel's depths (3 stages of 32 KB:
// one workgroup per CU; 2: several per CU).  fp8 stages are half as large:
// plan 2 takes 2 stages at d_h 128 (32 KB, four workgroups per CU, which the
// host fits its items to: 4 x 32K keys 67 us against 71 with three stages and
// three per CU) and 3 at d_h 64;
// plan 3 takes two wave groups with 6 stages (96 KB) at d_h 128 (8K decode
// cache: 12.3-12.6 us; 12.6-13.0 with 4 stages; one group of four waves
// 13.6-14.4) and one group with 4 stages (64 KB) at d_h 64.  With one group,
// deeper rings measured no faster on the 8K decode cache (5 to 7 stages:
// 13.5-15 us against 13.0-13.5) and slower on four 32K caches (they leave one
// workgroup per CU).
hipError_t launch_attn_fp8(const AttnArgs& a, int items, hipStream_t s) {
  if (items == 0) return hipSuccess;
  if ((a.qrows + 15) / 16 > 4) return hipErrorInvalidValue;
  if (a.nst >= 3) {
    if (a.d_h == 128 && a.sync != nullptr && a.merge_spread)
      launch((attn_ring64_fp8_kernel<128, 6, 2, 2>), dim3(items), dim3(512), 0, s, a);
    else if (a.d_h == 128 && a.sync != nullptr)
      launch((attn_ring64_fp8_kernel<128, 6, 2, 1>), dim3(items), dim3(512), 0, s, a);
    else if (a.d_h == 128) launch((attn_ring64_fp8_kernel<128, 6, 2>), dim3(items), dim3(512), 0, s, a);
    else launch((attn_ring64_fp8_kernel<64, 4>), dim3(items), dim3(256), 0, s, a);
  } else {
    if (a.d_h == 128) launch((attn_ring64_fp8_kernel<128, 2>), dim3(items), dim3(256), 0, s, a);
    else launch((attn_ring64_fp8_kernel<64, 3>), dim3(items), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dflash
