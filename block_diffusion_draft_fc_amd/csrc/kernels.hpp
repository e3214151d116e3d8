// Launch interface between the C-ABI host layer and the gfx950 kernels.
// Every struct here is passed by value as a kernel argument.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "dflash_common.hpp"

namespace dflash {

// Events that the kernel launches of the stage being enqueued attach to (set
// by the host timing layer, null when timing is off): the first launch takes
// `start`, every launch `stop`, so the pair spans the stage's kernels from the
// first one's start to the last one's end as the GPU executes them.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchEvents& launch_events();   // per host thread

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  LaunchEvents& ev = launch_events();
  if (ev.stop != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.start, ev.stop, 0u, args...);
    ev.start = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
  }
}

constexpr int kMaxSeqs = 64;

// ---------------------------------------------------------------- GEMM
// part[s][row_off + m][n] = sum over k in split s of A[m][k] * W[n][k], for the
// rows m of a virtual concatenation: m < m0 from x0, m0 <= m < m0 + m1 from x1
// (row stride K for both).  The partial buffer holds m_out rows per split.
struct GemmProb {
  const void* x0;
  const void* x1;
  const void* w;
  float* part;
  int32_t m0, m1;
  int32_t row_off, m_out;
  int32_t N, K;
  int32_t k_chunk;   // K per split, a multiple of 256 (one stage of 8 K-steps)
  int32_t splits;
  int32_t mt;        // 16-row tiles: ceil((m0 + m1) / 16)
  int32_t n_tiles;   // ceil(N / 64)
  int32_t blocks;    // n_tiles * splits
};
struct GemmArgs {
  GemmProb p[2];
  int32_t nprob;
};
// Rows handled by one weight-streaming problem.
constexpr int kSkinnyMaxM = 64;

// Tiled bf16 product for many rows: part[s][m][n] over the virtual rows
// [x0 (m0 rows); x1 (m1 rows)] (row stride K), 256x256 tiles, K and k_chunk
// multiples of 64.
struct TileProb {
  const bf16* x0;
  const bf16* x1;
  int32_t m0, m1;
  const bf16* w;     // [N][K]
  float* part;       // [splits][m0 + m1][N]
  int32_t N, K;
  int32_t k_chunk, splits, m_tiles, n_tiles;
};
// bn: output columns per tile, 256, 128 or 64 (n_tiles = ceil(N / bn)).
hipError_t launch_gemm_tile(const TileProb& p, int bn, hipStream_t s);
// Weight-streaming product for at most 64 rows (mt = ceil(M / 16) of 1 to 4):
// bf16, K a multiple of 64, N of 4, k_chunk == 512; the TileProb's n_tiles is
// ceil(N / (16 * gemm_stream_waves(mt))) and m_tiles is unused.
int gemm_stream_waves(int mt);
hipError_t launch_gemm_stream(const TileProb& p, int mt, hipStream_t s);

// Full-K product for at most 16 rows of the virtual concatenation [x0; x1]
// (bf16, K a multiple of 512, N of 4): exactly one of part (fp32 [M][N]) and
// out (bf16 [M][N], plus add when add is not null; out may alias add) is set.
struct FullkArgs {
  const bf16* x0;
  const bf16* x1;
  int32_t m0, m1;
  const bf16* w;     // [N][K]
  int32_t N, K;
  float* part;
  void* out;
  const void* add;
};
hipError_t launch_gemm_fullk(const FullkArgs& p, hipStream_t s);
// The same product with the (at most 16) activation rows resident in LDS and
// whole-K 16-column weight tiles streamed per wave, for very many columns:
// bf16, K a multiple of 64 and at most kResMaxK, N of 4; writes part (fp32
// [M][N]) only.
constexpr int kResMaxK = 4096;
hipError_t launch_gemm_resident(const FullkArgs& p, hipStream_t s);

// LDS budget for the staged activation slice of one gemm_lds_kernel workgroup.
constexpr int kLdsGemmBytes = 64 * 1024;
hipError_t launch_gemm_lds(int dtype, const GemmArgs& a, int max_mt, size_t lds_bytes, hipStream_t s);
// bf16, 33..128 rows (mt of 3 to 8, the same for both problems), K and
// k_chunk multiples of 512: the activation slice staged by direct copies in
// lds_bytes (at most kSlabLdsBytes) of LDS.
constexpr int kSlabLdsBytes = 160 * 1024;
hipError_t launch_gemm_slab(const GemmArgs& a, size_t lds_bytes, hipStream_t s);
// bf16 only, at most 32 rows (mt <= 2); 256-column tiles (n_tiles = ceil(N/256)).
hipError_t launch_gemm_wide(const GemmProb& p, hipStream_t s);

// out[m][n] = sum_s part[s][m][n] (+ add[m][n] when add is not null), written
// as fp32 (out_dtype 0) or bf16 (1); add has the output dtype.
hipError_t launch_splitk_reduce(int out_dtype, const float* part, int splits, int64_t M,
                                int64_t N, const void* add, void* out, hipStream_t s);

// C[t] = u[t] / sqrt(mean(u[t]^2) + eps) * gamma with u[t] = sum_s part[s][t],
// one row of d per workgroup; d % 4 == 0 and d <= 16384.
hipError_t launch_reduce_rmsnorm(int dtype, const float* part, int splits, int64_t T, int64_t d,
                                 const void* gamma, float eps, void* out, hipStream_t s);

// ---------------------------------------------------------------- QKV epilogue
struct SeqTable {
  int32_t L[kMaxSeqs];       // cache length before the call
  int32_t n[kMaxSeqs];       // new context rows
  int32_t cu[kMaxSeqs + 1];  // context row offsets
};
// A device-driven round's new context rows of sequence r, clamped to the
// 0..n_max the host planned capacity, pages and the attention split for: a
// row count out of range then cannot move a read or write past those bounds.
__device__ __forceinline__ int dev_rows_of(const int32_t* d_rows, int r, int n_max) {
  return min(max(d_rows[r], 0), n_max);
}

struct QkvEpiArgs {
  // Split-K partials: Q of block row b (0 <= b < R*B), split s, column c at
  // part_q[s * q_split + b * q_row + c]; K/V of context row m < T (K columns
  // first, then V) at part_kv[s * kv_split + m * kv_row + c], and of block
  // row b at part_kvh[s * kvh_split + b * kvh_row + c] (skvh splits).
  const float* part_q;
  const float* part_kv;
  const float* part_kvh;
  int64_t q_row, q_split, kv_row, kv_split, kvh_row, kvh_split;
  int32_t sq, skv, skvh;
  const void* gamma_q;
  const void* gamma_k;
  void* q_ws;            // [R][n_kv][qrows][d_h]
  CacheView cache;
  int32_t R, B, T, n_h, n_kv, d_h, qrows;
  float eps;
  double inv_freq[64];   // RoPE w_i, i < d_h/2, computed in fp64 on the host
  SeqTable seq;
  int32_t cache_fp8;     // 1: K/V go to the cache as E4M3 bytes of x / k_scale, x / v_scale
  float k_scale, v_scale;
  // device-driven rounds (d_rows not null): sequence r's cache length is
  // d_len[r] and its new context rows d_rows[r] <= n_max, at rows
  // r * n_max .. of C (the context rows past d_rows[r] are skipped); seq is
  // then unused
  const int32_t* d_len;
  const int32_t* d_rows;
  int32_t n_max;
  // the arrival words of an in-launch attention merge (n_sync heads), zeroed
  // here so that the attention launch that follows starts from zero
  uint32_t* attn_sync;
  int32_t n_sync;
};
hipError_t launch_qkv_epilogue(int dtype, const QkvEpiArgs& a, hipStream_t s);

// ---------------------------------------------------------------- attention
// Pages one attention work item may span (its chunk is limited to
// (kAttnMaxChunkPages - 2) pages of keys by the host planner).
constexpr int kAttnMaxChunkPages = 64;

struct AttnArgs {
  const void* q_ws;      // [R][n_kv][qrows][d_h]
  CacheView cache;
  void* part_o;          // [items][qrows][d_h], unnormalised O in the layer's
                         // storage type (bf16 or fp32)
  float* part_ml;        // [items][2][qrows]
  int32_t R, B, n_kv, group, qrows, d_h;
  int32_t chunk_keys;    // keys per work item (multiple of 64)
  int32_t rot;           // block order rotation multiplier (0: in order)
  int32_t nst;           // ring stages of the bf16 64-key-block kernel (2..4; 0: by item count)
  int32_t window;
  float scale_log2;      // d_h^-0.5 * log2(e) (times the key scale of an fp8 cache)
  float v_scale;         // value scale of an fp8 cache (the fp8 kernel scales its partial O)
  // sequence 0's key_lo, key_hi, qpos0 and chunks beside the scalars above,
  // so that a one-sequence launch reads everything its start needs from one
  // span of the arguments
  int32_t seq0[4];
  int32_t item_base[kMaxSeqs + 1];  // items of sequence r: [item_base[r], item_base[r+1])
  int32_t chunks[kMaxSeqs];         // items per (sequence, K/V head)
  int32_t key_lo[kMaxSeqs];         // first key any query may see
  int32_t key_hi[kMaxSeqs];         // keys in the cache after the append
  int32_t qpos0[kMaxSeqs];          // position of block row 0
  // device-driven rounds (d_rows not null): the lengths and new rows of the
  // round are read from device memory and key_lo / key_hi / qpos0 follow
  // from them (the host planned the items for upper bounds: items past a
  // sequence's keys hold no key); row counts are clamped to 0..n_max
  const int32_t* d_len;
  const int32_t* d_rows;
  int32_t n_max;
  // In-launch merge (sync not null; one sequence, n_kv a multiple of 8, at
  // most one item per CU): item x takes K/V head x % n_kv, chunk x / n_kv, so
  // the items of a head share an XCD (workgroups are dealt to the XCDs in
  // turn); once all of a head's items have stored their partials they merge
  // its rows and write the normalised output to `attn` ([B][n_h*d_h]).
  // sync[kAttnSyncStride * g ..]: head g's arrival word (u64: a byte per XCD,
  // each arrival adding one to its XCD's byte), the fallback count (u32) and,
  // in the next 128-byte line, one arrival flag per item of the head, all
  // zeroed by the q/k/v epilogue before every launch.
  uint32_t* sync;
  void* attn;
  // a diagnostic item order for the in-launch merge: chunk x % chunks of head
  // x / chunks, which deals a head's items to several XCDs (the merge's
  // write-back path); 0 in every ordinary call
  int32_t merge_spread;
  // polls before a wait of the in-launch merge gives up (kAttnSpinLimit in
  // every ordinary call; dflash_attn_set_spin_limit lowers it for tests of the
  // time-out path)
  int32_t spin_limit;
};
constexpr int kAttnSpinLimit = 1 << 18;   // polls (each a memory round trip): ~0.3 s
constexpr int kAttnSyncStride = 64;   // u32 words between heads' arrival words (256 bytes)
constexpr int kAttnSyncWords = 4;     // a head's words 0..3: arrival word, fallback count
constexpr int kAttnSyncFlags = 32;    // a head's words 32..63: the items' arrival flags
constexpr int kAttnMergeMaxItems = kAttnSyncStride - kAttnSyncFlags;   // items of a head merged in the launch
// Workgroups whose wait for the other items of their head timed out since the
// library was loaded (their rows are written as NaN); 0 in every correct run.
hipError_t attn_sync_timeouts(uint32_t* count);
hipError_t attn_fp8_sync_timeouts(uint32_t* count);   // the fp8-cache kernels' count

// Key range and block position of sequence r for one launch.
__device__ __forceinline__ void attn_seq_keys(const AttnArgs& a, int r, int& lo, int& hi, int& q0) {
  if (a.d_rows != nullptr) {
    q0 = a.d_len[r] + dev_rows_of(a.d_rows, r, a.n_max);
    hi = q0 + a.B;
    lo = a.window > 0 ? max(0, q0 - a.window + 1) : 0;
  } else {
    q0 = a.qpos0[r];
    hi = a.key_hi[r];
    lo = a.key_lo[r];
  }
}
hipError_t launch_attn_split(int dtype, const AttnArgs& a, int items, hipStream_t s);
// bf16 queries over an fp8 (E4M3) cache, any d_h of 64 / 128 and up to four
// 16-row query tiles; a.nst as for the bf16 64-key-block kernel.
hipError_t launch_attn_fp8(const AttnArgs& a, int items, hipStream_t s);

struct CombineArgs {
  // device-driven rounds: after the merge, d_len[r] += d_rows[r] + B (the
  // round's rows are in the cache; d_rows clamped to 0..n_max); null otherwise
  int32_t* d_len;
  const int32_t* d_rows;
  int32_t n_max;
  const void* part_o;    // the storage type of the layer
  const float* part_ml;
  void* attn;            // [R*B][n_h*d_h]
  int32_t R, B, n_kv, group, qrows, d_h;
  int32_t item_base[kMaxSeqs + 1];
  int32_t chunks[kMaxSeqs];
};
hipError_t launch_attn_combine(int dtype, const CombineArgs& a, hipStream_t s);

// ---------------------------------------------------------------- draft head
// x[m] = RMSNorm(h[r*B + 1 + j]) * gamma for m = r*(B-1) + j (the last B-1
// rows of every request's block), in the storage type.
hipError_t launch_head_norm(int dtype, const void* h, int64_t rows, int B, int64_t d, const void* gamma,
                            float eps, void* x, hipStream_t s);
// Columns per argmax segment (one workgroup per segment and row).
constexpr int kHeadSeg = 8192;
// ids[m] = the first argmax over n of sum_s part[s][m][n] (vocab % 4 == 0);
// max_logit[m] its value (when not null).  seg_val / seg_idx: [M][ceil(vocab /
// kHeadSeg)] scratch.
// acc[r] = leading matches of draft [R][B-1] against post [R][B] (position j+1
// against the prediction from j); next_rows = acc + 1 and next_anchor =
// post[r][acc] when not null.
hipError_t launch_accept(const int32_t* draft, const int32_t* post, int64_t R, int B, int32_t* acc,
                         int32_t* next_rows, int32_t* next_anchor, hipStream_t s);
hipError_t launch_head_argmax(const float* part, int splits, int64_t M, int64_t vocab, float* seg_val,
                              int32_t* seg_idx, int32_t* ids, float* max_logit, hipStream_t s);

// ---------------------------------------------------------------- device-side cache lengths
// d_len[r] = max(0, d_len[r] + delta) for r < R; or, with set != 0,
// d_len[r] = value[r].
struct LenArgs {
  int32_t* d_len;
  int32_t R, delta, set;
  int32_t value[kMaxSeqs];
};
hipError_t launch_len_update(const LenArgs& a, hipStream_t s);

// ---------------------------------------------------------------- measurement
// Reads bytes / 16 16-byte words of src (nothing is written).
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_mfma_peak(int iters, int64_t workgroups, float* sink, hipStream_t s);

// ---------------------------------------------------------------- cache
struct AppendArgs {
  const void* k_rows;    // [n_rows][n_kv][d_h]
  const void* v_rows;
  CacheView cache;
  int32_t n_seqs;
  int32_t L[kMaxSeqs];
  int32_t cu[kMaxSeqs + 1];
};
hipError_t launch_cache_append(int dtype, const AppendArgs& a, int64_t n_rows, hipStream_t s);

constexpr int kBtBatch = 240;
struct BtUpdateArgs {
  int32_t* table;
  int32_t count;
  int32_t index[kBtBatch];
  int32_t value[kBtBatch];
};
hipError_t launch_bt_update(const BtUpdateArgs& a, hipStream_t s);

}  // namespace dflash
